"""GPU parity of the expert-indexed GEMV (qmv_id) against the oracle."""
import numpy as np
import pytest
import torch

import gen
import oracle
from block_quantized_matrix_amd import bqm
from tests._gpu import DEV, check_close, host, packed, say, weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _oracle():
    oracle.build(force=False)


def run_id(fmt, E, N, K, ids_np, X, xts, xss, key):
    T, top_k = ids_np.shape
    Wi = weights(fmt, E * N, K, key)
    Wp = packed(fmt, Wi, E * N, K)
    ids = torch.from_numpy(ids_np).to(DEV)
    Y = torch.full((T, top_k, N), -7.0, device=DEV)
    bqm.qmv_id(fmt, Wp, E, N, K, ids, T, top_k, X, xts, xss, Y)
    # the oracle rejects ids >= E (a contract violation); give it those slots as padding
    ids_ok = np.where(ids_np >= E, -1, ids_np).astype(np.int32)
    Yr, S = oracle.qmv_id(fmt, host(Wi), E, N, K, ids_ok, host(X).reshape(-1), xts, xss)
    return host(Y), Yr, S


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("slots", ["broadcast", "per_slot"])
@pytest.mark.parametrize("E,N,K", [(5, 37, 96), (3, 300, 1536), (9, 64, 4096)])
def test_qmv_id_small(fmt, slots, E, N, K):
    say("qmv_id small", fmt, slots, E, N, K)
    ids = np.array([[3, 0, 4], [-1, 4, 2], [1, 3, -1], [0, 2, 4]], np.int32) % max(E, 1)
    ids[1, 0] = -1
    ids[2, 2] = -1
    T, top_k = ids.shape
    if slots == "broadcast":
        X = gen.normal((T, K), ("id-x", K), device=DEV)
        xts, xss = K, 0
    else:
        X = gen.normal((T, top_k, K), ("id-x2", K), device=DEV)
        xts, xss = top_k * K, K
    y, Yr, S = run_id(fmt, E, N, K, ids, X, xts, xss, ("id", fmt, E, N, K))
    check_close(y, Yr, S, f"qmv_id {fmt} {slots}")
    assert np.all(y[1, 0] == 0) and np.all(y[2, 2] == 0)


def test_qmv_id_many_tokens_per_expert():
    """20 tokens all routed to experts 0 and 1: passes of 8, 8 and 4 slots per expert."""
    E, N, K, T = 4, 80, 512, 20
    ids = np.tile(np.array([[1, 0]], np.int32), (T, 1))
    X = gen.normal((T, K), ("many-x",), device=DEV)
    y, Yr, S = run_id("q4_0", E, N, K, ids, X, K, 0, ("many",))
    check_close(y, Yr, S, "many tokens per expert")


def test_qmv_id_out_of_range_ids_give_nan():
    E, N, K = 3, 40, 64
    ids = np.array([[0, 3], [7, -1]], np.int32)
    X = gen.normal((2, K), ("oor-x",), device=DEV)
    y, Yr, S = run_id("q4_0", E, N, K, ids, X, K, 0, ("oor",))
    assert np.all(np.isnan(y[0, 1])) and np.all(np.isnan(y[1, 0]))
    assert np.all(y[1, 1] == 0)
    check_close(y[0, 0], Yr[0, 0], S[0, 0], "valid slot next to bad ids")


@pytest.mark.parametrize("T", [1, 16])
@pytest.mark.parametrize("proj", ["gate", "down"])
def test_qmv_id_moe_layer(T, proj):
    """128 experts, top-8, hidden 4096, expert FFN 1536, Q4_0; ids from the skewed router;
    gate/up take one input per token (broadcast), down one input per (token, slot)."""
    sh = gen.MOE_SHAPE
    E, top_k = sh["E"], sh["top_k"]
    ids = gen.router_ids(T, E, top_k, ("moe-router", T))
    if proj == "gate":
        N, K = sh["ffn"], sh["hidden"]
        X = gen.normal((T, K), ("moe-x", T, proj), device=DEV)
        xts, xss = K, 0
    else:
        N, K = sh["hidden"], sh["ffn"]
        X = gen.normal((T, top_k, K), ("moe-x", T, proj), device=DEV)
        xts, xss = top_k * K, K
    say("qmv_id moe", T, proj, "unique experts", len(np.unique(ids)))
    y, Yr, S = run_id("q4_0", E, N, K, ids, X, xts, xss, ("moe", proj))
    check_close(y, Yr, S, f"moe T={T} {proj}")


def test_qmv_id_deterministic():
    E, N, K, T = 16, 256, 1024, 12
    ids = gen.router_ids(T, E, 4, ("det-router",))
    Wp = packed("q4_0", weights("q4_0", E * N, K, ("det-id",)), E * N, K)
    X = gen.normal((T, K), ("det-id-x",), device=DEV)
    idd = torch.from_numpy(ids).to(DEV)
    Y1 = torch.empty((T, 4, N), device=DEV)
    Y2 = torch.empty((T, 4, N), device=DEV)
    bqm.qmv_id("q4_0", Wp, E, N, K, idd, T, 4, X, K, 0, Y1)
    bqm.qmv_id("q4_0", Wp, E, N, K, idd, T, 4, X, K, 0, Y2)
    assert torch.equal(Y1, Y2)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("T", [2, 3, 5, 8])
def test_qmv_id_batch_classes(fmt, T):
    """T tokens run in the batch class of min(T, 4) (2, 4, 4, 4): groups of every size,
    some shorter than the class, with padding slots among them."""
    E, N, K, top_k = 6, 130, 1184, 3
    ids = gen.router_ids(T, E, top_k, ("cls-router", T))
    ids[0, 1] = -1
    X = gen.normal((T, top_k, K), ("cls-x", T, fmt), device=DEV)
    say("qmv_id classes", fmt, T)
    y, Yr, S = run_id(fmt, E, N, K, ids, X, top_k * K, K, ("cls", fmt, T))
    check_close(y, Yr, S, f"qmv_id {fmt} T={T}")
    assert np.all(y[0, 1] == 0)


@pytest.mark.parametrize("T,K", [(16, 16384), (4, 32768), (1, 32768)])
def test_qmv_id_long_k_is_chunked(T, K):
    """Inputs of a long K do not fit the LDS at once: each group is walked in chunks of K
    with per-row partial sums."""
    E, N, top_k = 8, 100, 4
    ids = gen.router_ids(T, E, top_k, ("long-router", T))
    X = gen.normal((T, top_k, K), ("long-x", T, K), device=DEV)
    say("qmv_id long K", T, K)
    y, Yr, S = run_id("q8_0", E, N, K, ids, X, top_k * K, K, ("long", T, K))
    check_close(y, Yr, S, f"qmv_id long K T={T}")


def test_qmv_id_maximum_slots_and_experts():
    """T = 64 tokens x top_k = 32 slots over E = 4096 experts (the limits), with padding and
    out-of-range ids mixed in: the grouping tables at their largest."""
    from block_quantized_matrix_amd import bqm as b
    E, N, K, T, top_k = b.QMV_ID_MAX_E, 8, 64, b.QMV_ID_MAX_T, b.QMV_ID_MAX_TOPK
    rng = np.random.default_rng(7)
    ids = rng.integers(0, 64, size=(T, top_k)).astype(np.int32) * 64  # crowd 64 experts
    ids[::3, 5] = rng.integers(0, E, size=ids[::3, 5].shape)
    ids[1::7, 2] = -1
    ids[2::9, 9] = E + 5
    X = gen.normal((T, K), ("max-x",), device=DEV)
    say("qmv_id max slots")
    y, Yr, S = run_id("q4_0", E, N, K, ids, X, K, 0, ("max",))
    bad = ids >= E
    assert np.all(np.isnan(y[bad]))
    check_close(y[~bad], Yr[~bad], S[~bad], "qmv_id max slots")


def test_qmv_id_empty_k_and_no_experts():
    """K = 0: every valid slot's sum is empty (zeros); E = 0: every id is out of range."""
    ids = torch.tensor([[0, -1], [2, 5]], dtype=torch.int32, device=DEV)
    W = torch.zeros(256, dtype=torch.uint8, device=DEV)
    X = torch.zeros(64, device=DEV)
    Y = torch.full((2, 2, 24), -7.0, device=DEV)
    bqm.qmv_id("q4_0", W, 3, 24, 0, ids, 2, 2, X, 0, 0, Y)
    y = host(Y)
    assert np.all(y[0, 0] == 0) and np.all(y[0, 1] == 0) and np.all(y[1, 0] == 0)
    assert np.all(np.isnan(y[1, 1]))
    Y.fill_(-7.0)
    bqm.qmv_id("q4_0", W, 0, 24, 32, ids, 2, 2, X, 0, 0, Y)
    y = host(Y)
    assert np.all(y[0, 1] == 0)
    assert np.all(np.isnan(y[0, 0])) and np.all(np.isnan(y[1]))


def test_qmv_id_groups_split_between_workgroups():
    """Experts with more slots than one group holds, and groups whose rows are split between
    workgroups: every workgroup must form the same groups (slot order within an expert's
    run is by slot index), or some rows of a slot are never computed."""
    E, N, K, T, top_k = 3, 2048, 256, 16, 2
    ids = np.stack([np.zeros(T, np.int32), (np.arange(T) % 2 + 1).astype(np.int32)], axis=1)
    X = gen.normal((T, K), ("split-x",), device=DEV)
    say("qmv_id groups split between workgroups")
    y, Yr, S = run_id("q4_0", E, N, K, ids, X, K, 0, ("split",))
    check_close(y, Yr, S, "groups split between workgroups")


# --- fused gate+up ------------------------------------------------------------------------

def run_gate_up(fmt, E, N, K, ids_np, X, xts, xss, key):
    T, top_k = ids_np.shape
    Wg = weights(fmt, E * N, K, key + ("g",), std=0.05)
    Wu = weights(fmt, E * N, K, key + ("u",), std=0.05)
    Gp, Up = packed(fmt, Wg, E * N, K), packed(fmt, Wu, E * N, K)
    ids = torch.from_numpy(ids_np).to(DEV)
    Y = torch.full((T, top_k, N), -7.0, device=DEV)
    bqm.qmv_id_gate_up(fmt, Gp, Up, E, N, K, ids, T, top_k, X, xts, xss, Y)
    ids_ok = np.where(ids_np >= E, -1, ids_np).astype(np.int32)
    Yr, S = oracle.qmv_id_gate_up(fmt, host(Wg), host(Wu), E, N, K, ids_ok, host(X).reshape(-1), xts, xss)
    return host(Y), Yr, S


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("T", [1, 2, 3, 5, 16])
def test_gate_up_batch_classes(fmt, T):
    """silu(gate) * up for every batch class (1, 2, 4, 8), groups of one expert split over
    workgroups, a padding slot and an out-of-range id."""
    E, N, K, top_k = 6, 300, 1184, 3
    ids = gen.router_ids(T, E, top_k, ("gu-router", T))
    ids[0, 1] = -1
    if T > 1:
        ids[1, 2] = E + 2
    X = gen.normal((T, K), ("gu-x", T, fmt), device=DEV)
    say("gate_up classes", fmt, T)
    y, Yr, S = run_gate_up(fmt, E, N, K, ids, X, K, 0, ("gu", fmt, T))
    bad = ids >= E
    assert np.all(np.isnan(y[bad]))
    assert np.all(y[0, 1] == 0)
    check_close(y[~bad], Yr[~bad], S[~bad], f"gate_up {fmt} T={T}")


def test_gate_up_maximum_slots_and_experts():
    """The gate+up form at the limits: T = 64 tokens x top_k = 32 slots over E = 4096
    experts, crowded onto 64 of them, with padding and out-of-range ids mixed in."""
    from block_quantized_matrix_amd import bqm as b
    E, N, K, T, top_k = b.QMV_ID_MAX_E, 8, 64, b.QMV_ID_MAX_T, b.QMV_ID_MAX_TOPK
    rng = np.random.default_rng(17)
    ids = rng.integers(0, 64, size=(T, top_k)).astype(np.int32) * 64
    ids[::3, 5] = rng.integers(0, E, size=ids[::3, 5].shape)
    ids[1::7, 2] = -1
    ids[2::9, 9] = E + 5
    X = gen.normal((T, K), ("gu-max-x",), device=DEV)
    say("gate_up max slots")
    y, Yr, S = run_gate_up("q4_0", E, N, K, ids, X, K, 0, ("gu-max",))
    bad = ids >= E
    assert np.all(np.isnan(y[bad]))
    assert np.all(y[ids < 0] == 0)
    check_close(y[~bad], Yr[~bad], S[~bad], "gate_up max slots")


@pytest.mark.parametrize("T,K", [(16, 16384), (1, 32768)])
def test_gate_up_long_k_is_chunked(T, K):
    """Chunked K: each output row keeps two partial sums (gate and up) across the chunks."""
    E, N, top_k = 8, 100, 4
    ids = gen.router_ids(T, E, top_k, ("gu-long-router", T))
    X = gen.normal((T, top_k, K), ("gu-long-x", T, K), device=DEV)
    say("gate_up long K", T, K)
    y, Yr, S = run_gate_up("q8_0", E, N, K, ids, X, top_k * K, K, ("gu-long", T, K))
    check_close(y, Yr, S, f"gate_up long K T={T}")


@pytest.mark.parametrize("T", [1, 16])
def test_gate_up_moe_layer(T):
    """The MoE layer's gate/up shapes (1536 x 4096 per expert, 128 experts, top-8)."""
    sh = gen.MOE_SHAPE
    E, top_k, N, K = sh["E"], sh["top_k"], sh["ffn"], sh["hidden"]
    ids = gen.router_ids(T, E, top_k, ("moe-router", T))
    X = gen.normal((T, K), ("gu-moe-x", T), device=DEV)
    say("gate_up moe", T)
    y, Yr, S = run_gate_up("q4_0", E, N, K, ids, X, K, 0, ("gu-moe",))
    check_close(y, Yr, S, f"gate_up moe T={T}")


def test_gate_up_empty_k_and_matches_separate_calls():
    """K = 0 gives zeros for valid slots; with K > 0 the fused result equals silu of one
    qmv_id call times the other's, to the tolerance of the fused bound."""
    ids = torch.tensor([[0, -1], [2, 5]], dtype=torch.int32, device=DEV)
    W = torch.zeros(256, dtype=torch.uint8, device=DEV)
    X = torch.zeros(64, device=DEV)
    Y = torch.full((2, 2, 24), -7.0, device=DEV)
    bqm.qmv_id_gate_up("q4_0", W, W, 3, 24, 0, ids, 2, 2, X, 0, 0, Y)
    y = host(Y)
    assert np.all(y[0] == 0) and np.all(y[1, 0] == 0) and np.all(np.isnan(y[1, 1]))
    E, N, K, T, top_k = 5, 200, 2048, 4, 2
    idn = gen.router_ids(T, E, top_k, ("gu-sep",))
    Wg, Wu = weights("q4_0", E * N, K, ("gu-sep", "g")), weights("q4_0", E * N, K, ("gu-sep", "u"))
    Gp, Up = packed("q4_0", Wg, E * N, K), packed("q4_0", Wu, E * N, K)
    X = gen.normal((T, K), ("gu-sep-x",), device=DEV)
    idd = torch.from_numpy(idn).to(DEV)
    Yf = torch.empty((T, top_k, N), device=DEV)
    Yg = torch.empty((T, top_k, N), device=DEV)
    Yu = torch.empty((T, top_k, N), device=DEV)
    bqm.qmv_id_gate_up("q4_0", Gp, Up, E, N, K, idd, T, top_k, X, K, 0, Yf)
    bqm.qmv_id("q4_0", Gp, E, N, K, idd, T, top_k, X, K, 0, Yg)
    bqm.qmv_id("q4_0", Up, E, N, K, idd, T, top_k, X, K, 0, Yu)
    Yr, S = oracle.qmv_id_gate_up("q4_0", host(Wg), host(Wu), E, N, K, idn, host(X).reshape(-1), K, 0)
    sep = host(torch.nn.functional.silu(Yg) * Yu).astype(np.float64)
    check_close(host(Yf), sep, S, "fused vs separate")
    check_close(host(Yf), Yr, S, "fused vs oracle")


# --- router-weighted sum over each token's slots -------------------------------------------

def run_sum(fmt, E, N, K, ids_np, X, xts, xss, key, w_np=None):
    T, top_k = ids_np.shape
    Wi = weights(fmt, E * N, K, key)
    Wp = packed(fmt, Wi, E * N, K)
    if w_np is None:
        w_np = gen.router_weights(T, top_k, key + ("w",))
    ids = torch.from_numpy(ids_np).to(DEV)
    w = torch.from_numpy(w_np).to(DEV)
    Ys = torch.full((T, top_k, N), -7.0, device=DEV)
    Y = torch.full((T, N), -7.0, device=DEV)
    bqm.qmv_id_sum(fmt, Wp, E, N, K, ids, w, T, top_k, X, xts, xss, Ys, Y)
    ids_ok = np.where(ids_np >= E, -1, ids_np).astype(np.int32)
    Yr, S = oracle.qmv_id_sum(fmt, host(Wi), E, N, K, ids_ok, w_np, host(X).reshape(-1), xts, xss)
    Yid, Sid = oracle.qmv_id(fmt, host(Wi), E, N, K, ids_ok, host(X).reshape(-1), xts, xss)
    return host(Ys), host(Y), Yr, S, Yid, Sid, w_np


def slot_sum_fp32(ys, ids_np, E):
    """The weighted sum as the kernel defines it: fp32, slots in order, padding 0, bad NaN."""
    T, top_k, N = ys.shape
    out = np.zeros((T, N), np.float32)
    for t in range(T):
        acc = None
        for s in range(top_k):
            e = ids_np[t, s]
            v = np.full(N, np.nan, np.float32) if e >= E else (np.zeros(N, np.float32) if e < 0 else ys[t, s])
            acc = v.copy() if acc is None else (acc + v).astype(np.float32)
        out[t] = acc
    return out


def check_sum(ys, y, Yr, S, Yid, Sid, w_np, ids_np, E, what):
    T, top_k = ids_np.shape
    valid = (ids_np >= 0) & (ids_np < E)
    wb = w_np.astype(np.float64)[:, :, None]
    check_close(ys[valid], (wb * Yid)[valid], (np.abs(wb) * Sid)[valid], what + " slots")
    assert np.array_equal(y.view(np.uint32), slot_sum_fp32(ys, ids_np, E).view(np.uint32)), what
    ok = ~np.any(ids_np >= E, axis=1)
    check_close(y[ok], Yr[ok], S[ok], what)
    assert np.all(np.isnan(y[~ok]))


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("E,N,K", [(5, 37, 96), (3, 300, 1536), (9, 130, 4096)])
def test_qmv_id_sum_small(fmt, E, N, K):
    say("qmv_id_sum small", fmt, E, N, K)
    ids = np.array([[3, 0, 4], [-1, 4, 2], [1, 3, -1], [0, 0, 4]], np.int32) % max(E, 1)
    ids[1, 0] = -1
    ids[2, 2] = -1
    T, top_k = ids.shape
    X = gen.normal((T, top_k, K), ("sum-x", K), device=DEV)
    r = run_sum(fmt, E, N, K, ids, X, top_k * K, K, ("sum", fmt, E, N, K))
    check_sum(*r, ids, E, f"qmv_id_sum {fmt} {E}x{N}x{K}")


@pytest.mark.parametrize("T", [1, 16])
def test_qmv_id_sum_moe_down(T):
    """The MoE layer's down projection (4096 x 1536 per expert, 128 experts, top-8) with
    the router weights: the layer's output per token."""
    sh = gen.MOE_SHAPE
    E, top_k, N, K = sh["E"], sh["top_k"], sh["hidden"], sh["ffn"]
    ids = gen.router_ids(T, E, top_k, ("moe-router", T))
    X = gen.normal((T, top_k, K), ("sum-moe-x", T), device=DEV)
    say("qmv_id_sum moe down", T)
    r = run_sum("q4_0", E, N, K, ids, X, top_k * K, K, ("sum-moe",))
    check_sum(*r, ids, E, f"moe down sum T={T}")


def test_qmv_id_sum_bad_ids_empty_k_and_no_slots():
    """An id >= E makes its token's sum NaN; K = 0 gives 0 for tokens with valid slots;
    top_k = 0 gives 0 everywhere."""
    E, N, K = 3, 70, 64
    ids = np.array([[0, 3], [2, -1], [-1, -1]], np.int32)
    X = gen.normal((3, 2, K), ("sum-bad-x",), device=DEV)
    r = run_sum("q4_0", E, N, K, ids, X, 2 * K, K, ("sum-bad",))
    check_sum(*r, ids, E, "bad ids")
    y = r[1]
    assert np.all(np.isnan(y[0])) and np.all(y[2] == 0)
    idd = torch.from_numpy(ids).to(DEV)
    w = torch.ones((3, 2), device=DEV)
    W = torch.zeros(256, dtype=torch.uint8, device=DEV)
    Ys = torch.full((3, 2, N), -7.0, device=DEV)
    Y = torch.full((3, N), -7.0, device=DEV)
    bqm.qmv_id_sum("q4_0", W, E, N, 0, idd, w, 3, 2, X, 0, 0, Ys, Y)
    y = host(Y)
    assert np.all(np.isnan(y[0])) and np.all(y[1] == 0) and np.all(y[2] == 0)
    Y.fill_(-7.0)
    bqm.qmv_id_sum("q4_0", W, E, N, 64, idd, w, 3, 0, X, 0, 0, Ys, Y)
    assert torch.count_nonzero(Y).item() == 0


def test_qmv_id_sum_maximum_slots_and_repeat():
    """T = 64 tokens x top_k = 32 over crowded experts (the slot limits), with padding; two
    calls in a row give bit-identical outputs."""
    E, N, K, T, top_k = 256, 200, 128, bqm.QMV_ID_MAX_T, bqm.QMV_ID_MAX_TOPK
    rng = np.random.default_rng(11)
    ids = (rng.integers(0, 16, size=(T, top_k)) * 16).astype(np.int32)
    ids[1::7, 2] = -1
    X = gen.normal((T, top_k, K), ("sum-max-x",), device=DEV)
    say("qmv_id_sum max slots")
    r1 = run_sum("q4_0", E, N, K, ids, X, top_k * K, K, ("sum-max",))
    check_sum(*r1, ids, E, "max slots")
    r2 = run_sum("q4_0", E, N, K, ids, X, top_k * K, K, ("sum-max",))
    assert np.array_equal(r1[1].view(np.uint32), r2[1].view(np.uint32))


def test_qmv_id_sum_matches_weighted_qmv_id():
    """The fused sum equals the fp32 slot sum of qmv_id's rows times the weights, to the
    tolerance, for a ragged N (not a multiple of 64) and long K (chunked)."""
    E, N, K, T, top_k = 6, 1000, 16384, 3, 4
    ids = gen.router_ids(T, E, top_k, ("sum-vs",))
    X = gen.normal((T, top_k, K), ("sum-vs-x",), device=DEV)
    say("qmv_id_sum vs qmv_id")
    r = run_sum("q8_0", E, N, K, ids, X, top_k * K, K, ("sum-vs",))
    check_sum(*r, ids, E, "vs qmv_id")


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("T", [1, 2, 5])  # batch classes 1, 2 and 4
def test_indexed_neutral_codes_give_exact_zeros(fmt, T):
    """Codes all equal to the format's offset give exactly zero for any scale and input, in
    the indexed form and (silu(0) * 0) the gate+up form."""
    E, N, K, top_k = 4, 40, 4096, 2
    bb = gen.block_bytes(fmt)
    Wn = weights(fmt, E * N, K, ("neutral", fmt)).reshape(E * N, K // 32, bb).clone()
    Wn[:, :, 2:] = 0x88 if fmt == "q4_0" else 0
    Wp = packed(fmt, Wn.reshape(E * N, -1), E * N, K)
    ids = torch.from_numpy(gen.router_ids(T, E, top_k, ("neutral-ids", T))).to(DEV)
    X = gen.normal((T, K), ("neutral-x", T), device=DEV)
    Y = torch.full((T, top_k, N), float("nan"), device=DEV)
    bqm.qmv_id(fmt, Wp, E, N, K, ids, T, top_k, X, K, 0, Y)
    assert torch.all(Y == 0)
    Y.fill_(float("nan"))
    bqm.qmv_id_gate_up(fmt, Wp, Wp, E, N, K, ids, T, top_k, X, K, 0, Y)
    assert torch.all(Y == 0)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("T", [1, 2, 3, 5, 16])  # batch classes 1, 2, 2, 4, 4
def test_qmv_id_sum_batch_classes(fmt, T):
    """The router-weighted form at every batch class the indexed GEMV picks, with a padding
    slot and (T > 1) an out-of-range id: weighted slot rows against the oracle, the sums bit
    for bit against the slot rows added in slot order."""
    E, N, K, top_k = 6, 130, 1184, 3
    ids = gen.router_ids(T, E, top_k, ("sum-classes", T))
    ids[0, 1] = -1
    if T > 1:
        ids[1, 2] = E + 1
    X = gen.normal((T, top_k, K), ("sum-classes-x", T, fmt), device=DEV)
    say("qmv_id_sum classes", fmt, T)
    ys, y, Yr, S, Yid, Sid, w_np = run_sum(fmt, E, N, K, ids, X, top_k * K, K, ("sum-cl", fmt, T))
    check_sum(ys, y, Yr, S, Yid, Sid, w_np, ids, E, f"qmv_id_sum classes {fmt} T={T}")
