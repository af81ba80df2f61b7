"""GPU parity of the activation quantizer (bit exact) and the int8-MFMA prefill product."""
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


def quantize(X, M, K):
    Xq = torch.empty((M, K), dtype=torch.int8, device=DEV)
    dx = torch.empty((M, K // 32), dtype=torch.float32, device=DEV)
    bqm.bqm_quantize_q8_act(X, Xq, dx, M, K)
    return Xq, dx


@pytest.mark.parametrize("M,K", [(1, 32), (7, 96), (512, 5120)])
def test_quantize_q8_act_bitwise(M, K):
    say("quantize", M, K)
    X = gen.normal((M, K), ("qa", M, K), device=DEV)
    Xq, dx = quantize(X, M, K)
    Xq_r, dx_r = oracle.quantize_q8_act(host(X), K)
    assert np.array_equal(host(Xq), Xq_r)
    assert np.array_equal(host(dx).view(np.uint32), dx_r.view(np.uint32))


def test_quantize_q8_act_special_blocks():
    """Ties (x/dx exactly k + 1/2), zero blocks, subnormal blocks, the largest float below 1/2."""
    K = 256
    X = torch.zeros((4, K))
    X[0, :32] = torch.arange(-16, 16) * 0.5
    X[0, 31] = 127.0                                       # dx = 1: every half is a tie
    X[0, 32:38] = torch.tensor([127.0, 63.5, -0.5, 2.5, -2.5, 0.49999997])
    X[1, 64:96] = torch.arange(-16, 16) * 2.0 ** -149      # dx underflows to 0
    X[2, 96:128] = torch.arange(1, 33) * 2.0 ** -140       # subnormal dx
    X[3] = gen.normal((K,), ("qa-special",)) * 1e30
    Xd = X.to(DEV)
    Xq, dx = quantize(Xd, 4, K)
    Xq_r, dx_r = oracle.quantize_q8_act(X.numpy(), K)
    assert np.array_equal(host(Xq), Xq_r)
    assert np.array_equal(host(dx).view(np.uint32), dx_r.view(np.uint32))
    assert list(host(Xq)[0, 32:38]) == [127, 64, -1, 3, -3, 0]


FMTS = ["q8_0", "q4_0"]


def qmm(fmt):
    return getattr(bqm, f"qmm_{fmt}")


def qmm_oracle(fmt):
    return getattr(oracle, f"qmm_{fmt}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (5, 37, 96), (130, 129, 160), (256, 300, 1056),
                                   (129, 131, 4128)])
def test_qmm_parity_small(fmt, M, N, K):
    say("qmm small", fmt, M, N, K)
    Wi = weights(fmt, N, K, ("qmm", M, N, K))
    X = gen.normal((M, K), ("qmm-x", M, N, K), device=DEV)
    Xq, dx = quantize(X, M, K)
    Y = torch.full((M, N), float("nan"), device=DEV)
    qmm(fmt)(packed(fmt, Wi, N, K), Xq, dx, Y, M, N, K)
    Yr, S = qmm_oracle(fmt)(host(Wi), host(Xq), host(dx), N, K)
    check_close(host(Y), Yr, S, f"qmm {fmt} {M}x{N}x{K}")


def _exact_probe(fmt, M, N, K, rows=None):
    """qw in [-8, 8] (Q8_0) or every nibble (Q4_0: [-8, 7]), qx in [-8, 8], dw, dx in
    {0.5, 1, 2}: the block sums are exact integers and so is every fp32 step after them, so
    the output equals the oracle bit for bit; a single wrong integer block sum changes it."""
    if fmt == "q8_0":
        Wi = gen.raw_q8_0(N, K, ("qmm-probe", N, K), codes=(-8, 8), device=DEV)
    else:
        Wi = gen.raw_q4_0(N, K, ("qmm-probe4", N, K), codes=(0, 15), device=DEV)
    Xq = gen.small_int((M, K), ("qmm-probe-x", M, K), device=DEV, dtype=torch.int32).to(torch.int8)
    pick = gen.small_int((M, K // 32), ("qmm-probe-dx", M, K), 0, 2, device=DEV, dtype=torch.int32)
    dx = torch.tensor([0.5, 1.0, 2.0], device=DEV)[pick.long()]
    Y = torch.empty((M, N), device=DEV)
    qmm(fmt)(packed(fmt, Wi, N, K), Xq, dx, Y, M, N, K)
    Wh = host(Wi).reshape(N, -1)
    if rows is not None:
        Wh = Wh[rows]
    Yr, _ = qmm_oracle(fmt)(Wh, host(Xq), host(dx), Wh.shape[0], K)
    yg = host(Y) if rows is None else host(Y)[:, rows]
    assert np.array_equal(yg.astype(np.float64), Yr)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", [(3, 5, 64), (130, 129, 544), (128, 256, 5120)])
def test_qmm_exact_probe(fmt, M, N, K):
    say("qmm exact", fmt, M, N, K)
    _exact_probe(fmt, M, N, K)


@pytest.mark.parametrize("fmt", FMTS)
def test_qmm_exact_probe_prefill_shape(fmt):
    """The full 512 x 17408 x 5120 prefill shape, sampled output columns, bit exact."""
    say("qmm exact full shape", fmt)
    sh = gen.PREFILL_SHAPE
    rows = np.unique(np.random.default_rng(1).integers(0, sh["N"], 48))
    _exact_probe(fmt, sh["M"], sh["N"], sh["K"], rows)


@pytest.mark.parametrize("fmt", FMTS)
def test_qmm_prefill_shape(fmt):
    """Prefill GEMM: M=512 tokens, K=5120, N=17408, weights from N(0, 0.02) quantized to the
    format, activations N(0, 1) quantized per block; sampled output columns against the
    oracle."""
    sh = gen.PREFILL_SHAPE
    M, N, K = sh["M"], sh["N"], sh["K"]
    say("qmm prefill shape", fmt)
    Wi = weights(fmt, N, K, ("prefill", 0))
    X = gen.normal((M, K), ("prefill-x", 0), device=DEV)
    Xq, dx = quantize(X, M, K)
    Y = torch.empty((M, N), device=DEV)
    qmm(fmt)(packed(fmt, Wi, N, K), Xq, dx, Y, M, N, K)
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(2).integers(0, N, 64)]))
    Yr, S = qmm_oracle(fmt)(host(Wi).reshape(N, -1)[rows], host(Xq), host(dx), len(rows), K)
    check_close(host(Y)[:, rows], Yr, S, f"prefill {fmt}")


@pytest.mark.parametrize("fmt", FMTS)
def test_qmm_deterministic(fmt):
    M, N, K = 256, 384, 2048
    Wp = packed(fmt, weights(fmt, N, K, ("qmm-det",)), N, K)
    Xq, dx = quantize(gen.normal((M, K), ("qmm-det-x",), device=DEV), M, K)
    Y1 = torch.empty((M, N), device=DEV)
    Y2 = torch.empty((M, N), device=DEV)
    qmm(fmt)(Wp, Xq, dx, Y1, M, N, K)
    qmm(fmt)(Wp, Xq, dx, Y2, M, N, K)
    assert torch.equal(Y1, Y2)


@pytest.mark.parametrize("fmt", FMTS)
def test_qmm_empty_k_writes_zeros(fmt):
    M, N = 3, 70
    Y = torch.full((M, N), float("nan"), device=DEV)
    qmm(fmt)(None, None, None, Y, M, N, 0)
    assert torch.count_nonzero(Y).item() == 0


# --- expert-indexed prefill product ----------------------------------------------------------

def run_qmm_id(fmt, E, N, K, ids_np, rows, key, sample=None, exact=False):
    """qmm_id against the oracle; rows: 'broadcast' (one input row per token) or 'per_slot'.
    sample: slots to check (the oracle computes only those; others are given as padding)."""
    T, top_k = ids_np.shape
    if exact:
        Wi = (gen.raw_q8_0(E * N, K, key, codes=(-8, 8), device=DEV) if fmt == "q8_0"
              else gen.raw_q4_0(E * N, K, key, codes=(0, 15), device=DEV))
    else:
        Wi = weights(fmt, E * N, K, key)
    Wp = packed(fmt, Wi, E * N, K)
    nrows, xt, xs = (T, 1, 0) if rows == "broadcast" else (T * top_k, top_k, 1)
    if exact:
        Xq = gen.small_int((nrows, K), key + ("x",), device=DEV, dtype=torch.int32).to(torch.int8)
        pick = gen.small_int((nrows, K // 32), key + ("dx",), 0, 2, device=DEV, dtype=torch.int32)
        dx = torch.tensor([0.5, 1.0, 2.0], device=DEV)[pick.long()]
    else:
        Xq, dx = quantize(gen.normal((nrows, K), key + ("x",), device=DEV), nrows, K)
    ids = torch.from_numpy(ids_np).to(DEV)
    Y = torch.full((T, top_k, N), -7.0, device=DEV)
    bqm.qmm_id(fmt, Wp, E, N, K, ids, T, top_k, Xq, dx, xt, xs, Y)
    ids_or = np.where(ids_np >= E, -1, ids_np).astype(np.int32)
    if sample is not None:
        keep = np.zeros(T * top_k, bool)
        keep[sample] = True
        ids_or = np.where(keep.reshape(T, top_k), ids_or, -1).astype(np.int32)
    Yr, S = oracle.qmm_id(fmt, host(Wi), E, N, K, ids_or, host(Xq), host(dx), xt, xs)
    return host(Y), Yr, S


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows", ["broadcast", "per_slot"])
@pytest.mark.parametrize("E,N,K", [(5, 37, 96), (3, 300, 1056), (9, 129, 4128)])
def test_qmm_id_small(fmt, rows, E, N, K):
    say("qmm_id small", fmt, rows, E, N, K)
    ids = np.array([[3, 0, 4], [-1, 4, 2], [1, 3, -1], [0, 2, 4], [4, 4, 1]], np.int32) % E
    ids[1, 0] = -1
    ids[2, 2] = -1
    y, Yr, S = run_qmm_id(fmt, E, N, K, ids, rows, ("qmmid", fmt, rows, E, N, K))
    check_close(y, Yr, S, f"qmm_id {fmt} {rows}")
    assert np.all(y[1, 0] == 0) and np.all(y[2, 2] == 0)


@pytest.mark.parametrize("fmt", FMTS)
def test_qmm_id_exact_probe_and_many_slots_per_expert(fmt):
    """Integer-valued inputs (bit exact against the oracle), 300 tokens over 3 experts with
    one of them taking most slots: row tiles of 64 slots, several per expert, the last
    partial; bad ids give NaN rows."""
    E, N, K, T, top_k = 3, 200, 544, 300, 2
    ids = np.stack([np.zeros(T, np.int32), (np.arange(T) % 3).astype(np.int32)], axis=1)
    ids[5, 1] = -1
    ids[7, 1] = E + 2
    say("qmm_id exact", fmt)
    y, Yr, S = run_qmm_id(fmt, E, N, K, ids, "per_slot", ("qmmid-x", fmt), exact=True)
    bad = ids >= E
    assert np.all(np.isnan(y[bad]))
    assert np.array_equal(y[~bad].astype(np.float64), Yr[~bad])


@pytest.mark.parametrize("fmt", FMTS)
def test_qmm_id_exact_probe_tile_heights(fmt):
    """Bit exact against the oracle with per-expert slot counts on both sides of every cut
    between row tiles: 64-slot tiles while more than 32 slots are left, one 32-slot tile for
    a remainder that fits it, rescaling only its first 8 rows when it holds no more (counts
    1, 8, 9, 31, 32, 33, 63, 64, 65, 72, 73, 96, 97, 128 and none), slots of the experts
    interleaved in index order."""
    counts = [1, 8, 9, 31, 32, 33, 63, 64, 0, 65, 72, 73, 96, 97, 128]
    E, N, K, top_k = len(counts), 160, 288, 2
    flat = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])
    flat = flat[np.random.default_rng(11).permutation(flat.size)]
    flat = np.concatenate([flat, np.full((-flat.size) % top_k, -1, np.int32)])
    ids = flat.reshape(-1, top_k)
    say("qmm_id exact tile heights", fmt, ids.shape)
    y, Yr, S = run_qmm_id(fmt, E, N, K, ids, "per_slot", ("qmmid-h", fmt), exact=True)
    assert np.array_equal(y.astype(np.float64), Yr)


@pytest.mark.parametrize("proj", ["gate", "down"])
def test_qmm_id_moe_prefill(proj):
    """The MoE layer over a 512-token prompt (128 experts, top-8, skewed router), gate
    (4096 -> 1536, one input per token) or down (1536 -> 4096, one input per slot); 96
    sampled slots against the oracle, padding and every other slot present."""
    sh = gen.MOE_SHAPE
    E, top_k, T = sh["E"], sh["top_k"], gen.MOE_PREFILL_T
    N, K = (sh["ffn"], sh["hidden"]) if proj == "gate" else (sh["hidden"], sh["ffn"])
    ids = gen.router_ids(T, E, top_k, ("moe-prefill-router",))
    sample = np.unique(np.random.default_rng(3).integers(0, T * top_k, 96))
    say("qmm_id moe prefill", proj, "busiest expert", int(np.bincount(ids.ravel()).max()))
    y, Yr, S = run_qmm_id("q4_0", E, N, K, ids, "broadcast" if proj == "gate" else "per_slot",
                          ("qmmid-moe", proj), sample=sample)
    ys = y.reshape(T * top_k, N)[sample]
    check_close(ys, Yr.reshape(T * top_k, N)[sample], S.reshape(T * top_k, N)[sample],
                f"qmm_id moe prefill {proj}")


def test_qmm_id_deterministic_and_empty_k():
    E, N, K, T, top_k = 16, 256, 1024, 40, 4
    ids = torch.from_numpy(gen.router_ids(T, E, top_k, ("qmmid-det",))).to(DEV)
    Wp = packed("q8_0", weights("q8_0", E * N, K, ("qmmid-det",)), E * N, K)
    Xq, dx = quantize(gen.normal((T, K), ("qmmid-det-x",), device=DEV), T, K)
    Y1 = torch.empty((T, top_k, N), device=DEV)
    Y2 = torch.empty((T, top_k, N), device=DEV)
    bqm.qmm_id("q8_0", Wp, E, N, K, ids, T, top_k, Xq, dx, 1, 0, Y1)
    bqm.qmm_id("q8_0", Wp, E, N, K, ids, T, top_k, Xq, dx, 1, 0, Y2)
    assert torch.equal(Y1, Y2)
    idk = torch.tensor([[0, -1], [2, 5]], dtype=torch.int32, device=DEV)
    Y = torch.full((2, 2, 24), -7.0, device=DEV)
    bqm.qmm_id("q4_0", torch.zeros(256, dtype=torch.uint8, device=DEV), 3, 24, 0, idk, 2, 2,
               torch.zeros(64, dtype=torch.int8, device=DEV), torch.zeros(16, device=DEV), 1, 0, Y)
    y = host(Y)
    assert np.all(y[0] == 0) and np.all(y[1, 0] == 0) and np.all(np.isnan(y[1, 1]))


@pytest.mark.parametrize("T,top_k", [(bqm.QMM_ID_MAX_T, 2), (64, 32)])
def test_qmm_id_at_the_limits(T, top_k):
    """The largest token count (and the largest top-k) over the most experts, with short
    rows: every workgroup counts T * top_k ids; a sample of slots against the oracle, and
    the out-of-range ids (negative: zeros; >= E: NaN) checked everywhere."""
    E, N, K = bqm.QMV_ID_MAX_E, 64, 32
    rng = np.random.default_rng(11)
    ids = rng.integers(0, E, (T, top_k)).astype(np.int32)
    ids[0, 0] = -1
    ids[1, -1] = E
    ids[T - 1, 0] = E + 7
    sample = np.unique(np.concatenate([rng.integers(0, T * top_k, 160), [0, T * top_k - 1]]))
    say("qmm_id limits", T, top_k, E)
    y, Yr, S = run_qmm_id("q8_0", E, N, K, ids, "per_slot", ("qmmid-lim", T, top_k), sample=sample)
    flat, valid = y.reshape(T * top_k, N), (ids >= 0) & (ids < E)
    keep = valid.ravel()[sample]
    check_close(flat[sample][keep], Yr.reshape(T * top_k, N)[sample][keep],
                S.reshape(T * top_k, N)[sample][keep], "qmm_id at the limits")
    assert np.all(y[0, 0] == 0)
    assert np.all(np.isnan(y[1, -1])) and np.all(np.isnan(y[T - 1, 0]))
