"""GPU parity of the matrix-core form of the expert-indexed products (T >= 8 tokens, K a
multiple of 128): qmv_id, qmv_id_gate_up and qmv_id_sum against the oracle.

The form groups up to 16 slots per expert, splits each fp32 input into two bf16 parts, and
splits K between waves when a workgroup holds few tiles; the cases below reach each of these
(16-slot groups, experts with more than 16 slots, ragged row tiles, K splits of 2 to 16
shares, long K in chunks, the slot tables at their largest), and the exact probes check
every code, scale and index bit for bit."""
import numpy as np
import pytest
import torch

import gen
import oracle
from block_quantized_matrix_amd import bqm
from tests._gpu import DEV, check_close, host, packed, say, weights

pytestmark = pytest.mark.gpu

FMTS = ["q4_0", "q8_0"]


@pytest.fixture(scope="module", autouse=True)
def _oracle():
    oracle.build(force=False)


def _ids(T, E, top_k, key):
    return gen.router_ids(T, E, top_k, key)


def _run_id(fmt, Wi, E, N, K, ids, X, xts, xss):
    T, top_k = ids.shape
    Y = torch.full((T, top_k, N), float("nan"), device=DEV)
    bqm.qmv_id(fmt, packed(fmt, Wi, E * N, K), E, N, K, torch.from_numpy(ids).to(DEV), T, top_k, X,
               xts, xss, Y)
    ids_ok = np.where(ids >= E, -1, ids).astype(np.int32)
    Yr, S = oracle.qmv_id(fmt, host(Wi), E, N, K, ids_ok, host(X).reshape(-1), xts, xss)
    return host(Y), Yr, S


# (T, E, N, K, top_k): 16-slot groups of a skewed router; a ragged last row tile (N not a
# multiple of 16); experts with more than 16 slots (every token on a few experts); one tile
# per workgroup (K split 16 ways), a few (split 8 or 16 ways), many (split 2 ways); a ragged
# tile with 4-slot groups; long K in several staged chunks; a 15-slot group (one slot is
# padding) over long K with four tiles per pass (its inputs and scales in four chunks)
CASES = [(16, 32, 96, 4096, 8), (8, 6, 130, 1152, 3), (64, 4, 40, 256, 2), (8, 2, 16, 2048, 2),
         (16, 4, 4096, 1024, 2), (16, 40, 4096, 512, 8), (12, 5, 200, 1536, 4), (16, 4, 64, 16384, 2),
         (16, 1, 16384, 8192, 1)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("slots", ["broadcast", "per_slot"])
@pytest.mark.parametrize("T,E,N,K,top_k", CASES)
def test_mma_qmv_id(fmt, slots, T, E, N, K, top_k):
    say("mma qmv_id", fmt, slots, T, E, N, K, top_k)
    ids = _ids(T, E, top_k, ("mma-router", T, E, top_k))
    ids[0, -1] = -1                       # a padding slot
    Wi = weights(fmt, E * N, K, ("mma-w", fmt, T, E, N, K))
    if slots == "broadcast":
        X, xts, xss = gen.normal((T, K), ("mma-x", T, K), device=DEV), K, 0
    else:
        X, xts, xss = gen.normal((T, top_k, K), ("mma-x2", T, K), device=DEV), top_k * K, K
    y, Yr, S = _run_id(fmt, Wi, E, N, K, ids, X, xts, xss)
    check_close(y, Yr, S, f"mma qmv_id {fmt} {slots} T={T} E={E} N={N} K={K}")
    assert np.all(y[0, -1] == 0)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T,E,N,K,top_k", [(16, 8, 96, 4096, 4), (64, 3, 48, 512, 2), (8, 2, 16, 2048, 2)])
def test_mma_exact_probe(fmt, T, E, N, K, top_k):
    """Integer inputs in [-8, 8], scales in {0.5, 1, 2}, small codes: every product and sum
    is exact on both sides, so the outputs must match the oracle bit for bit (a wrong code,
    scale, slot or row shows up even where the tolerance could not see it)."""
    say("mma exact", fmt, T, E, N, K)
    ids = _ids(T, E, top_k, ("mma-probe-router", T, E))
    if fmt == "q4_0":
        Wi = gen.raw_q4_0(E * N, K, ("mma-probe", T, E, N, K), device=DEV)
    else:
        Wi = gen.raw_q8_0(E * N, K, ("mma-probe", T, E, N, K), codes=(-8, 8), device=DEV)
    X = gen.small_int((T, top_k, K), ("mma-probe-x", T, K), device=DEV)
    y, Yr, _ = _run_id(fmt, Wi, E, N, K, ids, X, top_k * K, K)
    assert np.array_equal(y.astype(np.float64), Yr)


@pytest.mark.parametrize("fmt", FMTS)
def test_mma_exact_probe_weighted_sum(fmt):
    """The weighted form with power-of-two router weights: exact as well."""
    T, E, N, K, top_k = 16, 6, 64, 1024, 4
    ids = _ids(T, E, top_k, ("mma-ws-router",))
    ids[3, 1] = -1
    if fmt == "q4_0":
        Wi = gen.raw_q4_0(E * N, K, ("mma-ws",), device=DEV)
    else:
        Wi = gen.raw_q8_0(E * N, K, ("mma-ws",), codes=(-8, 8), device=DEV)
    X = gen.small_int((T, top_k, K), ("mma-ws-x",), device=DEV)
    w = (2.0 ** np.random.default_rng(5).integers(-3, 2, (T, top_k))).astype(np.float32)
    say("mma exact weighted sum", fmt)
    Ys = torch.empty((T, top_k, N), device=DEV)
    Y = torch.empty((T, N), device=DEV)
    bqm.qmv_id_sum(fmt, packed(fmt, Wi, E * N, K), E, N, K, torch.from_numpy(ids).to(DEV),
                   torch.from_numpy(w).to(DEV), T, top_k, X, top_k * K, K, Ys, Y)
    Yr, _ = oracle.qmv_id_sum(fmt, host(Wi), E, N, K, ids, w, host(X).reshape(-1), top_k * K, K)
    assert np.array_equal(host(Y).astype(np.float64), Yr)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T,E,N,K,top_k", [(16, 8, 96, 4096, 4), (64, 3, 40, 512, 2), (8, 2, 16, 2048, 2)])
def test_mma_gate_up(fmt, T, E, N, K, top_k):
    say("mma gate_up", fmt, T, E, N, K)
    ids = _ids(T, E, top_k, ("mma-gu-router", T, E))
    ids[1, 0] = -1
    ids[2, 1] = E + 3                     # out of range: NaN row
    Wg = weights(fmt, E * N, K, ("mma-gu-g", fmt, T), std=0.05)
    Wu = weights(fmt, E * N, K, ("mma-gu-u", fmt, T), std=0.05)
    X = gen.normal((T, K), ("mma-gu-x", T, K), device=DEV)
    Y = torch.full((T, top_k, N), -7.0, device=DEV)
    bqm.qmv_id_gate_up(fmt, packed(fmt, Wg, E * N, K), packed(fmt, Wu, E * N, K), E, N, K,
                       torch.from_numpy(ids).to(DEV), T, top_k, X, K, 0, Y)
    ids_ok = np.where(ids >= E, -1, ids).astype(np.int32)
    Yr, S = oracle.qmv_id_gate_up(fmt, host(Wg), host(Wu), E, N, K, ids_ok, host(X).reshape(-1), K, 0)
    y = host(Y)
    assert np.all(np.isnan(y[2, 1])) and np.all(y[1, 0] == 0)
    ok = ids < E
    check_close(y[ok], Yr[ok], S[ok], f"mma gate_up {fmt} T={T}")


@pytest.mark.parametrize("fmt", FMTS)
def test_mma_weighted_sum(fmt):
    T, E, N, K, top_k = 16, 128, 48, 1536, 8
    ids = _ids(T, E, top_k, ("mma-wsum-router",))
    w = gen.router_weights(T, top_k, ("mma-wsum-w",))
    Wi = weights(fmt, E * N, K, ("mma-wsum", fmt))
    X = gen.normal((T, top_k, K), ("mma-wsum-x",), device=DEV)
    say("mma weighted sum", fmt)
    Ys = torch.empty((T, top_k, N), device=DEV)
    Y = torch.empty((T, N), device=DEV)
    bqm.qmv_id_sum(fmt, packed(fmt, Wi, E * N, K), E, N, K, torch.from_numpy(ids).to(DEV),
                   torch.from_numpy(w).to(DEV), T, top_k, X, top_k * K, K, Ys, Y)
    Yr, S = oracle.qmv_id_sum(fmt, host(Wi), E, N, K, ids, w, host(X).reshape(-1), top_k * K, K)
    check_close(host(Y), Yr, S, f"mma weighted sum {fmt}")


@pytest.mark.parametrize("fmt", FMTS)
def test_mma_subnormal_and_wide_range_inputs(fmt):
    """Inputs spanning fp32's range: subnormals (whose bf16 parts are subnormal too),
    values near 2^-120 and near 2^60 in the same rows, and all-subnormal input rows."""
    T, E, N, K, top_k = 16, 4, 48, 1024, 2
    ids = _ids(T, E, top_k, ("mma-sub-router",))
    Wi = weights(fmt, E * N, K, ("mma-sub", fmt))
    rng = np.random.default_rng(11)
    X = rng.standard_normal((T, K)).astype(np.float32)
    X[:, ::7] *= np.float32(2.0 ** -140)            # subnormal
    X[:, 3::11] *= np.float32(2.0 ** -120)
    X[:, 5::13] *= np.float32(2.0 ** 60)
    X[1] = (rng.integers(1, 1 << 20, K) * 2.0 ** -149).astype(np.float32) * rng.choice([-1, 1], K)
    Xd = torch.from_numpy(X).to(DEV)
    say("mma subnormal inputs", fmt)
    y, Yr, S = _run_id(fmt, Wi, E, N, K, ids, Xd, K, 0)
    check_close(y, Yr, S, f"mma subnormal {fmt}")


def test_mma_neutral_codes_give_exact_zeros():
    T, E, N, K, top_k = 16, 4, 64, 2048, 2
    Wi = weights("q4_0", E * N, K, ("mma-neutral",)).reshape(E * N, K // 32, 18).clone()
    Wi[:, :, 2:] = 0x88
    ids = _ids(T, E, top_k, ("mma-neutral-router",))
    X = gen.normal((T, K), ("mma-neutral-x",), device=DEV) * 1e3
    y, _, _ = _run_id("q4_0", Wi.reshape(E * N, -1), E, N, K, ids, X, K, 0)
    assert np.all(y == 0)


def test_mma_maximum_slots_and_experts():
    """T = 64 tokens x top_k = 32 over E = 4096 experts, K = 128: the slot tables at their
    largest beside the staged inputs, padding and out-of-range ids mixed in."""
    E, N, K, T, top_k = bqm.QMV_ID_MAX_E, 16, 128, bqm.QMV_ID_MAX_T, bqm.QMV_ID_MAX_TOPK
    rng = np.random.default_rng(9)
    ids = rng.integers(0, 64, size=(T, top_k)).astype(np.int32) * 64
    ids[::3, 5] = rng.integers(0, E, size=ids[::3, 5].shape)
    ids[1::7, 2] = -1
    ids[2::9, 9] = E + 5
    Wi = weights("q4_0", E * N, K, ("mma-max",))
    X = gen.normal((T, K), ("mma-max-x",), device=DEV)
    say("mma max slots")
    y, Yr, S = _run_id("q4_0", Wi, E, N, K, ids, X, K, 0)
    bad = ids >= E
    assert np.all(np.isnan(y[bad]))
    check_close(y[~bad], Yr[~bad], S[~bad], "mma max slots")


def test_mma_deterministic():
    T, E, N, K, top_k = 16, 16, 128, 4096, 4
    ids = torch.from_numpy(_ids(T, E, top_k, ("mma-det",))).to(DEV)
    Wp = packed("q4_0", weights("q4_0", E * N, K, ("mma-det",)), E * N, K)
    X = gen.normal((T, K), ("mma-det-x",), device=DEV)
    Y1 = torch.empty((T, top_k, N), device=DEV)
    Y2 = torch.empty((T, top_k, N), device=DEV)
    bqm.qmv_id("q4_0", Wp, E, N, K, ids, T, top_k, X, K, 0, Y1)
    bqm.qmv_id("q4_0", Wp, E, N, K, ids, T, top_k, X, K, 0, Y2)
    assert torch.equal(Y1, Y2)


def test_mma_q8_code_minus_128():
    """Q8_0 code -128 (accepted on read) through the matrix cores, exact probe: codes in
    [-128, 127] with -128 in every block, integer inputs, power-of-two scales."""
    T, E, N, K, top_k = 16, 4, 48, 1024, 2
    rng = np.random.default_rng(13)
    codes = rng.integers(-128, 128, (E * N, K // 32, 32))
    codes[:, :, 7] = -128
    d = rng.choice([0.5, 1.0, 2.0], (E * N, K // 32)).astype(np.float16)
    W = np.concatenate([d.view(np.uint8).reshape(E * N, K // 32, 2),
                        codes.astype(np.int8).view(np.uint8)], axis=2).reshape(E * N, -1)
    ids = _ids(T, E, top_k, ("mma-m128-router",))
    X = gen.small_int((T, K), ("mma-m128-x",), device=DEV)
    say("mma q8 code -128")
    y, Yr, _ = _run_id("q8_0", torch.from_numpy(W).to(DEV), E, N, K, ids, X, K, 0)
    assert np.array_equal(y.astype(np.float64), Yr)
