"""GPU parity of repack/unpack and the decode GEMVs (qmv_q4_0, qmv_q8_0) against the oracle."""
import numpy as np
import pytest
import torch

import gen
import oracle
from block_quantized_matrix_amd import bqm
from tests._gpu import DEV, check_close, host, packed, say, weights

pytestmark = pytest.mark.gpu

FMTS = ["q4_0", "q8_0"]
QMV = {"q4_0": bqm.qmv_q4_0, "q8_0": bqm.qmv_q8_0}


@pytest.fixture(scope="module", autouse=True)
def _oracle():
    oracle.build(force=False)


# ---- repack / unpack ---------------------------------------------------------------

@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(1, 32), (3, 96), (17, 160), (121, 32), (249, 32), (257, 4096),
                                 (64, 17408)])
def test_repack_roundtrip_bitwise(fmt, N, K):
    say("repack", fmt, N, K)
    bb = gen.block_bytes(fmt)
    W = torch.randint(0, 256, (N, K // 32 * bb), dtype=torch.uint8, device=DEV)
    P = torch.full((bqm.packed_bytes(fmt, N, K),), 0xAB, dtype=torch.uint8, device=DEV)
    bqm.bqm_repack(fmt, W, P, N, K)
    back = torch.empty_like(W)
    bqm.bqm_unpack(fmt, P, back, N, K)
    assert torch.equal(back, W)
    # the packed layout: codes section, then the scale section on a 256-byte boundary
    nb, cb = K // 32, 16 if fmt == "q4_0" else 32
    Ph, Wh = host(P), host(W).reshape(N, nb, bb)
    codes = Ph[:N * nb * cb].reshape(N, nb, cb)
    assert np.array_equal(codes, Wh[:, :, 2:])
    off = (N * nb * cb + 255) // 256 * 256
    assert np.array_equal(Ph[off:off + 2 * N * nb].reshape(N, nb, 2), Wh[:, :, :2])
    assert not Ph[N * nb * cb:off].any() and not Ph[off + 2 * N * nb:].any()  # padding zeroed


# ---- small shapes: several tiles and ragged tails -------------------------------------

SHAPES = [(1, 32), (3, 64), (17, 96), (64, 160), (300, 512), (129, 1536), (33, 4096), (70, 5120),
          (40, 17408)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("N,K", SHAPES)
def test_qmv_parity_small(fmt, M, N, K):
    say("qmv", fmt, M, N, K)
    Wi = weights(fmt, N, K, ("qmv-small", fmt, N, K))
    X = gen.normal((M, K), ("qmv-small-x", M, K), device=DEV)
    Y = torch.full((M, N), float("nan"), device=DEV)
    QMV[fmt](packed(fmt, Wi, N, K), X, Y, M, N, K)
    Yr, S = oracle.qmv(fmt, host(Wi), host(X), N, K)
    check_close(host(Y), Yr, S, f"{fmt} M={M} N={N} K={K}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 4, 8])
@pytest.mark.parametrize("N,K", [(67, 2048), (5, 17408)])
def test_qmv_exact_probe(fmt, M, N, K):
    """Integer x in [-8, 8], scales in {0.5, 1, 2}, small codes: every fp32 operation is
    exact, so the GPU result must equal the oracle bit for bit (any wrong code, scale or
    index shows up even where the 1e-3 tolerance could not see it)."""
    say("qmv exact", fmt, M, N, K)
    if fmt == "q4_0":
        Wi = gen.raw_q4_0(N, K, ("probe", N, K), device=DEV)
    else:
        Wi = gen.raw_q8_0(N, K, ("probe", N, K), codes=(-8, 8), device=DEV)
    X = gen.small_int((M, K), ("probe-x", M, K), device=DEV)
    Y = torch.empty((M, N), device=DEV)
    QMV[fmt](packed(fmt, Wi, N, K), X, Y, M, N, K)
    Yr, _ = oracle.qmv(fmt, host(Wi), host(X), N, K)
    assert np.array_equal(host(Y).astype(np.float64), Yr)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 2, 3, 8])  # every batch class (1, 2, 4, 8) and sum order
def test_qmv_invariants(fmt, M):
    N, K = 96, 5120
    say("qmv invariants", fmt, M)
    Wi = weights(fmt, N, K, ("inv", fmt))
    X = gen.normal((M, K), ("inv-x", M), device=DEV)
    bb = gen.block_bytes(fmt)
    # neutral codes: exactly zero output for any scale and input
    Wn = Wi.reshape(N, K // 32, bb).clone()
    Wn[:, :, 2:] = 0x88 if fmt == "q4_0" else 0
    Y = torch.full((M, N), float("nan"), device=DEV)
    QMV[fmt](packed(fmt, Wn.reshape(N, -1), N, K), X, Y, M, N, K)
    assert torch.all(Y == 0)
    # doubling every scale doubles every output bit for bit
    Y1 = torch.empty((M, N), device=DEV)
    QMV[fmt](packed(fmt, Wi, N, K), X, Y1, M, N, K)
    d = Wi.reshape(N, K // 32, bb)[:, :, :2].contiguous().view(torch.float16) * 2
    W2 = Wi.reshape(N, K // 32, bb).clone()
    W2[:, :, :2] = d.view(torch.uint8).reshape(N, K // 32, 2)
    Y2 = torch.empty((M, N), device=DEV)
    QMV[fmt](packed(fmt, W2.reshape(N, -1), N, K), X, Y2, M, N, K)
    assert torch.equal(Y2, 2 * Y1)
    # zero scales: zero output
    W0 = Wi.reshape(N, K // 32, bb).clone()
    W0[:, :, :2] = 0
    QMV[fmt](packed(fmt, W0.reshape(N, -1), N, K), X, Y, M, N, K)
    assert torch.all(Y == 0)


def test_qmv_k_zero_writes_zeros():
    Y = torch.full((2, 5), 7.0, device=DEV)
    X = torch.empty((2, 0), device=DEV)
    W = torch.empty(0, dtype=torch.uint8, device=DEV)
    bqm.qmv_q4_0(W, X, Y, 2, 5, 0)
    assert np.all(host(Y) == 0)


# ---- full-size workloads ------------------------------------------------------------

def test_qmv_q4_0_gemv_4096_full():
    """4096 x 4096 Q4_0 GEMV, batch 1, seed 0: every output against the oracle."""
    N = K = 4096
    say("qmv 4096 full")
    w = gen.normal((N, K), ("gemv4096", 0), std=0.02, device=DEV)
    Wi = gen.encode_q4_0(w)
    X = gen.normal((1, K), ("gemv4096-x", 0), device=DEV)
    Y = torch.empty((1, N), device=DEV)
    bqm.qmv_q4_0(packed("q4_0", Wi, N, K), X, Y, 1, N, K)
    Yr, S = oracle.qmv("q4_0", host(Wi), host(X), N, K)
    rel = check_close(host(Y), Yr, S, "gemv 4096")
    say("max |err|/S", rel)


def _sampled(fmt, M, N, K, key, n_sample=96):
    Wi = weights(fmt, N, K, key)
    X = gen.normal((M, K), key + ("x",), device=DEV)
    Y = torch.empty((M, N), device=DEV)
    QMV[fmt](packed(fmt, Wi, N, K), X, Y, M, N, K)
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(0).integers(0, N, n_sample)]))
    Wh = host(Wi).reshape(N, -1)[rows]
    Yr, S = oracle.qmv(fmt, Wh, host(X), len(rows), K)
    check_close(host(Y)[:, rows], Yr, S, f"{fmt} M={M} {N}x{K}")


@pytest.mark.parametrize("name,N,K", gen.DENSE27B_FUSED_SHAPES + (("k", 1024, 5120),))
def test_qmv_q4_0_27b_layer_shapes(name, N, K):
    """27B-dense layer shapes in the launch configuration the benchmark times (q|k|v and
    gate|up stacked), Q4_0, batch 1: sampled rows against the oracle."""
    say("qmv 27b", name, N, K)
    _sampled("q4_0", 1, N, K, ("27b", name))


@pytest.mark.parametrize("M", [1, 4, 8])
@pytest.mark.parametrize("name,N,K", gen.DENSE27B_FUSED_SHAPES)
def test_qmv_q8_0_27b_layer_shapes(name, N, K, M):
    say("qmv q8 27b", name, N, K, M)
    _sampled("q8_0", M, N, K, ("27b-q8", name, M))


# ---- robustness ---------------------------------------------------------------------

@pytest.mark.parametrize("fmt", FMTS)
def test_qmv_deterministic_and_stream(fmt):
    N, K, M = 513, 5120, 1
    say("qmv determinism", fmt)
    Wp = packed(fmt, weights(fmt, N, K, ("det", fmt)), N, K)
    X = gen.normal((M, K), ("det-x",), device=DEV)
    Y1 = torch.empty((M, N), device=DEV)
    Y2 = torch.empty((M, N), device=DEV)
    QMV[fmt](Wp, X, Y1, M, N, K)
    s = torch.cuda.Stream()
    torch.cuda.current_stream().synchronize()
    with torch.cuda.stream(s):
        QMV[fmt](Wp, X, Y2, M, N, K)
    s.synchronize()
    assert torch.equal(Y1, Y2)


def test_qmv_error_leaves_output_untouched():
    Y = torch.full((1, 8), 3.0, device=DEV)
    W = torch.zeros(4096, dtype=torch.uint8, device=DEV)
    X = torch.zeros((1, 64), device=DEV)
    with pytest.raises(bqm.BqmError):
        bqm.qmv_q4_0(W, X, Y, 1, 8, 48)        # K not a multiple of 32
    with pytest.raises(bqm.BqmError):
        bqm.qmv_q4_0(W, X, Y, 9, 8, 64)        # M > 8
    assert np.all(host(Y) == 3.0)


def test_qmv_output_guard_band():
    """Nothing is written past the end of Y."""
    N, K = 37, 96
    Wi = weights("q4_0", N, K, ("guard",))
    X = gen.normal((2, K), ("guard-x",), device=DEV)
    buf = torch.full((2 * N + 64,), 5.0, device=DEV)
    bqm.qmv_q4_0(packed("q4_0", Wi, N, K), X, buf, 2, N, K)
    assert np.all(host(buf)[2 * N:] == 5.0)
