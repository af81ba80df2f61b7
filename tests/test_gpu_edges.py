"""GPU parity on the inputs that stress how the single-precision sums are formed, against the
oracle under the acceptance bound |y - y_ref| <= 1e-3 S:

- near-neutral blocks: every code the format's offset (Q4_0 nibble 8, Q8_0 code 0) except a
  few at +-1, those placed on inputs of 1e-3..1e-2 and inputs of 100..300 everywhere else,
  so S is tiny against sum |d x|.  A kernel that sums unsigned codes and subtracts the
  offset times sum x afterwards loses these outputs to cancellation; run in the dense,
  indexed, gate+up and weighted-sum forms at batches 1, 2, 4 and 8;
- Q8_0 code -128 (accepted by the format reading, never produced by the quantizer);
- subnormal binary16 weight scales and subnormal fp32 inputs;
- the prefill products with code -128 and subnormal weight scales (exact probes).
The block formats are those of the format table of "V100跑Qwen 27B：量化与KV Cache调优，从4到
64 tok/s" (lmnt.cn), section 4.1.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from block_quantized_matrix_amd import bqm
from tests._gpu import DEV, check_close, host, packed, say

pytestmark = pytest.mark.gpu

QMV = {"q4_0": bqm.qmv_q4_0, "q8_0": bqm.qmv_q8_0}


@pytest.fixture(scope="module", autouse=True)
def _oracle():
    oracle.build(force=False)


def blocks_from(fmt, codes, d16):
    """Interchange bytes from signed codes [rows][nb][32] (Q4_0: value n - 8) and binary16
    scales [rows][nb]."""
    rows, nb, _ = codes.shape
    db = np.ascontiguousarray(d16.astype(np.float16)).view(np.uint8).reshape(rows, nb, 2)
    if fmt == "q4_0":
        n = (codes + 8).astype(np.uint8)
        qs = n[:, :, :16] | (n[:, :, 16:] << 4)
    else:
        qs = codes.astype(np.int8).view(np.uint8)
    return np.concatenate([db, qs], axis=2).reshape(rows, -1)


def near_neutral(fmt, rows, K, M, seed):
    """(W interchange bytes, X [M][K]): three input positions per block hold small values
    (the same positions in every input row), every other input is large; a row's codes are
    the offset except at a random subset of the small positions, where they are +-1."""
    rng = np.random.default_rng(seed)
    nb = K // 32
    small = np.zeros((nb, 32), bool)
    for b in range(nb):
        small[b, rng.choice(32, 3, replace=False)] = True
    sign = lambda shape: rng.choice([-1.0, 1.0], shape)
    X = rng.uniform(100, 300, (M, K)) * sign((M, K))
    sm = small.reshape(-1)
    X[:, sm] = rng.uniform(1e-3, 1e-2, (M, int(sm.sum()))) * sign((M, int(sm.sum())))
    codes = np.zeros((rows, nb, 32), np.int64)
    pick = rng.integers(-1, 2, (rows, nb, 32))
    codes[:, small] = pick[:, small]
    d = rng.uniform(0.005, 0.02, (rows, nb)) * sign((rows, nb))
    return blocks_from(fmt, codes, d), X.astype(np.float32)


def offset_form_err_scale(fmt, W, X, rows, K):
    """16 ulp of sum |d| |x| per block: the size of the cancellation error of the offset form."""
    bb = gen.block_bytes(fmt)
    d = W.reshape(rows, K // 32, bb)[:, :, :2].copy().view(np.float16)[:, :, 0].astype(np.float64)
    ax = np.abs(X.astype(np.float64)).reshape(X.shape[0], K // 32, 32).sum(axis=2)
    return 16 * 2.0 ** -24 * (ax @ np.abs(d).T)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("M", [1, 2, 4, 8])
@pytest.mark.parametrize("K", [4096, 17408])
def test_near_neutral_dense(fmt, M, K):
    N = 160
    W, X = near_neutral(fmt, N, K, M, gen.seed_of("nn-dense", fmt, M, K))
    Yr, S = oracle.qmv(fmt, W, X, N, K)
    # the construction is adversarial: the offset form's error would exceed the bar
    assert np.median(offset_form_err_scale(fmt, W, X, N, K) / (1e-3 * S)) > 1.0
    say("near-neutral dense", fmt, M, K)
    Wd = torch.from_numpy(W).to(DEV)
    Xd = torch.from_numpy(X).to(DEV)
    Y = torch.full((M, N), float("nan"), device=DEV)
    QMV[fmt](packed(fmt, Wd, N, K), Xd, Y, M, N, K)
    rel = check_close(host(Y), Yr, S, f"near-neutral {fmt} M={M} K={K}")
    say("max err/S", rel)


def _moe_near_neutral(fmt, E, N, K, T, top_k, seed, per_slot):
    rows_in = T * top_k if per_slot else T
    W, X = near_neutral(fmt, E * N, K, rows_in, seed)
    ids = gen.router_ids(T, E, top_k, ("nn-router", T, seed))
    return W, X, ids


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("T", [1, 2, 5, 16])   # batch classes 1, 2, 4 and 4 with long groups
def test_near_neutral_indexed(fmt, T):
    E, N, K, top_k = 6, 96, 4096, 3
    W, X, ids = _moe_near_neutral(fmt, E, N, K, T, top_k, 21 + T, per_slot=False)
    say("near-neutral indexed", fmt, T)
    Y = torch.full((T, top_k, N), float("nan"), device=DEV)
    bqm.qmv_id(fmt, packed(fmt, torch.from_numpy(W).to(DEV), E * N, K), E, N, K,
               torch.from_numpy(ids).to(DEV), T, top_k, torch.from_numpy(X).to(DEV), K, 0, Y)
    Yr, S = oracle.qmv_id(fmt, W, E, N, K, ids, X, K, 0)
    check_close(host(Y), Yr, S, f"near-neutral indexed {fmt} T={T}")


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("T", [1, 2, 5, 16])
def test_near_neutral_gate_up(fmt, T):
    E, N, K, top_k = 6, 96, 4096, 3
    Wg, X, ids = _moe_near_neutral(fmt, E, N, K, T, top_k, 41 + T, per_slot=False)
    # the up matrix: the gate's codes (so they sit on the same small inputs), other scales
    bb = gen.block_bytes(fmt)
    Wu = Wg.reshape(E * N, K // 32, bb).copy()
    d = np.random.default_rng(61 + T).uniform(0.005, 0.02, (E * N, K // 32)).astype(np.float16)
    Wu[:, :, :2] = d.view(np.uint8).reshape(E * N, K // 32, 2)
    Wu = Wu.reshape(E * N, -1)
    say("near-neutral gate_up", fmt, T)
    Y = torch.full((T, top_k, N), float("nan"), device=DEV)
    bqm.qmv_id_gate_up(fmt, packed(fmt, torch.from_numpy(Wg).to(DEV), E * N, K),
                       packed(fmt, torch.from_numpy(Wu).to(DEV), E * N, K), E, N, K,
                       torch.from_numpy(ids).to(DEV), T, top_k, torch.from_numpy(X).to(DEV), K, 0, Y)
    Yr, S = oracle.qmv_id_gate_up(fmt, Wg, Wu, E, N, K, ids, X, K, 0)
    check_close(host(Y), Yr, S, f"near-neutral gate_up {fmt} T={T}")
    # the gate and up sums each within their own bar: compare with the separate products
    g, Sg = oracle.qmv_id(fmt, Wg, E, N, K, ids, X, K, 0)
    Yg = torch.empty((T, top_k, N), device=DEV)
    bqm.qmv_id(fmt, packed(fmt, torch.from_numpy(Wg).to(DEV), E * N, K), E, N, K,
               torch.from_numpy(ids).to(DEV), T, top_k, torch.from_numpy(X).to(DEV), K, 0, Yg)
    check_close(host(Yg), g, Sg, f"near-neutral gate rows {fmt} T={T}")


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("T", [1, 2, 5, 16])
def test_near_neutral_weighted_sum(fmt, T):
    E, N, K, top_k = 6, 96, 4096, 3
    W, X, ids = _moe_near_neutral(fmt, E, N, K, T, top_k, 81 + T, per_slot=True)
    w = gen.router_weights(T, top_k, ("nn-w", T))
    say("near-neutral weighted sum", fmt, T)
    Ys = torch.full((T, top_k, N), float("nan"), device=DEV)
    Y = torch.full((T, N), float("nan"), device=DEV)
    bqm.qmv_id_sum(fmt, packed(fmt, torch.from_numpy(W).to(DEV), E * N, K), E, N, K,
                   torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), T, top_k,
                   torch.from_numpy(X).to(DEV), top_k * K, K, Ys, Y)
    Yr, S = oracle.qmv_id_sum(fmt, W, E, N, K, ids, w, X, top_k * K, K)
    check_close(host(Y), Yr, S, f"near-neutral weighted sum {fmt} T={T}")
    Yid, Sid = oracle.qmv_id(fmt, W, E, N, K, ids, X, top_k * K, K)
    wb = w.astype(np.float64)[:, :, None]
    check_close(host(Ys), wb * Yid, np.abs(wb) * Sid, f"near-neutral weighted slots {fmt} T={T}")


@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_q8_code_minus_128(M):
    """Q8_0 blocks holding code -128 (with every other code value) and random inputs."""
    N, K = 130, 5120
    rng = np.random.default_rng(M)
    codes = rng.integers(-128, 128, (N, K // 32, 32))
    codes[:, :, 5] = -128
    codes[::3, :, :] = -128
    d = rng.uniform(0.001, 0.02, (N, K // 32))
    W = blocks_from("q8_0", codes, d)
    X = rng.standard_normal((M, K)).astype(np.float32)
    say("q8 code -128", M)
    Y = torch.full((M, N), float("nan"), device=DEV)
    bqm.qmv_q8_0(packed("q8_0", torch.from_numpy(W).to(DEV), N, K), torch.from_numpy(X).to(DEV), Y, M, N, K)
    Yr, S = oracle.qmv("q8_0", W, X, N, K)
    check_close(host(Y), Yr, S, f"q8 -128 M={M}")
    # exact probe: codes in {-128} U [-8, 8], small integer inputs, power-of-two scales
    codes = rng.integers(-8, 9, (N, 32, 32))
    codes[:, :, 7] = -128
    K2 = 1024
    assert K2 // 32 * (31 * 8 + 128) * 8 * 2 / 0.5 < 2 ** 24
    W2 = blocks_from("q8_0", codes, rng.choice([0.5, 1.0, 2.0], (N, 32)))
    X2 = rng.integers(-8, 9, (M, K2)).astype(np.float32)
    Y2 = torch.full((M, N), float("nan"), device=DEV)
    bqm.qmv_q8_0(packed("q8_0", torch.from_numpy(W2).to(DEV), N, K2), torch.from_numpy(X2).to(DEV), Y2, M, N, K2)
    Yr2, _ = oracle.qmv("q8_0", W2, X2, N, K2)
    assert np.array_equal(host(Y2).astype(np.float64), Yr2)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("M", [1, 4])
def test_subnormal_scales_and_inputs(fmt, M):
    """Binary16 subnormal weight scales (down to 2^-24) in half the blocks, and fp32
    subnormal inputs (around 2^-130) at a quarter of the positions, mixed with normal
    values: every output within the bar, and exact with integer-valued inputs."""
    N, K = 96, 4096
    rng = np.random.default_rng(3 + M)
    lo, hi = (-8, 7) if fmt == "q4_0" else (-127, 127)
    codes = rng.integers(lo, hi + 1, (N, K // 32, 32))
    d = rng.uniform(0.005, 0.02, (N, K // 32))
    sub = rng.random((N, K // 32)) < 0.5
    d[sub] = rng.integers(1, 1024, int(sub.sum())) * 2.0 ** -24   # binary16 subnormals, exact
    W = blocks_from(fmt, codes, d)
    assert np.all(W.reshape(N, K // 32, -1)[:, :, :2].copy().view(np.uint16)[sub][:, 0] & 0x7C00 == 0)
    X = rng.standard_normal((M, K)).astype(np.float32)
    tiny = rng.random((M, K)) < 0.25
    X[tiny] = (rng.integers(1, 2 ** 20, int(tiny.sum())) * 2.0 ** -150).astype(np.float32)
    say("subnormal", fmt, M)
    Y = torch.full((M, N), float("nan"), device=DEV)
    QMV[fmt](packed(fmt, torch.from_numpy(W).to(DEV), N, K), torch.from_numpy(X).to(DEV), Y, M, N, K)
    Yr, S = oracle.qmv(fmt, W, X, N, K)
    check_close(host(Y), Yr, S, f"subnormal {fmt} M={M}")
    # all scales subnormal, integer inputs: every partial sum is a multiple of 2^-24 below 2^24
    d2 = rng.integers(1, 8, (N, K // 32)) * 2.0 ** -24
    c2 = rng.integers(-8, 8, (N, K // 32, 32))
    W2 = blocks_from(fmt, c2, d2)
    X2 = rng.integers(-8, 9, (M, K)).astype(np.float32)
    assert K * 8 * 8 * 8 < 2 ** 24
    Y2 = torch.full((M, N), float("nan"), device=DEV)
    QMV[fmt](packed(fmt, torch.from_numpy(W2).to(DEV), N, K), torch.from_numpy(X2).to(DEV), Y2, M, N, K)
    Yr2, _ = oracle.qmv(fmt, W2, X2, N, K)
    assert np.array_equal(host(Y2).astype(np.float64), Yr2)


# ---- prefill products --------------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
def test_qmm_subnormal_weight_scales_exact(fmt):
    """Prefill products with binary16 subnormal weight scales (k * 2^-24) and activation
    scales in {0.5, 1, 2}, codes with |q| <= 8 (Q8_0 also -128 at one position per block)
    and activation codes in [-8, 8]: block sums, scale products and their sum are exact, so
    the output equals the oracle bit for bit."""
    M, N, K = 64, 256, 1024
    rng = np.random.default_rng(9)
    nb = K // 32
    if fmt == "q8_0":
        codes = rng.integers(-8, 9, (N, nb, 32))
        codes[:, :, 11] = -128
    else:
        codes = rng.integers(-8, 8, (N, nb, 32))
    d = rng.integers(1, 8, (N, nb)) * 2.0 ** -24
    W = blocks_from(fmt, codes, d)
    Xq = rng.integers(-8, 9, (M, K)).astype(np.int8)
    dx = rng.choice([0.5, 1.0, 2.0], (M, nb)).astype(np.float32)
    # |y| / 2^-25 < 2^24: per block at most 31 * 8 * 8 + 128 * 8 in units of 2^-24 * 0.5
    assert nb * (31 * 64 + 1024) * 7 * 2 / 0.5 < 2 ** 24
    say("qmm subnormal scales", fmt)
    Y = torch.full((M, N), float("nan"), device=DEV)
    f = bqm.qmm_q8_0 if fmt == "q8_0" else bqm.qmm_q4_0
    f(packed(fmt, torch.from_numpy(W).to(DEV), N, K), torch.from_numpy(Xq).to(DEV),
      torch.from_numpy(dx).to(DEV), Y, M, N, K)
    o = oracle.qmm_q8_0 if fmt == "q8_0" else oracle.qmm_q4_0
    Yr, _ = o(W, Xq, dx, N, K)
    assert np.array_equal(host(Y).astype(np.float64), Yr)


def test_qmm_q8_code_minus_128_quantized_activations():
    """Q8_0 weight code -128 against activations from the quantizer (codes up to +-127):
    the integer block sums reach 32 * 128 * 127 and stay exact."""
    M, N, K = 96, 200, 2048
    rng = np.random.default_rng(13)
    codes = rng.integers(-128, 128, (N, K // 32, 32))
    codes[::2] = -128
    W = blocks_from("q8_0", codes, rng.uniform(0.001, 0.02, (N, K // 32)))
    Xh = rng.standard_normal((M, K)).astype(np.float32)
    Xh[0] = 1.0  # every activation code 127: the all -128 rows reach the extreme block sum
    X = torch.from_numpy(Xh).to(DEV)
    Xq = torch.empty((M, K), dtype=torch.int8, device=DEV)
    dx = torch.empty((M, K // 32), device=DEV)
    bqm.bqm_quantize_q8_act(X, Xq, dx, M, K)
    say("qmm q8 -128")
    Y = torch.full((M, N), float("nan"), device=DEV)
    bqm.qmm_q8_0(packed("q8_0", torch.from_numpy(W).to(DEV), N, K), Xq, dx, Y, M, N, K)
    Yr, S, isum = oracle.qmm_q8_0(W, host(Xq), host(dx), N, K, want_isum=True)
    assert isum.min() == -32 * 128 * 127
    check_close(host(Y), Yr, S, "qmm q8 -128")
