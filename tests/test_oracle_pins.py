"""Pins for the CPU oracle: hand-worked blocks, closed forms, invariants and an
independent NumPy brute force on tiny inputs.  CPU only."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import gen
from tests import _npref

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")))


def _x_named(name, K=32):
    j = np.arange(K, dtype=np.float32)
    return {
        "ones": np.ones(K, np.float32),
        "first16": (j < 16).astype(np.float32),
        "j_plus_1": j + 1,
        "j": j,
        "alternating": np.where(j % 2 == 0, 1.0, -1.0).astype(np.float32),
    }[name]


# --- binary16 decoding: all 65,536 patterns against numpy's conversion ---------------

def test_half_to_double_exhaustive(oracle_lib):
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle_lib.half_to_double(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin].view(np.uint64), ref[fin].view(np.uint64))  # bitwise, incl. -0
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got) & (got > 0), np.isinf(ref) & (ref > 0))
    assert np.array_equal(np.isinf(got) & (got < 0), np.isinf(ref) & (ref < 0))


# --- hand-worked blocks ---------------------------------------------------------------

@pytest.mark.parametrize("case", GOLDEN["qmv"], ids=lambda c: c["name"])
def test_hand_worked_qmv(oracle_lib, case):
    W = np.frombuffer(bytes.fromhex(case["block"]), np.uint8)
    x = _x_named(case["x"])
    Y, S = oracle_lib.qmv(case["fmt"], W, x[None, :], 1, 32)
    assert Y[0, 0] == case["y"]


def _qx_named(name, K):
    j = np.arange(K)
    if name == "j_minus_16":
        return (j - 16).astype(np.int8)
    if name == "block0_j_minus_16_block1_ones":
        return np.where(j < 32, j - 16, 1).astype(np.int8)
    raise KeyError(name)


@pytest.mark.parametrize("case", GOLDEN["qmm"], ids=lambda c: c["name"])
def test_hand_worked_qmm(oracle_lib, case):
    K = case["K"]
    blocks = b""
    for qw, db in zip(case["qw"], case["dw_bits"]):
        blocks += int(db).to_bytes(2, "little") + np.array(qw, np.int8).tobytes()
    W = np.frombuffer(blocks, np.uint8)
    qx = _qx_named(case["qx"], K)[None, :]
    dx = np.array(case["dx"], np.float32)[None, :]
    Y, S, isum = oracle_lib.qmm_q8_0(W, qx, dx, 1, K, want_isum=True)
    assert list(isum[0, 0]) == case["isum"]
    assert Y[0, 0] == case["y"]


def test_hand_worked_quantize_q8_act(oracle_lib):
    case = GOLDEN["quantize_q8_act"][0]
    x = np.zeros(32, np.uint32)
    x[:6] = [int(b, 16) for b in case["x_bits_first6"]]
    x = x.view(np.float32)
    Xq, dx = oracle_lib.quantize_q8_act(x[None, :], 32)
    assert dx[0, 0] == case["dx"]
    assert list(Xq[0, :6]) == case["q_first6"]
    assert not Xq[0, 6:].any()


# --- decoding against an independent NumPy decoder ------------------------------------

@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
def test_decode_matches_numpy(oracle_lib, fmt):
    rng = np.random.default_rng(1)
    N, K = 7, 96
    bb = 18 if fmt == "q4_0" else 34
    W = rng.integers(0, 256, size=(N, K // 32, bb), dtype=np.uint8)
    # scales: random finite binary16 patterns, including subnormals and negatives
    d = rng.integers(0, 0x7C00, size=(N, K // 32), dtype=np.uint16) | (
        rng.integers(0, 2, size=(N, K // 32), dtype=np.uint16) << 15)
    d[0, 0] = 0x0001  # smallest subnormal
    d[0, 1] = 0x8000  # -0
    W[:, :, 0:2] = d[:, :, None].view(np.uint8).reshape(N, K // 32, 2)
    ref = _npref.dequant(fmt, W.reshape(-1), N, K)
    for n in range(N):
        got = oracle_lib.decode_row(fmt, W[n].reshape(-1), K)
        assert np.array_equal(got, ref[n])


# --- products against a dense brute force ---------------------------------------------

@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("M,N,K", [(1, 5, 96), (3, 4, 64), (8, 3, 160)])
def test_qmv_bruteforce(oracle_lib, fmt, M, N, K):
    w = gen.normal((N, K), ("pin", fmt, M, N, K), std=0.02)
    W = (gen.encode_q4_0(w) if fmt == "q4_0" else gen.encode_q8_0(w)).numpy()
    X = gen.normal((M, K), ("pin-x", fmt, M, N, K)).numpy()
    Y, S = oracle_lib.qmv(fmt, W, X, N, K)
    Yr, Sr = _npref.qmv(fmt, W, X, N, K)
    assert Y.shape == (M, N)
    assert np.all(np.abs(Y - Yr) <= 1e-12 * Sr)
    assert np.allclose(S, Sr, rtol=1e-12, atol=0)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
def test_qmv_exact_probe(oracle_lib, fmt):
    """Integer inputs and power-of-two scales: every sum is exact, so equality is bitwise."""
    M, N, K = 4, 6, 128
    W = (gen.raw_q4_0(N, K, ("probe", 1)) if fmt == "q4_0" else gen.raw_q8_0(N, K, ("probe", 2))).numpy()
    X = gen.small_int((M, K), ("probe-x",)).numpy()
    Y, _ = oracle_lib.qmv(fmt, W, X, N, K)
    Yr, _ = _npref.qmv(fmt, W, X, N, K)
    assert np.array_equal(Y, Yr)


def _set_scales(W, fmt, N, K, fn):
    bb = 18 if fmt == "q4_0" else 34
    blk = W.reshape(N, K // 32, bb).copy()
    d = blk[:, :, 0:2].copy().view(np.float16)[:, :, 0]
    d = fn(d).astype(np.float16)
    blk[:, :, 0:2] = d[:, :, None].view(np.uint8).reshape(N, K // 32, 2)
    return blk.reshape(W.shape)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
def test_invariants(oracle_lib, fmt):
    M, N, K = 2, 5, 96
    w = gen.normal((N, K), ("inv", fmt), std=0.02)
    W = (gen.encode_q4_0(w) if fmt == "q4_0" else gen.encode_q8_0(w)).numpy()
    X = gen.normal((M, K), ("inv-x", fmt)).numpy()
    Y, S = oracle_lib.qmv(fmt, W, X, N, K)
    # neutral codes (8 for Q4_0, 0 for Q8_0) give exactly zero for any scale and input
    bb = 18 if fmt == "q4_0" else 34
    Wn = W.reshape(N, K // 32, bb).copy()
    Wn[:, :, 2:] = 0x88 if fmt == "q4_0" else 0
    Yn, Sn = oracle_lib.qmv(fmt, Wn.reshape(W.shape), X, N, K)
    assert np.all(Yn == 0) and np.all(Sn == 0)
    # zero scales give exactly zero
    Y0, _ = oracle_lib.qmv(fmt, _set_scales(W, fmt, N, K, lambda d: d * 0), X, N, K)
    assert np.all(Y0 == 0)
    # doubling every scale doubles every output bitwise
    Y2, _ = oracle_lib.qmv(fmt, _set_scales(W, fmt, N, K, lambda d: d * 2), X, N, K)
    assert np.array_equal(Y2, 2 * Y)
    # linearity in x (within fp64 rounding); dyadic inputs so that X1 + X2 is exact in fp32
    X1 = gen.small_int((M, K), ("inv-x1", fmt), -64, 64).numpy() / np.float32(16)
    X2 = gen.small_int((M, K), ("inv-x2", fmt), -64, 64).numpy() / np.float32(8)
    Y, S = oracle_lib.qmv(fmt, W, X1, N, K)
    Ya, Sa = oracle_lib.qmv(fmt, W, X1 + X2, N, K)
    Yb, Sb = oracle_lib.qmv(fmt, W, X2, N, K)
    assert np.all(np.abs(Ya - (Y + Yb)) <= 1e-12 * (S + Sb))


@pytest.mark.parametrize("x_slot_stride", ["broadcast", "per_slot"])
def test_qmv_id_bruteforce(oracle_lib, x_slot_stride):
    E, N, K, T, top_k = 5, 6, 64, 3, 2
    w = gen.normal((E * N, K), ("id", 1), std=0.02)
    W = gen.encode_q4_0(w).numpy()
    ids = np.array([[3, 0], [-1, 4], [1, 3]], np.int32)
    if x_slot_stride == "broadcast":
        X = gen.normal((T, K), ("id-x", 1)).numpy()
        xts, xss = K, 0
    else:
        X = gen.normal((T, top_k, K), ("id-x", 2)).numpy()
        xts, xss = top_k * K, K
    Y, S = oracle_lib.qmv_id("q4_0", W, E, N, K, ids, X, xts, xss)
    Wd = _npref.dequant("q4_0", W, E * N, K).reshape(E, N, K)
    Xf = X.reshape(-1)
    for t in range(T):
        for s in range(top_k):
            e = ids[t, s]
            if e < 0:
                assert np.all(Y[t, s] == 0) and np.all(S[t, s] == 0)
                continue
            x = Xf[t * xts + s * xss: t * xts + s * xss + K].astype(np.float64)
            yr = Wd[e] @ x
            sr = np.abs(Wd[e]) @ np.abs(x)
            assert np.all(np.abs(Y[t, s] - yr) <= 1e-12 * sr)
            assert np.all(sr > 0) and np.allclose(S[t, s], sr, rtol=1e-12, atol=0)


def test_qmv_id_rejects_out_of_range_id(oracle_lib):
    E, N, K = 2, 3, 32
    W = gen.raw_q4_0(E * N, K, ("rej",)).numpy()
    with pytest.raises(ValueError):
        oracle_lib.qmv_id("q4_0", W, E, N, K, np.array([[2]], np.int32),
                          np.zeros(K, np.float32), K, 0)


# --- router-weighted sum over each token's experts ---------------------------------------

@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
def test_qmv_id_sum_bruteforce(oracle_lib, fmt):
    """Y[t] = sum_s w[t][s] * W[e_ts] x_ts against a dense NumPy product per slot, with a
    padding slot and one expert chosen twice by the same token."""
    E, N, K, T, top_k = 5, 6, 96, 3, 3
    enc = gen.encode_q4_0 if fmt == "q4_0" else gen.encode_q8_0
    W = enc(gen.normal((E * N, K), ("idsum", fmt), std=0.05)).numpy()
    ids = np.array([[3, 0, 3], [-1, 4, 2], [1, 3, 0]], np.int32)
    w = gen.router_weights(T, top_k, ("idsum-w", fmt))
    w[2, 1] = -w[2, 1]  # any fp32 weight is valid; a negative one checks |w| in the scale
    X = gen.normal((T, top_k, K), ("idsum-x", fmt)).numpy()
    Y, S = oracle_lib.qmv_id_sum(fmt, W, E, N, K, ids, w, X, top_k * K, K)
    Wd = _npref.dequant(fmt, W, E * N, K).reshape(E, N, K)
    for t in range(T):
        yr = np.zeros(N)
        sr = np.zeros(N)
        for s in range(top_k):
            e = ids[t, s]
            if e < 0:
                continue
            x = X[t, s].astype(np.float64)
            yr += float(w[t, s]) * (Wd[e] @ x)
            sr += abs(float(w[t, s])) * (np.abs(Wd[e]) @ np.abs(x))
        assert np.all(np.abs(Y[t] - yr) <= 1e-12 * sr)
        assert np.allclose(S[t], sr, rtol=1e-12, atol=0)


def test_qmv_id_sum_one_hot_and_scaling(oracle_lib):
    """One-hot weights pick one slot's expert product (equal to qmv_id's row bit for bit);
    doubling every weight doubles every output bit for bit; all-padding tokens give 0."""
    E, N, K, T, top_k = 4, 5, 64, 3, 2
    W = gen.encode_q4_0(gen.normal((E * N, K), ("idsum1",), std=0.05)).numpy()
    ids = np.array([[2, 1], [0, 3], [-1, -1]], np.int32)
    X = gen.normal((T, top_k, K), ("idsum1-x",)).numpy()
    Yid, _ = oracle_lib.qmv_id("q4_0", W, E, N, K, ids, X, top_k * K, K)
    onehot = np.array([[0, 1], [1, 0], [1, 0]], np.float32)
    Y, S = oracle_lib.qmv_id_sum("q4_0", W, E, N, K, ids, onehot, X, top_k * K, K)
    assert np.array_equal(Y[0], Yid[0, 1]) and np.array_equal(Y[1], Yid[1, 0])
    assert np.all(Y[2] == 0) and np.all(S[2] == 0)
    w = gen.router_weights(T, top_k, ("idsum1-w",))
    Y1, _ = oracle_lib.qmv_id_sum("q4_0", W, E, N, K, ids, w, X, top_k * K, K)
    Y2, _ = oracle_lib.qmv_id_sum("q4_0", W, E, N, K, ids, 2 * w, X, top_k * K, K)
    assert np.array_equal(Y2, 2 * Y1)


# --- fused gate+up: silu and the product ------------------------------------------------

def test_silu_closed_forms(oracle_lib):
    """silu(z) = z * logistic(z): logistic(0) = 1/2, logistic(1) = e/(1+e), logistic(2) =
    e^2/(1+e^2) (textbook values); silu(z) - silu(-z) = z because logistic(z) +
    logistic(-z) = 1; silu(z) -> z for large z and -> 0 (from below) for very negative z."""
    import math
    assert oracle_lib.silu(0.0) == 0.0
    assert oracle_lib.silu(1.0) == pytest.approx(0.7310585786300049, rel=1e-15, abs=0)
    assert oracle_lib.silu(2.0) == pytest.approx(2 * 0.8807970779778823, rel=1e-15, abs=0)
    assert oracle_lib.silu(-1.0) == pytest.approx(-0.2689414213699951, rel=1e-15, abs=0)
    for z in (0.25, 1.0, 3.5, 7.0, 20.0):
        assert oracle_lib.silu(z) - oracle_lib.silu(-z) == pytest.approx(z, rel=1e-14, abs=0)
    assert oracle_lib.silu(60.0) == 60.0
    assert -1e-20 < oracle_lib.silu(-60.0) < 0
    assert oracle_lib.silu(-2.0) == pytest.approx(-2 / (1 + math.e ** 2), rel=1e-15, abs=0)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
def test_gate_up_bruteforce(oracle_lib, fmt):
    """Fused gate+up against the NumPy brute force: silu(Wg x) * (Wu x) per slot, padding
    slots zero, and the tolerance scale is at least |y| * 1e-3 and zero for padding."""
    E, N, K, T, top_k = 4, 5, 96, 3, 2
    enc = gen.encode_q4_0 if fmt == "q4_0" else gen.encode_q8_0
    Wg = enc(gen.normal((E * N, K), ("gu", "g", fmt), std=0.05)).numpy()
    Wu = enc(gen.normal((E * N, K), ("gu", "u", fmt), std=0.05)).numpy()
    ids = np.array([[3, 0], [-1, 2], [1, 3]], np.int32)
    X = gen.normal((T, top_k, K), ("gu-x", fmt)).numpy()
    Y, S = oracle_lib.qmv_id_gate_up(fmt, Wg, Wu, E, N, K, ids, X, top_k * K, K)
    Gd = _npref.dequant(fmt, Wg, E * N, K).reshape(E, N, K)
    Ud = _npref.dequant(fmt, Wu, E * N, K).reshape(E, N, K)
    for t in range(T):
        for s in range(top_k):
            e = ids[t, s]
            if e < 0:
                assert np.all(Y[t, s] == 0) and np.all(S[t, s] == 0)
                continue
            x = X[t, s].astype(np.float64)
            g, u = Gd[e] @ x, Ud[e] @ x
            yr = g / (1 + np.exp(-g)) * u
            assert np.all(np.abs(Y[t, s] - yr) <= 1e-12 * (np.abs(yr) + np.abs(g * u) + 1e-300))
            Sr = _npref.gate_up_scale(g, u, np.abs(Gd[e]) @ np.abs(x), np.abs(Ud[e]) @ np.abs(x))
            assert np.allclose(S[t, s], Sr, rtol=1e-9, atol=0)


# --- activation quantizer: special cases and properties --------------------------------

def _half_away_exact(v: np.float32) -> int:
    f = Fraction(float(v))
    r = int(abs(f) + Fraction(1, 2))  # floor(|v| + 1/2) in exact arithmetic
    return r if f >= 0 else -r


def test_quantize_q8_act_properties(oracle_lib):
    M, K = 6, 256
    X = gen.normal((M, K), ("qa",)).numpy()
    X[1, 32:64] = 0.0                       # zero block
    X[2, 64:96] = np.float32(2.0 ** -149) * np.arange(-16, 16, dtype=np.float32)  # dx = 16*2^-149/127 underflows to 0
    X[4, 96:128] = np.float32(2.0 ** -140) * np.arange(1, 33, dtype=np.float32)   # subnormal, non-zero dx
    X[3, :32] = np.float32(0.5) * np.arange(-16, 16, dtype=np.float32)  # many exact halves
    Xq, dx = oracle_lib.quantize_q8_act(X, K)
    nb = K // 32
    assert dx[1, 1] == 0 and not Xq[1, 32:64].any()
    assert dx[2, 2] == 0 and not Xq[2, 64:96].any()
    for m in range(M):
        for b in range(nb):
            xb = X[m, 32 * b:32 * b + 32]
            a = np.max(np.abs(xb))
            d = np.float32(a) / np.float32(127.0)
            assert dx[m, b] == (d if d != 0 else 0.0)
            if d == 0:
                continue
            qb = Xq[m, 32 * b:32 * b + 32].astype(int)
            for j in range(32):
                v = np.float32(xb[j]) / d
                assert qb[j] == max(-127, min(127, _half_away_exact(v)))
                assert abs(float(xb[j]) - qb[j] * float(d)) <= 0.5 * float(d) * (1 + 1e-6)
            k = int(np.argmax(np.abs(xb)))
            assert abs(qb[k]) == 127
    # sign symmetry and power-of-two scaling
    Xq_neg, dx_neg = oracle_lib.quantize_q8_act(-X, K)
    assert np.array_equal(Xq_neg, -Xq) and np.array_equal(dx_neg, dx)
    normal_rows = [0, 1, 3, 5]  # rows 2 and 4 hold subnormal blocks, where scaling is not exact
    Xq2, dx2 = oracle_lib.quantize_q8_act(X[normal_rows] * 4, K)
    assert np.array_equal(Xq2, Xq[normal_rows]) and np.array_equal(dx2, dx[normal_rows] * 4)


# --- prefill product ----------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(3, 4, 96), (5, 2, 64)])
def test_qmm_bruteforce(oracle_lib, M, N, K):
    W = gen.raw_q8_0(N, K, ("qmm", M, N, K), scales=(0.001, 0.0173, -0.02), codes=(-127, 127)).numpy()
    rng = np.random.default_rng(7)
    Xq = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    dx = (rng.random((M, K // 32)) * 0.05).astype(np.float32)
    Y, S, isum = oracle_lib.qmm_q8_0(W, Xq, dx, N, K, want_isum=True)
    iref = _npref.qmm_isum(W, Xq, N, K)
    assert np.array_equal(isum, iref)
    dw = _npref.q8_scales(W, N, K)                                   # [N][nb]
    scale = dw[None, :, :] * dx.astype(np.float64)[:, None, :]       # [M][N][nb]
    Yr = np.einsum("mnb,mnb->mn", scale, iref.astype(np.float64))
    assert np.all(np.abs(Y - Yr) <= 1e-12 * S)
    assert np.allclose(S, _npref.qmm_scale("q8_0", W, Xq, dx, N, K), rtol=1e-12, atol=0)


def test_qmm_single_block_is_one_product(oracle_lib):
    K = 32
    W = gen.raw_q8_0(3, K, ("qmm1",), scales=(0.5, 2.0), codes=(-127, 127)).numpy()
    Xq = np.arange(-16, 16, dtype=np.int8)[None, :]
    dx = np.array([[0.25]], np.float32)
    Y, S, isum = oracle_lib.qmm_q8_0(W, Xq, dx, 3, K, want_isum=True)
    dw = _npref.q8_scales(W, 3, K)[:, 0]
    assert np.array_equal(Y[0], dw * 0.25 * isum[0, :, 0])


@pytest.mark.parametrize("M,N,K", [(3, 4, 96), (2, 5, 64)])
def test_qmm_q4_bruteforce(oracle_lib, M, N, K):
    """Q4_0 prefill product: exact block sums against a NumPy decode of the nibbles, and
    the scaled sum against a dense fp64 contraction."""
    W = gen.raw_q4_0(N, K, ("qmm4", M, N, K), scales=(0.001, 0.0173, -0.02), codes=(0, 15)).numpy()
    rng = np.random.default_rng(11)
    Xq = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    dx = (rng.random((M, K // 32)) * 0.05).astype(np.float32)
    Y, S, isum = oracle_lib.qmm_q4_0(W, Xq, dx, N, K, want_isum=True)
    iref = _npref.qmm_q4_isum(W, Xq, N, K)
    assert np.array_equal(isum, iref)
    dw = _npref.q4_scales(W, N, K)
    scale = dw[None, :, :] * dx.astype(np.float64)[:, None, :]
    Yr = np.einsum("mnb,mnb->mn", scale, iref.astype(np.float64))
    assert np.all(np.abs(Y - Yr) <= 1e-12 * S)
    assert np.allclose(S, _npref.qmm_scale("q4_0", W, Xq, dx, N, K), rtol=1e-12, atol=0)


def test_qmm_q4_extreme_codes(oracle_lib):
    """Nibble 0 is the code -8 and nibble 15 the code +7: all-0x00 bytes against all-ones
    activations give -8 per weight, all-0xFF bytes +7."""
    K = 64
    W = gen.raw_q4_0(2, K, ("qmm4x",), scales=(1.0,), codes=(0, 0)).numpy().reshape(2, 2, 18)
    W[1, :, 2:] = 0xFF
    Xq = np.ones((1, K), np.int8)
    dx = np.array([[1.0, 0.5]], np.float32)
    Y, S, isum = oracle_lib.qmm_q4_0(W.reshape(-1), Xq, dx, 2, K, want_isum=True)
    assert np.array_equal(isum[0], [[-256, -256], [224, 224]])
    assert np.array_equal(Y[0], [-256 * 1.5, 224 * 1.5])


def test_qmm_q4_matches_qmv_on_dequantized_activations(oracle_lib):
    """qmm with activations dx*qx equals the fp64 Q4_0 GEMV with them."""
    M, N, K = 2, 3, 64
    W = gen.raw_q4_0(N, K, ("qmm4-qmv",), scales=(0.25, 0.5), codes=(0, 15)).numpy()
    rng = np.random.default_rng(5)
    Xq = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    dx = np.array([[0.5, 2.0], [0.125, 1.0]], np.float32)
    Y, _ = oracle_lib.qmm_q4_0(W, Xq, dx, N, K)
    Xd = (Xq.reshape(M, 2, 32) * dx[:, :, None]).reshape(M, K).astype(np.float32)
    Y2, _ = oracle_lib.qmv("q4_0", W, Xd, N, K)
    assert np.array_equal(Y, Y2)


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
@pytest.mark.parametrize("rows", ["broadcast", "per_slot"])
def test_qmm_id_bruteforce(oracle_lib, fmt, rows):
    """Expert-indexed prefill product: per slot, exact block sums of the selected expert's
    codes with the slot's input row (NumPy decode), scaled in fp64; padding slots 0."""
    E, N, K, T, top_k = 4, 5, 96, 3, 2
    raw = gen.raw_q8_0 if fmt == "q8_0" else gen.raw_q4_0
    codes = (-127, 127) if fmt == "q8_0" else (0, 15)
    W = raw(E * N, K, ("qmmid", fmt), scales=(0.001, 0.0173, -0.02), codes=codes).numpy()
    ids = np.array([[3, 0], [-1, 2], [1, 3]], np.int32)
    nrows, xt, xs = (T, 1, 0) if rows == "broadcast" else (T * top_k, top_k, 1)
    rng = np.random.default_rng(13)
    Xq = rng.integers(-127, 128, size=(nrows, K), dtype=np.int8)
    dx = (rng.random((nrows, K // 32)) * 0.05).astype(np.float32)
    Y, S = oracle_lib.qmm_id(fmt, W, E, N, K, ids, Xq, dx, xt, xs)
    nb = K // 32
    bb = 34 if fmt == "q8_0" else 18
    for t in range(T):
        for s in range(top_k):
            e = ids[t, s]
            if e < 0:
                assert np.all(Y[t, s] == 0) and np.all(S[t, s] == 0)
                continue
            r = t * xt + s * xs
            We = W.reshape(E, N * nb * bb)[e]
            isum = (_npref.qmm_isum if fmt == "q8_0" else _npref.qmm_q4_isum)(We, Xq[r:r + 1], N, K)[0]
            dw = (_npref.q8_scales if fmt == "q8_0" else _npref.q4_scales)(We, N, K)
            yr = (dw * dx[r].astype(np.float64)[None, :] * isum).sum(axis=1)
            assert np.all(np.abs(Y[t, s] - yr) <= 1e-12 * S[t, s])
            Sr = _npref.qmm_scale(fmt, We, Xq[r:r + 1], dx[r:r + 1], N, K)[0]
            assert np.all(Sr > 0) and np.allclose(S[t, s], Sr, rtol=1e-12, atol=0)


def test_qmm_matches_qmv_on_dequantized_activations(oracle_lib):
    """qmm with activations dx*qx equals the fp64 product of the Q8_0 weights with them."""
    M, N, K = 2, 3, 64
    W = gen.raw_q8_0(N, K, ("qmm-qmv",), scales=(0.25, 0.5), codes=(-127, 127)).numpy()
    rng = np.random.default_rng(3)
    Xq = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    dx = np.array([[0.5, 2.0], [0.125, 1.0]], np.float32)
    Y, _ = oracle_lib.qmm_q8_0(W, Xq, dx, N, K)
    Xd = (Xq.reshape(M, 2, 32) * dx[:, :, None]).reshape(M, K).astype(np.float32)  # exact
    Y2, _ = oracle_lib.qmv("q8_0", W, Xd, N, K)
    assert np.array_equal(Y, Y2)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
def test_gate_up_scale_exact_inputs(oracle_lib, fmt):
    """The gate+up tolerance scale, term by term, on inputs where every sum is exact
    (power-of-two scales, small integer codes and inputs), so both sides see the same g, u,
    Sg and Su and the scale must agree to rounding: rtol 1e-12."""
    E, N, K, T, top_k = 3, 7, 128, 2, 2
    raw = gen.raw_q4_0 if fmt == "q4_0" else gen.raw_q8_0
    Wg, Wu = raw(E * N, K, ("gus", "g", fmt)).numpy(), raw(E * N, K, ("gus", "u", fmt)).numpy()
    ids = np.array([[2, 0], [1, -1]], np.int32)
    X = gen.small_int((T, K), ("gus-x", fmt)).numpy()
    Y, S = oracle_lib.qmv_id_gate_up(fmt, Wg, Wu, E, N, K, ids, X, K, 0)
    Gd = _npref.dequant(fmt, Wg, E * N, K).reshape(E, N, K)
    Ud = _npref.dequant(fmt, Wu, E * N, K).reshape(E, N, K)
    for t in range(T):
        for s in range(top_k):
            e = ids[t, s]
            if e < 0:
                continue
            x = X[t].astype(np.float64)
            g, u = Gd[e] @ x, Ud[e] @ x
            Sr = _npref.gate_up_scale(g, u, np.abs(Gd[e]) @ np.abs(x), np.abs(Ud[e]) @ np.abs(x))
            assert np.allclose(S[t, s], Sr, rtol=1e-12, atol=0)
            assert np.allclose(Y[t, s], _npref.silu(g) * u, rtol=1e-12, atol=1e-300)


def test_qmv_scale_is_sum_of_abs_products(oracle_lib):
    """The GEMV tolerance scale S = sum |w x| against |W| |x| on signed scales and inputs."""
    M, N, K = 3, 4, 96
    W = gen.raw_q8_0(N, K, ("qs",), scales=(0.001, 0.0173, -0.02), codes=(-127, 127)).numpy()
    X = gen.normal((M, K), ("qs-x",)).numpy()
    _, S = oracle_lib.qmv("q8_0", W, X, N, K)
    Wd = _npref.dequant("q8_0", W, N, K)
    assert np.allclose(S, np.abs(X.astype(np.float64)) @ np.abs(Wd).T, rtol=1e-12, atol=0)
