"""Independent NumPy brute force used to pin the oracle on small inputs.

Written separately from oracle.c on purpose: the blocks are decoded with
vectorised bit operations and numpy's own binary16 conversion, and products
are formed as one dense fp64 matrix product (a different summation order
from the oracle's sequential sums).
"""
import numpy as np


def dequant(fmt: str, W: np.ndarray, N: int, K: int) -> np.ndarray:
    """Dense fp64 weights [N][K] from interchange bytes."""
    nb = K // 32
    bb = 18 if fmt == "q4_0" else 34
    blk = np.asarray(W, np.uint8).reshape(N, nb, bb)
    d = blk[:, :, 0:2].copy().view(np.float16)[:, :, 0].astype(np.float64)  # little endian
    qs = blk[:, :, 2:]
    if fmt == "q4_0":
        codes = np.concatenate([qs & 0x0F, qs >> 4], axis=2).astype(np.int64) - 8
    else:
        codes = qs.view(np.int8).astype(np.int64)
    return (codes * d[:, :, None]).reshape(N, K)


def qmv(fmt, W, X, N, K):
    Wd = dequant(fmt, W, N, K)
    X64 = np.asarray(X, np.float32).astype(np.float64).reshape(-1, K)
    Y = X64 @ Wd.T
    S = np.abs(X64) @ np.abs(Wd).T
    return Y, S


def qmm_isum(Wq8, Xq, N, K):
    """Exact int64 block sums [M][N][nb] by a dense integer product per block."""
    nb = K // 32
    blk = np.asarray(Wq8, np.uint8).reshape(N, nb, 34)
    qw = blk[:, :, 2:].view(np.int8).astype(np.int64)             # [N][nb][32]
    qx = np.asarray(Xq, np.int8).astype(np.int64).reshape(-1, nb, 32)  # [M][nb][32]
    return np.einsum("mbj,nbj->mnb", qx, qw)


def q8_scales(Wq8, N, K):
    nb = K // 32
    blk = np.asarray(Wq8, np.uint8).reshape(N, nb, 34)
    return blk[:, :, 0:2].copy().view(np.float16)[:, :, 0].astype(np.float64)


def q4_codes(Wq4, N, K):
    """Signed Q4_0 codes [N][nb][32] (nibble - 8): low nibbles are weights 0..15 of a
    block, high nibbles weights 16..31."""
    nb = K // 32
    qs = np.asarray(Wq4, np.uint8).reshape(N, nb, 18)[:, :, 2:]
    return np.concatenate([qs & 0x0F, qs >> 4], axis=2).astype(np.int64) - 8


def q4_scales(Wq4, N, K):
    nb = K // 32
    blk = np.asarray(Wq4, np.uint8).reshape(N, nb, 18)
    return blk[:, :, 0:2].copy().view(np.float16)[:, :, 0].astype(np.float64)


def qmm_q4_isum(Wq4, Xq, N, K):
    """Exact int64 block sums [M][N][nb] of Q4_0 weight codes with int8 activations."""
    nb = K // 32
    qx = np.asarray(Xq, np.int8).astype(np.int64).reshape(-1, nb, 32)
    return np.einsum("mbj,nbj->mnb", qx, q4_codes(Wq4, N, K))


def q8_codes(Wq8, N, K):
    """Signed Q8_0 codes [N][nb][32]."""
    nb = K // 32
    return np.asarray(Wq8, np.uint8).reshape(N, nb, 34)[:, :, 2:].view(np.int8).astype(np.int64)


def qmm_scale(fmt, W, Xq, dx, N, K):
    """Tolerance scale of the prefill product, from its definition:
    S[m][n] = sum_b |d_w[n][b] * dx[m][b]| * sum_j |qw[n][32b+j] * qx[m][32b+j]|,
    with the absolute block sums formed as one dense integer contraction per block."""
    nb = K // 32
    codes = q8_codes(W, N, K) if fmt == "q8_0" else q4_codes(W, N, K)       # [N][nb][32]
    dw = q8_scales(W, N, K) if fmt == "q8_0" else q4_scales(W, N, K)        # [N][nb]
    qx = np.asarray(Xq, np.int8).astype(np.int64).reshape(-1, nb, 32)      # [M][nb][32]
    aisum = np.einsum("mbj,nbj->mnb", np.abs(qx), np.abs(codes)).astype(np.float64)
    scale = np.abs(dw)[None, :, :] * np.abs(np.asarray(dx, np.float32).astype(np.float64))[:, None, :]
    return (scale * aisum).sum(axis=2)


def silu(z):
    return z / (1.0 + np.exp(-z))


def gate_up_scale(g, u, Sg, Su):
    """Tolerance scale of silu(g) * u when g and u each carry an error within 1e-3 of
    their own scales Sg, Su: the bound of the first-order expansion with |silu'| <= 1.1,
    term by term, plus 1e-3 |y| for evaluating silu and the product in single precision."""
    y = silu(g) * u
    return 1.1 * Sg * (np.abs(u) + 1e-3 * Su) + np.abs(silu(g)) * Su + 1e-3 * np.abs(y)
