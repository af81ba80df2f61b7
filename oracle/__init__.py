"""Python access to the plain CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only callers.  The GPU library never
imports this package, and this package never imports the GPU library.

All functions take and return NumPy arrays.  Weights are interchange bytes
(``uint8``, [rows, K/32 * block_bytes]); see oracle.c for the definitions.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test may point at another build of oracle.c (the planted-mistake check does).
_LIB_OVERRIDE = os.environ.get("BQM_ORACLE_LIB")

FMT = {"q4_0": 2, "q8_0": 8}
BLOCK_BYTES = {"q4_0": 18, "q8_0": 34}

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (no fast-math, no FP contraction, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_half_to_double.restype = ctypes.c_double
        lib.oracle_decode_row.argtypes = [I32, P, I64, P]
        lib.oracle_qmv.argtypes = [I32, P, P, I64, I64, I64, P, P]
        lib.oracle_qmv_id.argtypes = [I32, P, I64, I64, I64, P, I64, I64, P, I64, I64, P, P]
        lib.oracle_qmv_id_gate_up.argtypes = [I32, P, P, I64, I64, I64, P, I64, I64, P, I64, I64, P, P]
        lib.oracle_silu.argtypes = [ctypes.c_double]
        lib.oracle_silu.restype = ctypes.c_double
        lib.oracle_quantize_q8_act.argtypes = [P, I64, I64, P, P]
        lib.oracle_qmm_q8_0.argtypes = [P, P, P, I64, I64, I64, P, P, P]
        lib.oracle_qmm_q4_0.argtypes = [P, P, P, I64, I64, I64, P, P, P]
        lib.oracle_qmv_id_sum.argtypes = [I32, P, I64, I64, I64, P, P, I64, I64, P, I64, I64, P, P]
        lib.oracle_qmm_id.argtypes = [I32, P, I64, I64, I64, P, I64, I64, P, P, I64, I64, P, P]
        lib.oracle_threads.restype = I32
        lib.oracle_set_threads.argtypes = [I32]
        for f in ("oracle_decode_row", "oracle_qmv", "oracle_qmv_id", "oracle_qmv_id_gate_up", "oracle_qmv_id_sum",
                  "oracle_quantize_q8_act", "oracle_qmm_q8_0", "oracle_qmm_q4_0", "oracle_qmm_id"):
            getattr(lib, f).restype = I32
        _lib = lib
    return _lib


def _p(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


def threads() -> int:
    return _load().oracle_threads()


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def half_to_double(bits: int) -> float:
    return _load().oracle_half_to_double(int(bits) & 0xFFFF)


def decode_row(fmt: str, blocks, K: int) -> np.ndarray:
    b = _c(blocks, np.uint8)
    w = np.empty(K, np.float64)
    _check(_load().oracle_decode_row(FMT[fmt], _p(b), K, _p(w)), "decode_row")
    return w


def qmv(fmt: str, W, X, N: int, K: int):
    """Y, S = oracle of Y[M][N] = X[M][K] . dequant(W[N][K])^T (fp64)."""
    Wb = _c(W, np.uint8)
    Xf = _c(X, np.float32).reshape(-1, K)
    M = Xf.shape[0]
    assert Wb.size == N * (K // 32) * BLOCK_BYTES[fmt]
    Y = np.empty((M, N), np.float64)
    S = np.empty((M, N), np.float64)
    _check(_load().oracle_qmv(FMT[fmt], _p(Wb), _p(Xf), M, N, K, _p(Y), _p(S)), "qmv")
    return Y, S


def qmv_id(fmt: str, W, E: int, N: int, K: int, ids, X, x_tok_stride: int, x_slot_stride: int):
    """Y, S [T][top_k][N] of the expert-indexed product (negative id -> zero row)."""
    Wb = _c(W, np.uint8)
    ids32 = _c(ids, np.int32)
    T, top_k = ids32.shape
    Xf = _c(X, np.float32).reshape(-1)
    assert Wb.size == E * N * (K // 32) * BLOCK_BYTES[fmt]
    Y = np.empty((T, top_k, N), np.float64)
    S = np.empty((T, top_k, N), np.float64)
    _check(_load().oracle_qmv_id(FMT[fmt], _p(Wb), E, N, K, _p(ids32), T, top_k, _p(Xf),
                                 x_tok_stride, x_slot_stride, _p(Y), _p(S)), "qmv_id")
    return Y, S


def qmv_id_sum(fmt: str, W, E: int, N: int, K: int, ids, weights, X, x_tok_stride: int,
               x_slot_stride: int):
    """Y, S [T][N]: the router-weighted sum over each token's routed experts."""
    Wb = _c(W, np.uint8)
    ids32 = _c(ids, np.int32)
    T, top_k = ids32.shape
    wf = _c(weights, np.float32).reshape(T, top_k)
    Xf = _c(X, np.float32).reshape(-1)
    assert Wb.size == E * N * (K // 32) * BLOCK_BYTES[fmt]
    Y = np.empty((T, N), np.float64)
    S = np.empty((T, N), np.float64)
    _check(_load().oracle_qmv_id_sum(FMT[fmt], _p(Wb), E, N, K, _p(ids32), _p(wf), T, top_k,
                                     _p(Xf), x_tok_stride, x_slot_stride, _p(Y), _p(S)),
           "qmv_id_sum")
    return Y, S


def silu(z):
    """silu(z) = z / (1 + e^-z) in double precision (the oracle's own, from C)."""
    return _load().oracle_silu(float(z))


def qmv_id_gate_up(fmt: str, Wg, Wu, E: int, N: int, K: int, ids, X, x_tok_stride: int,
                   x_slot_stride: int):
    """Y, S [T][top_k][N] of the fused gate+up product silu(Wg x) * (Wu x) (padding -> 0)."""
    Wgb, Wub = _c(Wg, np.uint8), _c(Wu, np.uint8)
    ids32 = _c(ids, np.int32)
    T, top_k = ids32.shape
    Xf = _c(X, np.float32).reshape(-1)
    assert Wgb.size == Wub.size == E * N * (K // 32) * BLOCK_BYTES[fmt]
    Y = np.empty((T, top_k, N), np.float64)
    S = np.empty((T, top_k, N), np.float64)
    _check(_load().oracle_qmv_id_gate_up(FMT[fmt], _p(Wgb), _p(Wub), E, N, K, _p(ids32), T, top_k,
                                         _p(Xf), x_tok_stride, x_slot_stride, _p(Y), _p(S)),
           "qmv_id_gate_up")
    return Y, S


def quantize_q8_act(X, K: int):
    """Xq int8 [M][K], dx fp32 [M][K/32]."""
    Xf = _c(X, np.float32).reshape(-1, K)
    M = Xf.shape[0]
    Xq = np.empty((M, K), np.int8)
    dx = np.empty((M, K // 32), np.float32)
    _check(_load().oracle_quantize_q8_act(_p(Xf), M, K, _p(Xq), _p(dx)), "quantize_q8_act")
    return Xq, dx


def qmm_q8_0(W, Xq, dx, N: int, K: int, want_isum: bool = False):
    """Y, S [M][N] (fp64) and optionally the exact block sums isum [M][N][K/32]."""
    Wb = _c(W, np.uint8)
    Xq8 = _c(Xq, np.int8).reshape(-1, K)
    M = Xq8.shape[0]
    dxf = _c(dx, np.float32).reshape(M, K // 32)
    Y = np.empty((M, N), np.float64)
    S = np.empty((M, N), np.float64)
    isum = np.empty((M, N, K // 32), np.int32) if want_isum else None
    _check(_load().oracle_qmm_q8_0(_p(Wb), _p(Xq8), _p(dxf), M, N, K, _p(isum), _p(Y), _p(S)),
           "qmm_q8_0")
    return (Y, S, isum) if want_isum else (Y, S)


def qmm_q4_0(W, Xq, dx, N: int, K: int, want_isum: bool = False):
    """The Q4_0-weight prefill product: Y, S [M][N] and optionally isum [M][N][K/32]."""
    Wb = _c(W, np.uint8)
    Xq8 = _c(Xq, np.int8).reshape(-1, K)
    M = Xq8.shape[0]
    dxf = _c(dx, np.float32).reshape(M, K // 32)
    Y = np.empty((M, N), np.float64)
    S = np.empty((M, N), np.float64)
    isum = np.empty((M, N, K // 32), np.int32) if want_isum else None
    _check(_load().oracle_qmm_q4_0(_p(Wb), _p(Xq8), _p(dxf), M, N, K, _p(isum), _p(Y), _p(S)),
           "qmm_q4_0")
    return (Y, S, isum) if want_isum else (Y, S)


def qmm_id(fmt: str, W, E: int, N: int, K: int, ids, Xq, dx, x_tok_rows: int, x_slot_rows: int):
    """Y, S [T][top_k][N] of the expert-indexed prefill product (negative id -> zero row)."""
    Wb = _c(W, np.uint8)
    ids32 = _c(ids, np.int32)
    T, top_k = ids32.shape
    Xq8 = _c(Xq, np.int8).reshape(-1, K)
    dxf = _c(dx, np.float32).reshape(Xq8.shape[0], K // 32)
    assert Wb.size == E * N * (K // 32) * BLOCK_BYTES[fmt]
    Y = np.empty((T, top_k, N), np.float64)
    S = np.empty((T, top_k, N), np.float64)
    _check(_load().oracle_qmm_id(FMT[fmt], _p(Wb), E, N, K, _p(ids32), T, top_k, _p(Xq8), _p(dxf),
                                 x_tok_rows, x_slot_rows, _p(Y), _p(S)), "qmm_id")
    return Y, S
