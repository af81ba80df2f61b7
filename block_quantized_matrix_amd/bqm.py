"""Thin Python binding of libbqm.so (the C ABI in include/bqm.h).

Argument marshalling only: every function passes device pointers (``tensor.data_ptr()``),
sizes and the current HIP stream of torch to the C entry point of the same name and
raises ``BqmError`` on a non-zero status.  All computation happens in the HIP kernels;
there is no fallback of any kind: if the library is missing, importing the functions
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# BQM_LIB names another build of the same library (a host-sanitizer build, in the tests)
LIB_PATH = os.environ.get("BQM_LIB") or os.path.join(_HERE, "libbqm.so")

Q4_0 = 2
Q8_0 = 8
FMT = {"q4_0": Q4_0, "q8_0": Q8_0}
QMV_MAX_M = 8
QMV_ID_MAX_T = 64
QMM_ID_MAX_T = 16384
QMV_ID_MAX_TOPK = 32
QMV_ID_MAX_E = 4096
NOALLOC_SLOT_FLOATS = 1 << 20

_lib = None


class BqmError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn}: {strerror(status)} (status {status})")
        self.status = status


def lib():
    """Load libbqm.so (raises OSError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        L.bqm_packed_bytes.argtypes = [I, I64, I64]
        L.bqm_packed_bytes.restype = SZ
        L.bqm_repack.argtypes = [I, P, P, I64, I64, P]
        L.bqm_unpack.argtypes = [I, P, P, I64, I64, P]
        L.qmv_q4_0.argtypes = [P, P, P, I, I64, I64, P]
        L.qmv_q8_0.argtypes = [P, P, P, I, I64, I64, P]
        L.qmv_id.argtypes = [I, P, I, I64, I64, P, I, I, P, I64, I64, P, P]
        L.qmv_id_gate_up.argtypes = [I, P, P, I, I64, I64, P, I, I, P, I64, I64, P, P]
        L.qmv_id_sum.argtypes = [I, P, I, I64, I64, P, P, I, I, P, I64, I64, P, P, P]
        L.qmv_id_sum_noalloc.argtypes = [I, P, I, I64, I64, P, P, I, I, P, I64, I64, P, P]
        L.bqm_quantize_q8_act.argtypes = [P, P, P, I64, I64, P]
        L.qmm_q8_0.argtypes = [P, P, P, P, I64, I64, I64, P]
        L.qmm_q4_0.argtypes = [P, P, P, P, I64, I64, I64, P]
        L.qmm_id.argtypes = [I, P, I, I64, I64, P, I, I, P, P, I64, I64, P, P]
        L.bqm_chain_workspace_bytes.argtypes = [I]
        L.bqm_chain_workspace_bytes.restype = SZ
        L.bqm_chain_prepare.argtypes = [P, I, P, P]
        L.qmv_chain.argtypes = [I, I, P, I, P]
        L.bqm_chain_status.argtypes = [P, P]
        for f in ("bqm_chain_prepare", "qmv_chain", "bqm_chain_status"):
            getattr(L, f).restype = I
        L.bqm_strerror.argtypes = [I]
        L.bqm_strerror.restype = ctypes.c_char_p
        for f in ("bqm_repack", "bqm_unpack", "qmv_q4_0", "qmv_q8_0", "qmv_id", "qmv_id_gate_up",
                  "qmv_id_sum", "qmv_id_sum_noalloc", "bqm_quantize_q8_act", "qmm_q8_0", "qmm_q4_0",
                  "qmm_id"):
            getattr(L, f).restype = I
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().bqm_strerror(int(status)).decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr()) if t.numel() > 0 else ctypes.c_void_p(t.data_ptr() or None)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise BqmError(name, st)


def _fmt(fmt):
    return FMT[fmt] if isinstance(fmt, str) else int(fmt)


def packed_bytes(fmt, rows: int, K: int) -> int:
    return int(lib().bqm_packed_bytes(_fmt(fmt), rows, K))


def bqm_repack(fmt, w_interchange, w_packed, rows: int, K: int, stream=None):
    _call("bqm_repack", _fmt(fmt), _ptr(w_interchange), _ptr(w_packed), rows, K, _stream(stream))


def bqm_unpack(fmt, w_packed, w_interchange, rows: int, K: int, stream=None):
    _call("bqm_unpack", _fmt(fmt), _ptr(w_packed), _ptr(w_interchange), rows, K, _stream(stream))


def qmv_q4_0(w_packed, X, Y, M: int, N: int, K: int, stream=None):
    _call("qmv_q4_0", _ptr(w_packed), _ptr(X), _ptr(Y), M, N, K, _stream(stream))


def qmv_q8_0(w_packed, X, Y, M: int, N: int, K: int, stream=None):
    _call("qmv_q8_0", _ptr(w_packed), _ptr(X), _ptr(Y), M, N, K, _stream(stream))


def qmv_id(fmt, w_packed, E: int, N: int, K: int, ids, T: int, top_k: int, X,
           x_tok_stride: int, x_slot_stride: int, Y, stream=None):
    _call("qmv_id", _fmt(fmt), _ptr(w_packed), E, N, K, _ptr(ids), T, top_k, _ptr(X),
          x_tok_stride, x_slot_stride, _ptr(Y), _stream(stream))


def qmv_id_sum(fmt, w_packed, E: int, N: int, K: int, ids, weights, T: int, top_k: int, X,
               x_tok_stride: int, x_slot_stride: int, Y_slots, Y, stream=None):
    _call("qmv_id_sum", _fmt(fmt), _ptr(w_packed), E, N, K, _ptr(ids), _ptr(weights), T, top_k,
          _ptr(X), x_tok_stride, x_slot_stride, _ptr(Y_slots), _ptr(Y), _stream(stream))


def qmv_id_sum_noalloc(fmt, w_packed, E: int, N: int, K: int, ids, weights, T: int, top_k: int,
                       X, x_tok_stride: int, x_slot_stride: int, Y, stream=None):
    _call("qmv_id_sum_noalloc", _fmt(fmt), _ptr(w_packed), E, N, K, _ptr(ids), _ptr(weights), T,
          top_k, _ptr(X), x_tok_stride, x_slot_stride, _ptr(Y), _stream(stream))


def qmv_id_gate_up(fmt, w_gate, w_up, E: int, N: int, K: int, ids, T: int, top_k: int, X,
                   x_tok_stride: int, x_slot_stride: int, Y, stream=None):
    _call("qmv_id_gate_up", _fmt(fmt), _ptr(w_gate), _ptr(w_up), E, N, K, _ptr(ids), T, top_k,
          _ptr(X), x_tok_stride, x_slot_stride, _ptr(Y), _stream(stream))


def bqm_quantize_q8_act(X, Xq, dx, M: int, K: int, stream=None):
    _call("bqm_quantize_q8_act", _ptr(X), _ptr(Xq), _ptr(dx), M, K, _stream(stream))


def qmm_q8_0(w_packed, Xq, dx, Y, M: int, N: int, K: int, stream=None):
    _call("qmm_q8_0", _ptr(w_packed), _ptr(Xq), _ptr(dx), _ptr(Y), M, N, K, _stream(stream))


def qmm_q4_0(w_packed, Xq, dx, Y, M: int, N: int, K: int, stream=None):
    _call("qmm_q4_0", _ptr(w_packed), _ptr(Xq), _ptr(dx), _ptr(Y), M, N, K, _stream(stream))


def qmm_id(fmt, w_packed, E: int, N: int, K: int, ids, T: int, top_k: int, Xq, dx,
           x_tok_rows: int, x_slot_rows: int, Y, stream=None):
    _call("qmm_id", _fmt(fmt), _ptr(w_packed), E, N, K, _ptr(ids), T, top_k, _ptr(Xq), _ptr(dx),
          x_tok_rows, x_slot_rows, _ptr(Y), _stream(stream))


class Gemv(ctypes.Structure):
    """One GEMV of a chain (the C struct bqm_gemv)."""
    _fields_ = [("w_packed", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("fmt", ctypes.c_int32),
                ("wait", ctypes.c_int32), ("M", ctypes.c_int32), ("reserved", ctypes.c_int32)]


CHAIN_MAX_K = 32768


def chain_workspace_bytes(n: int) -> int:
    return int(lib().bqm_chain_workspace_bytes(n))


def bqm_chain_prepare(descs, workspace, stream=None):
    """descs: a sequence of Gemv (host memory); workspace: device tensor of
    chain_workspace_bytes(len(descs)) bytes.  Synchronizes the stream."""
    arr = (Gemv * len(descs))(*descs)
    _call("bqm_chain_prepare", ctypes.cast(arr, ctypes.c_void_p), len(descs), _ptr(workspace),
          _stream(stream))


def qmv_chain(fmt, M: int, workspace, n: int, stream=None):
    _call("qmv_chain", _fmt(fmt), M, _ptr(workspace), n, _stream(stream))


def bqm_chain_status(workspace, stream=None) -> int:
    return int(lib().bqm_chain_status(_ptr(workspace), _stream(stream)))


def gemv(fmt, w_packed, x, y, N: int, K: int, wait: bool, M: int = 1) -> Gemv:
    """Descriptor of one GEMV of a chain: x [M][K], y [M][N] (torch tensors on the device)."""
    return Gemv(w_packed.data_ptr(), x.data_ptr(), y.data_ptr(), N, K, _fmt(fmt), 1 if wait else 0, M, 0)


# ---- conveniences built only from the calls above (allocation through torch) ----

def repack(fmt, w_interchange: torch.Tensor, rows: int, K: int, stream=None) -> torch.Tensor:
    """Device interchange bytes -> a new packed uint8 tensor."""
    out = torch.empty(packed_bytes(fmt, rows, K), dtype=torch.uint8, device=w_interchange.device)
    bqm_repack(fmt, w_interchange, out, rows, K, stream)
    return out
