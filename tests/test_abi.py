"""The C-ABI library on the host: it loads, exports every symbol include/bqm.h declares,
and rejects bad arguments on the host before anything is launched.  No GPU needed: every
call below fails validation and returns before touching the HIP runtime."""
import ctypes
import os
import re

from block_quantized_matrix_amd import bqm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bqm.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([A-Za-z_]\w*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("bqm_packed_bytes", "bqm_repack", "bqm_unpack", "qmv_q4_0", "qmv_q8_0", "qmv_id",
              "qmv_id_gate_up", "qmv_id_sum", "bqm_quantize_q8_act", "qmm_q8_0", "qmm_q4_0", "qmm_id", "bqm_strerror"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(bqm.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), f"libbqm.so does not export {n}"


def test_packed_bytes():
    # Q4_0 4096 x 4096: 16 B of codes + 2 B of scale per block, sections 256-aligned, at
    # least 16 bytes of slack after the scales
    nb = 4096 * 4096 // 32
    assert bqm.packed_bytes("q4_0", 4096, 4096) == nb * 16 + nb * 2 + 256
    assert bqm.packed_bytes("q8_0", 17408, 5120) == 17408 * 5120 + 17408 * 160 * 2 + 256
    assert bqm.packed_bytes("q4_0", 3, 32) == 256 + 256    # 48 B codes -> 256, 6 + 16 B -> 256
    assert bqm.packed_bytes("q4_0", 1, 32 * 120) == 2048 + 256   # 240 B scales + 16 -> 256
    assert bqm.packed_bytes("q4_0", 1, 32 * 128) == 2048 + 512   # 256 B scales + 16 -> 512
    assert bqm.packed_bytes("q4_0", 0, 64) == 0
    assert bqm.packed_bytes("q4_0", 5, 33) == 0             # K not a multiple of 32
    assert bqm.packed_bytes(3, 5, 32) == 0                  # unknown format


def test_strerror():
    assert bqm.strerror(0) == "success"
    assert "multiple of 32" in bqm.strerror(2)
    assert bqm.strerror(99) == "unknown status"


def _st(fn, *args):
    return getattr(bqm.lib(), fn)(*args)


P = ctypes.c_void_p
GOOD = P(0x100000)      # 16-byte aligned fake addresses: never dereferenced on these paths
ODD = P(0x100008)


def test_host_validation_before_launch():
    L = bqm.lib()
    # K not a multiple of 32
    assert L.qmv_q4_0(GOOD, GOOD, GOOD, 1, 64, 48, None) == 2
    assert L.qmv_q8_0(GOOD, GOOD, GOOD, 1, 64, 33, None) == 2
    # M out of range
    assert L.qmv_q4_0(GOOD, GOOD, GOOD, 9, 64, 64, None) == 2
    assert L.qmv_q4_0(GOOD, GOOD, GOOD, -1, 64, 64, None) == 2
    # null pointers
    assert L.qmv_q4_0(None, GOOD, GOOD, 1, 64, 64, None) == 1
    assert L.qmv_q4_0(GOOD, None, GOOD, 1, 64, 64, None) == 1
    assert L.qmv_q4_0(GOOD, GOOD, None, 1, 64, 64, None) == 1
    # misaligned
    assert L.qmv_q4_0(ODD, GOOD, GOOD, 1, 64, 64, None) == 3
    assert L.qmv_q4_0(GOOD, ODD, GOOD, 1, 64, 64, None) == 3
    # unknown format
    assert L.bqm_repack(3, GOOD, GOOD, 4, 64, None) == 4
    assert L.qmv_id(5, GOOD, 4, 8, 64, GOOD, 1, 2, GOOD, 64, 0, GOOD, None) == 4
    # qmv_id limits and strides
    assert L.qmv_id(2, GOOD, 4, 8, 64, GOOD, 65, 2, GOOD, 64, 0, GOOD, None) == 2
    assert L.qmv_id(2, GOOD, 4097, 8, 64, GOOD, 1, 2, GOOD, 64, 0, GOOD, None) == 2
    assert L.qmv_id(2, GOOD, 4, 8, 64, GOOD, 1, 33, GOOD, 64, 0, GOOD, None) == 2
    assert L.qmv_id(2, GOOD, 4, 8, 64, GOOD, 1, 2, GOOD, 66, 0, GOOD, None) == 3
    assert L.qmv_id(2, GOOD, 4, 8, 64, None, 1, 2, GOOD, 64, 0, GOOD, None) == 1
    # qmv_id_gate_up: the same checks, and the up tensor too
    assert L.qmv_id_gate_up(5, GOOD, GOOD, 4, 8, 64, GOOD, 1, 2, GOOD, 64, 0, GOOD, None) == 4
    assert L.qmv_id_gate_up(2, GOOD, GOOD, 4, 8, 64, GOOD, 65, 2, GOOD, 64, 0, GOOD, None) == 2
    assert L.qmv_id_gate_up(2, GOOD, None, 4, 8, 64, GOOD, 1, 2, GOOD, 64, 0, GOOD, None) == 1
    assert L.qmv_id_gate_up(2, GOOD, ODD, 4, 8, 64, GOOD, 1, 2, GOOD, 64, 0, GOOD, None) == 3
    assert L.qmv_id_gate_up(2, None, GOOD, 4, 8, 64, GOOD, 1, 2, GOOD, 64, 0, GOOD, None) == 1
    assert L.qmv_id_gate_up(2, GOOD, GOOD, 4, 8, 64, GOOD, 1, 2, GOOD, 66, 0, GOOD, None) == 3
    # qmv_id_sum: qmv_id's checks, then Y, the weights and the counters
    assert L.qmv_id_sum(5, GOOD, 4, 8, 64, GOOD, GOOD, 1, 2, GOOD, 64, 0, GOOD, GOOD, None) == 4
    assert L.qmv_id_sum(2, GOOD, 4, 8, 64, GOOD, GOOD, 65, 2, GOOD, 64, 0, GOOD, GOOD, None) == 2
    assert L.qmv_id_sum(2, GOOD, 4, 8, 64, GOOD, GOOD, 1, 2, GOOD, 64, 0, GOOD, None, None) == 1
    assert L.qmv_id_sum(2, GOOD, 4, 8, 64, GOOD, GOOD, 1, 2, GOOD, 64, 0, GOOD, ODD, None) == 3
    assert L.qmv_id_sum(2, GOOD, 4, 8, 64, GOOD, None, 1, 2, GOOD, 64, 0, GOOD, GOOD, None) == 1
    assert L.qmv_id_sum(2, GOOD, 4, 8, 64, GOOD, P(0x100002), 1, 2, GOOD, 64, 0, GOOD, GOOD, None) == 3
    assert L.qmv_id_sum(2, GOOD, 4, 8, 64, None, GOOD, 1, 2, GOOD, 64, 0, GOOD, GOOD, None) == 1
    # qmv_id_sum_noalloc: qmv_id_sum's checks, and the slot rows must fit the library's array
    assert L.qmv_id_sum_noalloc(5, GOOD, 4, 8, 64, GOOD, GOOD, 1, 2, GOOD, 64, 0, GOOD, None) == 4
    assert L.qmv_id_sum_noalloc(2, GOOD, 4, 8, 64, GOOD, GOOD, 65, 2, GOOD, 64, 0, GOOD, None) == 2
    assert L.qmv_id_sum_noalloc(2, GOOD, 4, 8, 64, GOOD, GOOD, 1, 2, GOOD, 64, 0, None, None) == 1
    assert L.qmv_id_sum_noalloc(2, GOOD, 4, 8, 64, GOOD, GOOD, 1, 2, GOOD, 64, 0, ODD, None) == 3
    assert L.qmv_id_sum_noalloc(2, GOOD, 4, 8, 64, GOOD, None, 1, 2, GOOD, 64, 0, GOOD, None) == 1
    assert L.qmv_id_sum_noalloc(2, GOOD, 4, 1024, 64, GOOD, GOOD, 64, 32, GOOD, 64, 0, GOOD, None) == 2
    # quantizer and qmm
    assert L.bqm_quantize_q8_act(GOOD, GOOD, GOOD, 4, 40, None) == 2
    assert L.bqm_quantize_q8_act(GOOD, None, GOOD, 4, 64, None) == 1
    assert L.qmm_q8_0(GOOD, GOOD, GOOD, GOOD, 4, 8, 48, None) == 2
    assert L.qmm_q8_0(GOOD, ODD, GOOD, GOOD, 4, 8, 64, None) == 3
    assert L.qmm_q4_0(GOOD, GOOD, GOOD, GOOD, 4, 8, 48, None) == 2
    assert L.qmm_q4_0(GOOD, GOOD, GOOD, GOOD, -1, 8, 64, None) == 2
    assert L.qmm_q4_0(None, GOOD, GOOD, GOOD, 4, 8, 64, None) == 1
    assert L.qmm_q4_0(GOOD, GOOD, GOOD, ODD, 4, 8, 64, None) == 3
    # qmm_id: limits, strides, pointers
    assert L.qmm_id(5, GOOD, 4, 8, 64, GOOD, 1, 2, GOOD, GOOD, 1, 0, GOOD, None) == 4
    assert L.qmm_id(2, GOOD, 4, 8, 64, GOOD, 16385, 2, GOOD, GOOD, 1, 0, GOOD, None) == 2
    assert L.qmm_id(2, GOOD, 4, 8, 64, GOOD, 1, 33, GOOD, GOOD, 1, 0, GOOD, None) == 2
    assert L.qmm_id(2, GOOD, 4097, 8, 64, GOOD, 1, 2, GOOD, GOOD, 1, 0, GOOD, None) == 2
    assert L.qmm_id(2, GOOD, 4, 8, 48, GOOD, 1, 2, GOOD, GOOD, 1, 0, GOOD, None) == 2
    assert L.qmm_id(2, GOOD, 4, 8, 64, GOOD, 2, 2, GOOD, GOOD, 1 << 31, 0, GOOD, None) == 2
    assert L.qmm_id(2, GOOD, 4, 8, 64, GOOD, 1, 2, GOOD, GOOD, -1, 0, GOOD, None) == 2
    assert L.qmm_id(2, GOOD, 4, 8, 64, None, 1, 2, GOOD, GOOD, 1, 0, GOOD, None) == 1
    assert L.qmm_id(2, None, 4, 8, 64, GOOD, 1, 2, GOOD, GOOD, 1, 0, GOOD, None) == 1
    assert L.qmm_id(2, GOOD, 4, 8, 64, GOOD, 1, 2, GOOD, GOOD, 1, 0, ODD, None) == 3
    assert L.qmm_id(2, ODD, 4, 8, 64, GOOD, 1, 2, GOOD, GOOD, 1, 0, GOOD, None) == 3
    # prefill operands are addressed with 32-bit offsets: 2 GiB of activations or of one
    # matrix's codes is refused before any launch
    assert L.qmm_q8_0(GOOD, GOOD, GOOD, GOOD, 1 << 17, 8, 1 << 14, None) == 2
    assert L.qmm_q8_0(GOOD, GOOD, GOOD, GOOD, 4, 1 << 17, 1 << 14, None) == 2
    assert L.qmm_id(2, GOOD, 4, 8, 1 << 14, GOOD, 16384, 32, GOOD, GOOD, 32, 1, GOOD, None) == 2
    # repack alignment: interchange needs 2-byte alignment, packed 16
    assert L.bqm_repack(2, P(0x100001), GOOD, 4, 64, None) == 3
    assert L.bqm_repack(2, GOOD, ODD, 4, 64, None) == 3


def test_empty_sizes_are_no_ops():
    L = bqm.lib()
    # nothing to compute: success without any launch (null pointers are fine then)
    assert L.qmv_q4_0(None, None, None, 0, 64, 64, None) == 0
    assert L.qmv_q4_0(None, None, None, 1, 0, 64, None) == 0
    assert L.qmv_id(2, None, 4, 8, 64, None, 0, 8, None, 64, 0, None, None) == 0
    assert L.qmv_id_gate_up(2, None, None, 4, 8, 64, None, 0, 8, None, 64, 0, None, None) == 0
    assert L.qmv_id_sum(2, None, 4, 8, 64, None, None, 0, 8, None, 64, 0, None, None, None) == 0
    assert L.bqm_quantize_q8_act(None, None, None, 0, 64, None) == 0
    assert L.qmm_q8_0(None, None, None, None, 0, 8, 64, None) == 0
    assert L.qmm_q4_0(None, None, None, None, 4, 0, 64, None) == 0
    assert L.qmm_id(2, None, 4, 8, 64, None, 0, 2, None, None, 1, 0, None, None) == 0
    assert L.bqm_repack(2, None, None, 0, 64, None) == 0
    assert L.bqm_unpack(8, None, None, 4, 0, None) == 0


def _gemv(N, K, fmt="q4_0", ptr=0x10000, wait=0, M=1):
    return bqm.Gemv(ptr, ptr, ptr, N, K, bqm.FMT[fmt], wait, M, 0)


def test_chain_host_validation():
    """bqm_chain_prepare rejects bad descriptor lists on the host.  Host addresses stand in
    for device pointers: every case below is rejected before any device work (at most the
    CU count is queried), so nothing is dereferenced."""
    ws = 0x20000  # 16-byte aligned stand-in
    L = bqm.lib()

    def prep(descs, n=None, w=ws):
        arr = (bqm.Gemv * max(1, len(descs)))(*descs)
        return L.bqm_chain_prepare(ctypes.cast(arr, ctypes.c_void_p), len(descs) if n is None else n,
                                   ctypes.c_void_p(w), None)

    assert bqm.chain_workspace_bytes(0) == 0
    # per GEMV: its descriptor (56 bytes) and its segment's split (two int64)
    assert bqm.chain_workspace_bytes(2) - bqm.chain_workspace_bytes(1) == ctypes.sizeof(bqm.Gemv) + 16 == 72
    assert prep([], n=0) == 2                                    # empty chain
    assert prep([_gemv(64, 64)], w=0) == 1                       # no workspace
    assert prep([_gemv(64, 64)], w=ws + 8) == 3                  # misaligned workspace
    assert prep([_gemv(64, 64), _gemv(64, 64, "q8_0")]) == 4     # mixed formats
    assert prep([_gemv(64, 64), _gemv(64, 64, M=2)]) == 2        # mixed batch
    assert prep([_gemv(64, 64, M=0)]) == 2                       # batch 0
    assert prep([_gemv(64, 64, M=9)]) == 2                       # batch over 8
    assert prep([_gemv(64, 48)]) == 2                            # K % 32 != 0
    assert prep([_gemv(64, 32800)]) == 2                         # K over the chain limit
    assert prep([_gemv(0, 64)]) == 2                             # empty GEMV
    assert prep([_gemv(64, 64, ptr=0)]) == 1                     # null matrix
    assert prep([_gemv(64, 64, ptr=0x10008)]) == 3               # misaligned matrix
    # LDS: a 64-byte table row per GEMV, the split-tile parts (512 M bytes), 64 bytes of
    # counters, per-row partial sums and at least 32 staged blocks per input row must fit
    # 162816 bytes.  With 64 rows (one per workgroup) at M = 1 that allows 2462 GEMVs.
    assert prep([_gemv(64, 17408)] * 2463) == 2
    assert prep([_gemv(64, 17408, M=8)] * 2463) == 2
