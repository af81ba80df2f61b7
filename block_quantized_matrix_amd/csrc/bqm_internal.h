// Internal definitions of the gfx950 library: packed layout, launch helpers.
// Not part of the public ABI (include/bqm.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bqm.h"

namespace bqm {

constexpr int kQK = 32;  // weights per block

// Packed layout of a rows x K matrix (nb = K/32 blocks per row):
//   [0, codes_bytes)            code bytes, row-major, block-major within a row:
//                                 Q4_0: 16 bytes per block, the interchange nibble
//                                       order (byte j: weight j low, weight j+16 high)
//                                 Q8_0: 32 bytes per block = the int8 matrix [rows][K]
//   [scales_off, +rows*nb*2)    binary16 scales, [rows][nb]
// Both sections start on a 256-byte boundary.  At least 16 zero bytes follow the scales
// (so a 4-byte read at any scale stays inside the buffer), and the total is rounded up to
// 256 bytes; an empty matrix takes 0 bytes.
struct Layout {
  int64_t nb;
  int64_t code_bytes_per_block;
  int64_t codes_bytes;
  int64_t scales_off;
  int64_t total;
};

inline int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }

inline bool layout_of(int fmt, int64_t rows, int64_t K, Layout* L) {
  if ((fmt != BQM_Q4_0 && fmt != BQM_Q8_0) || rows < 0 || K < 0 || K % kQK != 0) return false;
  L->nb = K / kQK;
  L->code_bytes_per_block = fmt == BQM_Q4_0 ? 16 : 32;
  L->codes_bytes = rows * L->nb * L->code_bytes_per_block;
  L->scales_off = align256(L->codes_bytes);
  L->total = rows * L->nb == 0 ? 0 : align256(L->scales_off + rows * L->nb * 2 + 16);
  return true;
}

inline int interchange_block_bytes(int fmt) { return fmt == BQM_Q4_0 ? 18 : 34; }

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? BQM_OK : BQM_E_LAUNCH;
}

// ---- launchers implemented in the .hip files (arguments already validated) ----
int launch_repack(int fmt, const void* src, void* dst, int64_t rows, int64_t K, hipStream_t s);
int launch_unpack(int fmt, const void* src, void* dst, int64_t rows, int64_t K, hipStream_t s);
int launch_qmv(int fmt, const void* w, const float* X, float* Y, int M, int64_t N, int64_t K,
               hipStream_t s);
int launch_qmv_id(int fmt, const void* w, int E, int64_t N, int64_t K, const int32_t* ids, int T,
                  int top_k, const float* X, int64_t xts, int64_t xss, float* Y, hipStream_t s);
int launch_qmv_id_gate_up(int fmt, const void* w_gate, const void* w_up, int E, int64_t N, int64_t K,
                          const int32_t* ids, int T, int top_k, const float* X, int64_t xts,
                          int64_t xss, float* Y, hipStream_t s);
int launch_qmv_id_sum(int fmt, const void* w, int E, int64_t N, int64_t K, const int32_t* ids,
                      const float* rw, int T, int top_k, const float* X, int64_t xts, int64_t xss,
                      float* Y_slots, float* Y, hipStream_t s);
int launch_qmv_id_sum_noalloc(int fmt, const void* w, int E, int64_t N, int64_t K, const int32_t* ids,
                              const float* rw, int T, int top_k, const float* X, int64_t xts,
                              int64_t xss, float* Y, hipStream_t s);
int launch_quantize_q8_act(const float* X, int8_t* Xq, float* dx, int64_t M, int64_t K,
                           hipStream_t s);
int launch_qmm_q8_0(const void* w, const int8_t* Xq, const float* dx, float* Y, int64_t M,
                    int64_t N, int64_t K, hipStream_t s);
int launch_qmm_q4_0(const void* w, const int8_t* Xq, const float* dx, float* Y, int64_t M,
                    int64_t N, int64_t K, hipStream_t s);
int launch_qmm_id(int fmt, const void* w, int E, int64_t N, int64_t K, const int32_t* ids, int T,
                  int top_k, const int8_t* Xq, const float* dx, int64_t x_tok_rows,
                  int64_t x_slot_rows, float* Y, hipStream_t s);
int launch_fill(float* y, int64_t n, float v, hipStream_t s);
int cu_count();
int launch_id_mma(int fmt, const void* w, const void* w_up, int E, int64_t N, int64_t K,
                  const int32_t* ids, int T, int top_k, const float* X, int64_t xts, int64_t xss,
                  float* Y, hipStream_t s, const float* rw);
int64_t chain_max_k();
size_t chain_workspace_bytes(int n);
int chain_prepare(const bqm_gemv* descs, int n, void* ws, hipStream_t s);
int chain_launch(int fmt, int M, void* ws, int n, hipStream_t s);
int chain_status(const void* ws, hipStream_t s);

}  // namespace bqm
