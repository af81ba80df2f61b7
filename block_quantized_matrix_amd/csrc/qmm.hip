// Prefill: activation quantizer and the Q8_0 / Q4_0 x Q8-activation product on int8 MFMA,
// gfx950.  qw is the signed weight code: the int8 of Q8_0, the nibble - 8 of Q4_0.
//
//   isum[m][n][b] = sum_{j<32} qw[n][32b+j] * Xq[m][32b+j]        exact int32
//   Y[m][n]       = sum_b (d_w[n][b] * dx[m][b]) * isum[m][n][b]    fp32, b ascending
//
// The work is a dense contraction (M = 512 prompt tokens in the llama-bench pp512 shape
// of the "llama.cpp 0.9.0" analysis page (ai-v5 LLMNews), section 2), so it runs on the
// matrix cores: one v_mfma_i32_32x32x32_i8 covers exactly one 32-wide block, so every
// block's integer sum comes out of the MFMA on its own, exact, and is scaled in fp32 by
// the product of the two block scales.
#include "bqm_internal.h"

namespace bqm {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;

__device__ __forceinline__ float h2f(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// ---------------------------------------------------------------- quantizer ----
// Eight threads per 32-wide block, four values (one 16-byte load) each; the block's
// absolute maximum is combined with cross-lane shuffles inside the 8-lane group.
// Everything is IEEE single precision: a correctly rounded division for the scale and for
// each x / dx, roundf (half away from zero), no contraction (built with -ffp-contract=off).
__global__ __launch_bounds__(kThreads) void k_quantize_q8_act(const float4* __restrict__ X,
                                                              uint32_t* __restrict__ Xq,
                                                              float* __restrict__ dx,
                                                              int64_t n_quads) {
  const int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x;  // quad index
  const bool ok = i < n_quads;
  const float4 v = ok ? X[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
  const float d = a / 127.0f;
  uint32_t packed = 0;
  if (d != 0.0f) {
    const float q[4] = {v.x / d, v.y / d, v.z / d, v.w / d};
#pragma unroll
    for (int e = 0; e < 4; e++) {
      float r = roundf(q[e]);
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      packed |= ((uint32_t)(int32_t)r & 0xffu) << (8 * e);
    }
  }
  if (ok) {
    Xq[i] = packed;
    if ((i & 7) == 0) dx[i >> 3] = d == 0.0f ? 0.0f : d;
  }
}

// ---------------------------------------------------------------- qmm ----
// Workgroup tile 128 (m) x 128 (n), four waves as 2 x 2 of 64 x 64, each wave 2 x 2 MFMA
// tiles of 32 x 32.  K advances four blocks (128 bytes of codes per row) per LDS stage;
// the next stage's codes and scales are loaded into registers while the current one is
// computed.
//
// The block-scale epilogue, not the integer products, bounds this kernel: per 32 x 32 tile
// and block one int8 MFMA (32 cycles) meets 1024 fp32 rescales.  The scale product
// dx[m][b] * dw[n][b] of a tile is an outer product, so it goes to the matrix cores too:
// one bf16 MFMA with K = 6 used terms, dx split exactly into three truncated bf16 parts
// and dw (fp16, 11 significant bits) into two, every partial product exact in fp32.
// Per element and block the vector units then do one conversion and one FMA.
constexpr int BM = 128, BN = 128, BKB = 4;     // BKB blocks of 32 per stage
constexpr int ROWB = BKB * 32 + 16;            // LDS row stride in bytes (padding vs conflicts)

// v = hi + mid + lo exactly, each a truncated bf16 (returned as its 16 bits)
__device__ __forceinline__ void split3(float v, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const uint32_t h = __float_as_uint(v) & 0xFFFF0000u;
  const float r1 = v - __uint_as_float(h);
  const uint32_t m = __float_as_uint(r1) & 0xFFFF0000u;
  const float r2 = r1 - __uint_as_float(m);
  hi = h >> 16;
  mid = m >> 16;
  lo = __float_as_uint(r2) >> 16;
}

// MFMA operand rows of the scale outer product (k = 0..5 used, 6..15 zero):
//   A (row m): dx parts  {hi, hi, mid, mid, lo, lo}
//   B (col n): dw parts  {hi, lo, hi, lo, hi, lo}
// so that sum_k A[m][k] B[k][n] = (dx_hi + dx_mid + dx_lo) (dw_hi + dw_lo).
__device__ __forceinline__ u32x4 dx_operand(float dx) {
  uint32_t h, m, l;
  split3(dx, h, m, l);
  return u32x4{h | (h << 16), m | (m << 16), l | (l << 16), 0u};
}
__device__ __forceinline__ u32x4 dw_operand(uint32_t dw_bits) {
  const float d = h2f(dw_bits);
  const uint32_t h = __float_as_uint(d) & 0xFFFF0000u;
  const uint32_t l = __float_as_uint(d - __uint_as_float(h)) >> 16;
  const uint32_t w = (h >> 16) | (l << 16);
  return u32x4{w, w, w, 0u};
}

// Q4_0 codes: a 16-byte block holds weight j in the low nibble of byte j and weight j + 16
// in the high one.  Each half expands to four signed bytes per word (nibble - 8) without a
// borrow between bytes: set bit 7, subtract 8, flip bit 7 back.
__device__ __forceinline__ uint32_t nib_to_i8(uint32_t v) {  // v: four nibbles 0..15
  return ((v | 0x80808080u) - 0x08080808u) ^ 0x80808080u;
}
__device__ __forceinline__ void expand_q4(const u32x4& q, u32x4& lo, u32x4& hi) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    lo[i] = nib_to_i8(q[i] & 0x0F0F0F0Fu);
    hi[i] = nib_to_i8((q[i] >> 4) & 0x0F0F0F0Fu);
  }
}

// One workgroup tile of Y.  FMT selects how the weight codes arrive: Q8_0 as int8 rows
// [N][K]; Q4_0 as 16-byte blocks [N][nb][16], expanded to int8 while they are staged, so
// that the LDS layout and everything after it are the same for both.
template <int FMT>
__device__ __forceinline__ void qmm_tile(const uint8_t* __restrict__ Wc, const uint16_t* __restrict__ Wd,
                                         const int8_t* __restrict__ Xq, const float* __restrict__ dx,
                                         float* __restrict__ Y, int M, int N, int nb, int tiles_m,
                                         int tiles_n) {
  constexpr bool Q4 = FMT == BQM_Q4_0;
  constexpr int NPB = Q4 ? 2 : 4;   // 16-byte pieces of weight codes per thread and stage
  __shared__ __attribute__((aligned(16))) int8_t sA[BM * ROWB];
  __shared__ __attribute__((aligned(16))) int8_t sB[BN * ROWB];
  __shared__ u32x4 sXs[BKB * BM + 1];  // dx operands per (block, m); the last: zeros
  __shared__ u32x4 sWs[BKB * BN];      // dw operands per (block, n)

  // Workgroups are dealt round-robin to the eight XCDs; give the workgroups of one XCD
  // neighbouring tiles (all m-tiles of a few n-tiles) so they share W rows in that L2.
  const int nwg = tiles_m * tiles_n;
  const int bid = blockIdx.x;
  int tile = bid;
  if (nwg % 8 == 0) tile = (bid % 8) * (nwg / 8) + bid / 8;
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int K = nb * 32;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave & 1) * 64, wn = (wave >> 1) * 64;
  const int l32 = lane & 31, lh = lane >> 5;
  if (tid == 0) sXs[BKB * BM] = u32x4{0u, 0u, 0u, 0u};

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) acc[i][j] = f32x16{};

  // staging: 128 rows x 128 bytes per operand = 1024 16-byte pieces, 4 per thread; 512
  // scales per operand, 2 per thread
  // (Q4_0: 128 rows x 4 blocks of 16 bytes, 2 per thread)
  const int64_t wrow = Q4 ? (int64_t)nb * 16 : (int64_t)K;  // bytes per weight row
  u32x4 pa0, pa1, pa2, pa3, pb0, pb1, pb2 = {}, pb3 = {};
  float px0, px1;
  uint32_t pw0, pw1;
#define BQM_FETCH(B0)                                                                          \
  {                                                                                            \
    const int bn_ = min(BKB, nb - (B0));                                                       \
    u32x4* pa_[4] = {&pa0, &pa1, &pa2, &pa3};                                                  \
    u32x4* pb_[4] = {&pb0, &pb1, &pb2, &pb3};                                                  \
    _Pragma("unroll") for (int p = 0; p < 4; p++) {                                            \
      const int piece = tid + p * kThreads, row = piece >> 3, c16 = piece & 7;                 \
      const bool kin = (c16 >> 1) < bn_;                                                       \
      u32x4 va = {0u, 0u, 0u, 0u};                                                             \
      if (kin && m0 + row < M)                                                                 \
        va = *reinterpret_cast<const u32x4*>(Xq + (size_t)(m0 + row) * K + (size_t)(B0) * 32 + c16 * 16); \
      *pa_[p] = va;                                                                            \
    }                                                                                          \
    _Pragma("unroll") for (int p = 0; p < NPB; p++) {                                          \
      const int piece = tid + p * kThreads;                                                    \
      const int row = Q4 ? piece >> 2 : piece >> 3, c16 = Q4 ? piece & 3 : piece & 7;          \
      const int kb_ = Q4 ? c16 : c16 >> 1;                                                     \
      u32x4 vb = {0u, 0u, 0u, 0u};                                                             \
      if (kb_ < bn_ && n0 + row < N)                                                           \
        vb = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(                       \
            Wc + (size_t)(n0 + row) * wrow + (size_t)(B0) * (Q4 ? 16 : 32) + c16 * 16));       \
      *pb_[p] = vb;                                                                            \
    }                                                                                          \
    float* px_[2] = {&px0, &px1};                                                              \
    uint32_t* pw_[2] = {&pw0, &pw1};                                                           \
    _Pragma("unroll") for (int q = 0; q < 2; q++) {                                            \
      const int e = tid + q * kThreads, kb = e >> 7, r = e & 127;                              \
      const bool kin = kb < bn_;                                                               \
      *px_[q] = (kin && m0 + r < M) ? dx[(size_t)(m0 + r) * nb + (B0) + kb] : 0.f;             \
      *pw_[q] = (kin && n0 + r < N) ? (uint32_t)Wd[(size_t)(n0 + r) * nb + (B0) + kb] : 0u;   \
    }                                                                                          \
  }

  BQM_FETCH(0)
  for (int b0 = 0; b0 < nb; b0 += BKB) {
    const int bn = min(BKB, nb - b0);
    __syncthreads();  // every wave is done with the previous stage
    {
      const u32x4 pa_[4] = {pa0, pa1, pa2, pa3};
      const u32x4 pb_[4] = {pb0, pb1, pb2, pb3};
#pragma unroll
      for (int p = 0; p < 4; p++) {
        const int piece = tid + p * kThreads, row = piece >> 3, c16 = piece & 7;
        *reinterpret_cast<u32x4*>(sA + row * ROWB + c16 * 16) = pa_[p];
      }
#pragma unroll
      for (int p = 0; p < NPB; p++) {
        const int piece = tid + p * kThreads;
        if constexpr (Q4) {
          const int row = piece >> 2, kb = piece & 3;
          u32x4 lo, hi;
          expand_q4(pb_[p], lo, hi);
          *reinterpret_cast<u32x4*>(sB + row * ROWB + kb * 32) = lo;
          *reinterpret_cast<u32x4*>(sB + row * ROWB + kb * 32 + 16) = hi;
        } else {
          const int row = piece >> 3, c16 = piece & 7;
          *reinterpret_cast<u32x4*>(sB + row * ROWB + c16 * 16) = pb_[p];
        }
      }
      const float px_[2] = {px0, px1};
      const uint32_t pw_[2] = {pw0, pw1};
#pragma unroll
      for (int q = 0; q < 2; q++) {
        const int e = tid + q * kThreads;  // = kb * 128 + r
        sXs[e] = dx_operand(px_[q]);
        sWs[e] = dw_operand(pw_[q]);
      }
    }
    __syncthreads();
    if (b0 + BKB < nb) BQM_FETCH(b0 + BKB)  // in flight while this stage is computed

    for (int kb = 0; kb < bn; kb++) {
      i32x4 a[2], bq[2];
      bf16x8 as[2], bs[2];
#pragma unroll
      for (int i = 0; i < 2; i++) {
        a[i] = *reinterpret_cast<const i32x4*>(sA + (wm + i * 32 + l32) * ROWB + kb * 32 + lh * 16);
        // lanes 32..63 hold k = 8..15 of the scale product: zeros
        const u32x4* p = lh ? &sXs[BKB * BM] : &sXs[kb * BM + wm + i * 32 + l32];
        as[i] = __builtin_bit_cast(bf16x8, *p);
      }
#pragma unroll
      for (int j = 0; j < 2; j++) {
        bq[j] = *reinterpret_cast<const i32x4*>(sB + (wn + j * 32 + l32) * ROWB + kb * 32 + lh * 16);
        const u32x4* p = lh ? &sXs[BKB * BM] : &sWs[kb * BN + wn + j * 32 + l32];
        bs[j] = __builtin_bit_cast(bf16x8, *p);
      }
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) {
          const i32x16 isum = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], bq[j], i32x16{}, 0, 0, 0);
          const f32x16 sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as[i], bs[j], f32x16{}, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 16; r++) acc[i][j][r] = fmaf(sc[r], (float)isum[r], acc[i][j][r]);
        }
    }
  }
#undef BQM_FETCH

  // a lane's 16 results of a 32 x 32 tile: rows 8 (r / 4) + 4 lh + r % 4, column l32
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int n = n0 + wn + j * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int m = m0 + wm + i * 32 + 8 * (r / 4) + 4 * lh + (r % 4);
        if (m < M && n < N) Y[(size_t)m * N + n] = acc[i][j][r];
      }
    }
}

#define BQM_QMM_KERNEL(NAME, FMT)                                                              \
  __global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void NAME( \
      const uint8_t* __restrict__ Wc, const uint16_t* __restrict__ Wd,                         \
      const int8_t* __restrict__ Xq, const float* __restrict__ dx, float* __restrict__ Y,      \
      int M, int N, int nb, int tiles_m, int tiles_n) {                                        \
    qmm_tile<FMT>(Wc, Wd, Xq, dx, Y, M, N, nb, tiles_m, tiles_n);                              \
  }
BQM_QMM_KERNEL(k_qmm_q8_0, BQM_Q8_0)
BQM_QMM_KERNEL(k_qmm_q4_0, BQM_Q4_0)
#undef BQM_QMM_KERNEL

}  // namespace

int launch_quantize_q8_act(const float* X, int8_t* Xq, float* dx, int64_t M, int64_t K,
                           hipStream_t s) {
  const int64_t quads = M * K / 4;
  const int64_t grid = (quads + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(k_quantize_q8_act, dim3((unsigned)grid), dim3(kThreads), 0, s,
                     reinterpret_cast<const float4*>(X), reinterpret_cast<uint32_t*>(Xq), dx, quads);
  return launch_status();
}

static int launch_qmm(int fmt, const void* w, const int8_t* Xq, const float* dx, float* Y,
                      int64_t M, int64_t N, int64_t K, hipStream_t s) {
  Layout L;
  layout_of(fmt, N, K, &L);
  const uint8_t* Wc = static_cast<const uint8_t*>(w);
  const uint16_t* Wd = reinterpret_cast<const uint16_t*>(Wc + L.scales_off);
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  hipLaunchKernelGGL(fmt == BQM_Q4_0 ? k_qmm_q4_0 : k_qmm_q8_0, dim3((unsigned)(tiles_m * tiles_n)),
                     dim3(kThreads), 0, s, Wc, Wd, Xq, dx, Y, (int)M, (int)N, (int)L.nb, tiles_m,
                     tiles_n);
  return launch_status();
}

int launch_qmm_q8_0(const void* w, const int8_t* Xq, const float* dx, float* Y, int64_t M,
                    int64_t N, int64_t K, hipStream_t s) {
  return launch_qmm(BQM_Q8_0, w, Xq, dx, Y, M, N, K, s);
}

int launch_qmm_q4_0(const void* w, const int8_t* Xq, const float* dx, float* Y, int64_t M,
                    int64_t N, int64_t K, hipStream_t s) {
  return launch_qmm(BQM_Q4_0, w, Xq, dx, Y, M, N, K, s);
}

}  // namespace bqm
