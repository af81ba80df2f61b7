// Prefill: activation quantizer and the Q8_0 x Q8-activation product on int8 MFMA, gfx950.
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
// tiles of 32 x 32.  K advances four blocks (128 bytes of codes per row) per LDS stage.
constexpr int BM = 128, BN = 128, BKB = 4;     // BKB blocks of 32 per stage
constexpr int ROWB = BKB * 32 + 16;            // LDS row stride in bytes (padding vs conflicts)

__global__ __launch_bounds__(kThreads) void k_qmm_q8_0(const int8_t* __restrict__ Wc,   // [N][K]
                                                       const uint16_t* __restrict__ Wd,  // [N][nb]
                                                       const int8_t* __restrict__ Xq,    // [M][K]
                                                       const float* __restrict__ dx,     // [M][nb]
                                                       float* __restrict__ Y, int M, int N, int nb,
                                                       int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) int8_t sA[BM * ROWB];
  __shared__ __attribute__((aligned(16))) int8_t sB[BN * ROWB];
  __shared__ float sdx[BKB][BM];
  __shared__ float sdw[BKB][BN];

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

  float acc[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

  // staging assignment: 128 rows x 128 bytes per operand = 1024 16-byte pieces, 4/thread
  for (int b0 = 0; b0 < nb; b0 += BKB) {
    const int bn = min(BKB, nb - b0);
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 4; p++) {
      const int piece = tid + p * kThreads;   // 0..1023
      const int row = piece >> 3, c16 = piece & 7;   // 8 pieces of 16 B per row
      const bool kin = (c16 >> 1) < bn;             // 2 pieces per block
      u32x4 va = {0u, 0u, 0u, 0u}, vb = {0u, 0u, 0u, 0u};
      if (kin && m0 + row < M)
        va = *reinterpret_cast<const u32x4*>(Xq + (size_t)(m0 + row) * K + (size_t)b0 * 32 + c16 * 16);
      if (kin && n0 + row < N)
        vb = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(Wc + (size_t)(n0 + row) * K + (size_t)b0 * 32 + c16 * 16));
      *reinterpret_cast<u32x4*>(sA + row * ROWB + c16 * 16) = va;
      *reinterpret_cast<u32x4*>(sB + row * ROWB + c16 * 16) = vb;
    }
    for (int e = tid; e < BKB * BM; e += kThreads) {
      const int kb = e / BM, r = e % BM;
      const bool kin = kb < bn;
      sdx[kb][r] = (kin && m0 + r < M) ? dx[(size_t)(m0 + r) * nb + b0 + kb] : 0.f;
      sdw[kb][r] = (kin && n0 + r < N) ? h2f(Wd[(size_t)(n0 + r) * nb + b0 + kb]) : 0.f;
    }
    __syncthreads();

    for (int kb = 0; kb < bn; kb++) {
      i32x4 a[2], bfrag[2];
#pragma unroll
      for (int i = 0; i < 2; i++)
        a[i] = *reinterpret_cast<const i32x4*>(sA + (wm + i * 32 + l32) * ROWB + kb * 32 + lh * 16);
#pragma unroll
      for (int j = 0; j < 2; j++)
        bfrag[j] = *reinterpret_cast<const i32x4*>(sB + (wn + j * 32 + l32) * ROWB + kb * 32 + lh * 16);
      float dwv[2];
#pragma unroll
      for (int j = 0; j < 2; j++) dwv[j] = sdw[kb][wn + j * 32 + l32];
#pragma unroll
      for (int i = 0; i < 2; i++) {
        // the 16 rows this lane holds in a 32x32 tile: 8*(r/4) + 4*lh + r%4
        float dxv[16];
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const float4 t = *reinterpret_cast<const float4*>(&sdx[kb][wm + i * 32 + 8 * q + 4 * lh]);
          dxv[4 * q + 0] = t.x; dxv[4 * q + 1] = t.y; dxv[4 * q + 2] = t.z; dxv[4 * q + 3] = t.w;
        }
#pragma unroll
        for (int j = 0; j < 2; j++) {
          const i32x16 zero = {};
          const i32x16 isum = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], bfrag[j], zero, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 16; r++)
            acc[i][j][r] = fmaf(dxv[r] * dwv[j], (float)isum[r], acc[i][j][r]);
        }
      }
    }
  }

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

}  // namespace

int launch_quantize_q8_act(const float* X, int8_t* Xq, float* dx, int64_t M, int64_t K,
                           hipStream_t s) {
  const int64_t quads = M * K / 4;
  const int64_t grid = (quads + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(k_quantize_q8_act, dim3((unsigned)grid), dim3(kThreads), 0, s,
                     reinterpret_cast<const float4*>(X), reinterpret_cast<uint32_t*>(Xq), dx, quads);
  return launch_status();
}

int launch_qmm_q8_0(const void* w, const int8_t* Xq, const float* dx, float* Y, int64_t M,
                    int64_t N, int64_t K, hipStream_t s) {
  Layout L;
  layout_of(BQM_Q8_0, N, K, &L);
  const int8_t* Wc = static_cast<const int8_t*>(w);
  const uint16_t* Wd = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(w) + L.scales_off);
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  hipLaunchKernelGGL(k_qmm_q8_0, dim3((unsigned)(tiles_m * tiles_n)), dim3(kThreads), 0, s, Wc, Wd,
                     Xq, dx, Y, (int)M, (int)N, (int)L.nb, tiles_m, tiles_n);
  return launch_status();
}

}  // namespace bqm
