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
// Row tile of the dense product and workgroups per CU: 64 rows (waves 2 x 2, each 1 x 2
// MFMA tiles, 156-158 VGPRs) let three workgroups share a CU, which hides more of each
// wave's MFMA-to-epilogue latency than a 128-row tile's reuse saves (512 x 5120 x 17408:
// Q8_0 392 -> 426 TOP/s, Q4_0 393 -> 445 against 128 rows with two per CU).
#ifndef BQM_QMM_ROWS
#define BQM_QMM_ROWS 64
#endif
#ifndef BQM_QMM_WAVES
#define BQM_QMM_WAVES 3
#endif
constexpr int BM = BQM_QMM_ROWS, BN = 128, BKB = 4;  // BKB blocks of 32 per stage
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
// in the high one.  Each nibble becomes the int8 16 (n - 8), four to a word with no carry
// between bytes: flipping bit 3 of a nibble gives n - 8 as a 4-bit two's complement number,
// which read as the high half of a byte (the high nibble masked in place, the low one
// shifted up) is the int8 16 (n - 8).  The sums come out 16 times too large (exactly: at most
// 2^19 in magnitude); the epilogue takes the factor out.
constexpr uint32_t kQ4Flip = 0x88888888u, kHighNibbles = 0xF0F0F0F0u;
__device__ __forceinline__ void expand_q4(const u32x4& q, u32x4& lo, u32x4& hi) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint32_t v = q[i] ^ kQ4Flip;
    lo[i] = (v << 4) & kHighNibbles;
    hi[i] = v & kHighNibbles;
  }
}

// One workgroup tile of Y: TBM = 32 WGM TI rows (m) by BN columns (n); the four waves form
// a WGM x (4 / WGM) grid, each wave TI x TJ MFMA tiles of 32 x 32.  FMT selects how the
// weight codes arrive: Q8_0 as int8 rows [N][K]; Q4_0 as 16-byte blocks [N][nb][16],
// expanded to int8 while they are staged, so that the LDS layout and everything after it
// are the same for both.  Rows: dense (GATHER false), tile row r is input and output row
// m0 + r (< M); gathered, tile row r reads input row xrow[r] and writes output row yrow[r]
// (LDS tables, -1 past the tile's rows).  NQ < 4: only the first 8 NQ rows of each MFMA
// tile hold inputs, and the rescale skips the rest of a lane's results (rows 8 q .. 8 q + 7
// are its results 4 q .. 4 q + 3).
template <int FMT, int WGM, int TI, int TJ, bool GATHER, int NQ = 4>
__device__ __forceinline__ void qmm_core(const uint8_t* __restrict__ Wc, const uint16_t* __restrict__ Wd,
                                         const int8_t* __restrict__ Xq, const float* __restrict__ dx,
                                         int64_t x_rows, float* __restrict__ Y, int N, int nb, int n0,
                                         int m0, int M, const int* xrow, const int* yrow, int8_t* sA,
                                         int8_t* sB, u32x4* sXs, u32x4* sWs) {
  constexpr bool Q4 = FMT == BQM_Q4_0;
  constexpr int TBM = 32 * WGM * TI;
  constexpr int PA = TBM * 8 / kThreads;    // 16-byte pieces of activation codes per thread and stage
  constexpr int NXS = BKB * TBM;            // activation scales per stage ...
  constexpr int QX = (NXS + kThreads - 1) / kThreads;  // ... per thread
  constexpr int NPB = Q4 ? 2 : 4;           // 16-byte pieces of weight codes per thread and stage
  constexpr uint32_t kOob = 0x80000000u;    // a buffer offset past every descriptor: reads 0
  static_assert(PA >= 1 && PA <= 4 && QX >= 1 && QX <= 2, "tile shape");
  static_assert((4 / WGM) * 32 * TJ == BN, "the waves cover the BN columns");
  const int K = nb * 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave % WGM) * 32 * TI, wn = (wave / WGM) * 32 * TJ;
  const int l32 = lane & 31, lh = lane >> 5;
  // dx operands in LDS as [BKB][2][TBM]: the second half stays zero (lanes 32..63 of the
  // scale product's A operand hold its k = 8..15, which must be zero)
  for (int e = tid; e < NXS; e += kThreads) sXs[(e / TBM * 2 + 1) * TBM + e % TBM] = u32x4{0u, 0u, 0u, 0u};
  // input row of tile row r, or -1
  auto in_row = [&](int r) -> int {
    if constexpr (GATHER) return xrow[r];
    else return m0 + r < M ? m0 + r : -1;
  };

  // Gathered rows fill a tile from its first row, so a wave whose first row has no input
  // row has nothing to compute (it still loads and stages its pieces for the other waves).
  const bool live = !GATHER || __builtin_amdgcn_readfirstlane(in_row(wm)) >= 0;

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; i++)
#pragma unroll
    for (int j = 0; j < TJ; j++) acc[i][j] = f32x16{};

  // Loads go through buffer descriptors: each lane's offset is fixed for the whole K loop
  // (row and place in the stage), the stage's block offset is a scalar.  A lane's piece
  // past the rows, or (last stage) past K, reads zeros through an offset past the
  // descriptor; every other access lies inside the operand by construction.
  const int64_t wrow = Q4 ? (int64_t)nb * 16 : (int64_t)K;  // bytes per weight row
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void*)Xq, (short)0, (int)(x_rows * K), 0x00020000);
  const __amdgpu_buffer_rsrc_t rX = __builtin_amdgcn_make_buffer_rsrc((void*)dx, (short)0, (int)(x_rows * nb * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc((void*)Wc, (short)0, (int)(N * wrow), 0x00020000);
  const __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc((void*)Wd, (short)0, (int)((int64_t)N * nb * 2), 0x00020000);
  uint32_t oA[PA], oB[NPB], oX[QX], oW[2];
  int bA[PA], bB[NPB], bX[QX], bW[2];  // block of the stage each piece belongs to
#pragma unroll
  for (int p = 0; p < PA; p++) {
    const int piece = tid + p * kThreads, row = piece >> 3, c16 = piece & 7;
    const int xr = in_row(row);
    oA[p] = xr >= 0 ? (uint32_t)xr * (uint32_t)K + c16 * 16 : kOob;
    bA[p] = c16 >> 1;
  }
#pragma unroll
  for (int p = 0; p < NPB; p++) {
    const int piece = tid + p * kThreads;
    const int row = Q4 ? piece >> 2 : piece >> 3, c16 = Q4 ? piece & 3 : piece & 7;
    oB[p] = n0 + row < N ? (uint32_t)((n0 + row) * wrow) + c16 * 16 : kOob;
    bB[p] = Q4 ? c16 : c16 >> 1;
  }
#pragma unroll
  for (int q = 0; q < QX; q++) {
    const int e = tid + q * kThreads, kb = e / TBM, r = e % TBM;
    const int xr = e < NXS ? in_row(r) : -1;
    oX[q] = xr >= 0 ? ((uint32_t)xr * (uint32_t)nb + kb) * 4u : kOob;
    bX[q] = kb;
  }
#pragma unroll
  for (int q = 0; q < 2; q++) {
    const int e = tid + q * kThreads, kb = e >> 7, r = e & 127;
    oW[q] = n0 + r < N ? ((uint32_t)(n0 + r) * (uint32_t)nb + kb) * 2u : kOob;
    bW[q] = kb;
  }

  // two register sets of staged pieces: the loads of stage s + 2 are issued while stage s is
  // computed, stage s + 1's already in flight
  u32x4 pa[2][PA], pb[2][NPB];
  uint32_t px[2][QX], pw[2][2];
  auto fetch = [&](auto SET, int b0) {
    constexpr int S = decltype(SET)::value;
    const int bn_ = min(BKB, nb - b0);
    const bool full = bn_ == BKB;
#pragma unroll
    for (int p = 0; p < PA; p++)
      pa[S][p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     rA, full || bA[p] < bn_ ? oA[p] : kOob, b0 * 32, 0));
#pragma unroll
    for (int p = 0; p < NPB; p++)
      pb[S][p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     rB, full || bB[p] < bn_ ? oB[p] : kOob, b0 * (Q4 ? 16 : 32), 0));
#pragma unroll
    for (int q = 0; q < QX; q++)
      px[S][q] = __builtin_amdgcn_raw_buffer_load_b32(rX, full || bX[q] < bn_ ? oX[q] : kOob, b0 * 4, 0);
#pragma unroll
    for (int q = 0; q < 2; q++)
      pw[S][q] = (uint32_t)__builtin_bit_cast(uint16_t, __builtin_amdgcn_raw_buffer_load_b16(
                     rW, full || bW[q] < bn_ ? oW[q] : kOob, b0 * 2, 0));
  };

  auto stage = [&](auto SET, int b0) {
    constexpr int S = decltype(SET)::value;
    const int bn = min(BKB, nb - b0);
    __syncthreads();  // every wave is done with the previous stage
#pragma unroll
    for (int p = 0; p < PA; p++) {
      const int piece = tid + p * kThreads, row = piece >> 3, c16 = piece & 7;
      *reinterpret_cast<u32x4*>(sA + row * ROWB + c16 * 16) = pa[S][p];
    }
#pragma unroll
    for (int p = 0; p < NPB; p++) {
      const int piece = tid + p * kThreads;
      if constexpr (Q4) {
        const int row = piece >> 2, kb = piece & 3;
        u32x4 lo, hi;
        expand_q4(pb[S][p], lo, hi);
        *reinterpret_cast<u32x4*>(sB + row * ROWB + kb * 32) = lo;
        *reinterpret_cast<u32x4*>(sB + row * ROWB + kb * 32 + 16) = hi;
      } else {
        const int row = piece >> 3, c16 = piece & 7;
        *reinterpret_cast<u32x4*>(sB + row * ROWB + c16 * 16) = pb[S][p];
      }
    }
#pragma unroll
    for (int q = 0; q < QX; q++) {
      const int e = tid + q * kThreads;  // = kb * TBM + r
      if (e < NXS) sXs[(e / TBM * 2) * TBM + e % TBM] = dx_operand(__uint_as_float(px[S][q]));
    }
#pragma unroll
    for (int q = 0; q < 2; q++) sWs[tid + q * kThreads] = dw_operand(pw[S][q]);  // kb * BN + r
    __syncthreads();
    if (b0 + 2 * BKB < nb) fetch(SET, b0 + 2 * BKB);

    // unrolled over the stage's blocks, so every LDS read has an immediate offset
#pragma unroll
    for (int kb = 0; kb < BKB; kb++) {
      if (kb < bn && live) {
        i32x4 a[TI], bq[TJ];
        bf16x8 as[TI], bs[TJ];
#pragma unroll
        for (int i = 0; i < TI; i++) {
          a[i] = *reinterpret_cast<const i32x4*>(sA + (wm + i * 32 + l32) * ROWB + kb * 32 + lh * 16);
          as[i] = __builtin_bit_cast(bf16x8, sXs[(kb * 2 + lh) * TBM + wm + i * 32 + l32]);
        }
#pragma unroll
        for (int j = 0; j < TJ; j++) {
          bq[j] = *reinterpret_cast<const i32x4*>(sB + (wn + j * 32 + l32) * ROWB + kb * 32 + lh * 16);
          // lanes 32..63 read the same operand row: it meets the zero half of A
          bs[j] = __builtin_bit_cast(bf16x8, sWs[kb * BN + wn + j * 32 + l32]);
        }
#pragma unroll
        for (int i = 0; i < TI; i++)
#pragma unroll
          for (int j = 0; j < TJ; j++) {
            const i32x16 isum = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], bq[j], i32x16{}, 0, 0, 0);
            const f32x16 sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as[i], bs[j], f32x16{}, 0, 0, 0);
            // a lane's results r = 4 q .. 4 q + 3 lie in the tile's rows 8 q .. 8 q + 7
#pragma unroll
            for (int r = 0; r < 4 * NQ; r++) acc[i][j][r] = fmaf(sc[r], (float)isum[r], acc[i][j][r]);
          }
      }
    }
  };

  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  fetch(Set0{}, 0);
  if (BKB < nb) fetch(Set1{}, BKB);
  for (int b0 = 0; b0 < nb; b0 += 2 * BKB) {
    stage(Set0{}, b0);
    if (b0 + BKB < nb) stage(Set1{}, b0 + BKB);
  }

  // a lane's 16 results of a 32 x 32 tile: rows 8 (r / 4) + 4 lh + r % 4, column l32.  Q4_0
  // sums carry the factor 16 of the expanded codes: every rounding step above saw exactly 16
  // times the values of the unscaled sums, so the product with 1/16 is the unscaled result
  // (outside fp32's subnormal range, where the scaled sums kept more bits)
  constexpr float kOut = Q4 ? 0.0625f : 1.0f;
#pragma unroll
  for (int i = 0; i < TI; i++)
#pragma unroll
    for (int j = 0; j < TJ; j++) {
      const int n = n0 + wn + j * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int tr = wm + i * 32 + 8 * (r / 4) + 4 * lh + (r % 4);
        if constexpr (GATHER) {
          const int yr = yrow[tr];
          if (yr >= 0 && n < N) Y[(size_t)yr * N + n] = acc[i][j][r] * kOut;
        } else {
          const int m = m0 + tr;
          if (m < M && n < N) Y[(size_t)m * N + n] = acc[i][j][r] * kOut;
        }
      }
    }
}

template <int FMT>
__device__ __forceinline__ void qmm_dense(const uint8_t* __restrict__ Wc, const uint16_t* __restrict__ Wd,
                                          const int8_t* __restrict__ Xq, const float* __restrict__ dx,
                                          float* __restrict__ Y, int M, int N, int nb, int tiles_m,
                                          int tiles_n) {
  __shared__ __attribute__((aligned(16))) int8_t sA[BM * ROWB];
  __shared__ __attribute__((aligned(16))) int8_t sB[BN * ROWB];
  __shared__ u32x4 sXs[BKB * 2 * BM];  // dx operands per (block, m), each block's zero half after it
  __shared__ u32x4 sWs[BKB * BN];      // dw operands per (block, n)
  // Workgroups are dealt round-robin to the eight XCDs; give the workgroups of one XCD
  // neighbouring tiles (all m-tiles of a few n-tiles) so they share W rows in that L2.
  const int nwg = tiles_m * tiles_n;
  const int bid = blockIdx.x;
  int tile = bid;
  if (nwg % 8 == 0) tile = (bid % 8) * (nwg / 8) + bid / 8;
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  constexpr int WGM = BM == 32 ? 1 : 2;  // waves along m; each covers 128 / (4 / WGM) columns
  qmm_core<FMT, WGM, BM / (32 * WGM), WGM, false>(Wc, Wd, Xq, dx, M, Y, N, nb, tn * BN, tm * BM,
                                                  M, nullptr, nullptr, sA, sB, sXs, sWs);
}

// Exclusive prefix sum of v over the workgroup's threads (thread order).
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(x, o, 64);
    if (lane >= o) x += u;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; w++) base += wsum[w];
  __syncthreads();
  return base + x - v;
}

// Exclusive prefix sums of u and v over the workgroup's threads (thread order), and their
// totals.
__device__ __forceinline__ void block_exclusive_scan2(int& u, int& v, int* wsum, int& tu, int& tv) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = u, y = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int p = __shfl_up(x, o, 64), q = __shfl_up(y, o, 64);
    if (lane >= o) {
      x += p;
      y += q;
    }
  }
  if (lane == 63) {
    wsum[2 * wave] = x;
    wsum[2 * wave + 1] = y;
  }
  __syncthreads();
  int bu = 0, bv = 0;
  tu = tv = 0;
  for (int w = 0; w < kThreads / 64; w++) {
    if (w < wave) {
      bu += wsum[2 * w];
      bv += wsum[2 * w + 1];
    }
    tu += wsum[2 * w];
    tv += wsum[2 * w + 1];
  }
  __syncthreads();
  u = bu + x - u;
  v = bv + y - v;
}

// Expert-indexed prefill product.  Every workgroup counts the slots per expert and cuts each
// expert's slots (in index order) into row tiles: tall tiles of kIdTall slots while more
// than kIdShort are left, then one short tile of kIdShort for a remainder that fits one.
// The tall tiles of all experts are numbered first (experts ascending), then the short
// ones; workgroup b takes row tile b / tiles_n, column tile b % tiles_n, and workgroups past
// the last row tile only take part in the padding fill.  A tall tile runs its four waves
// as 2 x 2 (each 32 rows x 64 columns), a short one as 1 x 4 (each 32 x 32): measured on
// the 512-token MoE prefill (128 experts, top-8, a skewed router: half the experts hold two
// slots or fewer, the busiest about 500), a short remainder in a tall tile left the two
// waves of its empty half with nothing to compute, and 32-row tiles throughout (waves
// 1 x 4) lost on the busy experts' reuse of each weight tile.
constexpr int kIdTall = 64, kIdShort = 32;
constexpr int kIdChunk = 16;  // slot ids a thread loads at once
// A short tile holding at most kIdFew slots (most of the rarely chosen experts' tiles) rescales
// only the MFMA results of its first kIdFew rows: a separate instantiation, since a branch per
// row group inside the block loop cost more than it saved (it splits the MFMA and VALU
// stream the compiler interleaves).
constexpr int kIdFew = 8;

template <int FMT>
__device__ __forceinline__ void qmm_indexed(const uint8_t* __restrict__ Wc, const uint16_t* __restrict__ Wd,
                                            const int8_t* __restrict__ Xq, const float* __restrict__ dx,
                                            const int32_t* __restrict__ ids, float* __restrict__ Y,
                                            int E, int N, int nb, int TS, int top_k, int xtr, int xsr,
                                            int64_t x_rows,
                                            int tiles_n) {
  __shared__ __attribute__((aligned(16))) int8_t sA[kIdTall * ROWB];
  __shared__ __attribute__((aligned(16))) int8_t sB[BN * ROWB];  // first: per-expert counts
  __shared__ u32x4 sXs[BKB * 2 * kIdTall];
  __shared__ u32x4 sWs[BKB * BN];
  __shared__ int xrow[kIdTall], yrow[kIdTall];
  __shared__ int wsum[2 * (kThreads / 64)];
  __shared__ int tile_e, tile_m0, tile_h, tile_rows;
  const int tid = threadIdx.x;
  // Thread t owns the slots [s0, s1).  Their ids are read in chunks of kIdChunk through a
  // buffer descriptor, every load of a chunk issued before the first is used (a slot past the
  // thread's range reads its neighbour's id, or 0 past TS, and is masked); the first chunk
  // stays in registers for both passes over the slots.  (Read one at a time, the ids cost
  // each workgroup two or three dependent round trips per slot it owns: on the 512-token MoE
  // prefill, a quarter of the kernel's time.)
  const int sper = (TS + kThreads - 1) / kThreads;
  const int s0 = min(TS, tid * sper), s1 = min(TS, s0 + sper);
  const __amdgpu_buffer_rsrc_t rI = __builtin_amdgcn_make_buffer_rsrc((void*)ids, (short)0, TS * 4, 0x00020000);
  auto load_chunk = [&](int c0, int* v) {
#pragma unroll
    for (int k = 0; k < kIdChunk; k++) v[k] = __builtin_amdgcn_raw_buffer_load_b32(rI, (c0 + k) * 4, 0, 0);
  };
  int v0[kIdChunk];
  load_chunk(s0, v0);
  // rows of slots that no tile computes, each by one workgroup (slots blockIdx.x + j gridDim.x,
  // their ids read four at a time alongside the chunk): a padding slot (negative id) gives
  // zeros, an id >= E NaN
  for (int i0 = blockIdx.x; i0 < TS; i0 += 4 * gridDim.x) {
    int f[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int64_t i = i0 + (int64_t)j * gridDim.x;
      f[j] = __builtin_amdgcn_raw_buffer_load_b32(rI, (int)(i < TS ? i : TS) * 4, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int64_t i = i0 + (int64_t)j * gridDim.x;
      const int e = f[j];
      if (i >= TS || (e >= 0 && e < E)) continue;
      const float v = e < 0 ? 0.0f : __builtin_nanf("");
      for (int n = tid; n < N; n += kThreads) Y[(size_t)i * N + n] = v;
    }
  }
  // f(slot, id) for every slot of [s0, s1), in order
  auto for_slots = [&](auto&& f) {
#pragma unroll
    for (int k = 0; k < kIdChunk; k++)
      if (s0 + k < s1) f(s0 + k, v0[k]);
    for (int c0 = s0 + kIdChunk; c0 < s1; c0 += kIdChunk) {
      int v[kIdChunk];
      load_chunk(c0, v);
#pragma unroll
      for (int k = 0; k < kIdChunk; k++)
        if (c0 + k < s1) f(c0 + k, v[k]);
    }
  };
  int* cnt = reinterpret_cast<int*>(sB);
  for (int e = tid; e < E; e += kThreads) cnt[e] = 0;
  if (tid == 0) tile_e = -1;
  __syncthreads();
  for_slots([&](int, int e) {
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  });
  __syncthreads();
  // tall and short tiles of an expert with c slots
  auto tall = [](int c) { return c / kIdTall + (c % kIdTall > kIdShort ? 1 : 0); };
  auto short_ = [](int c) { const int r = c % kIdTall; return r > 0 && r <= kIdShort ? 1 : 0; };
  // find this workgroup's row tile: thread t holds experts [e0, e1) and their tile counts
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int per = (E + kThreads - 1) / kThreads;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int mt = 0, ms = 0;
  for (int e = e0; e < e1; e++) {
    mt += tall(cnt[e]);
    ms += short_(cnt[e]);
  }
  int ft = mt, fs = ms, nt, ns;
  block_exclusive_scan2(ft, fs, wsum, nt, ns);
  if (tm >= ft && tm < ft + mt) {
    int t = ft;
    for (int e = e0; e < e1; e++) {
      const int k = tall(cnt[e]);
      if (tm < t + k) {
        tile_e = e;
        tile_m0 = (tm - t) * kIdTall;
        tile_h = kIdTall;
        tile_rows = min(kIdTall, cnt[e] - tile_m0);
        break;
      }
      t += k;
    }
  } else if (tm >= nt + fs && tm < nt + fs + ms) {
    int t = nt + fs;
    for (int e = e0; e < e1; e++) {
      if (short_(cnt[e]) && tm == t++) {
        tile_e = e;
        tile_m0 = cnt[e] / kIdTall * kIdTall;
        tile_h = kIdShort;
        tile_rows = cnt[e] - tile_m0;
        break;
      }
    }
  }
  for (int r = tid; r < kIdTall; r += kThreads) xrow[r] = yrow[r] = -1;
  __syncthreads();
  const int e = tile_e;
  if (e < 0) return;  // past the last row tile (uniform)
  const int m0 = tile_m0, h = __builtin_amdgcn_readfirstlane(tile_h), rows = __builtin_amdgcn_readfirstlane(tile_rows);
  // the expert's slots of ranks m0 .. m0 + h - 1 (rank: place among its slots in index order)
  int c = 0;
  for_slots([&](int, int id) { c += id == e; });
  int rank = block_exclusive_scan(c, wsum);
  for_slots([&](int i, int id) {
    if (id == e) {
      const int r = rank - m0;
      if (r >= 0 && r < h) {
        const int t = i / top_k;
        xrow[r] = t * xtr + (i - t * top_k) * xsr;
        yrow[r] = i;
      }
      ++rank;
    }
  });
  __syncthreads();
  const int64_t wrow = FMT == BQM_Q4_0 ? (int64_t)nb * 16 : (int64_t)nb * 32;
  const uint8_t* We = Wc + (int64_t)e * N * wrow;
  const uint16_t* De = Wd + (int64_t)e * N * nb;
  if (h == kIdTall)
    qmm_core<FMT, 2, 1, 2, true>(We, De, Xq, dx, x_rows, Y, N, nb, tn * BN, 0, 0, xrow, yrow, sA, sB, sXs, sWs);
  else if (rows > kIdFew)
    qmm_core<FMT, 1, 1, 1, true>(We, De, Xq, dx, x_rows, Y, N, nb, tn * BN, 0, 0, xrow, yrow, sA, sB, sXs, sWs);
  else
    qmm_core<FMT, 1, 1, 1, true, kIdFew / 8>(We, De, Xq, dx, x_rows, Y, N, nb, tn * BN, 0, 0, xrow, yrow, sA, sB,
                                             sXs, sWs);
}

#define BQM_QMM_KERNEL(NAME, FMT)                                                              \
  __global__ __launch_bounds__(kThreads)                                                       \
  __attribute__((amdgpu_waves_per_eu(BQM_QMM_WAVES, BQM_QMM_WAVES))) void NAME(                \
      const uint8_t* __restrict__ Wc, const uint16_t* __restrict__ Wd,                         \
      const int8_t* __restrict__ Xq, const float* __restrict__ dx, float* __restrict__ Y,      \
      int M, int N, int nb, int tiles_m, int tiles_n) {                                        \
    qmm_dense<FMT>(Wc, Wd, Xq, dx, Y, M, N, nb, tiles_m, tiles_n);                             \
  }
BQM_QMM_KERNEL(k_qmm_q8_0, BQM_Q8_0)
BQM_QMM_KERNEL(k_qmm_q4_0, BQM_Q4_0)
#undef BQM_QMM_KERNEL

#ifndef BQM_QMM_ID_WAVES
#define BQM_QMM_ID_WAVES 3  // waves per SIMD (workgroups per CU) the indexed kernel is built for
#endif
#define BQM_QMM_ID_KERNEL(NAME, FMT)                                                           \
  __global__ __launch_bounds__(kThreads)                                                       \
  __attribute__((amdgpu_waves_per_eu(BQM_QMM_ID_WAVES, BQM_QMM_ID_WAVES))) void NAME(          \
      const uint8_t* __restrict__ Wc, const uint16_t* __restrict__ Wd,                         \
      const int8_t* __restrict__ Xq, const float* __restrict__ dx,                             \
      const int32_t* __restrict__ ids, float* __restrict__ Y, int E, int N, int nb, int TS,    \
      int top_k, int xtr, int xsr, int64_t x_rows, int tiles_n) {                              \
    qmm_indexed<FMT>(Wc, Wd, Xq, dx, ids, Y, E, N, nb, TS, top_k, xtr, xsr, x_rows, tiles_n);  \
  }
BQM_QMM_ID_KERNEL(k_qmm_id_q8_0, BQM_Q8_0)
BQM_QMM_ID_KERNEL(k_qmm_id_q4_0, BQM_Q4_0)
#undef BQM_QMM_ID_KERNEL

}  // namespace

int launch_quantize_q8_act(const float* X, int8_t* Xq, float* dx, int64_t M, int64_t K,
                           hipStream_t s) {
  const int64_t quads = M * K / 4;
  const int64_t grid = (quads + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(k_quantize_q8_act, dim3((unsigned)grid), dim3(kThreads), 0, s,
                     reinterpret_cast<const float4*>(X), reinterpret_cast<uint32_t*>(Xq), dx, quads);
  return launch_status();
}

// The kernels address each operand through a buffer descriptor with 32-bit offsets.
static bool fits_descriptors(int fmt, int64_t x_rows, int64_t N, int64_t K) {
  const int64_t lim = (int64_t)1 << 31;
  const int64_t wrow = fmt == BQM_Q4_0 ? K / 2 : K;  // code bytes per weight row
  return x_rows * K < lim && x_rows * (K / 32) * 4 < lim && N * wrow < lim && N * (K / 32) * 2 < lim;
}

static int launch_qmm(int fmt, const void* w, const int8_t* Xq, const float* dx, float* Y,
                      int64_t M, int64_t N, int64_t K, hipStream_t s) {
  if (!fits_descriptors(fmt, M, N, K)) return BQM_E_SHAPE;
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

int launch_qmm_id(int fmt, const void* w, int E, int64_t N, int64_t K, const int32_t* ids, int T,
                  int top_k, const int8_t* Xq, const float* dx, int64_t x_tok_rows,
                  int64_t x_slot_rows, float* Y, hipStream_t s) {
  Layout L;
  layout_of(fmt, (int64_t)E * N, K, &L);
  const uint8_t* Wc = static_cast<const uint8_t*>(w);
  const uint16_t* Wd = reinterpret_cast<const uint16_t*>(Wc + L.scales_off);
  const int TS = T * top_k;
  const int tiles_n = (int)((N + BN - 1) / BN);
  // row tiles: at most one partial tile per expert that has slots, plus the full ones
  const int64_t max_tm = (TS < E ? TS : E) + (TS + kIdTall - 1) / kIdTall;
  const int64_t grid = max_tm * tiles_n;
  // input rows the slots can address: row (T - 1) x_tok_rows + (top_k - 1) x_slot_rows at most
  const int64_t x_rows = (int64_t)(T - 1) * x_tok_rows + (int64_t)(top_k - 1) * x_slot_rows + 1;
  if (grid >= ((int64_t)1 << 31) || !fits_descriptors(fmt, x_rows, N, K)) return BQM_E_SHAPE;
  hipLaunchKernelGGL(fmt == BQM_Q4_0 ? k_qmm_id_q4_0 : k_qmm_id_q8_0, dim3((unsigned)grid),
                     dim3(kThreads), 0, s, Wc, Wd, Xq, dx, ids, Y, E, (int)N, (int)L.nb, TS, top_k,
                     (int)x_tok_rows, (int)x_slot_rows, x_rows, tiles_n);
  return launch_status();
}

}  // namespace bqm
