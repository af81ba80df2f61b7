// Operands of the bf16 matrix-core products over packed codes, gfx950 (device code; included
// by the matrix-core GEMV kernels).
//
// Codes enter v_mfma_f32_16x16x32_bf16 as exact bf16 signed values (Q4_0 as 16 (n - 8), Q8_0
// the int8 code), inputs as two bf16 parts of x * 2^kXShift (see split): bf16 products are
// exact in fp32, so a block sum carries the MFMA's fp32 accumulation error plus at most
// 2^-14 sum_j |c_j x_j| from the part of x left out.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bqm {
namespace mma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float sbyte(uint32_t v, int b) {
  return (float)(int8_t)(v >> (8 * b));  // v_cvt_f32_i32 with a sign-extending byte select
}
// Two floats whose low 16 bits are zero (exact bf16 values) -> one bf16 pair, f0 low.
__device__ __forceinline__ uint32_t bf_pair(float f0, float f1) {
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f1), __builtin_bit_cast(uint32_t, f0),
                               0x07060302u);
}
// One word of Q4_0 codes (bytes 4q..4q+3 of a block) -> an MFMA operand: 16 (n - 8) of the
// low nibbles (positions 4q..4q+3), then of the high ones (16+4q..16+4q+3).  n ^ 8 is n - 8
// in four-bit two's complement; placed at the top of a byte it reads as 16 (n - 8).
__device__ __forceinline__ bf16x8 q4_operand(uint32_t w) {
  const uint32_t lo = ((w << 4) ^ 0x80808080u) & 0xF0F0F0F0u;
  const uint32_t hi = (w ^ 0x80808080u) & 0xF0F0F0F0u;
  const u32x4 v{bf_pair(sbyte(lo, 0), sbyte(lo, 1)), bf_pair(sbyte(lo, 2), sbyte(lo, 3)),
                bf_pair(sbyte(hi, 0), sbyte(hi, 1)), bf_pair(sbyte(hi, 2), sbyte(hi, 3))};
  return __builtin_bit_cast(bf16x8, v);
}
// Eight Q8_0 codes (bytes 8q..8q+7 of a block) -> an MFMA operand.
__device__ __forceinline__ bf16x8 q8_operand(uint32_t w0, uint32_t w1) {
  const u32x4 v{bf_pair(sbyte(w0, 0), sbyte(w0, 1)), bf_pair(sbyte(w0, 2), sbyte(w0, 3)),
                bf_pair(sbyte(w1, 0), sbyte(w1, 1)), bf_pair(sbyte(w1, 2), sbyte(w1, 3))};
  return __builtin_bit_cast(bf16x8, v);
}

// Inputs enter scaled by 2^kXShift (exact), which lifts every fp32 subnormal into the
// range where the two bf16 parts keep all but 2^-14 of it (a bf16 part cannot hold a value
// below 2^-133, and the smallest fp32 subnormal is 2^-149); the block scale carries
// 2^-kXShift back.  The price: |x| must stay below 2^86 for the partial sums (codes up to
// 128 = 2^7 times 32 terms) to stay below fp32's limit.
constexpr int kXShift = 30;
// x -> (x_hi, x_lo) bits of x * 2^kXShift: truncated to bf16, and the exact remainder
// truncated to bf16 (zero when x is not finite: x_hi carries the infinity or NaN).
__device__ __forceinline__ void split(float x, uint32_t& hi, uint32_t& lo) {
  const float f = x * 0x1p30f;
  static_assert(kXShift == 30, "the literal above");
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  hi = u & 0xFFFF0000u;
  const float r = f - __builtin_bit_cast(float, hi);
  lo = __builtin_isfinite(f) ? __builtin_bit_cast(uint32_t, r) & 0xFFFF0000u : 0u;
}
// Eight consecutive inputs (k-group order) -> their two bf16 parts, each as 16 bytes.
__device__ __forceinline__ void split8(const float (&f)[8], u32x4& hi, u32x4& lo) {
  uint32_t hb[8], lb[8];
#pragma unroll
  for (int k = 0; k < 8; k++) split(f[k], hb[k], lb[k]);
  hi = u32x4{(hb[1] & 0xFFFF0000u) | (hb[0] >> 16), (hb[3] & 0xFFFF0000u) | (hb[2] >> 16),
             (hb[5] & 0xFFFF0000u) | (hb[4] >> 16), (hb[7] & 0xFFFF0000u) | (hb[6] >> 16)};
  lo = u32x4{(lb[1] & 0xFFFF0000u) | (lb[0] >> 16), (lb[3] & 0xFFFF0000u) | (lb[2] >> 16),
             (lb[5] & 0xFFFF0000u) | (lb[4] >> 16), (lb[7] & 0xFFFF0000u) | (lb[6] >> 16)};
}

// v_permlane32_swap: rows 2-3 (lanes 32-63) of a <-> rows 0-1 of b; v_permlane16_swap:
// rows 1 and 3 of a <-> rows 0 and 2 of b (a row is 16 lanes)
__device__ __forceinline__ void swap32(uint32_t& x, uint32_t& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  x = r[0];
  y = r[1];
}
__device__ __forceinline__ void swap16(uint32_t& x, uint32_t& y) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, y, false, false);
  x = r[0];
  y = r[1];
}
// A 16-byte code load in which lane group g (lanes 16g..16g+15, one row each) holds bytes
// 16g..16g+15 of a 64-byte piece of its row -> the words the MFMA operands take.  Q4_0 (the
// piece is blocks 0-3, 16 bytes each): afterwards word u of lane group q is word q of block u
// (a 4 x 4 transpose between the lane groups and the words).  Q8_0 (the piece is blocks 0-1,
// 32 bytes each): afterwards words 0-1 of lane group q are bytes 8q..8q+7 of block 0, words
// 2-3 those of block 1.
template <bool Q4>
__device__ __forceinline__ void exchange(u32x4& v) {
  uint32_t r0 = v.x, r1 = v.y, r2 = v.z, r3 = v.w;
  if constexpr (Q4) {
    swap32(r0, r2);
    swap32(r1, r3);
    swap16(r0, r1);
    swap16(r2, r3);
  } else {
    swap16(r0, r2);
    swap16(r1, r3);
    swap32(r0, r2);
    swap32(r1, r3);
  }
  v = u32x4{r0, r1, r2, r3};
}

}  // namespace mma
}  // namespace bqm
