// Decode GEMV / small-batch GEMV over packed Q4_0 and Q8_0 weights, gfx950.
//
// Y[m][n] = sum_k dequant(W)[n][k] * X[m][k]. Decode reads every weight once per token
// ("V100跑Qwen 27B：量化与KV Cache调优" (lmnt.cn), section 1.2), so the kernels are built
// around streaming the packed codes from HBM once, at full 16-byte load width, and doing as
// little VALU work per weight as the format allows.
//
// Work mapping.  A row of the matrix is handled by a group of 16 lanes; lane g of the group
// owns blocks g, g+16, g+32, ... of the row, one whole 32-weight block per 16-byte (Q4_0) or
// 2x16-byte (Q8_0) load.  A lane holds R rows at once (two for most batch sizes), so the
// inputs it reads from LDS for one block serve R rows.
//
// Activations.  The M inputs are staged once per workgroup into LDS, one block per 144
// bytes (128 bytes of x and 16 unused, a stride at which eight neighbouring blocks start in
// eight different bank groups); rows too long for the LDS budget are staged in chunks.
//
// Arithmetic.  Every code becomes its signed value exactly before it meets x (a Q4_0 nibble
// as 16 (n - 8) in a byte, a Q8_0 code as is, each through a sign-extending byte
// conversion), and each block's 32 products are summed by fused multiply-adds, then scaled by
// d (Q4_0: d / 16): the rounding error of a block stays proportional to sum |(n - 8) d x|, its
// share of the tolerance scale, and neutral codes give exactly zero.  The signed codes of a
// block are formed once and shared by the M inputs.
//
// Reduction: DPP exchanges inside the 16-lane group, then one lane stores the row; a tile
// split between waves is finished through LDS in wave order.  No atomics on data; the
// summation order is fixed for a given launch shape.
#include "bqm_internal.h"
#include "mma_ops.h"
#include "slot_groups.h"

#include <algorithm>
#include <atomic>
#include <type_traits>
#include <mutex>
#include <unordered_map>
#include <vector>

namespace bqm {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__device__ __forceinline__ float h2f(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}
__device__ __forceinline__ float ub(uint32_t v, int k) {
  return (float)((v >> (8 * k)) & 0xffu);  // v_cvt_f32_ubyte{k}
}

enum { FQ4 = 0, FQ8 = 1 };

template <int FMT> struct Codes;
template <> struct Codes<FQ4> { u32x4 a; };
template <> struct Codes<FQ8> { u32x4 a, b; };

// ---- persistent GEMV chain ------------------------------------------------------------
// Decode is bandwidth-critical, so the batch-M (M <= 8) product gets its own kernel shaped
// around the VALU budget and around the cost of starting a kernel (Q4_0 at 8 TB/s delivers
// 14.2 T weights/s against 39.3 T fp32 lane-ops/s, about 2.8 ops per weight).  One launch
// runs a chain of GEMVs in order (a single GEMV is a chain of one):
//  - One 1024-thread workgroup per CU owns, for each GEMV, a contiguous range of rows and
//    stages that GEMV's M inputs into LDS.  Blocks are 144 bytes apart in LDS (128 bytes of
//    x and 16 unused): with that stride eight neighbouring blocks start in eight different
//    16-byte bank groups, so the per-lane block reads are conflict-free with immediate
//    offsets.
//  - When M inputs of K do not fit, a GEMV is walked in chunks of kc blocks of K: the
//    workgroup stages one chunk of x at a time and keeps each row's partial sums in LDS,
//    adding the chunks in order.
//  - Codes and scales come through buffer loads: the per-lane part of the offset is a
//    constant register, the per-step part a scalar, so a load costs no VALU address
//    arithmetic.  Lanes past the workgroup's last row (or past K in a ragged last step)
//    use an offset beyond the descriptor and read zeros.
//  - Each lane keeps P blocks in flight in a register ring consumed in place (the loop is
//    unrolled by P).  The ring runs ahead across GEMV and chunk boundaries: the weights of
//    the next GEMV do not depend on its input, so they stream while the workgroup waits for
//    the previous GEMV's outputs (device-wide barrier) and stages the new x.
// Arithmetic per block and row (see chain_block): Q4_0 12 integer ops and 32 sign-extending
// conversions give the signed codes, Q8_0 32 conversions; then per input 32 fp32 FMAs and
// acc += d * sum.
constexpr int kP1Waves = 16;  // waves of a workgroup (8 for the widest batch: registers)
constexpr int kBlkLds = 144;  // LDS bytes per staged block
constexpr int kChainMaxM = 8;
// A row's blocks are taken by a group of kG lanes (lane g: blocks g, g + kG, ...), kGpw
// groups per wave.  Narrow groups are faster on every shape measured (16 lanes against the
// 64 or 32 that leave as few idle lanes, e.g. 4096 x 4096 Q4_0: +18 %): a row's sum is
// reduced over fewer lanes and once per more blocks, and the lanes of a wave read fewer
// distinct staged input blocks per step (LDS broadcasts the rest).
#ifndef BQM_LG2G
#define BQM_LG2G 4
#endif
constexpr int kLg2G = BQM_LG2G, kG = 1 << kLg2G, kGpw = 64 >> kLg2G;
static_assert(kLg2G >= 3 && kLg2G <= 4, "group_sum covers 8 or 16 lanes");

// ---- per-block arithmetic ------------------------------------------------------------
// Each code is turned into its signed value exactly (Q4_0: nibble - 8, Q8_0: the int8 code)
// before it meets x, and a block's 32 products are summed by fused multiply-adds in a fixed
// order (chain_block): a product is exact inside its FMA, so the block sum carries at most
// 32 roundings of partial sums that are each bounded by sum_j |code_j x_j|, the block's
// share of S = sum |w x|.  (Summing unsigned codes and subtracting the offset times sum x
// afterwards cancels: its error grows with sum (n + 8)|x| and can swallow a whole
// near-neutral block.)  All-neutral codes give exactly zero.

// Q4_0 codes as bytes holding 16 (n - 8): a nibble n with its top bit flipped, n ^ 8, is the
// two's complement of n - 8 in four bits, so (w ^ 0x80808080) & 0xF0F0F0F0 leaves the high
// nibbles (positions 16 + 4k + b of word k) as 16 (n - 8) at the top of their bytes and
// ((w << 4) ^ 0x80808080) & 0xF0F0F0F0 the low ones (positions 4k + b); one shift and two
// three-input bit operations (v_bitop3_b32) per word.  A sign-extending byte conversion
// (v_cvt_f32_i32 with an SDWA byte select) then gives 16 (n - 8) exactly, and the 1/16 goes
// into the block's scale (d / 16 is exact for every binary16 d).  Measured on gfx950: plain fp32 FMAs issue about twice as
// fast as v_fma_mix_f32, the packed binary16 ops and the conversions, so this form (3 integer
// ops and 8 conversions per 8 codes, then plain FMAs) beats binary16 code pairs fed to
// v_fma_mix from batch 2 on and matches them at batch 1.
struct Q4Bytes {
  uint32_t lo, hi;  // byte b: 16 (n - 8) of position 4k + b, and of 16 + 4k + b
};
__device__ __forceinline__ Q4Bytes q4_bytes(uint32_t w) {
  return Q4Bytes{((w << 4) ^ 0x80808080u) & 0xF0F0F0F0u, (w ^ 0x80808080u) & 0xF0F0F0F0u};
}
__device__ __forceinline__ float sbyte(uint32_t v, int b) {
  return (float)(int8_t)(v >> (8 * b));  // v_cvt_f32_i32 with a sign-extending byte select
}

// One block of codes against MM staged input blocks (input m at xb + m * mstride bytes):
// c[m] = sum_{j < 32} code_j * x_mj (Q4_0: 16 times that) by FMA chains in a fixed order.  A
// word's signed codes are formed once and shared by the MM inputs.  The order only changes
// which registers stay live (any fixed order meets the bound), so it is picked per format
// and batch class:
//  - batches 1-2: Q4_0 word-major, one chain: for word k positions 4k..4k+3 then
//    16+4k..16+4k+3, so a word's codes die at once; Q8_0 eight chains of four positions (one
//    per 16-byte piece of the staged input) added as ((c0 + c1) + (c2 + c3)) + ((c4 + c5) +
//    (c6 + c7)): each piece's reads are used at once (with one or two chains the scheduler
//    hoisted every read and batch 2 with two steps in flight spilled registers);
//  - batches 4-8: one chain in position order 0..31 (Q4_0: the low nibbles of the four words,
//    then the high ones), so each input's two staged chunks are not live together.
template <int FMT, int MM, int WIDE = (MM > 2)>  // WIDE: the order of batches 4-8
__device__ __forceinline__ void chain_block(const Codes<FMT>& q, const char* xb, int mstride,
                                            float (&c)[MM]) {
  auto xm = [&](int m, int k) { return *reinterpret_cast<const f32x4*>(xb + m * mstride + k * 16); };
  if constexpr (FMT == FQ4) {
    const uint32_t w[4] = {q.a.x, q.a.y, q.a.z, q.a.w};
    if constexpr (!WIDE) {
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const Q4Bytes p = q4_bytes(w[k]);
        const float l0 = sbyte(p.lo, 0), l1 = sbyte(p.lo, 1), l2 = sbyte(p.lo, 2), l3 = sbyte(p.lo, 3);
        const float h0 = sbyte(p.hi, 0), h1 = sbyte(p.hi, 1), h2 = sbyte(p.hi, 2), h3 = sbyte(p.hi, 3);
#pragma unroll
        for (int m = 0; m < MM; m++) {
          const f32x4 a = xm(m, k), b = xm(m, k + 4);
          float t = k == 0 ? l0 * a.x : fmaf(l0, a.x, c[m]);
          t = fmaf(l1, a.y, t);
          t = fmaf(l2, a.z, t);
          t = fmaf(l3, a.w, t);
          t = fmaf(h0, b.x, t);
          t = fmaf(h1, b.y, t);
          t = fmaf(h2, b.z, t);
          c[m] = fmaf(h3, b.w, t);
        }
      }
    } else {
      Q4Bytes p[4];
#pragma unroll
      for (int k = 0; k < 4; k++) p[k] = q4_bytes(w[k]);
      float t[MM];
#pragma unroll
      for (int half = 0; half < 2; half++) {
#pragma unroll
        for (int k = 0; k < 4; k++) {  // half 0: low nibbles (positions 4k..), 1: high (16 + 4k..)
          const uint32_t v = half ? p[k].hi : p[k].lo;
          const float v0 = sbyte(v, 0), v1 = sbyte(v, 1), v2 = sbyte(v, 2), v3 = sbyte(v, 3);
#pragma unroll
          for (int m = 0; m < MM; m++) {
            const f32x4 a = xm(m, k + 4 * half);
            float u = half == 0 && k == 0 ? v0 * a.x : fmaf(v0, a.x, t[m]);
            u = fmaf(v1, a.y, u);
            u = fmaf(v2, a.z, u);
            t[m] = fmaf(v3, a.w, u);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < MM; m++) c[m] = t[m];
    }
  } else {
    const uint32_t w[8] = {q.a.x, q.a.y, q.a.z, q.a.w, q.b.x, q.b.y, q.b.z, q.b.w};
    constexpr bool kTree = !WIDE;
    float pr[MM], qd[MM], hf[MM];  // the tree's partial sums: pair, quad, half
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const float v0 = sbyte(w[k], 0), v1 = sbyte(w[k], 1), v2 = sbyte(w[k], 2), v3 = sbyte(w[k], 3);
#pragma unroll
      for (int m = 0; m < MM; m++) {
        const f32x4 a = xm(m, k);
        float t = k == 0 || kTree ? v0 * a.x : fmaf(v0, a.x, c[m]);
        t = fmaf(v1, a.y, t);
        t = fmaf(v2, a.z, t);
        t = fmaf(v3, a.w, t);
        if constexpr (kTree) {
          if (k % 2 == 0) pr[m] = t;
          else pr[m] = pr[m] + t;
          if (k % 4 == 1) qd[m] = pr[m];
          if (k % 4 == 3) qd[m] = qd[m] + pr[m];
          if (k == 3) hf[m] = qd[m];
          if (k == 7) c[m] = hf[m] + qd[m];
        } else {
          c[m] = t;
        }
      }
    }
  }
}

// The block scale as the FMA that applies it takes it: d, or for Q4_0 (whose block sums are
// 16 times too large) d / 16, exact for every binary16 d.
template <int FMT>
__device__ __forceinline__ float block_scale(uint32_t dbits) {
  return FMT == FQ4 ? h2f(dbits) * 0.0625f : h2f(dbits);
}

// Sum over the lane group of 16 (or 8) lanes holding one row (every lane gets the sum): DPP
// exchanges within the 16-lane row.  The partners of each step add the same two values, so
// all lanes hold bitwise the same result.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v),
                                                               __builtin_bit_cast(int, v), CTRL, 0xF,
                                                               0xF, false));
}
__device__ __forceinline__ float group_sum(float v) {
  v = v + dpp<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  v = v + dpp<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  v = v + dpp<0x141>(v);  // row_half_mirror: the other quad of the 8
  if constexpr (kLg2G >= 4) v = v + dpp<0x140>(v);  // row_mirror: the other 8 of the 16
  return v;
}

// Description of one GEMV of a chain (the device image of bqm_gemv).
struct GemvDesc {
  const uint8_t* w;
  const float* x;
  float* y;
  int64_t N, K;
  int32_t fmt, wait, M, reserved;
};
static_assert(sizeof(GemvDesc) == sizeof(bqm_gemv), "bqm_gemv layout");

// The expert-indexed form (qmv_id): `one` is the expert tensor as one matrix of E * N rows
// (N = rows per expert), its x and y the bases of X and Y.
struct IdxArgs {
  const int32_t* ids;      // [T][top_k]
  const uint16_t* scales;  // the scales of all E * N rows
  const uint8_t* up;       // gate+up form: the up tensor's codes (E * N rows) ...
  const uint16_t* up_scales;  // ... and scales; the gate tensor is `one.w`
  int E, TS, top_k;        // experts; slots T * top_k; slots per token
  int64_t xts, xss;        // input strides (floats) per token and per slot
  const float* rw;         // indexed form: router weights [T][top_k] the rows are scaled by, or null
};

struct ChainArgs {
  const GemvDesc* descs;  // n descriptors in device memory, or null: use `one`
  const int64_t* seg;     // per GEMV {blocks before it in its segment, blocks of the segment}
  GemvDesc one;
  int n;
  int kc;                 // K blocks staged at a time (`one` only; else in the workspace)
  int pacc_rows;          // rows per workgroup of the partial-sum buffer (likewise)
  uint32_t* sync;         // workspace words (see grid_barrier); null for a chain of one
  IdxArgs ix;             // the expert-indexed form only
};

// Per-GEMV values of one workgroup, computed once at kernel start (one thread per GEMV)
// into a table in LDS, so moving to the next GEMV costs a few LDS reads.
struct StageRow {
  const uint8_t* codes;     // this workgroup's first row of codes
  const uint16_t* scales;   // ... and of scales
  const float* x;           // input row 0
  float* y;                 // output row 0, this workgroup's first row
  int32_t nrows, nb;        // rows of this workgroup; blocks per row
  int32_t wait, M;
  int32_t xstride, ystride; // floats between input rows (K) and between output rows (N)
  int32_t nchunks;          // chunks of kc blocks
  int32_t next;             // the next GEMV this workgroup enters (see link_units), or n
};
static_assert(sizeof(StageRow) == 64, "stage table row");

// Rows of a GEMV before flattened position v of its segment, whose rows (nb blocks each)
// start at position sbase.
__device__ __forceinline__ int rows_before(int64_t v, int64_t sbase, int nb, int N) {
  if (v <= sbase) return 0;
  const int64_t r = (v - sbase + nb - 1) / nb;
  return r < N ? (int)r : N;
}

// A segment is a run of GEMVs that starts with a waiting one (or the chain's first) and
// holds no other: its GEMVs may run at once.  The weight blocks of a segment, its GEMVs'
// rows one after another, are split evenly between the workgroups at row boundaries: a
// row belongs to the workgroup whose share holds its first block.  A workgroup thus works
// on the few GEMVs its share touches, and meets the others only at the waits.
template <int FMT>
__device__ __forceinline__ StageRow make_stage(const GemvDesc& d, int64_t sbase, int64_t sblocks, int kc) {
  constexpr int CB = FMT == FQ4 ? 16 : 32;
  const int nb = (int)(d.K >> 5);
  const int N = (int)d.N;
  const int grid = (int)gridDim.x, b = (int)blockIdx.x;
  const int r0 = rows_before(b * sblocks / grid, sbase, nb, N);
  const int r1 = rows_before((b + 1) * sblocks / grid, sbase, nb, N);
  const int64_t code_bytes = (int64_t)N * nb * CB;
  StageRow st;
  st.codes = d.w + (int64_t)r0 * nb * CB;
  st.scales = reinterpret_cast<const uint16_t*>(d.w + ((code_bytes + 255) & ~int64_t(255))) +
              (int64_t)r0 * nb;
  st.x = d.x;
  st.y = d.y + r0;
  st.nrows = r1 - r0;
  st.nb = nb;
  st.wait = d.wait ? 1 : 0;
  st.M = d.M;
  st.xstride = (int)d.K;
  st.ystride = N;
  st.nchunks = (nb + kc - 1) / kc;
  st.next = 0;  // set by link_units
  return st;
}

// Uniform values of one chunk of one GEMV for one wave.
struct Stage {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint8_t* codes2;    // gate+up form: the up rows (the gate rows are `codes`)
  const uint16_t* scales2;
  const float* x;
  float* y;
  int nrows, nb, nbc, kb0, ns, S, start, end, M, xstride, ystride, nchunks, lo;
  int th;                   // matrix-core form: rows per tile
  int next;                 // chains: the next GEMV the workgroup enters
  bool wait, first, last;
};

// __builtin_amdgcn_readfirstlane is 32 bits wide: a 64-bit value takes two.
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// The chunk-dependent values of a stage whose GEMV-level values are set.
template <int LGW, int R, int RT = R>  // log2 of the waves; rows per lane; distinct rows per lane
__device__ __forceinline__ void stage_chunk(int c, int kc, int wave, int wait, Stage& s) {
  s.kb0 = c * kc;
  s.nbc = min(kc, s.nb - s.kb0);
  s.first = c == 0;
  s.last = c == s.nchunks - 1;
  s.wait = wait != 0 && c == 0;
  s.ns = (s.nbc + kG - 1) >> kLg2G;
  // tiles of RT * kGpw rows, ns steps each, in row order; the waves take equal contiguous
  // ranges of the tile-major step sequence (a tile may be split between waves)
  const int ntiles = (s.nrows + RT * kGpw - 1) / (RT * kGpw);
  s.S = ntiles * s.ns;
  s.start = (wave * s.S) >> LGW;
  s.end = ((wave + 1) * s.S) >> LGW;
}

template <int LGW, int R>
__device__ __forceinline__ void load_stage(const StageRow* t, int i, int c, int kc, int wave, Stage& s) {
  const StageRow r = t[i];
  s.codes = reinterpret_cast<const uint8_t*>(uniform64(reinterpret_cast<uint64_t>(r.codes)));
  s.scales = reinterpret_cast<const uint16_t*>(uniform64(reinterpret_cast<uint64_t>(r.scales)));
  s.x = reinterpret_cast<const float*>(uniform64(reinterpret_cast<uint64_t>(r.x)));
  s.y = reinterpret_cast<float*>(uniform64(reinterpret_cast<uint64_t>(r.y)));
  s.nrows = __builtin_amdgcn_readfirstlane(r.nrows);
  s.nb = __builtin_amdgcn_readfirstlane(r.nb);
  s.M = __builtin_amdgcn_readfirstlane(r.M);
  s.xstride = __builtin_amdgcn_readfirstlane(r.xstride);
  s.ystride = __builtin_amdgcn_readfirstlane(r.ystride);
  s.nchunks = __builtin_amdgcn_readfirstlane(r.nchunks);
  s.next = __builtin_amdgcn_readfirstlane(r.next);
  s.lo = 0;
  stage_chunk<LGW, R>(c, kc, wave, __builtin_amdgcn_readfirstlane(r.wait), s);
}

// Expert-indexed form: unit i is a group of up to MM slots routed to one expert (`groups`:
// expert, first slot in the sorted list, slots).  The units' rows, N each, one unit after
// another, are split evenly between the workgroups; this one holds flattened rows
// [flo, fhi).  `base`: expert 0's row 0 (codes, scales), x and y bases, nb, nchunks.
template <int LGW, int R, int CB, bool GU>
__device__ __forceinline__ void load_unit(const int* groups, const Stage& base, int i, int c, int kc,
                                          int wave, int N, int64_t flo, int64_t fhi, Stage& s) {
  const int e = __builtin_amdgcn_readfirstlane(groups[3 * i]);
  const int64_t u0 = (int64_t)i * N;
  const int r0 = (int)(flo - u0 < 0 ? 0 : flo - u0 > N ? N : flo - u0);
  const int r1 = (int)(fhi - u0 < 0 ? 0 : fhi - u0 > N ? N : fhi - u0);
  const int64_t row = (int64_t)e * N + r0;
  s = base;
  s.codes = base.codes + row * base.nb * CB;
  s.scales = base.scales + row * base.nb;
  if constexpr (GU) {
    s.codes2 = base.codes2 + row * base.nb * CB;
    s.scales2 = base.scales2 + row * base.nb;
  }
  s.y = base.y + r0;
  s.nrows = r1 - r0;
  s.lo = __builtin_amdgcn_readfirstlane(groups[3 * i + 1]);
  s.M = __builtin_amdgcn_readfirstlane(groups[3 * i + 2]);
  stage_chunk<LGW, R, GU ? 1 : R>(c, kc, wave, 0, s);
}

// Device-wide barrier between the GEMVs of a chain.  Workspace words: [0] the last epoch
// (read at the start of a launch), [2] error, [3] n, [4] format, [5] kc, [6] partial-sum rows,
// [7] M class; then one arrival flag per workgroup, each on its own 128-byte line (no
// contended atomic).  Every workgroup writes the barrier's epoch to its flag and waits until
// all flags have reached it, one thread per flag.  (Workgroup 0 gathering the flags and
// publishing one release word for the others to poll took a memory round trip more: the
// dependent 27B Q4_0 pass 3-4 % slower, Q8_0 M = 4 2.5 %.  Polling all flags when they were
// packed into a few lines was slower than both: every line had 256 pollers.)  Data crossing
// the barrier (the outputs y and the next inputs x) is written and read with agent-coherent
// (sc1) accesses, so no L2-wide write-back or invalidation is needed; the outputs must only
// have landed before a workgroup arrives (see the wait below).  Every wait is bounded: on
// timeout the error word is set and all workgroups leave.
constexpr int kChainHeaderWords = 64;      // 256 bytes
constexpr int kFlagStrideWords = 32;       // 128 bytes
constexpr int kChainMaxWorkgroups = 512;
constexpr uint32_t kSpinLimit = 1u << 22;

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Before a wave arrives, its output stores must have landed.  Every store is followed by
// at least LOADS loads (its step's refill), and vector memory operations complete in issue
// order, so vmcnt <= LOADS suffices, while the weights prefetched for the next GEMV may
// stay in flight.
// `lds_ok` is set once per launch and only ever cleared.  The error word is read only while
// a flag keeps a thread waiting, every 64th poll, so that each poll costs one memory round
// trip and a passing workgroup none at all (reading it after every wait, and after every
// poll, cost the dependent 27B Q4_0 pass several percent); after a timeout the others
// still leave within 64 polls of their next wait, and the word reports the launch invalid.
template <int LOADS>
__device__ __forceinline__ bool grid_barrier(uint32_t* ws, uint32_t epoch, bool* lds_ok) {
  static_assert(LOADS >= 1 && LOADS <= 15, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | LOADS);  // vmcnt(LOADS); expcnt, lgkmcnt: no wait
  __syncthreads();
  uint32_t* flags = ws + kChainHeaderWords;
  if (threadIdx.x == 0) st_agent(flags + blockIdx.x * kFlagStrideWords, epoch);
  // every workgroup waits for every flag (one thread per flag)
  for (uint32_t b = threadIdx.x; b < gridDim.x; b += blockDim.x) {
    uint32_t spins = 0;
    // a workgroup past this barrier may already have arrived at the next: epochs only grow
    while ((int32_t)(ld_agent(flags + b * kFlagStrideWords) - epoch) < 0) {
      if ((++spins & 63u) == 0 && (spins > kSpinLimit || ld_agent(ws + 2) != 0)) {
        st_agent(ws + 2, 1u);
        *lds_ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  if (threadIdx.x == 0 && blockIdx.x == 0) st_agent(ws, epoch);  // the epoch the next launch starts from
  __syncthreads();
  return *lds_ok;
}

// The GEMVs of a chain that a workgroup enters: those with rows in its share, and, when the
// workgroups wait for each other, every waiting one after the first (all take part in each
// wait).  Walking the whole table instead, one stage read per GEMV on both sides of every
// wave, cost a chain of 63 independent 4096 x 4096 Q4_0 GEMVs a quarter of its time: each
// workgroup's share touches one or two of them.  The entered GEMVs are linked once per
// launch: table[i].next is the first one after i (n if none), first[0] the first of all, so
// that a step of the walk is a field of the stage row just read (a scan of a bit mask at
// every step cost the dependent 27B passes 1-2 %: its branches sit before each wait).
// LDS: mask, one bit per GEMV (64-bit words, at most 64 of them: n <= 4096); first, 64 ints
// (per word, the first entered GEMV in it or a later word).  Every thread calls it once the
// table is complete; a barrier must follow.
__device__ __forceinline__ void link_units(StageRow* table, int n, bool sync, uint64_t* mask, int* first) {
  const int lane = threadIdx.x & 63;
  const int nw = (n + 63) >> 6;
  for (int i0 = threadIdx.x & ~63; i0 < n; i0 += blockDim.x) {
    const int i = i0 + lane;
    const bool v = i < n && (table[i].nrows > 0 || (sync && i > 0 && table[i].wait != 0));
    const uint64_t m = __ballot(v);
    if (lane == 0) mask[i0 >> 6] = m;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const uint64_t m = lane < nw ? mask[lane] : 0;
    int f = m ? lane * 64 + __builtin_ctzll(m) : n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {  // the minimum over this word and the later ones
      const int g = __shfl_down(f, o, 64);
      if (lane + o < 64) f = min(f, g);
    }
    first[lane] = f;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int b = i & 63, w1 = (i >> 6) + 1;
    const uint64_t m = b == 63 ? 0 : mask[i >> 6] >> (b + 1);  // entered GEMVs after i in its word
    table[i].next = m ? i + 1 + __builtin_ctzll(m) : w1 < 64 ? first[w1] : n;
  }
}

// Largest batch class (slots per group) of the indexed form.
constexpr int kIdMaxClass = 4;
// LDS rows (64 bytes) the indexed form's tables take: per-expert counts (E + 1), the slots
// grouped by expert (TS) and the groups (3 ints each, at most TS).
__host__ __device__ inline int idx_table_rows(int E, int TS) { return (4 * (E + 1) + 16 * TS + 63) / 64; }

// Dynamic LDS of a chain launch, in bytes from the start: the stage table, the split-tile
// parts, their counters, the per-row partial sums of chunked GEMVs, the staged inputs.
struct ChainLds {
  int part, done, pacc, x, mask, first, total;
};
// Bytes of link_units' mask for a table of n rows (whole 16 bytes); its 64 ints follow.
__host__ __device__ inline int unit_mask_bytes(int n) { return ((n + 127) / 128) * 16; }
__host__ __device__ inline ChainLds chain_lds(int n, int mm, int r, int pacc_rows, int kc) {
  ChainLds L;
  L.part = (n * 64 + 15) & ~15;
  L.done = L.part + kP1Waves * 2 * kGpw * r * mm * 4;
  L.pacc = L.done + kP1Waves * 4;
  L.x = L.pacc + ((pacc_rows * mm * 4 + 15) & ~15);
  L.mask = L.x + mm * kc * kBlkLds;
  L.first = L.mask + unit_mask_bytes(n);
  L.total = L.first + 256;
  return L;
}

// MODE 0: chains of GEMVs; 1: the expert-indexed form; 2: the expert-indexed gate+up form
// (a lane's two rows are gate row n and up row n of one expert; outputs silu(g) * u).
template <int FMT, int P, int MM, int LGW, int R, int MODE>
__global__ __launch_bounds__(64 << LGW) void k_qmv_chain(ChainArgs a) {
  constexpr bool IDX = MODE != 0, GU = MODE == 2;
  static_assert(!GU || R == 2, "gate+up pairs take the two rows of a lane");
  constexpr int RT = GU ? 1 : R;  // distinct output rows per lane
  constexpr int NW = 1 << LGW, NT = 64 << LGW;  // waves, threads
  extern __shared__ float4 smem[];
  constexpr int CB = FMT == FQ4 ? 16 : 32;     // code bytes per block
  constexpr uint32_t kOob = 0x80000000u;       // lane offset past every descriptor: reads 0
  constexpr int LOADS = R * (FMT == FQ4 ? 2 : 3);  // loads per step (R rows)
  constexpr bool kPrioFeedback = MM == 1 || (MM == 2 && !IDX);
  __shared__ bool lds_ok;
  __shared__ uint32_t lds_epoch;
  const int tid = threadIdx.x, lane = tid & 63;
  if (a.sync && (a.sync[3] != (uint32_t)a.n || a.sync[4] != (uint32_t)(FMT == FQ4 ? BQM_Q4_0 : BQM_Q8_0) ||
                 a.sync[7] != (uint32_t)MM)) {
    // the workspace was prepared for another chain: flag it, compute nothing
    if (blockIdx.x == 0 && tid == 0)
      __hip_atomic_store(a.sync + 2, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep in SGPRs
  const int kc = a.sync ? (int)a.sync[5] : a.kc;
  const int pacc_rows = a.sync ? (int)a.sync[6] : a.pacc_rows;
  const int TS = IDX ? a.ix.TS : 0;
  const ChainLds ly = chain_lds(IDX ? idx_table_rows(a.ix.E, TS) : a.n, MM, R, pacc_rows, kc);
  char* lds = reinterpret_cast<char*>(smem);
  StageRow* table = reinterpret_cast<StageRow*>(lds);
  float* part = reinterpret_cast<float*>(lds + ly.part);
  int* done = reinterpret_cast<int*>(lds + ly.done);
  float* pacc = reinterpret_cast<float*>(lds + ly.pacc);
  char* xlds = lds + ly.x;
  uint64_t* umask = reinterpret_cast<uint64_t*>(lds + ly.mask);
  int* ufirst = reinterpret_cast<int*>(lds + ly.first);
  const int mstride = kc * kBlkLds;  // bytes between the staged inputs
  // indexed form: per-expert counts, then starts; the valid slots grouped by expert; the
  // groups (expert, first position in srt, slots)
  int* cnt = reinterpret_cast<int*>(lds);
  int* srt = cnt + (IDX ? a.ix.E + 1 : 0);
  int* groups = srt + TS;
  __shared__ int lds_units;
  __shared__ int scan_w[2 * NW];
  Stage ibase;  // indexed form: expert 0, bases
  // the id of this workgroup's first slot in the padding fill below, read now, together with
  // the ids the slot sort reads (after the sort it would be a memory round trip more)
  int fill_e0 = 0;
  if constexpr (IDX) fill_e0 = (int)blockIdx.x < TS ? a.ix.ids[blockIdx.x] : 0;
  if constexpr (IDX) {
    // the slots grouped by expert, groups of at most MM slots (srt is first read after the
    // barrier below)
    group_slots<NT, MM, false>(a.ix.ids, a.ix.E, TS, cnt, srt, groups, scan_w, &lds_units);
    const int N = (int)a.one.N, nb = (int)(a.one.K >> 5);
    ibase.codes = a.one.w;
    ibase.scales = a.ix.scales;
    ibase.codes2 = a.ix.up;
    ibase.scales2 = a.ix.up_scales;
    ibase.x = a.one.x;
    ibase.y = a.one.y;
    ibase.nrows = 0;
    ibase.nb = nb;
    ibase.xstride = nb * kQK;
    ibase.ystride = N;
    ibase.nchunks = (nb + kc - 1) / kc;
    ibase.M = 1;
    ibase.lo = 0;
  } else {
    for (int i = tid; i < a.n; i += NT) {
      const GemvDesc d = a.descs ? a.descs[i] : a.one;
      table[i] = a.seg ? make_stage<FMT>(d, a.seg[2 * i], a.seg[2 * i + 1], kc)
                       : make_stage<FMT>(d, 0, d.N * (d.K >> 5), kc);
      if (a.n == 1) {  // one GEMV (a single call): entered if it has rows here
        table[0].next = 1;
        ufirst[0] = table[0].nrows > 0 ? 0 : 1;
      }
    }
    if (a.n > 1) {
      __syncthreads();
      link_units(table, a.n, a.sync != nullptr, umask, ufirst);
    }
  }
  if (tid < NW) done[tid] = 0;
  if (tid == 0 && a.sync) lds_epoch = ld_agent(a.sync);  // stable until all have arrived once
  if (tid == 0) lds_ok = true;
  __syncthreads();
  uint32_t epoch = a.sync ? lds_epoch : 0u;
  // units of work: the GEMVs, or (indexed form) the groups; none when K = 0
  const int n_units = IDX ? (a.one.K > 0 ? __builtin_amdgcn_readfirstlane(lds_units) : 0) : a.n;
  // this workgroup's units [u_begin, u_end) and (indexed form) flattened rows [flo, fhi)
  int u_begin = 0, u_end = n_units;
  int64_t flo = 0, fhi = 0;
  if constexpr (IDX) {
    // Workgroup b runs on XCD b mod 8; taking the flattened rows in the order of
    // lb = (b mod 8) * (grid / 8) + b / 8 gives each XCD one contiguous range.  The groups
    // of an expert are consecutive units, so the workgroups streaming the same expert rows
    // for its successive groups share an L2 and the rows cross HBM about once.
    // (floor(lb * rows / G) as q lb + floor(r lb / G) with rows = q G + r: small 32-bit
    // divisions instead of 64-bit ones, which take a long software sequence)
    const int64_t rows = (int64_t)n_units * a.one.N;
    const int G = (int)gridDim.x, b = (int)blockIdx.x;
    const int lb = G % 8 == 0 ? (b % 8) * (G / 8) + b / 8 : b;
    const int64_t q = rows / G;  // one 64-bit division, uniform
    const int rr = (int)(rows - q * G);
    flo = q * lb + (rr * lb) / G;
    fhi = q * (lb + 1) + (rr * (lb + 1)) / G;
    if (fhi > flo) {
      const int N = (int)a.one.N;
      if (fhi <= 0x7FFFFFFF) {
        u_begin = (int)flo / N;
        u_end = ((int)fhi - 1) / N + 1;
      } else {
        u_begin = (int)(flo / N);
        u_end = (int)((fhi - 1) / N) + 1;
      }
    } else {
      u_end = 0;
    }
  }
  if constexpr (IDX) {
    // rows of slots that no group computes, each by one workgroup: a negative id gives
    // zeros, an id >= E NaN; with K = 0 every valid slot's sums are empty (zeros)
    const int N = (int)a.one.N;
    for (int ts = blockIdx.x; ts < TS; ts += gridDim.x) {
      const int e = ts == (int)blockIdx.x ? fill_e0 : a.ix.ids[ts];
      const bool valid = e >= 0 && e < a.ix.E;
      if (valid && n_units > 0) continue;
      const float v = valid || e < 0 ? 0.0f : __builtin_nanf("");
      for (int n = tid; n < N; n += NT) a.one.y[(int64_t)ts * N + n] = v;
    }
    if (n_units == 0) return;
  }
  auto load = [&](int i, int c, Stage& st) {
    if constexpr (IDX) load_unit<LGW, R, CB, GU>(groups, ibase, i, c, kc, wave, (int)a.one.N, flo, fhi, st);
    else load_stage<LGW, R>(table, i, c, kc, wave, st);
  };
  // input and output row of batch entry m of the current unit: m itself, or (indexed form)
  // the m-th slot of the group
  auto slot_of = [&](const Stage& st, int m) {
    return IDX ? __builtin_amdgcn_readfirstlane(srt[st.lo + m]) : m;
  };

  // Both sides walk the same sequence of steps: for each (GEMV, chunk) in which this wave
  // has steps, its steps padded to a multiple of P (padding steps load nothing useful and
  // compute nothing), so a chunk always ends at the end of an unrolled group.  Every step
  // issues its loads, real or past the descriptor, so the number of loads in flight is the
  // same on every path through the loop.

  // ---------------- issue side: P steps ahead ----------------
  int gi = u_begin - 1, ci = 0;  // unit and chunk being issued
  const int g_first = IDX ? 0 : __builtin_amdgcn_readfirstlane(ufirst[0]);  // the first GEMV entered
  Stage si;
  si.nchunks = 0;
  int it = 0, ij = 0;        // this wave's tile, step in tile
  int ireal = 0, ipad = 0;   // real steps left; steps left with padding
  __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(nullptr, (short)0, 0, 0x00020000);
  __amdgpu_buffer_rsrc_t rs = rc;
  __amdgpu_buffer_rsrc_t rc2 = rc, rs2 = rc;  // gate+up form: the up rows
  // lane offsets of its rows (ilg, and ilg + gpw when R = 2, in the tile) in the current
  // tile, and at the tile's last step (past K in a ragged row: zeros).  Named scalars, not
  // arrays: an array shared by the lambdas may be kept in scratch memory.
  uint32_t vc0 = kOob, vs0 = kOob, vcl0 = kOob, vsl0 = kOob;
  uint32_t vc1 = kOob, vs1 = kOob, vcl1 = kOob, vsl1 = kOob;
  int ig = 0, ilg = 0;
  auto tile_offsets = [&]() {
    const bool past_k = ((si.ns - 1) << kLg2G) + ig >= si.nbc;
    const int row = it * RT * kGpw + ilg;
    const bool ok0 = row < si.nrows;  // rows past the range read zeros
    vc0 = ok0 ? ((uint32_t)ilg * si.nb + ig) * CB : kOob;
    vs0 = ok0 ? ((uint32_t)ilg * si.nb + ig) * 2 : kOob;
    vcl0 = past_k ? kOob : vc0;
    vsl0 = past_k ? kOob : vs0;
    if constexpr (GU) {  // the up row: same row, other tensor
      vc1 = vc0;
      vs1 = vs0;
      vcl1 = vcl0;
      vsl1 = vsl0;
    } else if constexpr (R == 2) {
      const bool ok1 = row + kGpw < si.nrows;
      vc1 = ok1 ? ((uint32_t)(kGpw + ilg) * si.nb + ig) * CB : kOob;
      vs1 = ok1 ? ((uint32_t)(kGpw + ilg) * si.nb + ig) * 2 : kOob;
      vcl1 = past_k ? kOob : vc1;
      vsl1 = past_k ? kOob : vs1;
    }
  };
  auto next_issue = [&]() {  // the next (GEMV, chunk) with steps for this wave, if any
    ireal = 0;
    ipad = 0;
    while (ipad == 0) {
      if (ci + 1 < si.nchunks) {
        ++ci;
      } else {
        const int g = IDX ? gi + 1 : gi < 0 ? g_first : si.next;
        if (g >= u_end) break;
        gi = g;
        ci = 0;
      }
      load(gi, ci, si);
      if (si.nrows == 0) ci = si.nchunks - 1;  // none of its rows here: skip its chunks
      ireal = si.end - si.start;
      ipad = (ireal + P - 1) / P * P;
    }
    if (ipad > 0) {
      rc = __builtin_amdgcn_make_buffer_rsrc((void*)si.codes, (short)0,
                                             (int)((uint32_t)si.nrows * si.nb * CB), 0x00020000);
      // +2: a scale is read as 4 bytes (the packed layout leaves slack after the scales)
      rs = __builtin_amdgcn_make_buffer_rsrc((void*)si.scales, (short)0,
                                             (int)((uint32_t)si.nrows * si.nb * 2 + 2), 0x00020000);
      if constexpr (GU) {
        rc2 = __builtin_amdgcn_make_buffer_rsrc((void*)si.codes2, (short)0,
                                                (int)((uint32_t)si.nrows * si.nb * CB), 0x00020000);
        rs2 = __builtin_amdgcn_make_buffer_rsrc((void*)si.scales2, (short)0,
                                                (int)((uint32_t)si.nrows * si.nb * 2 + 2), 0x00020000);
      }
      ig = lane & (kG - 1);
      ilg = lane >> kLg2G;
      it = si.start / si.ns;
      ij = si.start - it * si.ns;
      tile_offsets();
    }
  };
  next_issue();

  auto issue = [&](Codes<FMT> (&q)[R], uint32_t (&d)[R]) {
    // arithmetic, not branches or selects (which the compiler may turn into branches with
    // the loads duplicated): one load sequence for real and padding steps.  Once the range
    // is done the lane offsets are past the descriptor: zeros, no memory traffic.
    const uint32_t live = ireal > 0 ? 1u : 0u;
    const uint32_t so = ((uint32_t)(it * RT * kGpw) * si.nb + (uint32_t)si.kb0 + (uint32_t)(ij << kLg2G)) * live;
    const uint32_t lm = 0u - (uint32_t)(ij == si.ns - 1);  // all ones at a tile's last step
#pragma unroll
    for (int r = 0; r < R; r++) {
      const uint32_t c = r == 0 ? (vcl0 & lm) | (vc0 & ~lm) : (vcl1 & lm) | (vc1 & ~lm);
      const uint32_t e = r == 0 ? (vsl0 & lm) | (vs0 & ~lm) : (vsl1 & lm) | (vs1 & ~lm);
      const __amdgpu_buffer_rsrc_t rcr = GU && r == 1 ? rc2 : rc;
      const __amdgpu_buffer_rsrc_t rsr = GU && r == 1 ? rs2 : rs;
      if constexpr (FMT == FQ4) {
        q[r].a = __builtin_amdgcn_raw_buffer_load_b128(rcr, c, so * CB, 0);
      } else {
        q[r].a = __builtin_amdgcn_raw_buffer_load_b128(rcr, c, so * CB, 0);
        q[r].b = __builtin_amdgcn_raw_buffer_load_b128(rcr, c + 16, so * CB, 0);
      }
      // the scale and the next 2 bytes (ignored): a whole-register load, which the compiler
      // neither widens nor merges, so the ring is waited on per slot
      d[r] = __builtin_amdgcn_raw_buffer_load_b32(rsr, e, so * 2, 0);
    }
    if (ireal > 0) {
      if (--ireal == 0) {  // padding steps follow: read nothing
        vc0 = vs0 = vcl0 = vsl0 = vc1 = vs1 = vcl1 = vsl1 = kOob;
      } else if (++ij == si.ns) {
        ij = 0;
        ++it;
        tile_offsets();
      }
    }
    if (ipad > 0 && --ipad == 0) next_issue();
  };

  Codes<FMT> ring_q[P][R];
  uint32_t ring_d[P][R];  // low 16 bits: the scale
#pragma unroll
  for (int p = 0; p < P; p++) issue(ring_q[p], ring_d[p]);

  // ---------------- consume side ----------------
  // A tile within one wave's range is reduced and stored by that wave.  A tile split
  // between waves w0..wl: each part leaves its row sums in `part` (slot 1: the part that
  // holds the tile's first step, slot 0: later parts) and counts itself in done[w0]; the
  // part that completes the count adds the parts in wave order, stores the rows and resets
  // the count.  A chunked GEMV adds each chunk's row sums into `pacc` and stores at its last
  // chunk.  Every store is followed by its step's loads.
  int gc = u_begin - 1, cc = 0;                      // unit and chunk being consumed
  int ct = 0, cj = 0, creal = 0, cpad = 0;           // tile, step in tile, steps left
  int creal0 = 1;                                    // steps of this wave in the chunk
  Stage sc;
  sc.nchunks = 0;
  const char* lds_lane = xlds;   // this lane's first block of a tile
  const char* lds_last = xlds;   // ... its block at the tile's last step (past K: the last block)
  int cg = 0, clg = 0;
  float acc[R][MM];
  float wslot[MM];  // weighted-sum form: the router weights of the current group's slots
#pragma unroll
  for (int m = 0; m < MM; m++) wslot[m] = 1.0f;
#pragma unroll
  for (int r = 0; r < R; r++)
#pragma unroll
    for (int m = 0; m < MM; m++) acc[r][m] = 0.f;
  bool alive = true;
  // Enter the next (unit, chunk) with rows in this workgroup: wait for earlier outputs
  // where a unit asks (also for a unit with none of its rows here: every workgroup takes
  // part in every wait), then, once all waves finished reading the staged x, stage the new
  // x.  Every wave enters the same (unit, chunk)s, in order.  False when
  // no unit is left or a wait failed.
  auto enter = [&]() -> bool {
    bool waited = false;  // a device-wide wait, which ends with a workgroup barrier, was passed
    for (;;) {
      if (cc + 1 < sc.nchunks) {
        ++cc;
      } else {
        const int g = IDX ? gc + 1 : gc < 0 ? g_first : sc.next;
        if (g >= u_end) return false;
        gc = g;
        cc = 0;
      }
      load(gc, cc, sc);
      if (sc.wait && gc > 0 && a.sync) {
        alive = grid_barrier<LOADS>(a.sync, ++epoch, &lds_ok);
        if (!alive) return false;
        waited = true;
      }
      if (sc.nrows > 0) break;
      cc = sc.nchunks - 1;  // none of its rows here: skip its chunks
    }
    creal = sc.end - sc.start;
    creal0 = creal > 0 ? creal : 1;
    if constexpr (kPrioFeedback) __builtin_amdgcn_s_setprio(3);
    cpad = (creal + P - 1) / P * P;
    ct = sc.start / sc.ns;
    cj = sc.start - ct * sc.ns;
    cg = lane & (kG - 1);
    clg = lane >> kLg2G;
    // every wave is done with the staged inputs before they are replaced (after a device-wide
    // wait they are already)
    if (!waited) __syncthreads();
    // x comes through agent-coherent loads (other workgroups may have written it), 16
    // bytes per lane: a pass of a wave stages 8 whole blocks of each input.  Inputs m >= M
    // are staged as zeros (their results are not stored).
    if constexpr (IDX && !GU) {  // read here, off the store path (the staging waits anyway)
      if (a.ix.rw) {
#pragma unroll
        for (int m = 0; m < MM; m++) wslot[m] = m < sc.M ? a.ix.rw[slot_of(sc, m)] : 0.0f;
      }
    }
    const int nch = sc.nbc * 8;  // 16-byte pieces per input
    __amdgpu_buffer_rsrc_t rx[MM];
#pragma unroll
    for (int m = 0; m < MM; m++) {
      int64_t xo = 0;  // input row of entry m (entries m >= M read nothing)
      if (m < sc.M) {
        if constexpr (IDX) {
          const int ts = slot_of(sc, m), t = ts / a.ix.top_k;
          xo = t * a.ix.xts + (ts - t * a.ix.top_k) * a.ix.xss;
        } else {
          xo = (int64_t)m * sc.xstride;
        }
      }
      const float* xrow = sc.x + xo + (int64_t)sc.kb0 * kQK;
      rx[m] = __builtin_amdgcn_make_buffer_rsrc((void*)xrow, (short)0, m < sc.M ? sc.nbc * 128 : 0,
                                                0x00020000);
    }
    // Loads per lane in flight taken over the inputs and the passes together: MB inputs at a
    // time, QC passes each (eight loads; four for the widest batch, whose registers are
    // spent).  Staging the inputs one after another cost a memory round trip per input after
    // every wait.
    constexpr int MB = MM >= 8 ? 4 : MM, QC = MM >= 8 ? 1 : 8 / MM;
#pragma unroll
    for (int mb = 0; mb < MM; mb += MB) {
      for (int c00 = wave * 64; c00 < nch; c00 += QC * NT) {
        f32x4 v[MB][QC];
#pragma unroll
        for (int q = 0; q < QC; q++)
#pragma unroll
          for (int m = 0; m < MB; m++) {  // a pass wholly past the end loads nothing (uniform)
            v[m][q] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (c00 + q * NT < nch)  // lanes past the end read zeros
              v[m][q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rx[mb + m], (c00 + q * NT + lane) * 16, 0, 16));
          }
#pragma unroll
        for (int q = 0; q < QC; q++) {
          const int c = c00 + q * NT + lane;
          if (c < nch) {
            const int blk = c >> 3, i = c & 7;
#pragma unroll
            for (int m = 0; m < MB; m++)
              *reinterpret_cast<f32x4*>(xlds + (mb + m) * mstride + blk * kBlkLds + i * 16) = v[m][q];
          }
        }
      }
    }
    __syncthreads();
    lds_lane = xlds + cg * kBlkLds;
    lds_last = ((sc.ns - 1) << kLg2G) + cg < sc.nbc ? lds_lane + (sc.ns - 1) * (kG * kBlkLds)
                                                      : xlds + (sc.nbc - 1) * kBlkLds;  // its d is 0
    return true;
  };

  bool more = enter();
  while (more) {
    if (cpad > 0) {
#pragma unroll
      for (int p = 0; p < P; p++) {
        if (creal > 0) {  // uniform: a real step of this wave
          const char* xb = cj == sc.ns - 1 ? lds_last : lds_lane + cj * (kG * kBlkLds);
#pragma unroll
          for (int r = 0; r < R; r++) {
            float c[MM];
            chain_block<FMT, MM>(ring_q[p][r], xb, mstride, c);
            const float dsc = block_scale<FMT>(ring_d[p][r]);
#pragma unroll
            for (int m = 0; m < MM; m++) acc[r][m] = fmaf(dsc, c[m], acc[r][m]);
          }
          --creal;
          ++cj;
          // A SIMD issues from its oldest wave first, so with equal step counts the younger
          // waves of a workgroup finish microseconds later and the whole workgroup waits
          // for them.  Each wave's issue priority follows the share of its steps still
          // left: a wave that falls behind keeps a higher priority than those ahead of it.
          // (Measured: 8% faster on the dependent batch-1 chain, 3% at batch 2, 2-4% on the
          // indexed form's batch-1 groups (MoE decode at T = 1); 4-6 times slower for the
          // chain at batches 4 and 8 and 3.5 times for the indexed form's class 4, which keep
          // the default.)
          if constexpr (kPrioFeedback) {  // quarter of the steps left: 3 .. 0 (no division)
            const int c4 = 4 * creal;
            if (c4 >= 3 * creal0) __builtin_amdgcn_s_setprio(3);
            else if (c4 >= 2 * creal0) __builtin_amdgcn_s_setprio(2);
            else if (c4 >= creal0) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
          }
          if (cj == sc.ns || creal == 0) {  // this wave's part of the tile is done
            float v[R][MM];
#pragma unroll
            for (int r = 0; r < R; r++)
#pragma unroll
              for (int m = 0; m < MM; m++) v[r][m] = group_sum(acc[r][m]);
            // waves holding the tile: the wave of step s is (NW s + NW - 1) / S; when S < NW
            // each non-empty wave holds one step
            const int t0 = ct * sc.ns, t1 = t0 + sc.ns;
            const int w0 = (NW * t0 + NW - 1) / sc.S, wl = (NW * (t1 - 1) + NW - 1) / sc.S;
            const int parts = sc.S >= NW ? wl - w0 + 1 : sc.ns;
            bool put = parts == 1;
            if (!put) {  // rows of the tile: r * kGpw + clg
              float* mine = part + ((wave * 2 + (t0 >= sc.start ? 1 : 0)) * kGpw * R + clg) * MM;
              if (cg == 0) {
#pragma unroll
                for (int r = 0; r < R; r++)
#pragma unroll
                  for (int m = 0; m < MM; m++) mine[r * kGpw * MM + m] = v[r][m];
              }
              asm volatile("" ::: "memory");
              int before = 0;
              if (lane == 0)
                before = __hip_atomic_fetch_add(&done[w0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
              before = __builtin_amdgcn_readfirstlane(before);
              asm volatile("" ::: "memory");
              if (before == parts - 1) {  // the last part in: every part is in `part`
#pragma unroll
                for (int r = 0; r < R; r++) {
                  const float* p0 = part + ((w0 * 2 + 1) * kGpw * R + r * kGpw + clg) * MM;
#pragma unroll
                  for (int m = 0; m < MM; m++) v[r][m] = p0[m];
                }
                for (int u = w0 + 1; u <= wl; u++)
                  if (sc.S >= NW || ((u * sc.S) >> LGW) < (((u + 1) * sc.S) >> LGW)) {
#pragma unroll
                    for (int r = 0; r < R; r++) {
                      const float* pu = part + ((u * 2) * kGpw * R + r * kGpw + clg) * MM;
#pragma unroll
                      for (int m = 0; m < MM; m++) v[r][m] = v[r][m] + pu[m];
                    }
                  }
                if (lane == 0) done[w0] = 0;
                put = true;
              }
            }
#pragma unroll
            for (int r = 0; r < R; r++) {
              // the output row (gate+up form: both of the lane's rows are row n)
              const int row = GU ? ct * kGpw + clg : ct * R * kGpw + r * kGpw + clg;
              if (put && cg == 0 && row < sc.nrows) {
                bool store = true;
                if (sc.nchunks > 1) {  // chunk sums, added in chunk order
                  float* pa = pacc + (GU ? 2 * row + r : row) * MM;
#pragma unroll
                  for (int m = 0; m < MM; m++) {
                    if (!sc.first) v[r][m] = pa[m] + v[r][m];
                    pa[m] = v[r][m];
                  }
                  store = sc.last;
                }
                if (store && (!GU || r == 1)) {
#pragma unroll
                  for (int m = 0; m < MM; m++)
                    if (m < sc.M) {  // agent-coherent: a later GEMV may read it
                      float out = v[r][m];
                      const int ts = slot_of(sc, m);
                      if constexpr (GU) {  // silu(g) * u, g the gate row's sum
                        const float g = v[0][m];
                        out = g / (1.0f + expf(-g)) * v[1][m];
                      } else if constexpr (IDX) {
                        if (a.ix.rw) out = out * wslot[m];  // router weight of the slot
                      }
                      __hip_atomic_store((__attribute__((address_space(1))) float*)sc.y +
                                             (int64_t)ts * sc.ystride + row,
                                         out, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
              }
            }
            asm volatile("" ::: "memory");  // keep the store ahead of this step's loads
#pragma unroll
            for (int r = 0; r < R; r++)
#pragma unroll
              for (int m = 0; m < MM; m++) acc[r][m] = 0.f;
            if (cj == sc.ns) {
              cj = 0;
              ++ct;
            }
          }
        }
        issue(ring_q[p], ring_d[p]);  // refill the slot just consumed
      }
      cpad -= P;
    }
    if (cpad == 0) more = enter();
  }
}

// ---- the chain on the matrix cores (batches of 3 to 8 inputs) ----------------------------
// From three inputs on, the fp32 FMAs of a block (one per code and input) outgrow what the
// vector ALU issues beside the stream (27B Q8_0 pass at M = 8: 12 lane operations per weight,
// 27 % of HBM).  This form takes the products to the matrix cores, as the expert-indexed
// form does: every 32-weight block of 16 rows goes through v_mfma_f32_16x16x32_bf16 twice (the
// two bf16 parts of the inputs) for all M inputs at once, and the vector work per weight (the
// code conversion and the block-scale FMA) does not grow with M.  Operands and exactness as
// in mma_ops.h: codes exact, inputs in two bf16 parts of x * 2^30, blocks in ascending order
// per row (each block sum scaled by d and added in fp32).
//
// The chain's structure is kept: per GEMV a workgroup's rows (the same block-balanced split),
// the device-wide barrier at waits, the inputs staged in LDS per (GEMV, chunk of K), a
// register ring that runs ahead across GEMVs and chunks.  What changes is the step: a
// 16-row tile and 128 bytes of each of its rows (Q4_0 eight blocks, Q8_0 four), two 16-byte
// code loads per lane (lane group q: bytes 16q.. of each 64-byte piece) and one load of the
// row's scales for the step's blocks, exchanged between the lane groups into the MFMA's
// operand layout (mma::exchange).  A wave's steps are a contiguous range of the tile-major
// step sequence, as in the vector form; a tile split between waves is finished in LDS in
// wave order.  The inputs are staged compactly, per block and part the M inputs' 16-byte
// pieces of each k-group ([k-group][input]) and one zero piece, which the MFMA rows past M
// read.  K must be a multiple of 128 (Q8_0) or 256 (Q4_0), so that steps and chunks hold whole
// 128-byte pieces of a row.
constexpr int kMcRows = 16;                              // rows of a tile (the MFMA's columns)
constexpr int kMcMaxM = 8;                               // inputs at most
constexpr int kMcPartBytes = kP1Waves * 2 * kMcRows * kMcMaxM * 4;  // split-tile parts
constexpr int kMcClassBit = 0x100;                       // header word 7: a plan for this form
__host__ __device__ inline int mc_blk_bytes(int M) { return 32 * (4 * M + 1); }
__host__ __device__ inline ChainLds chain_lds_mc(int n, int M, int pacc_rows, int kc) {
  ChainLds L;
  L.part = (n * 64 + 15) & ~15;
  L.done = L.part + kMcPartBytes;
  L.pacc = L.done + kP1Waves * 4;
  L.x = L.pacc + ((pacc_rows * kMcMaxM * 4 + 15) & ~15);
  L.mask = L.x + kc * mc_blk_bytes(M);
  L.first = L.mask + unit_mask_bytes(n);
  L.total = L.first + 256;
  return L;
}

// The chunk-dependent values of a stage: steps of 128 bytes per row (UB blocks), the
// waves' equal contiguous ranges of the tile-major step sequence.  The rows are cut into the
// fewest tiles of at most 16, all but the last of th rows each, th as even as it gets (20
// rows: two of 10, not 16 and 4), so that the waves' steps carry equal shares of the rows.
template <int UB>
__device__ __forceinline__ void stage_chunk_mc(int c, int kc, int wave, int wait, Stage& s) {
  s.kb0 = c * kc;
  s.nbc = min(kc, s.nb - s.kb0);
  s.first = c == 0;
  s.last = c == s.nchunks - 1;
  s.wait = wait != 0 && c == 0;
  s.ns = s.nbc / UB;
  const int ntiles = (s.nrows + kMcRows - 1) / kMcRows;
  s.th = ntiles > 0 ? (s.nrows + ntiles - 1) / ntiles : kMcRows;
  s.S = ntiles * s.ns;
  s.start = (wave * s.S) >> 4;
  s.end = ((wave + 1) * s.S) >> 4;
}

template <int FMT, int P>
__global__ __launch_bounds__(1024) void k_qmv_chain_mc(ChainArgs a) {
  constexpr int NW = 16, NT = 1024;
  extern __shared__ float4 smem[];
  constexpr int CB = FMT == FQ4 ? 16 : 32;     // code bytes per block
  constexpr int UB = FMT == FQ4 ? 8 : 4;       // blocks per step: 128 bytes of a row
  constexpr uint32_t kOob = 0x80000000u;       // lane offset past every descriptor: reads 0
  constexpr int LOADS = 3;                     // loads per step: two of codes, one of scales
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  using ScaleRegs = typename std::conditional<FMT == FQ4, u32x4, u32x2>::type;
  __shared__ bool lds_ok;
  __shared__ uint32_t lds_epoch;
  const int tid = threadIdx.x, lane = tid & 63;
  if (a.sync && (a.sync[3] != (uint32_t)a.n || a.sync[4] != (uint32_t)(FMT == FQ4 ? BQM_Q4_0 : BQM_Q8_0) ||
                 (a.sync[7] & kMcClassBit) == 0)) {
    if (blockIdx.x == 0 && tid == 0)
      __hip_atomic_store(a.sync + 2, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kc = a.sync ? (int)a.sync[5] : a.kc;
  const int pacc_rows = a.sync ? (int)a.sync[6] : a.pacc_rows;
  const int M = a.sync ? (int)a.sync[8] : a.one.M;  // inputs of every GEMV of the chain
  const ChainLds ly = chain_lds_mc(a.n, M, pacc_rows, kc);
  char* lds = reinterpret_cast<char*>(smem);
  StageRow* table = reinterpret_cast<StageRow*>(lds);
  float* part = reinterpret_cast<float*>(lds + ly.part);
  int* done = reinterpret_cast<int*>(lds + ly.done);
  float* pacc = reinterpret_cast<float*>(lds + ly.pacc);
  char* xl = lds + ly.x;
  uint64_t* umask = reinterpret_cast<uint64_t*>(lds + ly.mask);
  int* ufirst = reinterpret_cast<int*>(lds + ly.first);
  const int bxb = mc_blk_bytes(M), xpp = bxb / 2;  // staged bytes per block; per part
  for (int i = tid; i < a.n; i += NT) {
    const GemvDesc d = a.descs ? a.descs[i] : a.one;
    table[i] = a.seg ? make_stage<FMT>(d, a.seg[2 * i], a.seg[2 * i + 1], kc)
                     : make_stage<FMT>(d, 0, d.N * (d.K >> 5), kc);
    if (a.n == 1) {  // one GEMV (a single call): entered if it has rows here
      table[0].next = 1;
      ufirst[0] = table[0].nrows > 0 ? 0 : 1;
    }
  }
  if (a.n > 1) {
    __syncthreads();
    link_units(table, a.n, a.sync != nullptr, umask, ufirst);
  }
  if (tid < NW) done[tid] = 0;
  if (tid == 0 && a.sync) lds_epoch = ld_agent(a.sync);
  if (tid == 0) lds_ok = true;
  __syncthreads();
  uint32_t epoch = a.sync ? lds_epoch : 0u;
  const int n_units = a.n;
  // lane (j, q): row j of a tile (MFMA column), k-group / 16-byte piece q
  const int j = lane & 15, q = lane >> 4;
  // this lane's A-operand piece in a staged block: input j's k-group q, or the zero piece
  const int xo = j < M ? (q * M + j) * 16 : 4 * M * 16;
  auto load = [&](int i, int c, Stage& st) {
    const StageRow r = table[i];
    st.codes = reinterpret_cast<const uint8_t*>(uniform64(reinterpret_cast<uint64_t>(r.codes)));
    st.scales = reinterpret_cast<const uint16_t*>(uniform64(reinterpret_cast<uint64_t>(r.scales)));
    st.x = reinterpret_cast<const float*>(uniform64(reinterpret_cast<uint64_t>(r.x)));
    st.y = reinterpret_cast<float*>(uniform64(reinterpret_cast<uint64_t>(r.y)));
    st.nrows = __builtin_amdgcn_readfirstlane(r.nrows);
    st.nb = __builtin_amdgcn_readfirstlane(r.nb);
    st.M = __builtin_amdgcn_readfirstlane(r.M);
    st.xstride = __builtin_amdgcn_readfirstlane(r.xstride);
    st.ystride = __builtin_amdgcn_readfirstlane(r.ystride);
    st.nchunks = __builtin_amdgcn_readfirstlane(r.nchunks);
    st.next = __builtin_amdgcn_readfirstlane(r.next);
    st.lo = 0;
    stage_chunk_mc<UB>(c, kc, wave, __builtin_amdgcn_readfirstlane(r.wait), st);
  };

  // ---------------- issue side: P steps ahead (as in the vector form) ----------------
  int gi = -1, ci = 0;
  const int g_first = __builtin_amdgcn_readfirstlane(ufirst[0]);  // the first GEMV entered
  Stage si;
  si.nchunks = 0;
  int it = 0, ij = 0, ireal = 0, ipad = 0;
  __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(nullptr, (short)0, 0, 0x00020000);
  __amdgpu_buffer_rsrc_t rs = rc;
  uint32_t vc = kOob, vs = kOob;  // lane offsets of its row in the current tile
  auto tile_offsets = [&]() {
    const int row = it * si.th + j;
    const bool ok = j < si.th && row < si.nrows;  // lanes past the tile's rows read zeros
    vc = ok ? (uint32_t)j * si.nb * CB + q * 16 : kOob;
    vs = ok ? (uint32_t)j * si.nb * 2 : kOob;
  };
  auto next_issue = [&]() {
    ireal = 0;
    ipad = 0;
    while (ipad == 0) {
      if (ci + 1 < si.nchunks) {
        ++ci;
      } else {
        const int g = gi < 0 ? g_first : si.next;
        if (g >= n_units) break;
        gi = g;
        ci = 0;
      }
      load(gi, ci, si);
      if (si.nrows == 0) ci = si.nchunks - 1;
      ireal = si.end - si.start;
      ipad = (ireal + P - 1) / P * P;
    }
    if (ipad > 0) {
      rc = __builtin_amdgcn_make_buffer_rsrc((void*)si.codes, (short)0,
                                             (int)((uint32_t)si.nrows * si.nb * CB), 0x00020000);
      rs = __builtin_amdgcn_make_buffer_rsrc((void*)si.scales, (short)0,
                                             (int)((uint32_t)si.nrows * si.nb * 2), 0x00020000);
      it = si.start / si.ns;
      ij = si.start - it * si.ns;
      tile_offsets();
    }
  };
  next_issue();

  auto issue = [&](u32x4 (&cq)[2], ScaleRegs& sq) {
    const uint32_t live = ireal > 0 ? 1u : 0u;
    // blocks before the step: the tile's rows, the chunk, the step in the tile
    const uint32_t so = ((uint32_t)(it * si.th) * si.nb + (uint32_t)si.kb0 + (uint32_t)(ij * UB)) * live;
    cq[0] = __builtin_amdgcn_raw_buffer_load_b128(rc, vc, so * CB, 0);
    cq[1] = __builtin_amdgcn_raw_buffer_load_b128(rc, vc + 64, so * CB, 0);
    if constexpr (FMT == FQ4) sq = __builtin_amdgcn_raw_buffer_load_b128(rs, vs, so * 2, 0);
    else sq = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, vs, so * 2, 0));
    if (ireal > 0) {
      if (--ireal == 0) {
        vc = vs = kOob;
      } else if (++ij == si.ns) {
        ij = 0;
        ++it;
        tile_offsets();
      }
    }
    if (ipad > 0 && --ipad == 0) next_issue();
  };

  u32x4 ring_c[P][2];
  ScaleRegs ring_s[P];
#pragma unroll
  for (int p = 0; p < P; p++) issue(ring_c[p], ring_s[p]);

  // ---------------- consume side ----------------
  int gc = -1, cc = 0;
  int ct = 0, cj = 0, creal = 0, cpad = 0, creal0 = 1;
  Stage sc;
  sc.nchunks = 0;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  bool alive = true;
  auto enter = [&]() -> bool {
    bool waited = false;
    for (;;) {
      if (cc + 1 < sc.nchunks) {
        ++cc;
      } else {
        const int g = gc < 0 ? g_first : sc.next;
        if (g >= n_units) return false;
        gc = g;
        cc = 0;
      }
      load(gc, cc, sc);
      if (sc.wait && gc > 0 && a.sync) {
        alive = grid_barrier<LOADS>(a.sync, ++epoch, &lds_ok);
        if (!alive) return false;
        waited = true;
      }
      if (sc.nrows > 0) break;
      cc = sc.nchunks - 1;
    }
    creal = sc.end - sc.start;
    creal0 = creal > 0 ? creal : 1;
    __builtin_amdgcn_s_setprio(3);
    cpad = (creal + P - 1) / P * P;
    ct = sc.start / sc.ns;
    cj = sc.start - ct * sc.ns;
    if (!waited) __syncthreads();
    // stage the chunk's inputs: per (block, k-group, input) both bf16 parts of 8 inputs,
    // through agent-coherent loads (other workgroups may have written them); each block's
    // zero pieces
    const int nbc = sc.nbc;
    for (int b = tid; b < nbc; b += NT) {
      *reinterpret_cast<u32x4*>(xl + b * bxb + 4 * M * 16) = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(xl + b * bxb + xpp + 4 * M * 16) = u32x4{0u, 0u, 0u, 0u};
    }
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(sc.x + (int64_t)sc.kb0 * kQK), (short)0,
        (int)(((uint32_t)(M - 1) * (uint32_t)sc.xstride + (uint32_t)nbc * kQK) * 4u), 0x00020000);
    // jobs (block, k-group, group of four inputs): a job's four loads fly together, and with
    // at most 1024 jobs (the plan keeps kc so) the staging takes one memory round trip
    const int MG = (M + 3) >> 2, njx = nbc * 4 * MG;
#pragma unroll 1
    for (int jb = tid; jb < njx; jb += NT) {
      const int kq = jb & 3, t = jb >> 2;
      const int bl = MG == 2 ? t >> 1 : t, m0 = MG == 2 ? 4 * (t & 1) : 0;
      // k-group kq: Q4_0 positions 4kq..4kq+3 and 16+4kq..; Q8_0 8kq..8kq+7
      const uint32_t o0 = ((uint32_t)bl * kQK + (FMT == FQ4 ? 4 * kq : 8 * kq)) * 4u;
      char* dst = xl + bl * bxb + kq * M * 16;
      f32x4 v[4][2];
#pragma unroll
      for (int r = 0; r < 4; r++) {
        v[r][0] = v[r][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (m0 + r < M) {
          const uint32_t o = o0 + (uint32_t)(m0 + r) * (uint32_t)sc.xstride * 4u;
          v[r][0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, o, 0, 16));
          v[r][1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rx, o + (FMT == FQ4 ? 64u : 16u), 0, 16));
        }
      }
#pragma unroll
      for (int r = 0; r < 4; r++) {
        if (m0 + r < M) {
          const float f[8] = {v[r][0].x, v[r][0].y, v[r][0].z, v[r][0].w,
                              v[r][1].x, v[r][1].y, v[r][1].z, v[r][1].w};
          u32x4 hi, lo;
          mma::split8(f, hi, lo);
          *reinterpret_cast<u32x4*>(dst + (m0 + r) * 16) = hi;
          *reinterpret_cast<u32x4*>(dst + xpp + (m0 + r) * 16) = lo;
        }
      }
    }
    __syncthreads();
    return true;
  };

  bool more = enter();
  while (more) {
    if (cpad > 0) {
#pragma unroll
      for (int p = 0; p < P; p++) {
        if (creal > 0) {  // uniform: a real step of this wave
          mma::exchange<FMT == FQ4>(ring_c[p][0]);
          mma::exchange<FMT == FQ4>(ring_c[p][1]);
          const char* xs = xl + (cj * UB) * bxb + xo;
#pragma unroll
          for (int u = 0; u < UB; u++) {
            const mma::bf16x8 ahi = *reinterpret_cast<const mma::bf16x8*>(xs + u * bxb);
            const mma::bf16x8 alo = *reinterpret_cast<const mma::bf16x8*>(xs + u * bxb + xpp);
            mma::bf16x8 b;
            if constexpr (FMT == FQ4) {
              b = mma::q4_operand(ring_c[p][u >> 2][u & 3]);
            } else {
              const u32x4& w = ring_c[p][u >> 1];
              b = mma::q8_operand(w[2 * (u & 1)], w[2 * (u & 1) + 1]);
            }
            f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, b, d, 0, 0, 0);
            const uint32_t sw = ring_s[p][u >> 1];
            // d, times 1/16 for the Q4_0 codes' 16 (n - 8), times 2^-30 for the inputs
            const float s = h2f((u & 1) ? sw >> 16 : sw) * (FMT == FQ4 ? 0x1p-34f : 0x1p-30f);
#pragma unroll
            for (int r = 0; r < 4; r++) acc[r] = fmaf(s, d[r], acc[r]);
          }
          --creal;
          ++cj;
          {  // issue priority from the share of the wave's steps left, as in the vector form
            // (measured on the dependent 27B Q8_0 pass: M = 8 8.65 -> 8.45 ms, M = 4 6.99 ->
            // 6.72 ms; the spread between a workgroup's first and last wave on gate_up at M = 4
            // 20 -> 7.5 us)
            const int c4 = 4 * creal;
            if (c4 >= 3 * creal0) __builtin_amdgcn_s_setprio(3);
            else if (c4 >= 2 * creal0) __builtin_amdgcn_s_setprio(2);
            else if (c4 >= creal0) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
          }
          if (cj == sc.ns || creal == 0) {  // this wave's part of the tile is done
            // lane (j, q) holds row j for inputs 4q .. 4q + 3 (q < 2 for M <= 8)
            float v[4] = {acc[0], acc[1], acc[2], acc[3]};
            const int t0 = ct * sc.ns, t1 = t0 + sc.ns;
            const int w0 = (NW * t0 + NW - 1) / sc.S, wl = (NW * (t1 - 1) + NW - 1) / sc.S;
            const int parts = sc.S >= NW ? wl - w0 + 1 : sc.ns;
            bool put = parts == 1;
            if (!put) {  // [part slot][input][row]
              float* mine = part + (wave * 2 + (t0 >= sc.start ? 1 : 0)) * (kMcRows * kMcMaxM);
              if (q < 2) {
#pragma unroll
                for (int r = 0; r < 4; r++) mine[(4 * q + r) * kMcRows + j] = v[r];
              }
              asm volatile("" ::: "memory");
              int before = 0;
              if (lane == 0)
                before = __hip_atomic_fetch_add(&done[w0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
              before = __builtin_amdgcn_readfirstlane(before);
              asm volatile("" ::: "memory");
              if (before == parts - 1) {
                if (q < 2) {
                  const float* p0 = part + (w0 * 2 + 1) * (kMcRows * kMcMaxM);
#pragma unroll
                  for (int r = 0; r < 4; r++) v[r] = p0[(4 * q + r) * kMcRows + j];
                  for (int u = w0 + 1; u <= wl; u++)
                    if (sc.S >= NW || ((u * sc.S) >> 4) < (((u + 1) * sc.S) >> 4)) {
                      const float* pu = part + (u * 2) * (kMcRows * kMcMaxM);
#pragma unroll
                      for (int r = 0; r < 4; r++) v[r] = v[r] + pu[(4 * q + r) * kMcRows + j];
                    }
                }
                if (lane == 0) done[w0] = 0;
                put = true;
              }
            }
            const int row = ct * sc.th + j;
            if (put && q < 2 && j < sc.th && row < sc.nrows) {
              bool store = true;
              if (sc.nchunks > 1) {  // chunk sums, added in chunk order
                float* pa = pacc + row * kMcMaxM + 4 * q;
#pragma unroll
                for (int r = 0; r < 4; r++) {
                  if (!sc.first) v[r] = pa[r] + v[r];
                  pa[r] = v[r];
                }
                store = sc.last;
              }
              if (store) {
#pragma unroll
                for (int r = 0; r < 4; r++)
                  if (4 * q + r < sc.M)  // agent-coherent: a later GEMV may read it
                    __hip_atomic_store((__attribute__((address_space(1))) float*)sc.y +
                                           (int64_t)(4 * q + r) * sc.ystride + row,
                                       v[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              }
            }
            asm volatile("" ::: "memory");  // keep the store ahead of this step's loads
            acc = f32x4{0.f, 0.f, 0.f, 0.f};
            if (cj == sc.ns) {
              cj = 0;
              ++ct;
            }
          }
        }
        issue(ring_c[p], ring_s[p]);  // refill the slot just consumed
      }
      cpad -= P;
    }
    if (cpad == 0) more = enter();
  }
}

__global__ void k_fill(float* __restrict__ y, int64_t n, float v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    y[i] = v;
}

// ---------------------------------------------------------------- host side ----

// Kernels using more than 64 KB of dynamic LDS must say so once.
template <typename Kern>
void allow_lds(Kern k, size_t bytes) {
  if (bytes > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

#ifndef BQM_P1_P
#define BQM_P1_P 4  // blocks in flight per lane (Q4_0; Q8_0 blocks are twice as long: half)
#endif
constexpr int kP1StaticLds = 1024;                   // reserved for the kernel's own __shared__
constexpr int kP1MaxLds = 160 * 1024 - kP1StaticLds;  // dynamic LDS of a chain launch
static_assert(kP1MaxLds / 64 <= 64 * 64, "link_units: a table that fits holds at most 64 mask words");

using ChainKernel = void (*)(ChainArgs);

// M class: the kernel instantiation that takes M inputs (1, 2, 4 or 8).
int m_class(int M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8; }

// Ring depth: a step of a wider batch computes longer, so fewer steps in flight cover the
// memory latency, and its registers go to the batch's sums.  Batches 1 and 4 take two
// rows per lane (two blocks per step), where a shallower ring is best (measured: also less
// padding at the end of each GEMV's share; batch 4 with two steps would spill); batch 8
// keeps one step, so that its sums fit 16 waves per CU.
template <int FMT, int MM>
constexpr int chain_ring() {
  if (MM == 1) return FMT == FQ4 ? 2 : 1;
  if (MM == 4 || MM >= 8) return 1;
  return (FMT == FQ4 ? BQM_P1_P : BQM_P1_P / 2) / (MM >= 4 && FMT == FQ4 ? 2 : 1);
}
// log2 of the waves per workgroup: 16 waves.  The indexed forms (mode 1, 2) at batch
// classes 1 and 2 take 8 waves: their calls are small (T = 1: 28 MB per MoE projection,
// ≈ 110 KB per workgroup) and a lighter workgroup starts and drains sooner (per call on the
// 128-expert MoE layer, 8 against 16 waves: T = 1 qmv_id 13.5 / 15.4 us, gate+up 18.8 /
// 18.8; T = 2 24.2 / 23.9, gate+up 32.8 / 34.8; class 4 keeps 16: T = 4 38.2 / 37.4,
// gate+up 61.2 / 57.3).
constexpr int chain_lgw(int mm, int mode = 0) { return mode != 0 && mm <= 2 ? 3 : 4; }
// rows per lane: one read of the staged inputs serves the codes of two rows, halving the
// LDS reads per weight byte (batch 1: 8 bytes of x per Q4_0 code byte otherwise; measured
// +6% on the 27B Q4_0 pass, +6% on the 27B Q8_0 pass at M = 4).  Batch 2 keeps one row per
// lane, and so does batch 8: two rows of eight sums need more than the 128 registers a lane
// has when 16 waves share a CU.  Measured on the 27B Q8_0 pass at M = 8, one row per lane,
// one step in flight and 16 waves against two rows, two steps and 8 waves: the dependent
// pass 2.10 -> 2.22 TB/s (the waits' ramps are shorter with more waves), the same GEMVs
// streamed without waits 3.05 -> 2.88 TB/s (two rows share each input read).
constexpr int chain_r(int mm) { return mm == 2 || mm >= 8 ? 1 : 2; }
// rows per lane of a mode: the gate+up form always pairs two rows
constexpr int mode_r(int mm, int mode) { return mode == 2 ? 2 : chain_r(mm); }
template <int FMT, int MODE>
ChainKernel chain_kernel_f(int mm) {
  switch (mm) {
    case 1: return k_qmv_chain<FMT, chain_ring<FMT, 1>(), 1, chain_lgw(1, MODE), mode_r(1, MODE), MODE>;
    // batch 2: one step in flight for the chain (R = 1), the batch-1 ring for the indexed
    // forms (two rows per lane); deeper rings spill registers
    case 2: return k_qmv_chain<FMT, MODE == 0 ? 1 : chain_ring<FMT, 1>(), 2, chain_lgw(2, MODE), mode_r(2, MODE), MODE>;
    case 4: return k_qmv_chain<FMT, chain_ring<FMT, 4>(), 4, chain_lgw(4, MODE), mode_r(4, MODE), MODE>;
    default:  // the indexed forms run at most class 4 (launch_id): no class 8 for them
      if constexpr (MODE != 0) return chain_kernel_f<FMT, MODE>(4);
      else return k_qmv_chain<FMT, chain_ring<FMT, 8>(), 8, chain_lgw(8, MODE), mode_r(8, MODE), MODE>;
  }
}
template <int MODE>
ChainKernel chain_kernel_m(int fmt, int mm) {
  return fmt == BQM_Q4_0 ? chain_kernel_f<FQ4, MODE>(mm) : chain_kernel_f<FQ8, MODE>(mm);
}
ChainKernel chain_kernel(int fmt, int mm, int mode) {
  return mode == 2 ? chain_kernel_m<2>(fmt, mm) : mode == 1 ? chain_kernel_m<1>(fmt, mm) : chain_kernel_m<0>(fmt, mm);
}
// A single GEMV call (qmv_q4_0 / qmv_q8_0, not a chain) at batch 1 or 2 runs on 8-wave
// workgroups: a lighter workgroup starts and drains sooner, which is most of a single call's
// time (4096 x 4096 Q4_0: 10.96 -> 9.96 us per call, median of 256; chains keep 16 waves,
// which stream large matrices and the dependent pass 2 % faster).
constexpr int kLightLgw = 3;
template <int FMT>
ChainKernel chain_kernel_light_f(int mm) {
  return mm == 1 ? k_qmv_chain<FMT, chain_ring<FMT, 1>(), 1, kLightLgw, chain_r(1), 0>
                 : k_qmv_chain<FMT, 1, 2, kLightLgw, chain_r(2), 0>;
}
ChainKernel chain_kernel_light(int fmt, int mm) {
  return fmt == BQM_Q4_0 ? chain_kernel_light_f<FQ4>(mm) : chain_kernel_light_f<FQ8>(mm);
}

}  // namespace

// Compute units of the current device, queried once per device (threads racing on the first
// call store the same value).
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

int launch_fill(float* y, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return BQM_OK;
  const int64_t blocks = (n + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(k_fill, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(kThreads), 0, s,
                     y, n, v);
  return launch_status();
}

// Largest K a chain GEMV may have.
int64_t chain_max_k() { return 32768; }

// Staging plan of a chain: kc (K blocks staged at a time) and the rows of the per-row
// partial-sum buffer (0 when no GEMV is walked in chunks).  Whole GEMVs are staged when
// the table, the split-tile parts and M inputs of the longest K fit; otherwise every GEMV
// longer than kc goes in chunks, and the partial sums are sized for the most rows a
// workgroup holds of one such GEMV.  `nbs` and `rows`: per GEMV, its blocks per row and the
// most rows a workgroup holds of it.  Returns false when even 32-block chunks do not fit.
bool chain_plan(int n, int mm, const int64_t* nbs, const int64_t* rows, int count, int* kc,
                int* pacc_rows) {
  int64_t max_nb = 0;
  for (int i = 0; i < count; i++) max_nb = nbs[i] > max_nb ? nbs[i] : max_nb;
  const int64_t fixed = chain_lds(n, mm, chain_r(mm), 0, 0).total;
  if (fixed + (int64_t)mm * max_nb * kBlkLds <= kP1MaxLds) {
    *kc = (int)max_nb;
    *pacc_rows = 0;
    return true;
  }
  // the largest kc (a multiple of 16) whose chunked GEMVs' partial sums fit beside it
  for (int64_t k = (max_nb - 1) & ~int64_t(15); k >= 32; k -= 16) {
    int64_t prow = 0;
    for (int i = 0; i < count; i++)
      if (nbs[i] > k && rows[i] > prow) prow = rows[i];
    const int64_t pacc = (prow * mm * 4 + 15) & ~int64_t(15);
    if (fixed + pacc + (int64_t)mm * k * kBlkLds <= kP1MaxLds) {
      *kc = (int)k;
      *pacc_rows = (int)prow;
      return true;
    }
  }
  return false;
}
bool chain_plan(int n, int mm, int64_t nb, int64_t rows, int* kc, int* pacc_rows) {
  return chain_plan(n, mm, &nb, &rows, 1, kc, pacc_rows);
}

// Launch a chain (descriptors in device memory, or `one` when descs is null), or with
// `ix` the expert-indexed form of `one`.  `coop`: some GEMV waits for the others, so all
// workgroups must be resident at once (a cooperative launch, which costs 15-20 us more).
int launch_chain(int fmt, int mm, const GemvDesc* descs, const int64_t* seg, const GemvDesc* one,
                 int n, int kc, int pacc_rows, uint32_t* sync, bool coop, hipStream_t s,
                 const IdxArgs* ix = nullptr) {
  ChainArgs a;
  a.descs = descs;
  a.seg = seg;
  if (one) a.one = *one; else a.one = GemvDesc{nullptr, nullptr, nullptr, 0, 0, fmt, 0, 1, 0};
  a.n = n;
  a.kc = kc;
  a.pacc_rows = pacc_rows;
  a.sync = sync;
  if (ix) a.ix = *ix; else a.ix = IdxArgs{nullptr, nullptr, nullptr, nullptr, 0, 0, 0, 0, 0, nullptr};
  const int mode = ix ? (ix->up ? 2 : 1) : 0;
  const bool light = !ix && one != nullptr && mm <= 2;  // a single GEMV call
  ChainKernel k = light ? chain_kernel_light(fmt, mm) : chain_kernel(fmt, mm, mode);
  // per kernel: 1 = its static LDS fits the reserve, -1 = it does not (checked once; threads
  // racing on the first call store the same answer)
  static std::atomic<int> static_ok[4][2][4];
  std::atomic<int>& okc =
      static_ok[light ? 3 : mode][fmt == BQM_Q4_0 ? 0 : 1][mm == 1 ? 0 : mm == 2 ? 1 : mm == 4 ? 2 : 3];
  int ok = okc.load(std::memory_order_relaxed);
  if (ok == 0) {
    hipFuncAttributes fa;
    ok = hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(k)) == hipSuccess &&
                 fa.sharedSizeBytes <= (size_t)kP1StaticLds ? 1 : -1;
    okc.store(ok, std::memory_order_relaxed);
  }
  if (ok < 0) return BQM_E_LAUNCH;
  allow_lds(k, kP1MaxLds);
  const int grid = cu_count();
  const int threads = 64 << (light ? kLightLgw : chain_lgw(mm, mode));
  if (coop) {
    // workgroups wait for each other: they must all be resident at once
    void* args[] = {&a};
    if (hipLaunchCooperativeKernel(reinterpret_cast<const void*>(k), dim3(grid), dim3(threads), args,
                                   kP1MaxLds, s) != hipSuccess)
      return BQM_E_LAUNCH;
    return launch_status();
  }
  hipLaunchKernelGGL(k, dim3(grid), dim3(threads), kP1MaxLds, s, a);
  return launch_status();
}

// The matrix-core chain (k_qmv_chain_mc) takes batches from BQM_MC_MIN_M inputs on, when
// every GEMV's K holds whole 128-byte pieces of a row.
// Measured on the dependent 27B Q8_0 pass (ms, this form / the vector form): M = 8 8.45 /
// 9.87-10.35, M = 4 6.72 / 6.02-6.16 (at M = 4 the vector form issues few enough FMAs, and
// its input staging is a copy where this form splits every input into two bf16 parts).
#ifndef BQM_MC_MIN_M
#define BQM_MC_MIN_M 5
#endif
#ifndef BQM_MC_P
#define BQM_MC_P 2  // steps in flight per wave
#endif
static bool mc_eligible(int fmt, int M, int64_t nb) {
  return M >= BQM_MC_MIN_M && M <= kMcMaxM && nb % (fmt == BQM_Q4_0 ? 8 : 4) == 0;
}
// Staging plan of the matrix-core chain, as chain_plan: kc (a multiple of 8 blocks, so that a
// chunk holds whole steps of either format) and the partial-sum rows.
static bool chain_plan_mc(int n, int M, const int64_t* nbs, const int64_t* rows, int count, int* kc,
                   int* pacc_rows) {
  int64_t max_nb = 0;
  for (int i = 0; i < count; i++) max_nb = nbs[i] > max_nb ? nbs[i] : max_nb;
  const int64_t fixed = chain_lds_mc(n, M, 0, 0).total;
  const int64_t bxb = mc_blk_bytes(M);
  // at most 1024 staging jobs per chunk (4 per block and group of four inputs): one round
  const int64_t kmax = 256 / ((M + 3) / 4);
  if (max_nb <= kmax && fixed + max_nb * bxb <= kP1MaxLds) {
    *kc = (int)max_nb;
    *pacc_rows = 0;
    return true;
  }
  for (int64_t k = std::min(max_nb - 1, kmax) & ~int64_t(7); k >= 8; k -= 8) {
    int64_t prow = 0;
    for (int i = 0; i < count; i++)
      if (nbs[i] > k && rows[i] > prow) prow = rows[i];
    const int64_t pacc = (prow * kMcMaxM * 4 + 15) & ~int64_t(15);
    if (fixed + pacc + k * bxb <= kP1MaxLds) {
      *kc = (int)k;
      *pacc_rows = (int)prow;
      return true;
    }
  }
  return false;
}
template <int FMT>
static ChainKernel chain_kernel_mc_f() { return k_qmv_chain_mc<FMT, BQM_MC_P>; }
static int launch_chain_mc(int fmt, const GemvDesc* descs, const int64_t* seg, const GemvDesc* one, int n,
                    int kc, int pacc_rows, uint32_t* sync, bool coop, hipStream_t s) {
  ChainArgs a;
  a.descs = descs;
  a.seg = seg;
  if (one) a.one = *one; else a.one = GemvDesc{nullptr, nullptr, nullptr, 0, 0, fmt, 0, 1, 0};
  a.n = n;
  a.kc = kc;
  a.pacc_rows = pacc_rows;
  a.sync = sync;
  a.ix = IdxArgs{nullptr, nullptr, nullptr, nullptr, 0, 0, 0, 0, 0, nullptr};
  ChainKernel k = fmt == BQM_Q4_0 ? chain_kernel_mc_f<FQ4>() : chain_kernel_mc_f<FQ8>();
  static std::atomic<int> static_ok[2];
  std::atomic<int>& okc = static_ok[fmt == BQM_Q4_0 ? 0 : 1];
  int ok = okc.load(std::memory_order_relaxed);
  if (ok == 0) {
    hipFuncAttributes fa;
    ok = hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(k)) == hipSuccess &&
                 fa.sharedSizeBytes <= (size_t)kP1StaticLds ? 1 : -1;
    okc.store(ok, std::memory_order_relaxed);
  }
  if (ok < 0) return BQM_E_LAUNCH;
  allow_lds(k, kP1MaxLds);
  const int grid = cu_count();
  if (coop) {
    void* args[] = {&a};
    if (hipLaunchCooperativeKernel(reinterpret_cast<const void*>(k), dim3(grid), dim3(1024), args,
                                   kP1MaxLds, s) != hipSuccess)
      return BQM_E_LAUNCH;
    return launch_status();
  }
  hipLaunchKernelGGL(k, dim3(grid), dim3(1024), kP1MaxLds, s, a);
  return launch_status();
}

// ---- chain API.  Workspace: 64 header words {release epoch, -, error, n, fmt, kc,
// partial-sum rows, M class, ...}, one 128-byte arrival flag per workgroup (at most
// kChainMaxWorkgroups), then the descriptors, then per descriptor its segment's split
// {blocks before it in its segment, blocks of the segment}.
constexpr int64_t kChainSyncBytes = (kChainHeaderWords + kChainMaxWorkgroups * kFlagStrideWords) * 4;
constexpr int64_t kSegBytes = 2 * sizeof(int64_t);

size_t chain_workspace_bytes(int n) {
  return n < 1 ? 0 : (size_t)(kChainSyncBytes + (int64_t)n * (int64_t)(sizeof(GemvDesc) + kSegBytes));
}

// Per prepared workspace (set by chain_prepare): whether its chain has a waiting GEMV, and
// whether it was planned for the matrix-core form.  A workspace this process did not
// prepare is taken to have a wait and the vector form (the kernel checks the plan's header
// and reports a mismatch).
struct ChainPlan {
  bool waits, mc;
};
static std::mutex g_waits_mutex;
static std::unordered_map<const void*, ChainPlan> g_chain_waits;

int chain_prepare(const bqm_gemv* descs, int n, void* ws, hipStream_t s) {
  const int fmt = descs[0].fmt, M = descs[0].M;
  if (fmt != BQM_Q4_0 && fmt != BQM_Q8_0) return BQM_E_UNSUPPORTED;
  const int CB = fmt == BQM_Q4_0 ? 16 : 32;
  // checks of the descriptors alone first (no HIP call before they pass)
  for (int i = 0; i < n; i++) {
    const bqm_gemv& d = descs[i];
    if (d.fmt != fmt) return BQM_E_UNSUPPORTED;
    if (d.M != M || M < 1 || M > kChainMaxM) return BQM_E_SHAPE;
    if (d.N < 1 || d.N > ((int64_t)1 << 30) || d.K < kQK || d.K % kQK != 0 || d.K > chain_max_k())
      return BQM_E_SHAPE;
  }
  for (int i = 0; i < n; i++) {
    const bqm_gemv& d = descs[i];
    if (!d.w_packed || !d.x || !d.y) return BQM_E_NULL;
    if (((uintptr_t)d.w_packed & 15) || ((uintptr_t)d.x & 15) || ((uintptr_t)d.y & 3))
      return BQM_E_ALIGN;
  }
  // segments: each waiting GEMV (and the first) starts one; its GEMVs' blocks are split
  // between the workgroups (see make_stage)
  std::vector<int64_t> seg(2 * (size_t)n);
  for (int i = 0, j; i < n; i = j) {
    int64_t blocks = 0;
    for (j = i; j < n && (j == i || !descs[j].wait); j++) {
      seg[2 * j] = blocks;
      blocks += descs[j].N * (descs[j].K / kQK);
    }
    for (int k = i; k < j; k++) seg[2 * k + 1] = blocks;
  }
  // then the checks that depend on the device: a workgroup's rows of one GEMV (at most
  // ceil(share / nb) for a share of ceil(blocks / workgroups) blocks) stay below 2 GiB
  const int cus = cu_count();
  if (cus > kChainMaxWorkgroups) return BQM_E_UNSUPPORTED;
  std::vector<int64_t> nbs(n), wrows(n);
  for (int i = 0; i < n; i++) {
    const bqm_gemv& d = descs[i];
    const int64_t nb = d.K / kQK, share = (seg[2 * i + 1] + cus - 1) / cus;
    int64_t rows = (share + nb - 1) / nb;  // rows whose first block is in the share
    rows = rows < d.N ? rows : d.N;
    if ((rows + 1) * nb * CB >= ((int64_t)1 << 31)) return BQM_E_SHAPE;
    nbs[i] = nb;
    wrows[i] = rows;
  }
  const int mm = m_class(M);
  bool mc = true;
  for (int i = 0; i < n; i++) mc = mc && mc_eligible(fmt, M, nbs[i]);
  int kc = 0, pacc_rows = 0;
  if (mc && !chain_plan_mc(n, M, nbs.data(), wrows.data(), n, &kc, &pacc_rows)) mc = false;
  if (!mc && !chain_plan(n, mm, nbs.data(), wrows.data(), n, &kc, &pacc_rows)) return BQM_E_SHAPE;
  uint32_t head[9] = {0, 0, 0, (uint32_t)n, (uint32_t)fmt, (uint32_t)kc, (uint32_t)pacc_rows,
                      (uint32_t)(mc ? mm | kMcClassBit : mm), (uint32_t)M};
  char* wsb = static_cast<char*>(ws);
  if (hipMemsetAsync(ws, 0, kChainSyncBytes, s) != hipSuccess ||
      hipMemcpyAsync(ws, head, sizeof(head), hipMemcpyHostToDevice, s) != hipSuccess ||
      hipMemcpyAsync(wsb + kChainSyncBytes, descs, (size_t)n * sizeof(GemvDesc),
                     hipMemcpyHostToDevice, s) != hipSuccess ||
      hipMemcpyAsync(wsb + kChainSyncBytes + (int64_t)n * sizeof(GemvDesc), seg.data(),
                     (size_t)n * kSegBytes, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return BQM_E_LAUNCH;
  bool waits = false;
  for (int i = 1; i < n; i++) waits = waits || descs[i].wait != 0;
  std::lock_guard<std::mutex> lock(g_waits_mutex);
  g_chain_waits[ws] = ChainPlan{waits, mc};
  return BQM_OK;
}

int chain_launch(int fmt, int M, void* ws, int n, hipStream_t s) {
  char* wsb = static_cast<char*>(ws);
  const GemvDesc* d = reinterpret_cast<const GemvDesc*>(wsb + kChainSyncBytes);
  const int64_t* seg = reinterpret_cast<const int64_t*>(wsb + kChainSyncBytes + (int64_t)n * sizeof(GemvDesc));
  ChainPlan plan{true, false};
  {
    std::lock_guard<std::mutex> lock(g_waits_mutex);
    auto it = g_chain_waits.find(ws);
    if (it != g_chain_waits.end()) plan = it->second;
  }
  if (plan.mc) return launch_chain_mc(fmt, d, seg, nullptr, n, 0, 0, static_cast<uint32_t*>(ws), plan.waits, s);
  return launch_chain(fmt, m_class(M), d, seg, nullptr, n, 0, 0, static_cast<uint32_t*>(ws), plan.waits, s);
}

int chain_status(const void* ws, hipStream_t s) {
  uint32_t err = 0;
  if (hipMemcpyAsync(&err, static_cast<const uint32_t*>(ws) + 2, 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return -1;
  return (int)err;
}

// Batch-M GEMV: a chain of one (no device-wide barrier), chunked along K when the M inputs
// do not fit the LDS.
int launch_qmv(int fmt, const void* w, const float* X, float* Y, int M, int64_t N, int64_t K,
               hipStream_t s) {
  if (M == 0 || N == 0) return BQM_OK;
  if (K == 0) return launch_fill(Y, (int64_t)M * N, 0.0f, s);
  const int mm = m_class(M);
  const int cus = cu_count();
  const int64_t rows = (N + cus - 1) / cus;
  const int CB = fmt == BQM_Q4_0 ? 16 : 32;
  if ((rows + 1) * (K / kQK) * CB >= ((int64_t)1 << 31)) return BQM_E_SHAPE;
  int kc = 0, pacc_rows = 0;
  const GemvDesc d{static_cast<const uint8_t*>(w), X, Y, N, K, fmt, 0, M, 0};
  const int64_t nb = K / kQK;
  if (mc_eligible(fmt, M, nb) && chain_plan_mc(1, M, &nb, &rows, 1, &kc, &pacc_rows))
    return launch_chain_mc(fmt, nullptr, nullptr, &d, 1, kc, pacc_rows, nullptr, false, s);
  if (!chain_plan(1, mm, nb, rows, &kc, &pacc_rows)) return BQM_E_SHAPE;
  return launch_chain(fmt, mm, nullptr, nullptr, &d, 1, kc, pacc_rows, nullptr, false, s);
}

// Tokens from which the indexed forms run on the matrix cores.  Measured on the 128-expert
// MoE layer (Q4_0, top-8, skewed routing), per call, matrix cores against the vector form:
// T = 2 38.6 / 23.9 us, T = 4 42.6 / 37.4, T = 8 51.5 / 51.2 (gate+up 77.8 / 81.9),
// T = 16 65.8 / 80.0 (gate+up 103 / 137): the matrix-core form has a fixed cost (16 input
// slots staged, most of them empty at small T) and wins once experts get several groups
// of 4 slots.
#ifndef BQM_MMA_MIN_T
#define BQM_MMA_MIN_T 8
#endif

// Expert-indexed GEMV: the chain kernel's indexed form, with E * N rows as one matrix.  The
// batch class is that of min(T, 4): one token usually adds at most one slot to an expert,
// so up to 4 tokens stream each selected expert once; an expert with more slots is
// streamed once per group of 4.  With `w_up`, the gate+up form: each lane takes gate row n
// and up row n of the expert, and the output is silu(gate) * up.
static int launch_id(int fmt, const void* w, const void* w_up, int E, int64_t N, int64_t K,
              const int32_t* ids, int T, int top_k, const float* X, int64_t xts, int64_t xss,
              float* Y, hipStream_t s, const float* rw = nullptr) {
  // From BQM_MMA_MIN_T tokens on, the matrix-core form: each expert's rows stream once for
  // up to 16 of its slots and the vector work per weight does not grow with the slots
  if (T >= BQM_MMA_MIN_T) {
    const int st = launch_id_mma(fmt, w, w_up, E, N, K, ids, T, top_k, X, xts, xss, Y, s, rw);
    if (st != BQM_E_UNSUPPORTED) return st;
  }
  const int TS = T * top_k;
  Layout L;
  layout_of(fmt, (int64_t)E * N, K, &L);
  const int CB = fmt == BQM_Q4_0 ? 16 : 32;
  // Groups of at most 4 slots (batch class 4, 16 waves): with top-8 routing an expert
  // rarely gets more than a few of T tokens, so a class-8 group mostly computes empty
  // inputs on half the waves (128-expert MoE layer, T = 16: 0.271 -> 0.183 ms per layer;
  // class 2 re-reads the popular experts too often: 0.190).
  const int mm = m_class(T < kIdMaxClass ? T : kIdMaxClass);
  const int cus = cu_count();
  // a workgroup's rows of one group: its share of the groups' rows (at most TS groups of N)
  int64_t rows = ((int64_t)TS * N + cus - 1) / cus;
  rows = rows < N ? rows : N;
  if ((rows + 1) * L.nb * CB >= ((int64_t)1 << 31)) return BQM_E_SHAPE;
  int kc = 0, pacc_rows = 0;
  // the gate+up form keeps two partial sums per output row
  if (!chain_plan(idx_table_rows(E, TS), mm, L.nb, w_up ? 2 * rows : rows, &kc, &pacc_rows))
    return BQM_E_SHAPE;
  if (kc < 1) kc = 1;  // K = 0: nothing is staged, but chunk counts divide by kc
  const uint8_t* codes = static_cast<const uint8_t*>(w);
  const uint8_t* up = static_cast<const uint8_t*>(w_up);
  const IdxArgs ix{ids, reinterpret_cast<const uint16_t*>(codes + L.scales_off), up,
                   up ? reinterpret_cast<const uint16_t*>(up + L.scales_off) : nullptr,
                   E, TS, top_k, xts, xss, rw};
  const GemvDesc d{codes, X, Y, N, K, fmt, 0, 1, 0};
  return launch_chain(fmt, mm, nullptr, nullptr, &d, 1, kc, pacc_rows, nullptr, false, s, &ix);
}

int launch_qmv_id(int fmt, const void* w, int E, int64_t N, int64_t K, const int32_t* ids, int T,
                  int top_k, const float* X, int64_t xts, int64_t xss, float* Y, hipStream_t s) {
  return launch_id(fmt, w, nullptr, E, N, K, ids, T, top_k, X, xts, xss, Y, s);
}

int launch_qmv_id_gate_up(int fmt, const void* w_gate, const void* w_up, int E, int64_t N, int64_t K,
                          const int32_t* ids, int T, int top_k, const float* X, int64_t xts,
                          int64_t xss, float* Y, hipStream_t s) {
  return launch_id(fmt, w_gate, w_up, E, N, K, ids, T, top_k, X, xts, xss, Y, s);
}

// Y[t][n] = sum over s < top_k of Y_slots[t][s][n], s ascending, fp32: one thread per (t, n),
// the slots' loads in flight together, eight at a time.
__global__ __launch_bounds__(256) void k_slot_sum(const float* __restrict__ ys, float* __restrict__ y,
                                                  int64_t N, int64_t TN, int top_k) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= TN) return;
  const int64_t t = i / N, n = i - t * N;
  const float* p = ys + t * top_k * N + n;
  float sum = 0.0f;
  for (int kb = 0; kb < top_k; kb += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; j++) v[j] = kb + j < top_k ? p[(int64_t)(kb + j) * N] : 0.0f;
#pragma unroll
    for (int j = 0; j < 8; j++)
      if (kb + j < top_k) sum = kb + j == 0 ? v[j] : sum + v[j];
  }
  y[i] = sum;
}

int launch_qmv_id_sum(int fmt, const void* w, int E, int64_t N, int64_t K, const int32_t* ids,
                      const float* rw, int T, int top_k, const float* X, int64_t xts, int64_t xss,
                      float* Y_slots, float* Y, hipStream_t s) {
  if (int st = launch_id(fmt, w, nullptr, E, N, K, ids, T, top_k, X, xts, xss, Y_slots, s, rw))
    return st;
  const int64_t TN = (int64_t)T * N;
  hipLaunchKernelGGL(k_slot_sum, dim3((unsigned)((TN + 255) / 256)), dim3(256), 0, s, Y_slots, Y, N,
                     TN, top_k);
  return launch_status();
}

// ---- the weighted sum without a caller buffer -------------------------------------------
// For callers that cannot allocate: the weighted slot rows live in a file-scope device array
// of BQM_NOALLOC_SLOT_FLOATS floats (4 MiB), one copy per GPU, held until the process ends.
// Its address is a device address only through hipGetSymbolAddress (the array's name in host
// code is a host-side stand-in), taken once per device with that device current and kept.
// Every slot row is written by the product before the slot sum reads it, so nothing has to
// start at zero; calls that overlap in time on one GPU share the array and race.
static __device__ __align__(256) float scratch[BQM_NOALLOC_SLOT_FLOATS];

namespace {
std::mutex g_scratch_mutex;
float* g_scratch_ptr[64] = {};

int scratch_on_current_device(float** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return BQM_E_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BQM_E_LAUNCH;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return BQM_OK;
}
}  // namespace

int launch_qmv_id_sum_noalloc(int fmt, const void* w, int E, int64_t N, int64_t K, const int32_t* ids,
                              const float* rw, int T, int top_k, const float* X, int64_t xts,
                              int64_t xss, float* Y, hipStream_t s) {
  if ((int64_t)T * top_k * N > BQM_NOALLOC_SLOT_FLOATS) return BQM_E_SHAPE;
  float* slots = nullptr;
  if (int st = scratch_on_current_device(&slots)) return st;
  return launch_qmv_id_sum(fmt, w, E, N, K, ids, rw, T, top_k, X, xts, xss, slots, Y, s);
}

}  // namespace bqm
