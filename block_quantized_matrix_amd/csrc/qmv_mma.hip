// Expert-indexed GEMV on the matrix cores, gfx950.
//
// The slots routed to one expert (mul_mat_id, on the page "ik_llama.cpp 老工作站多 GPU 部署
// Qwen3-235B-A22B 实战指南" (nxmr.cn), background section) all multiply the same expert rows:
// for a group of up to 16 of them, Y[s][n] = sum_k W[e][n][k] x_s[k] is a 16-column matrix
// product.  Here each 32-weight block of 16 rows goes through v_mfma_f32_16x16x32_bf16 once
// for all the group's slots, instead of one fp32 FMA per weight and slot on the vector ALU:
// the expert's rows stream from HBM once per group of 16 (with T <= 16 tokens, once), and
// the vector work per weight (code conversion and the block-scale FMA) does not grow with
// the number of slots.
//
// Operands.  MFMA rows i = slots of the group, columns j = 16 expert rows, k = the 32
// positions of one block (so the block's scale applies to the whole product).  Lane l holds
// A[i = l % 16][k-group l / 16] and B[k-group][j = l % 16]: 8 values each.  A lane's eight
// positions are those of one 4-byte word of Q4_0 codes (the low nibbles are positions
// 4q..4q+3, the high ones 16+4q..16+4q+3) or of 8 bytes of Q8_0 codes (8q..8q+7); the inputs
// are staged in LDS in the same order.  D[i][j] comes back as 4 values per lane: slots
// 4 (l / 16) + r, row l % 16.
//
// Exactness.  Codes enter as bf16 signed values, exact (Q4_0 as 16 (n - 8), Q8_0 the int8
// code).  Each fp32 input x, scaled by 2^30 (exact; undone in the block scale), is split
// into two bf16 parts: x_hi, truncated to 8 significant bits, and x_lo, the remainder
// (exact in fp32) truncated likewise; the part left out is below 2^-14 |x| for every fp32 x
// below 2^86 in magnitude (larger inputs can overflow the partial sums).  Products of bf16 values are exact in fp32, so a block sum carries
// the MFMA's fp32 accumulation error plus at most 2^-14 sum_j |c_j x_j|; then acc += d * sum
// in fp32 as in the vector kernels, blocks in ascending order.  Total error far below
// 1e-3 sum |w x|; neutral codes give exactly zero; integer inputs and power-of-two scales
// give exact results.
//
// Work.  Every workgroup (one per compute unit, 16 waves) sorts the slots by expert (the
// stable counting sort of slot_groups.h) and cuts each expert's run into groups of up to 16.  The
// 16-row tiles of all groups are split evenly over the workgroups.  A workgroup walks its
// tiles in passes of one group each: it stages the group's inputs (both bf16 parts) for a
// chunk of K in LDS, its waves compute their tiles over the chunk, and so on along K.  When
// a pass has fewer tiles than waves, the waves also split each chunk's blocks between them
// and the partial sums are added through LDS in a fixed order, so results are deterministic.
#include "bqm_internal.h"
#include "mma_ops.h"
#include "slot_groups.h"

#include <algorithm>

namespace bqm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum { MQ4 = 0, MQ8 = 1 };

constexpr int kMWaves = 16, kMThreads = 64 * kMWaves;
constexpr int kGroupSlots = 16;                     // slots per group: the MFMA's 16 rows
constexpr int kXBlk = 2 * 64 * 16;                  // LDS bytes per staged block: 2 parts x 64 lanes x 16 B
constexpr int kMStaticLds = 1024;
constexpr int kMMaxLds = 160 * 1024 - kMStaticLds;  // dynamic LDS of a launch
constexpr uint32_t kOob = 0x80000000u;              // a lane offset past every descriptor: reads 0
constexpr int kJobs = 4;                            // staging jobs per thread whose loads fly together

struct MmaArgs {
  const uint8_t* codes;    // the (gate) expert tensor: codes of E * N rows ...
  const uint16_t* scales;  // ... and their scales
  const uint8_t* codes2;   // gate+up form: the up tensor
  const uint16_t* scales2;
  const int32_t* ids;      // [T][top_k]
  const float* x;
  float* y;                // [T * top_k][N]
  const float* rw;         // router weights [T][top_k] the rows are scaled by, or null
  int E, N, nb, TS, top_k, kc;  // kc: the staging area's bytes / kXBlk
  int64_t xts, xss;        // input strides (floats) per token and per slot
};

// LDS: the slot table (per-expert counts then starts, E + 1; slots sorted by expert, TS;
// groups of 3 ints, at most TS), then the staging area: a pass's inputs and scales chunk by
// chunk, and its K-split partial sums at the end.
__host__ __device__ inline int mma_table_bytes(int E, int TS) { return ((E + 1 + 4 * TS) * 4 + 15) & ~15; }
// Tiles per wave in a pass (their loads, two units of 128 bytes per row in flight, and sums
// fit 128 registers).
__host__ __device__ constexpr int mma_tpw(bool q4, bool gu) { return (void)q4, gu ? 1 : 2; }
// Rows of a pass's scales at most, over both tensors: every wave's tiles.
__host__ __device__ constexpr int mma_max_rows(bool q4, bool gu) { return kMWaves * mma_tpw(q4, gu) * 16 * (gu ? 2 : 1); }
// The K-split partial sums at most: every wave but those of the first share, TPW tiles of
// 16 x 16 floats per tensor each.
__host__ __device__ constexpr int mma_part_bytes(bool q4, bool gu) {
  return (kMWaves - 1) * mma_tpw(q4, gu) * (gu ? 2 : 1) * 1024;
}

__device__ __forceinline__ float h2f(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

template <int FMT, bool GU>
__global__ __launch_bounds__(kMThreads) void k_qmv_id_mma(MmaArgs a) {
  constexpr int CB = FMT == MQ4 ? 16 : 32;         // code bytes per block
  constexpr int LW = FMT == MQ4 ? 1 : 2;           // 16-byte code loads per lane, tile and quad
  constexpr int NG = GU ? 2 : 1;                   // tensors (gate+up: two)
  constexpr int TPW = mma_tpw(FMT == MQ4, GU);
  extern __shared__ float4 smem[];
  char* lds = reinterpret_cast<char*>(smem);
  __shared__ int s_ng;
  __shared__ int s_scan[2 * kMWaves];
  __shared__ int64_t s_xoff[kGroupSlots];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = a.E, TS = a.TS, N = a.N, nb = a.nb;
  int* cnt = reinterpret_cast<int*>(lds);
  int* srt = cnt + E + 1;
  int* grp = srt + TS;
  char* xl = lds + mma_table_bytes(E, TS);

  // the id of this workgroup's first slot in the padding fill below, read now, together with
  // the ids the slot sort reads (after the sort it would be a memory round trip more)
  const int fill_e0 = (int)blockIdx.x < TS ? a.ids[blockIdx.x] : 0;
  // the slots grouped by expert, groups of up to 16
  group_slots<kMThreads, kGroupSlots>(a.ids, E, TS, cnt, srt, grp, s_scan, &s_ng);
  const int ng = s_ng;

  // rows of slots that no group computes, each by one workgroup: a negative id gives zeros,
  // an id >= E NaN; with K = 0 every valid slot's sums are empty (zeros)
  for (int ts = blockIdx.x; ts < TS; ts += gridDim.x) {
    const int e = ts == (int)blockIdx.x ? fill_e0 : a.ids[ts];
    const bool valid = e >= 0 && e < E;
    if (valid && nb > 0) continue;
    const float v = valid || e < 0 ? 0.0f : __builtin_nanf("");
    for (int n = tid; n < N; n += kMThreads) a.y[(int64_t)ts * N + n] = v;
  }
  if (nb == 0 || ng == 0) return;

  // ---- this workgroup's tiles ----
  // With no more groups than workgroups, each group's tiles go to its own run of workgroups
  // (the tiles split evenly between them), so a workgroup streams one expert in one pass.  (Split evenly over all
  // tiles, a workgroup whose share straddled two groups ran two passes, each with its own
  // staging and sums, and finished 30 us after the others on the MoE layer at T = 16.)  With
  // more groups than workgroups, the tiles of all groups are split evenly.
  const int tpg = (N + 15) >> 4;  // 16-row tiles per group
  const int64_t tt = (int64_t)ng * tpg;
  const int G = (int)gridDim.x, b = (int)blockIdx.x;
  int64_t t_begin, t_end;
  if (ng <= G) {
    // Each group gets a base of workgroups (below), and the others are shared out by weight:
    // 4 + 2 chunks, the chunks of K its slots' inputs need (estimated at the even share of
    // tiles, at most 3 counted).  A group of many slots stages its inputs in more chunks, each a memory
    // round trip more, and its workgroups then take fewer rows.  (Measured on the MoE gate
    // projection at T = 16, 16 tiles per workgroup: 48-50 us with one chunk, 54-58 with two,
    // 63 with three, about 2.2 us per tile.)  Group g's workgroups: from g base + floor(P_g
    // (G - ng base) / W) to the next group's first, P_g the weights before it, W their sum.
    {
      const int nt0 = (int)std::min<int64_t>(kMWaves * TPW, (tt + G - 1) / G);
      const int R0 = nt0 * 16;
      constexpr int KQ0 = FMT == MQ4 ? 8 : 4;
      int wv = 0;  // thread g < ng: group g's weight (ng <= G <= kMThreads)
      if (tid < ng) {
        const int c = grp[3 * tid + 2];
        int kcp = (a.kc * kXBlk - 16 * NG * R0) / (2 * (4 * c + 1) * 16 + 2 * NG * R0);
        kcp = std::max(KQ0, kcp & ~(KQ0 - 1));
        wv = 4 + 2 * std::min((nb + kcp - 1) / kcp, 3);
      }
      // exclusive prefix of the weights: a scan in each wave, then the waves' totals (s_scan is
      // free after the sort)
      int inc = wv;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(inc, o, 64);
        if (lane >= o) inc += u;
      }
      if (lane == 63) s_scan[wave] = inc;
      __syncthreads();
      int before = 0, W = 0;
      for (int w = 0; w < kMWaves; w++) {
        before += w < wave ? s_scan[w] : 0;
        W += s_scan[w];
      }
      // every group first gets the workgroups that keep its tiles within one pass (a round of
      // the waves, kMWaves * TPW tiles), where the grid allows, else one; then its weighted
      // share of the rest.  (Without the first part, gate+up at T = 16 (16 tiles a pass) gave
      // some workgroups 17-19 tiles, whose second pass ended the call 27 us after the median.)
      const int bmin = (tpg + kMWaves * TPW - 1) / (kMWaves * TPW);
      const int base = (int64_t)ng * bmin <= G ? bmin : 1;
      if (tid < ng) {  // is this workgroup one of group tid's?  (products below 2^31)
        const int P = before + inc - wv, E = G - ng * base;
        const int f0 = tid * base + P * E / W, f1 = (tid + 1) * base + (P + wv) * E / W;
        if (f0 <= b && b < f1) {
          s_xoff[0] = tid;
          s_xoff[1] = f0;
          s_xoff[2] = f1 - f0;
        }
      }
      __syncthreads();
    }
    const int g = (int)s_xoff[0], w0 = (int)s_xoff[1], nw = (int)s_xoff[2], i = b - w0;
    t_begin = (int64_t)g * tpg + (int64_t)tpg * i / nw;
    t_end = (int64_t)g * tpg + (int64_t)tpg * (i + 1) / nw;
    __syncthreads();  // read by every thread before the first pass writes s_xoff
  } else {
    t_begin = tt * b / G;
    t_end = tt * (b + 1) / G;
  }
  const int j = lane & 15, q = lane >> 4;
  for (int64_t t = t_begin; t < t_end;) {
    const int g = (int)(t / tpg), ta = (int)(t - (int64_t)g * tpg);
    const int64_t left = t_end - t;
    int nt = tpg - ta;
    if (left < nt) nt = (int)left;
    if (nt > kMWaves * TPW) nt = kMWaves * TPW;
    t += nt;
    const int e = grp[3 * g], s0 = grp[3 * g + 1], c = grp[3 * g + 2];
    // The pass's tiles in sets of TPW, one set per wave; with fewer sets than waves the waves
    // also split each chunk's blocks into KS shares: wave w takes set w % TSN, share w / TSN
    // (waves past TSN * KS only help stage the inputs).  Every busy wave then holds TPW tiles'
    // loads in flight.
    const int TSN = (nt + TPW - 1) / TPW, KS = kMWaves / TSN;
    const int tsi = wave % TSN, ks = wave / TSN;
    const int mt = ks < KS ? min(TPW, nt - tsi * TPW) : 0;  // this wave's tiles
    const int tb = ta + tsi * TPW;                          // its first tile
    // the group's input rows (slot si: token * xts + slot * xss floats into x), read by the
    // staging after the barrier that follows (the previous pass read them before two)
    if (tid < c) {
      const int ts = srt[s0 + tid];
      const int tok = ts / a.top_k, sl = ts - tok * a.top_k;
      s_xoff[tid] = tok * a.xts + sl * a.xss;
    }
    const int64_t erow = (int64_t)e * N;
    const uint32_t ecb = (uint32_t)N * (uint32_t)nb * CB;  // one expert's code bytes (< 2^31)
    __amdgpu_buffer_rsrc_t rc[NG], rs[NG];
    rc[0] = __builtin_amdgcn_make_buffer_rsrc((void*)(a.codes + erow * nb * CB), (short)0, (int)ecb, 0x00020000);
    rs[0] = __builtin_amdgcn_make_buffer_rsrc((void*)(a.scales + erow * nb), (short)0, (int)((uint32_t)N * nb * 2),
                                              0x00020000);
    if constexpr (GU) {
      rc[1] = __builtin_amdgcn_make_buffer_rsrc((void*)(a.codes2 + erow * nb * CB), (short)0, (int)ecb, 0x00020000);
      rs[1] = __builtin_amdgcn_make_buffer_rsrc((void*)(a.scales2 + erow * nb), (short)0,
                                                (int)((uint32_t)N * nb * 2), 0x00020000);
    }
    // lane offsets of its row in each of its tiles' codes (its word or two of a block); rows
    // past N and tiles the wave does not have read zeros
    uint32_t vc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; i++) {
      const int n = (tb + i) * 16 + j;
      const bool ok = i < mt && n < N;
      vc[i] = ok ? (uint32_t)n * (uint32_t)nb * CB + (uint32_t)q * 16 : kOob;
    }
    // The pass's scales are staged in LDS with its inputs, chunk by chunk: R rows (the pass's
    // tiles) per tensor, each a run of kcp 2-byte scales at a stride of sst bytes.  Read
    // straight from memory, 8 bytes per row and quad, every row kept a 128-byte scale line
    // in use for 16 quads: 32 CUs x 16 waves x 64 rows of them, as much as an XCD's L2 holds
    // while the codes stream through it, and most came back from HBM again and again
    // (measured on the MoE layer at T = 16: 5x the scale bytes).  Staged, each chunk's scales
    // of a row are read in one contiguous run.  The chunk (kcp blocks, a multiple of 4) is
    // the longest that leaves room for both, evened out over the chunks of K; the stride is
    // twice an odd number of words, so that the 16 rows of one 8-byte read meet 32 distinct
    // banks.
    //
    // The inputs are staged compactly: per block and bf16 part, the c slots' pieces of the 4
    // k-groups ([k-group][slot], 16 bytes each), then one zero piece, which the lanes of the
    // MFMA rows past c read.  (All 16 rows staged, a group of a few slots spent most of the
    // staging on zeros, and the chunks of K it fitted in were three times as many.)
    const int R = nt * 16;
    const int xpp = (4 * c + 1) * 16;  // bytes per block and part
    const int bxb = 2 * xpp;           // staged input bytes per block
    constexpr int KQ = FMT == MQ4 ? 8 : 4;  // blocks per 128 bytes of a row: chunks start on lines
    int kcp = (a.kc * kXBlk - 16 * NG * R) / (bxb + 2 * NG * R);
    kcp = max(KQ, kcp & ~(KQ - 1));
    {
      const int nch = (nb + kcp - 1) / kcp;
      kcp = min(kcp, (((nb + nch - 1) / nch) + KQ - 1) & ~(KQ - 1));
    }
    int sdw = kcp / 2 + 2;
    if (((sdw >> 1) & 1) == 0) sdw += 2;
    const int sst = 4 * sdw;
    char* scl = xl + kcp * bxb;
    // this lane's input piece (slot j, k-group q) in a block's first part (the second is xpp
    // bytes on); lanes past the group's slots read the zero piece
    const int xo = j < c ? (q * c + j) * 16 : 4 * c * 16;
    int srow[TPW];  // this lane's row in the scale area, per tile (tiles it does not have: row 0)
#pragma unroll
    for (int i = 0; i < TPW; i++) srow[i] = i < mt ? (tsi * TPW + i) * 16 + j : 0;
    float acc[TPW][NG][4];
#pragma unroll
    for (int i = 0; i < TPW; i++)
#pragma unroll
      for (int h = 0; h < NG; h++)
#pragma unroll
        for (int r = 0; r < 4; r++) acc[i][h][r] = 0.0f;

    // One quad (4 blocks) of a wave's tiles: 16-byte code loads of each tile and tensor (the
    // scales come from LDS).  A load covers 64 contiguous bytes of each of the tile's 16 rows (lane
    // group q: Q4_0 block q of the quad; Q8_0 half q % 2 of block q / 2, twice), so every
    // load instruction reads whole 64-byte pieces; lane exchanges then give each lane group
    // its word (Q4_0) or 8 bytes (Q8_0) of every block.
    struct Quad {
      u32x4 c[TPW][NG][LW];
    };
    // issue a quad's loads; `live` false: offsets past the descriptors, nothing is read
    auto issue = [&](Quad& Qd, int kb, bool live) {
      const uint32_t m = live ? 0u : kOob;
#pragma unroll
      for (int i = 0; i < TPW; i++)
#pragma unroll
        for (int h = 0; h < NG; h++) {
#pragma unroll
          for (int w = 0; w < LW; w++)
            Qd.c[i][h][w] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc[h], (vc[i] | m) + w * 64, kb * CB, 0));
        }
    };
    // a quad's products: block u of the chunk-local quad `ql`
    auto consume = [&](Quad& Qd, int ql) {
      // the 4 scales of each tile's row j (lanes of one row read the same 8 bytes)
      u32x2 sq[TPW][NG];
#pragma unroll
      for (int i = 0; i < TPW; i++)
#pragma unroll
        for (int h = 0; h < NG; h++)
          sq[i][h] = *reinterpret_cast<const u32x2*>(scl + (h * R + srow[i]) * sst + 8 * ql);
#pragma unroll
      for (int i = 0; i < TPW; i++)
#pragma unroll
        for (int h = 0; h < NG; h++)
#pragma unroll
          for (int w = 0; w < LW; w++) mma::exchange<FMT == MQ4>(Qd.c[i][h][w]);
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int bl = 4 * ql + u;
        const char* xb = xl + bl * bxb + xo;
        const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(xb);
        const bf16x8 alo = *reinterpret_cast<const bf16x8*>(xb + xpp);
        // every tile of the set, also those past the pass's end (whose codes and scales read
        // as zeros): no branches, so the tiles' products and sums interleave
        f32x4 d[TPW][NG];
#pragma unroll
        for (int i = 0; i < TPW; i++)
#pragma unroll
          for (int h = 0; h < NG; h++) {
            const u32x4& v = Qd.c[i][h][FMT == MQ4 ? 0 : u >> 1];
            const bf16x8 b = FMT == MQ4 ? mma::q4_operand(v[u]) : mma::q8_operand(v[2 * (u & 1)], v[2 * (u & 1) + 1]);
            d[i][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            d[i][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, b, d[i][h], 0, 0, 0);
          }
#pragma unroll
        for (int i = 0; i < TPW; i++)
#pragma unroll
          for (int h = 0; h < NG; h++) {
            const uint32_t sw = (u & 2) ? sq[i][h].y : sq[i][h].x;
            // d, times 1/16 for the Q4_0 codes' 16 (n - 8), times 2^-kXShift for the inputs
            const float sc = h2f((u & 1) ? sw >> 16 : sw) * (FMT == MQ4 ? 0x1p-34f : 0x1p-30f);
#pragma unroll
            for (int r = 0; r < 4; r++) acc[i][h][r] = fmaf(sc, d[i][h][r], acc[i][h][r]);
          }
      }
    };

    for (int kb0 = 0; kb0 < nb; kb0 += kcp) {
      const int kcb = min(kcp, nb - kb0);  // a multiple of 4, as nb and kcp are
      // The chunk's quads in units of 128 bytes of each row (Q4_0: two quads, issued together),
      // the units split into KS shares; a wave keeps two units of loads in registers and issues
      // the next into each as soon as its products are taken, so one unit is always in flight.
      // (Quads issued one ahead of their products asked for the second half of a line while
      // the first was still in flight, and more lines crossed HBM twice: 1.45x -> 1.66x the
      // algorithmic bytes on the MoE layer at T = 16.)
      constexpr int UQ = FMT == MQ4 ? 2 : 1;
      const int nq = kcb >> 2, nu = (nq + UQ - 1) / UQ;
      const int u0 = ks < KS ? nu * ks / KS : 0, u1 = ks < KS ? nu * (ks + 1) / KS : 0;
      Quad UA[UQ], UB[UQ];
      auto issue_unit = [&](Quad* U, int un, bool live) {
#pragma unroll
        for (int sq = 0; sq < UQ; sq++) issue(U[sq], kb0 + 4 * (UQ * un + sq), live && UQ * un + sq < nq);
      };
      auto consume_unit = [&](Quad* U, int un) {
#pragma unroll
        for (int sq = 0; sq < UQ; sq++)
          if (UQ * un + sq < nq) consume(U[sq], UQ * un + sq);
      };
      // the first unit's weights do not depend on the inputs: fetch them across the staging
      issue_unit(UA, u0, u0 < u1);
      __syncthreads();  // the previous chunk's inputs are no longer read
      // stage the group's inputs for blocks kb0 .. kb0 + kcb: per (block, k-group, slot) both
      // parts, and each block's zero pieces; a thread's jobs in rounds of kJobs, each round's
      // loads in flight together
      for (int b = tid; b < kcb; b += kMThreads) {
        *reinterpret_cast<u32x4*>(xl + b * bxb + 4 * c * 16) = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(xl + b * bxb + xpp + 4 * c * 16) = u32x4{0u, 0u, 0u, 0u};
      }
      const int njx = kcb * 4 * c;
      for (int jb0 = 0; jb0 < njx; jb0 += kJobs * kMThreads) {
        f32x4 v[kJobs][2];
#pragma unroll
        for (int r = 0; r < kJobs; r++) {
          const int jb = jb0 + r * kMThreads + tid;
          const int bl = jb / (4 * c), pq = jb - bl * 4 * c, sq = pq / c, si = pq - sq * c;
          v[r][0] = v[r][1] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (jb < njx) {
            const float* xr = a.x + s_xoff[si] + (int64_t)(kb0 + bl) * 32;
            v[r][0] = *reinterpret_cast<const f32x4*>(xr + (FMT == MQ4 ? 4 * sq : 8 * sq));
            v[r][1] = *reinterpret_cast<const f32x4*>(xr + (FMT == MQ4 ? 16 + 4 * sq : 8 * sq + 4));
          }
        }
#pragma unroll
        for (int r = 0; r < kJobs; r++) {
          const int jb = jb0 + r * kMThreads + tid;
          if (jb < njx) {
            const int bl = jb / (4 * c), pq = jb - bl * 4 * c;  // pq = k-group * c + slot
            const float f[8] = {v[r][0].x, v[r][0].y, v[r][0].z, v[r][0].w,
                                v[r][1].x, v[r][1].y, v[r][1].z, v[r][1].w};
            u32x4 hi, lo;
            mma::split8(f, hi, lo);
            *reinterpret_cast<u32x4*>(xl + bl * bxb + pq * 16) = hi;
            *reinterpret_cast<u32x4*>(xl + bl * bxb + xpp + pq * 16) = lo;
          }
        }
      }
      // stage the pass's scales for the chunk: per tensor, row r's kcb scales as 16-byte pieces
      // (8 blocks; else 8-byte pieces of 4), consecutive pieces of a
      // row to consecutive threads, kSJobs rows per thread in flight together (one memory round
      // trip for up to 8 * 1024 pieces; staged 8 bytes at a time, 4 in flight, a pass of 400
      // rows took four); rows past N read zeros
      {
        constexpr int kSJobs = 8;
        // 16-byte pieces only where each starts on a 16-byte boundary (nb, kb0, kcb multiples of 8)
        const bool p16 = ((nb | kb0 | kcb) & 7) == 0;
        const int pcs = p16 ? kcb >> 3 : kcb >> 2;  // pieces per row
        const int rpr = kMThreads / pcs;            // rows per round of the threads
        const int myr = tid / pcs, pc = tid - myr * pcs;
        const int pbytes = p16 ? 16 : 8;
#pragma unroll
        for (int h = 0; h < NG; h++)
          for (int r0 = 0; r0 < R; r0 += kSJobs * rpr) {
            u32x4 v[kSJobs];
#pragma unroll
            for (int k = 0; k < kSJobs; k++) {
              const int row = r0 + k * rpr + myr, n = ta * 16 + row;
              const bool ok = myr < rpr && row < R && n < N;
              const uint32_t off = ok ? (uint32_t)n * (uint32_t)nb * 2u + (uint32_t)(kb0 + pc * (p16 ? 8 : 4)) * 2u : kOob;
              if (p16) {
                v[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs[h], off, 0, 0));
              } else {
                const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs[h], off, 0, 0));
                v[k] = u32x4{w.x, w.y, 0u, 0u};
              }
            }
#pragma unroll
            for (int k = 0; k < kSJobs; k++) {
              const int row = r0 + k * rpr + myr;
              if (myr < rpr && row < R) {
                char* dst = scl + (h * R + row) * sst + pbytes * pc;  // 8-byte aligned
                *reinterpret_cast<u32x2*>(dst) = u32x2{v[k].x, v[k].y};
                if (p16) *reinterpret_cast<u32x2*>(dst + 8) = u32x2{v[k].z, v[k].w};
              }
            }
          }
      }
      __syncthreads();
      if (u0 + 1 < u1) issue_unit(UB, u0 + 1, true);
      for (int un = u0; un < u1; un += 2) {
        // issue priority from the share of the wave's units left: a SIMD issues from its
        // oldest wave first, and without it the waves of a workgroup finished up to 18 us
        // apart on the MoE layer at T = 16
        {
          const int c4 = 4 * (u1 - un), n4 = u1 - u0;
          if (c4 >= 3 * n4) __builtin_amdgcn_s_setprio(3);
          else if (c4 >= 2 * n4) __builtin_amdgcn_s_setprio(2);
          else if (c4 >= n4) __builtin_amdgcn_s_setprio(1);
          else __builtin_amdgcn_s_setprio(0);
        }
        consume_unit(UA, un);
        if (un + 2 < u1) issue_unit(UA, un + 2, true);
        if (un + 1 < u1) {
          consume_unit(UB, un + 1);
          if (un + 3 < u1) issue_unit(UB, un + 3, true);
        }
      }
    }

    // K split between waves: the shares after the first go through LDS (the staging area,
    // free once every wave is past the last chunk) and are added to the first share's sums in
    // share order
    if (KS > 1) {
      float* part = reinterpret_cast<float*>(xl);
      __syncthreads();
      if (ks > 0 && mt > 0) {
#pragma unroll
        for (int i = 0; i < TPW; i++)
          if (i < mt)
#pragma unroll
            for (int h = 0; h < NG; h++)
              *reinterpret_cast<f32x4*>(part + ((((ks - 1) * TSN + tsi) * TPW + i) * NG + h) * 256 + lane * 4) =
                  f32x4{acc[i][h][0], acc[i][h][1], acc[i][h][2], acc[i][h][3]};
      }
      __syncthreads();
      if (ks == 0 && mt > 0) {
        for (int kk = 1; kk < KS; kk++) {
#pragma unroll
          for (int i = 0; i < TPW; i++)
            if (i < mt)
#pragma unroll
              for (int h = 0; h < NG; h++) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(
                    part + ((((kk - 1) * TSN + tsi) * TPW + i) * NG + h) * 256 + lane * 4);
                acc[i][h][0] += v.x;
                acc[i][h][1] += v.y;
                acc[i][h][2] += v.z;
                acc[i][h][3] += v.w;
              }
        }
      }
    }
    // store: lane (j, q) holds row j of each tile for slots 4q .. 4q + 3 of the group
    if (ks == 0) {
#pragma unroll
      for (int i = 0; i < TPW; i++) {
        const int n = (tb + i) * 16 + j;
        if (i < mt && n < N) {
#pragma unroll
          for (int r = 0; r < 4; r++) {
            const int si = 4 * q + r;
            if (si < c) {
              const int ts = srt[s0 + si];
              float v = acc[i][0][r];
              if constexpr (GU) v = v / (1.0f + expf(-v)) * acc[i][NG - 1][r];  // silu(g) * u
              if (a.rw) v *= a.rw[ts];
              a.y[(int64_t)ts * N + n] = v;
            }
          }
        }
      }
    }
  }
}

using MmaKernel = void (*)(MmaArgs);
MmaKernel mma_kernel(int fmt, bool gu) {
  if (fmt == BQM_Q4_0) return gu ? k_qmv_id_mma<MQ4, true> : k_qmv_id_mma<MQ4, false>;
  return gu ? k_qmv_id_mma<MQ8, true> : k_qmv_id_mma<MQ8, false>;
}

}  // namespace

// The matrix-core form of the expert-indexed GEMV (plain, router-weighted with `rw`, or
// gate+up with `w_up`).  Returns BQM_E_UNSUPPORTED when the shape does not suit it (K not a
// multiple of 128, an expert of 2 GiB of codes or more, or the slot table leaving no room
// for a chunk of inputs); the caller then uses the vector form.
int launch_id_mma(int fmt, const void* w, const void* w_up, int E, int64_t N, int64_t K,
                  const int32_t* ids, int T, int top_k, const float* X, int64_t xts, int64_t xss,
                  float* Y, hipStream_t s, const float* rw) {
  const int64_t nb = K / kQK;
  if (nb % 4 != 0) return BQM_E_UNSUPPORTED;
  const int CB = fmt == BQM_Q4_0 ? 16 : 32;
  if (N * nb * CB >= ((int64_t)1 << 31)) return BQM_E_UNSUPPORTED;
  const int TS = T * top_k;
  const bool gu = w_up != nullptr;
  const int fixed = mma_table_bytes(E, TS);
  // the staging area: all the LDS the slot table leaves, in units of one block's inputs (a
  // pass takes its chunks' inputs and scales from it, and the K-split partial sums at the end)
  const int64_t kc = (kMMaxLds - fixed) / kXBlk;
  const int64_t xbytes = std::max<int64_t>(kc * kXBlk, mma_part_bytes(fmt == BQM_Q4_0, gu));
  if (fixed + xbytes > kMMaxLds) return BQM_E_UNSUPPORTED;
  // room for a chunk of 4 blocks with the scales of the largest pass
  if (kc * kXBlk < 4 * (kXBlk + 32) + 24 * mma_max_rows(fmt == BQM_Q4_0, gu)) return BQM_E_UNSUPPORTED;
  Layout L;
  layout_of(fmt, (int64_t)E * N, K, &L);
  const uint8_t* codes = static_cast<const uint8_t*>(w);
  const uint8_t* up = static_cast<const uint8_t*>(w_up);
  MmaArgs a;
  a.codes = codes;
  a.scales = reinterpret_cast<const uint16_t*>(codes + L.scales_off);
  a.codes2 = up;
  a.scales2 = up ? reinterpret_cast<const uint16_t*>(up + L.scales_off) : nullptr;
  a.ids = ids;
  a.x = X;
  a.y = Y;
  a.rw = rw;
  a.E = E;
  a.N = (int)N;
  a.nb = (int)nb;
  a.TS = TS;
  a.top_k = top_k;
  a.kc = (int)kc;
  a.xts = xts;
  a.xss = xss;
  MmaKernel k = mma_kernel(fmt, gu);
  const int lds = fixed + (int)xbytes;
  if (lds > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  hipLaunchKernelGGL(k, dim3((unsigned)cu_count()), dim3(kMThreads), lds, s, a);
  return launch_status();
}

}  // namespace bqm
