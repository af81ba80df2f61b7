// The slots of an expert-indexed product grouped by expert, in LDS, for the vector and the
// matrix-core forms of the indexed GEMV (device code; included by qmv.hip and qmv_mma.hip).
#pragma once

#include "bqm_internal.h"

namespace bqm {

// Slots of the indexed forms, at most (T * top_k at their limits).
constexpr int kIdMaxSlots = BQM_QMV_ID_MAX_T * BQM_QMV_ID_MAX_TOPK;

// A counting sort of the T * top_k slots by expert that is stable: within an expert's run the
// slots are in index order, so every workgroup forms the same groups (the workgroups split a
// group's rows between them, and each must know the same slots).  Each run is cut into groups
// of at most GMAX slots.  LDS arrays: cnt, E + 1 ints (the counts, then each expert's first
// place in srt; bucket E takes the ids out of range, which join no group); srt, TS ints (the
// valid slots, by expert); grp, 3 ints per group {expert, first place in srt, slots}, at most
// TS groups; scan, 2 ints per wave.  Every thread of the workgroup (NT threads) calls it; the
// group count is left in *ngroups (readable on return), and srt is complete after the next
// barrier: the function's own last one with SYNC, else the caller's.
template <int NT, int GMAX, bool SYNC = true>
__device__ __forceinline__ void group_slots(const int32_t* __restrict__ ids, int E, int TS, int* cnt, int* srt,
                                            int* grp, int* scan, int* ngroups) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: an SGPR
  for (int e = tid; e <= E; e += NT) cnt[e] = 0;
  __syncthreads();
  constexpr int SPT = (kIdMaxSlots + NT - 1) / NT;
  int key[SPT], pos[SPT];
#pragma unroll
  for (int k = 0; k < SPT; k++) {
    const int i = tid + k * NT;
    key[k] = E;
    pos[k] = 0;
    if (i < TS) {
      const int e = ids[i];
      key[k] = e >= 0 && e < E ? e : E;
      pos[k] = atomicAdd(&cnt[key[k]], 1);
    }
  }
  __syncthreads();
  // exclusive scans over e = 0..E of the slot counts and of the group counts; thread t owns
  // entries [t * per, (t + 1) * per)
  const int per = (E + 1 + NT - 1) / NT;
  const int e0 = min(E + 1, tid * per), e1 = min(E + 1, e0 + per);
  int ls = 0, lg = 0;
  for (int e = e0; e < e1; e++) {
    const int c = cnt[e];
    ls += c;
    lg += e < E ? (c + GMAX - 1) / GMAX : 0;
  }
  int is = ls, ig = lg;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(is, o, 64), v = __shfl_up(ig, o, 64);
    if (lane >= o) {
      is += u;
      ig += v;
    }
  }
  if (lane == 63) {
    scan[2 * wave] = is;
    scan[2 * wave + 1] = ig;
  }
  __syncthreads();
  int s0 = is - ls, g0 = ig - lg;
  for (int w = 0; w < wave; w++) {
    s0 += scan[2 * w];
    g0 += scan[2 * w + 1];
  }
  for (int e = e0; e < e1; e++) {
    const int c = cnt[e];
    cnt[e] = s0;
    if (e < E)
      for (int j = 0; j < c; j += GMAX) {
        grp[3 * g0] = e;
        grp[3 * g0 + 1] = s0 + j;
        grp[3 * g0 + 2] = min(GMAX, c - j);
        g0++;
      }
    s0 += c;
  }
  if (tid == NT - 1) *ngroups = g0;  // the last thread's range ends at E + 1: g0 is the total
  __syncthreads();
  // each slot at the place its counting atomic returned (an order that differs between
  // workgroups), then at its rank by index within its run
#pragma unroll
  for (int k = 0; k < SPT; k++) {
    const int i = tid + k * NT;
    if (i < TS && key[k] < E) srt[cnt[key[k]] + pos[k]] = i;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < SPT; k++) {
    const int i = tid + k * NT;
    if (i < TS && key[k] < E) {
      const int q0 = cnt[key[k]], q1 = cnt[key[k] + 1];
      int r = q0;
      for (int q = q0; q < q1; q++) r += srt[q] < i;
      pos[k] = r;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < SPT; k++) {
    const int i = tid + k * NT;
    if (i < TS && key[k] < E) srt[pos[k]] = i;
  }
  if constexpr (SYNC) __syncthreads();
}

}  // namespace bqm
