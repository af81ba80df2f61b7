// One-time layout transform between the interchange blocks (scale + codes, 18 or 34 bytes,
// only 2-byte aligned) and the packed layout read by the products (16-byte aligned code
// section + separate scale section; see bqm_internal.h).  Weights are re-laid out once for
// the unit that runs them, as the offline interleaved repack does for CPUs on the page
// "ik_llama.cpp 老工作站多 GPU 部署 Qwen3-235B-A22B 实战指南" (nxmr.cn), section on -rtr.
// The code bytes keep their order, so no arithmetic is involved: both directions are
// byte-exact and one thread moves one block.
#include "bqm_internal.h"

namespace bqm {
namespace {

constexpr int kThreads = 256;

template <int CB>  // code bytes per block: 16 (Q4_0) or 32 (Q8_0)
__global__ __launch_bounds__(kThreads) void k_repack(const uint16_t* __restrict__ src,
                                                     uint32_t* __restrict__ codes,
                                                     uint16_t* __restrict__ scales,
                                                     int64_t nblocks, uint8_t* __restrict__ pad0,
                                                     int pad0_n, uint8_t* __restrict__ pad1,
                                                     int pad1_n) {
  constexpr int HW = 1 + CB / 2;  // halfwords per interchange block
  const int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x;
  if (i < pad0_n) pad0[i] = 0;
  if (i < pad1_n) pad1[i] = 0;
  if (i >= nblocks) return;
  const uint16_t* b = src + i * HW;
  scales[i] = b[0];
  uint32_t* c = codes + i * (CB / 4);
#pragma unroll
  for (int k = 0; k < CB / 4; k++) c[k] = (uint32_t)b[1 + 2 * k] | ((uint32_t)b[2 + 2 * k] << 16);
}

template <int CB>
__global__ __launch_bounds__(kThreads) void k_unpack(const uint32_t* __restrict__ codes,
                                                     const uint16_t* __restrict__ scales,
                                                     uint16_t* __restrict__ dst, int64_t nblocks) {
  constexpr int HW = 1 + CB / 2;
  const int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x;
  if (i >= nblocks) return;
  uint16_t* b = dst + i * HW;
  b[0] = scales[i];
  const uint32_t* c = codes + i * (CB / 4);
#pragma unroll
  for (int k = 0; k < CB / 4; k++) {
    const uint32_t v = c[k];
    b[1 + 2 * k] = (uint16_t)(v & 0xffffu);
    b[2 + 2 * k] = (uint16_t)(v >> 16);
  }
}

}  // namespace

int launch_repack(int fmt, const void* src, void* dst, int64_t rows, int64_t K, hipStream_t s) {
  Layout L;
  layout_of(fmt, rows, K, &L);
  const int64_t nblocks = rows * L.nb;
  uint8_t* base = static_cast<uint8_t*>(dst);
  uint8_t* pad0 = base + L.codes_bytes;
  const int pad0_n = (int)(L.scales_off - L.codes_bytes);
  uint8_t* pad1 = base + L.scales_off + nblocks * 2;
  const int pad1_n = (int)(L.total - (L.scales_off + nblocks * 2));
  // one thread per block, and enough threads for each padding run (the run after the
  // scales can exceed 256 bytes: up to 255 of alignment plus the 16-byte slack)
  int64_t work = nblocks;
  work = work > pad0_n ? work : pad0_n;
  work = work > pad1_n ? work : pad1_n;
  const int64_t grid = (work + kThreads - 1) / kThreads;
  uint32_t* codes = reinterpret_cast<uint32_t*>(base);
  uint16_t* scales = reinterpret_cast<uint16_t*>(base + L.scales_off);
  const uint16_t* in = static_cast<const uint16_t*>(src);
  if (fmt == BQM_Q4_0)
    hipLaunchKernelGGL(k_repack<16>, dim3((unsigned)grid), dim3(kThreads), 0, s, in, codes, scales,
                       nblocks, pad0, pad0_n, pad1, pad1_n);
  else
    hipLaunchKernelGGL(k_repack<32>, dim3((unsigned)grid), dim3(kThreads), 0, s, in, codes, scales,
                       nblocks, pad0, pad0_n, pad1, pad1_n);
  return launch_status();
}

int launch_unpack(int fmt, const void* src, void* dst, int64_t rows, int64_t K, hipStream_t s) {
  Layout L;
  layout_of(fmt, rows, K, &L);
  const int64_t nblocks = rows * L.nb;
  if (nblocks == 0) return BQM_OK;
  const uint8_t* base = static_cast<const uint8_t*>(src);
  const uint32_t* codes = reinterpret_cast<const uint32_t*>(base);
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(base + L.scales_off);
  uint16_t* out = static_cast<uint16_t*>(dst);
  const int64_t grid = (nblocks + kThreads - 1) / kThreads;
  if (fmt == BQM_Q4_0)
    hipLaunchKernelGGL(k_unpack<16>, dim3((unsigned)grid), dim3(kThreads), 0, s, codes, scales,
                       out, nblocks);
  else
    hipLaunchKernelGGL(k_unpack<32>, dim3((unsigned)grid), dim3(kThreads), 0, s, codes, scales,
                       out, nblocks);
  return launch_status();
}

}  // namespace bqm
