// Device code shared by the layout kernels: moe_layout's assign kernel and
// the fused decode dispatch (moe_layout_scatter_quant).
#pragma once

#include "mxq_device.hpp"

namespace mxq {

// Region starts from each expert's total (thread e < E holds total_e), a
// block-wide scan of the padded sizes into off[0..E]; block 0 also
// publishes counts, region starts, masked_m and the overflow flag.
__device__ __forceinline__ void region_scan(
    int total, int32_t E, int32_t kind, int32_t block_e, int32_t cap,
    int32_t* off, int32_t* wsum, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ masked_m,
    int32_t* __restrict__ overflow) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  int padded = 0;
  if (tid < E)
    padded = kind == 0 ? (total + block_e - 1) / block_e * block_e : cap;
  int incl = padded;
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int before = 0, grand = 0;
  const int nwaves = blockDim.x >> 6;
  for (int w = 0; w < nwaves; ++w) {
    before += (w < wv) ? wsum[w] : 0;
    grand += wsum[w];
  }
  if (tid < E) off[tid] = before + incl - padded;
  if (tid == 0) off[E] = grand;
  if (blockIdx.x == 0) {
    if (tid < E) {
      counts[tid] = total;
      offsets[tid] = before + incl - padded;
      if (masked_m != nullptr)
        masked_m[tid] = kind == 1 ? min(total, cap) : total;
    }
    if (tid == 0) offsets[E] = grand;
    const int ovf = (tid < E && kind == 1 && total > cap) ? 1 : 0;
    const int any = __syncthreads_or(ovf);
    if (tid == 0) *overflow = any ? 1 : 0;
  }
}

}  // namespace mxq
