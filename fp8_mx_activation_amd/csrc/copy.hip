// mxq_copy16: a plain 16-byte-vector device copy, the bandwidth reference
// the path's kernels are compared with (it moves bytes the way they do:
// 16-byte loads, several in flight per lane, then 16-byte stores, each
// optionally non-temporal).
#include "mxq_device.hpp"
#include "mxq_host.hpp"

namespace {

using namespace mxq;

constexpr int kCopyUnroll = 4;  // 16-byte loads in flight per lane

template <bool NT_STORE, bool NT_LOAD>
__global__ __launch_bounds__(256) void copy16_kernel(
    const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i0 = (int64_t)blockIdx.x * blockDim.x * kCopyUnroll +
                    threadIdx.x;
       i0 < n; i0 += stride * kCopyUnroll) {
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = i0 + (int64_t)u * blockDim.x;
      const u32x4* p = src + (i < n ? i : n - 1);  // clamped: no branch
      v[u] = NT_LOAD ? load16_nt(p) : *p;
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = i0 + (int64_t)u * blockDim.x;
      if (i < n) {
        if (NT_STORE)
          store16_nt(dst + i, v[u]);
        else
          dst[i] = v[u];
      }
    }
  }
}

}  // namespace

extern "C" mxq_status mxq_copy16(const void* src, void* dst, int64_t bytes,
                                 int32_t nontemporal, void* stream) {
  if (bytes < 0 || bytes % 16 != 0 || nontemporal < 0 || nontemporal > 3)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (bytes == 0) return MXQ_OK;
  if (src == nullptr || dst == nullptr || !aligned16(src) || !aligned16(dst))
    return MXQ_ERR_INVALID_ARGUMENT;
  const int64_t n = bytes / 16;
  int64_t blocks = ceil_div(n, 256 * kCopyUnroll);
  if (blocks > 8192) blocks = 8192;
  hipStream_t s = as_stream(stream);
  const u32x4* a = static_cast<const u32x4*>(src);
  u32x4* b = static_cast<u32x4*>(dst);
  const unsigned g = (unsigned)blocks;
  switch (nontemporal) {
    case 0:
      copy16_kernel<false, false><<<g, 256, 0, s>>>(a, b, n);
      break;
    case 1:
      copy16_kernel<true, false><<<g, 256, 0, s>>>(a, b, n);
      break;
    case 2:
      copy16_kernel<false, true><<<g, 256, 0, s>>>(a, b, n);
      break;
    default:
      copy16_kernel<true, true><<<g, 256, 0, s>>>(a, b, n);
      break;
  }
  return launch_status();
}
