// Bandwidth references the path's kernels are compared with (not steps of
// the method):
//   mxq_copy16        a plain 16-byte-vector device copy (16-byte loads,
//                     several in flight per lane, then 16-byte stores, each
//                     optionally non-temporal);
//   mxq_gather_read16 the combine's reads alone: block g reads the rows its
//                     `group` indices name, a lane 16 bytes of each with all
//                     of a group's loads in flight (non-temporal), and writes
//                     only the XOR of what it read;
//   mxq_fill_rows16   the combine's writes alone: one block per row, 16-byte
//                     streaming stores of a 32-bit pattern.
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

// XOR of v over the block (blockDim.x a multiple of 64, at most 1024).
__device__ __forceinline__ uint32_t block_xor(uint32_t v, uint32_t* red) {
  for (int d = 32; d >= 1; d >>= 1) v ^= (uint32_t)__shfl_xor((int)v, d);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t x = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) x ^= red[w];
  return x;
}

__global__ __launch_bounds__(1024) void gather_read16_kernel(
    const uint8_t* __restrict__ rows, int64_t ld, int64_t num_rows,
    const int32_t* __restrict__ idx, int32_t group, int64_t row_bytes,
    uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[16];
  const int64_t g = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int32_t d_lane = idx[g * group + min(lane, group - 1)];
  uint32_t acc = 0;
  for (int64_t c = (int64_t)threadIdx.x * 16; c < row_bytes;
       c += (int64_t)blockDim.x * 16) {
    for (int j0 = 0; j0 < group; j0 += 8) {
      u32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u;
        const int64_t d =
            j < group ? (int64_t)__builtin_amdgcn_readlane(d_lane, j) : -1;
        v[u] = (d >= 0 && d < num_rows) ? load16_nt(rows + d * ld + c)
                                        : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
  const uint32_t x = block_xor(acc, red);
  if (threadIdx.x == 0) sink[g] = x;
}

__global__ __launch_bounds__(1024) void fill_rows16_kernel(
    uint8_t* __restrict__ dst, int64_t ld, int64_t row_bytes,
    uint32_t pattern) {
  uint8_t* r = dst + (int64_t)blockIdx.x * ld;
  const u32x4 v{pattern, pattern, pattern, pattern};
  for (int64_t c = (int64_t)threadIdx.x * 16; c < row_bytes;
       c += (int64_t)blockDim.x * 16)
    store16_nt(r + c, v);
}

}  // namespace

extern "C" mxq_status mxq_gather_read16(const void* rows, int64_t ld,
                                        int64_t num_rows, const int32_t* idx,
                                        int64_t groups, int32_t group,
                                        int64_t row_bytes, uint32_t* sink,
                                        void* stream) {
  if (groups < 0 || groups > INT32_MAX || group < 1 || group > 64 ||
      row_bytes < 0 || row_bytes % 16 != 0 || num_rows < 0 || ld < row_bytes ||
      ld % 16 != 0)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (groups == 0) return MXQ_OK;
  if (idx == nullptr || sink == nullptr ||
      (num_rows > 0 && row_bytes > 0 && (rows == nullptr || !aligned16(rows))))
    return MXQ_ERR_INVALID_ARGUMENT;
  const int threads = row_block_threads(row_bytes > 0 ? row_bytes : 16, 16);
  gather_read16_kernel<<<(unsigned)groups, threads, 0, as_stream(stream)>>>(
      static_cast<const uint8_t*>(rows), ld, num_rows, idx, group, row_bytes,
      sink);
  return launch_status();
}

extern "C" mxq_status mxq_fill_rows16(void* dst, int64_t ld, int64_t rows,
                                      int64_t row_bytes, uint32_t pattern,
                                      void* stream) {
  if (rows < 0 || rows > INT32_MAX || row_bytes < 0 || row_bytes % 16 != 0 ||
      ld < row_bytes || ld % 16 != 0)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (rows == 0 || row_bytes == 0) return MXQ_OK;
  if (dst == nullptr || !aligned16(dst)) return MXQ_ERR_INVALID_ARGUMENT;
  const int threads = row_block_threads(row_bytes, 16);
  fill_rows16_kernel<<<(unsigned)rows, threads, 0, as_stream(stream)>>>(
      static_cast<uint8_t*>(dst), ld, row_bytes, pattern);
  return launch_status();
}

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
