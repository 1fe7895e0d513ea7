// Repack between a dispatcher's expanded (psum) layout and the masked slab.
//
// The expanded layout is the one the DeepEPv2 page describes (key source
// snippets, _build_layout): expert e owns rows [start_e, psum[e]) with
// start_e = align(psum[e-1]) and psum[-1] = 0.  Three operations from that
// page (implementation breakdown item 3; review highlights):
//   moe_m_indices_from_psum    m_indices of the contiguous GEMM, with the
//                              tail of every range masked to -1;
//   moe_expand_to_masked_slab  expanded rows (and their scales, copied by
//                              explicit source strides) -> [E, max_m] slab
//                              plus masked_m; over-capacity experts raise a
//                              flag instead of being truncated silently;
//   moe_masked_slab_to_expand  slab -> expanded rows with the top-k weight
//                              applied on real rows only;
//   moe_scatter_rows           the prefill path: a dispatcher's quantized
//                              rows and scales written into the contiguous
//                              layout (psum offsets) by src2dst.
// The copies launch blocks per (expert, range of slab rows); a block deals
// its rows' 16-byte vectors to its threads and issues a round of loads
// before the stores.  All grids depend only on host arguments, so every call
// can be captured in a hipGraph.
#include "mxq_device.hpp"
#include "mxq_host.hpp"

namespace {

using namespace mxq;

__device__ __forceinline__ int64_t psum_start(const int32_t* psum, int e,
                                              int32_t align) {
  int64_t prev = e == 0 ? 0 : (int64_t)psum[e - 1];
  if (prev < 0) prev = 0;
  return (prev + align - 1) / align * align;
}

__device__ __forceinline__ int64_t psum_count(const int32_t* psum, int e,
                                              int32_t align) {
  const int64_t c = (int64_t)psum[e] - psum_start(psum, e, align);
  return c > 0 ? c : 0;
}

__global__ __launch_bounds__(1024) void m_indices_from_psum_kernel(
    const int32_t* __restrict__ psum, int32_t E, int32_t align,
    int64_t num_rows, int32_t* __restrict__ m_indices) {
  extern __shared__ int64_t rng[];  // [E] starts, [E] ends
  int64_t* st = rng;
  int64_t* en = rng + E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    st[e] = psum_start(psum, e, align);
    en[e] = st[e] + psum_count(psum, e, align);
  }
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
       r < num_rows; r += stride) {
    int32_t v = -1;
    if (r >= st[0]) {
      int lo = 0, hi = E - 1;  // largest e with start_e <= r
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (st[mid] <= r) lo = mid; else hi = mid - 1;
      }
      if (r < en[lo]) v = lo;
    }
    m_indices[r] = v;
  }
}

constexpr int kCopyThreads = 1024;
constexpr int kVecPerThread = 8;  // 16-byte loads in flight per thread

// Launch shape of the copy kernels, from host arguments only.  The grid has
// a block for every (expert, range of slab rows), most of them empty when
// few rows are live, so:
//   slabs of more than 4M 16-byte vectors: 1024-thread blocks of about 3584
//   vectors (3.5 per thread, one round of loads);
//   smaller (decode-sized) slabs: 256-thread blocks of about 1024 vectors,
//   so the blocks of rows that do not exist launch fewer wavefronts;
// and at most 1024 blocks per expert.  Measured on MI355X with 7168-wide
// rows: 32 experts x 2048 slab rows, 50282 live, expand 129.8 us and
// slab-to-expand 248.4 us (144.9 and 293.1 us with 1024-thread blocks of
// 32 rows); 32 x 128 slab rows, 140 live, 6.4 and 7.7 us (6.5 and 9.2 us
// with 1024-thread blocks of 8 rows).
struct CopyShape {
  int64_t rows_per_block;
  int threads;
};

inline CopyShape copy_shape(int32_t E, int32_t max_m, int64_t vec_per_row) {
  const int64_t v = vec_per_row > 0 ? vec_per_row : 1;
  const bool small = (int64_t)E * max_m * v <= ((int64_t)4 << 20);
  const int threads = small ? 256 : kCopyThreads;
  int64_t rpb = (small ? 1024 : 3584) / v;
  const int64_t floor_rows = ceil_div(max_m, 1024);
  if (rpb < floor_rows) rpb = floor_rows;
  if (rpb < 1) rpb = 1;
  return {rpb, threads};
}

// Block (e, b) copies rows [b*rpb, (b+1)*rpb) of expert e's slab, limited to
// the rows that exist.  The rows' 16-byte vectors are numbered and dealt
// round-robin to the threads; each thread issues up to kVecPerThread loads
// before its stores, so a block of the sizes copy_shape picks costs about
// one memory round trip.
// Block 0 also writes masked_m and the flags for every expert.
__global__ __launch_bounds__(kCopyThreads) void expand_to_slab_kernel(
    const uint8_t* __restrict__ x, int64_t ld_x, int64_t src_rows,
    int64_t row_bytes, const uint8_t* __restrict__ xs, int64_t xs_rs,
    int64_t xs_cs, int32_t s_cols, int32_t s_elem,
    const int32_t* __restrict__ psum, int32_t E, int32_t align, int32_t max_m,
    int32_t rpb, uint8_t* __restrict__ slab, int64_t ld_slab,
    uint8_t* __restrict__ ss, int64_t ss_rs, int64_t ss_cs,
    int32_t* __restrict__ masked_m, int32_t* __restrict__ flags) {
  const int nb = (max_m + rpb - 1) / rpb;
  const int e = blockIdx.x / nb;
  const int b = blockIdx.x % nb;
  if (blockIdx.x == 0) {  // one writer for masked_m and the flags word
    int f = 0;
    for (int ee = threadIdx.x; ee < E; ee += blockDim.x) {
      const int64_t s2 = psum_start(psum, ee, align);
      int64_t c2 = psum_count(psum, ee, align);
      if (c2 > max_m) { f |= 1; c2 = max_m; }
      if (s2 + c2 > src_rows) {
        f |= 2;
        c2 = src_rows > s2 ? src_rows - s2 : 0;
      }
      masked_m[ee] = (int32_t)c2;
    }
    const int any1 = __syncthreads_or(f & 1);
    const int any2 = __syncthreads_or(f & 2);
    if (threadIdx.x == 0) *flags = (any1 ? 1 : 0) | (any2 ? 2 : 0);
  }
  const int64_t s = psum_start(psum, e, align);
  int64_t c = psum_count(psum, e, align);
  if (c > max_m) c = max_m;
  if (s + c > src_rows) c = src_rows > s ? src_rows - s : 0;
  const int64_t j0 = (int64_t)b * rpb;
  const int64_t nrows = min(j0 + rpb, c) - j0;
  if (nrows <= 0) return;
  // a block's items fit in 32 bits (checked on the host)
  const uint32_t nvec = (uint32_t)(row_bytes / 16);
  const uint32_t items = (uint32_t)nrows * nvec;
  const uint32_t per_round = blockDim.x * kVecPerThread;
  const uint8_t* src0 = x + (s + j0) * ld_x;
  uint8_t* dst0 = slab + ((int64_t)e * max_m + j0) * ld_slab;
  // loads use an index clamped into range (no branch), so every load of a
  // round is issued before the first wait; only the stores are guarded
  for (uint32_t base = 0; base < items; base += per_round) {
    u32x4 v[kVecPerThread];
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      const uint32_t i = min(base + u * blockDim.x + threadIdx.x, items - 1);
      v[u] = load16(src0 + (int64_t)(i / nvec) * ld_x + (i % nvec) * 16);
    }
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      const uint32_t i = base + u * blockDim.x + threadIdx.x;
      if (i < items)
        store16(dst0 + (int64_t)(i / nvec) * ld_slab + (i % nvec) * 16, v[u]);
    }
  }
  if (xs != nullptr && s_cols > 0) {
    const uint32_t sitems = (uint32_t)nrows * (uint32_t)s_cols;
    for (uint32_t i = threadIdx.x; i < sitems; i += blockDim.x) {
      const int64_t j = j0 + i / (uint32_t)s_cols;
      const int64_t g = i % (uint32_t)s_cols;
      const uint8_t* sp = xs + (s + j) * xs_rs + g * xs_cs;
      uint8_t* dp = ss + ((int64_t)e * max_m + j) * ss_rs + g * ss_cs;
      if (s_elem == 4) {
        uint32_t w;
        __builtin_memcpy(&w, sp, 4);
        __builtin_memcpy(dp, &w, 4);
      } else {
        *dp = *sp;
      }
    }
  }
}

__device__ __forceinline__ uint32_t scale_bf16x2(uint32_t v, float w) {
  const float a = __uint_as_float(v << 16) * w;
  const float b = __uint_as_float(v & 0xFFFF0000u) * w;
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

// Block (e, b) writes expanded rows start_e + j for j in [b*rpb,
// (b+1)*rpb), j < min(masked_m[e], max_m) and start_e + j < out_rows, from
// slab row e*max_m + j, times w[start_e + j] when weighted; loads issued a
// round at a time as in expand_to_slab_kernel.
template <bool WEIGHTED>
__global__ __launch_bounds__(kCopyThreads) void slab_to_expand_kernel(
    const uint16_t* __restrict__ slab, int64_t ld_slab, int32_t H,
    const int32_t* __restrict__ masked_m, const int32_t* __restrict__ psum,
    int32_t align, int32_t max_m, int32_t rpb, const float* __restrict__ w,
    uint16_t* __restrict__ out, int64_t ld_out, int64_t out_rows) {
  const int nb = (max_m + rpb - 1) / rpb;
  const int e = blockIdx.x / nb;
  const int b = blockIdx.x % nb;
  const int64_t s = psum_start(psum, e, align);
  int64_t c = masked_m[e];
  if (c > max_m) c = max_m;
  if (s + c > out_rows) c = out_rows > s ? out_rows - s : 0;
  const int64_t j0 = (int64_t)b * rpb;
  const int64_t nrows = min(j0 + rpb, c) - j0;
  if (nrows <= 0) return;
  // a block's items fit in 32 bits (checked on the host)
  const uint32_t nvec = (uint32_t)H / 8;
  const uint32_t items = (uint32_t)nrows * nvec;
  const uint32_t per_round = blockDim.x * kVecPerThread;
  const uint16_t* src0 = slab + ((int64_t)e * max_m + j0) * ld_slab;
  uint16_t* dst0 = out + (s + j0) * ld_out;
  for (uint32_t base = 0; base < items; base += per_round) {
    u32x4 v[kVecPerThread];
    float wv[kVecPerThread];
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      const uint32_t i = min(base + u * blockDim.x + threadIdx.x, items - 1);
      v[u] = load16(src0 + (int64_t)(i / nvec) * ld_slab + (i % nvec) * 8);
      wv[u] = WEIGHTED ? w[s + j0 + i / nvec] : 1.0f;
    }
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      const uint32_t i = base + u * blockDim.x + threadIdx.x;
      if (i < items) {
        u32x4 o = v[u];
        if (WEIGHTED) {
          o.x = scale_bf16x2(o.x, wv[u]);
          o.y = scale_bf16x2(o.y, wv[u]);
          o.z = scale_bf16x2(o.z, wv[u]);
          o.w = scale_bf16x2(o.w, wv[u]);
        }
        store16(dst0 + (int64_t)(i / nvec) * ld_out + (i % nvec) * 8, o);
      }
    }
  }
}

// One block per token: each thread loads its 16-byte vectors of the row once
// and stores them to every destination of the token (streaming stores);
// scale entries are copied through their strides.
__global__ __launch_bounds__(1024) void scatter_rows_kernel(
    const uint8_t* __restrict__ x, int64_t ld_x, int64_t row_bytes,
    const uint8_t* __restrict__ xs, int64_t xs_rs, int64_t xs_cs,
    int32_t s_cols, int32_t s_elem, const int32_t* __restrict__ src2dst,
    int32_t K, int64_t num_rows, uint8_t* __restrict__ out, int64_t ld_out,
    uint8_t* __restrict__ os, int64_t os_rs, int64_t os_cs) {
  const int64_t t = blockIdx.x;
  const int32_t* dl = src2dst + t * K;
  const uint8_t* src = x + t * ld_x;
  const int64_t nvec = row_bytes / 16;
  for (int64_t v = threadIdx.x; v < nvec; v += blockDim.x) {
    const u32x4 val = load16(src + v * 16);
    for (int j = 0; j < K; ++j) {
      const int64_t d = dl[j];
      if (d >= 0 && d < num_rows) store16_nt(out + d * ld_out + v * 16, val);
    }
  }
  if (xs == nullptr) return;
  for (int g = threadIdx.x; g < s_cols; g += blockDim.x) {
    const uint8_t* sp = xs + t * xs_rs + (int64_t)g * xs_cs;
    uint32_t w = 0;
    if (s_elem == 4)
      __builtin_memcpy(&w, sp, 4);
    else
      w = *sp;
    for (int j = 0; j < K; ++j) {
      const int64_t d = dl[j];
      if (d < 0 || d >= num_rows) continue;
      uint8_t* dp = os + d * os_rs + (int64_t)g * os_cs;
      if (s_elem == 4)
        __builtin_memcpy(dp, &w, 4);
      else
        *dp = (uint8_t)w;
    }
  }
}

}  // namespace

extern "C" mxq_status moe_scatter_rows(
    const void* x, int64_t ld_x, int64_t T, int64_t row_bytes,
    const void* x_scales, int64_t xs_row_stride, int64_t xs_col_stride,
    int32_t scale_cols, int32_t scale_elem_bytes, const int32_t* src2dst,
    int32_t K, int64_t num_rows, void* out, int64_t ld_out, void* out_scales,
    int64_t os_row_stride, int64_t os_col_stride, void* stream) {
  if (T < 0 || T > INT32_MAX || K < 0 || K > MXQ_MAX_TOPK || row_bytes < 0 ||
      num_rows < 0)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (row_bytes % 16 != 0) return MXQ_ERR_UNSUPPORTED;
  if (T == 0 || K == 0 || num_rows == 0) return MXQ_OK;
  if (x == nullptr || src2dst == nullptr || out == nullptr)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || ld_x % 16 != 0 || ld_x < row_bytes ||
      !aligned16(out) || ld_out % 16 != 0 || ld_out < row_bytes)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (x_scales != nullptr) {
    if (out_scales == nullptr || scale_cols < 0 ||
        (scale_elem_bytes != 1 && scale_elem_bytes != 4))
      return MXQ_ERR_INVALID_ARGUMENT;
    if (scale_elem_bytes == 4 &&
        (((reinterpret_cast<uintptr_t>(x_scales) |
           reinterpret_cast<uintptr_t>(out_scales)) & 3) != 0 ||
         (xs_row_stride | xs_col_stride | os_row_stride | os_col_stride) % 4))
      return MXQ_ERR_INVALID_ARGUMENT;
  }
  const int threads = row_block_threads(row_bytes > 0 ? row_bytes : 16, 16);
  scatter_rows_kernel<<<(unsigned)T, threads, 0, as_stream(stream)>>>(
      static_cast<const uint8_t*>(x), ld_x, row_bytes,
      static_cast<const uint8_t*>(x_scales), xs_row_stride, xs_col_stride,
      scale_cols, scale_elem_bytes, src2dst, K, num_rows,
      static_cast<uint8_t*>(out), ld_out, static_cast<uint8_t*>(out_scales),
      os_row_stride, os_col_stride);
  return launch_status();
}

extern "C" mxq_status moe_m_indices_from_psum(const int32_t* psum, int32_t E,
                                              int32_t align, int64_t num_rows,
                                              int32_t* m_indices,
                                              void* stream) {
  if (E < 1 || E > MXQ_MAX_LOCAL_EXPERTS || align < 1 || num_rows < 0 ||
      num_rows > INT32_MAX)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (num_rows == 0) return MXQ_OK;
  if (psum == nullptr || m_indices == nullptr) return MXQ_ERR_INVALID_ARGUMENT;
  int64_t blocks = ceil_div(num_rows, 1024 * 4);
  if (blocks > 256) blocks = 256;
  m_indices_from_psum_kernel<<<(unsigned)blocks, 1024,
                               (size_t)2 * E * sizeof(int64_t),
                               as_stream(stream)>>>(psum, E, align, num_rows,
                                                    m_indices);
  return launch_status();
}

extern "C" mxq_status moe_expand_to_masked_slab(
    const void* x, int64_t ld_x, int64_t src_rows, int64_t row_bytes,
    const void* x_scales, int64_t xs_row_stride, int64_t xs_col_stride,
    int32_t scale_cols, int32_t scale_elem_bytes, const int32_t* psum,
    int32_t E, int32_t align, int32_t max_m, void* slab, int64_t ld_slab,
    void* slab_scales, int64_t ss_row_stride, int64_t ss_col_stride,
    int32_t* masked_m, int32_t* flags, void* stream) {
  if (E < 1 || E > MXQ_MAX_LOCAL_EXPERTS || align < 1 || max_m < 1 ||
      src_rows < 0 || row_bytes < 0)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (row_bytes % 16 != 0) return MXQ_ERR_UNSUPPORTED;
  if (psum == nullptr || masked_m == nullptr || flags == nullptr ||
      slab == nullptr)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (src_rows > 0 && x == nullptr) return MXQ_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || ld_x % 16 != 0 || ld_x < row_bytes ||
      !aligned16(slab) || ld_slab % 16 != 0 || ld_slab < row_bytes)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (x_scales != nullptr) {
    if (slab_scales == nullptr || scale_cols < 0 ||
        (scale_elem_bytes != 1 && scale_elem_bytes != 4))
      return MXQ_ERR_INVALID_ARGUMENT;
    if (scale_elem_bytes == 4 &&
        (((reinterpret_cast<uintptr_t>(x_scales) |
           reinterpret_cast<uintptr_t>(slab_scales)) & 3) != 0 ||
         (xs_row_stride | xs_col_stride | ss_row_stride | ss_col_stride) % 4))
      return MXQ_ERR_INVALID_ARGUMENT;
  }
  const CopyShape cs = copy_shape(E, max_m, row_bytes / 16);
  const int64_t rpb = cs.rows_per_block;
  const int64_t blocks = (int64_t)E * ceil_div(max_m, rpb);
  if (blocks > INT32_MAX ||
      rpb * (row_bytes / 16 + scale_cols) > (int64_t)INT32_MAX / 2)
    return MXQ_ERR_UNSUPPORTED;
  expand_to_slab_kernel<<<(unsigned)blocks, cs.threads, 0,
                          as_stream(stream)>>>(
      static_cast<const uint8_t*>(x), ld_x, src_rows, row_bytes,
      static_cast<const uint8_t*>(x_scales), xs_row_stride, xs_col_stride,
      scale_cols, scale_elem_bytes, psum, E, align, max_m, (int32_t)rpb,
      static_cast<uint8_t*>(slab), ld_slab, static_cast<uint8_t*>(slab_scales),
      ss_row_stride, ss_col_stride, masked_m, flags);
  return launch_status();
}

extern "C" mxq_status moe_masked_slab_to_expand(
    const void* slab_bf16, int64_t ld_slab, int32_t H, const int32_t* masked_m,
    const int32_t* psum, int32_t E, int32_t align, int32_t max_m,
    const float* weights, void* out_bf16, int64_t ld_out, int64_t out_rows,
    void* stream) {
  if (E < 1 || E > MXQ_MAX_LOCAL_EXPERTS || align < 1 || max_m < 1 ||
      H <= 0 || H % 8 != 0 || out_rows < 0)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (out_rows == 0) return MXQ_OK;
  if (slab_bf16 == nullptr || masked_m == nullptr || psum == nullptr ||
      out_bf16 == nullptr)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (!aligned16(slab_bf16) || (ld_slab * 2) % 16 != 0 || ld_slab < H ||
      !aligned16(out_bf16) || (ld_out * 2) % 16 != 0 || ld_out < H)
    return MXQ_ERR_INVALID_ARGUMENT;
  const CopyShape cs = copy_shape(E, max_m, H / 8);
  const int64_t rpb = cs.rows_per_block;
  const int64_t blocks = (int64_t)E * ceil_div(max_m, rpb);
  if (blocks > INT32_MAX || rpb * (H / 8) > (int64_t)INT32_MAX / 2)
    return MXQ_ERR_UNSUPPORTED;
  const uint16_t* sl = static_cast<const uint16_t*>(slab_bf16);
  uint16_t* o = static_cast<uint16_t*>(out_bf16);
  if (weights != nullptr)
    slab_to_expand_kernel<true><<<(unsigned)blocks, cs.threads, 0,
                                  as_stream(stream)>>>(
        sl, ld_slab, H, masked_m, psum, align, max_m, (int32_t)rpb, weights,
        o, ld_out, out_rows);
  else
    slab_to_expand_kernel<false><<<(unsigned)blocks, cs.threads, 0,
                                   as_stream(stream)>>>(
        sl, ld_slab, H, masked_m, psum, align, max_m, (int32_t)rpb, nullptr,
        o, ld_out, out_rows);
  return launch_status();
}
