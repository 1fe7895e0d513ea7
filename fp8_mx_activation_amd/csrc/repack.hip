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
// The copies of large slabs launch blocks per (expert, range of slab rows);
// a block deals its rows' 16-byte vectors to its threads and issues a round
// of loads before the stores.  Small slabs with at most 64 experts use a
// fixed grid that deals (real row, chunk) units to wavefronts instead.  All
// grids depend only on host arguments, so every call can be captured in a
// hipGraph.
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

// One row per thread and pass: each row's expert is a binary search over the
// starts in LDS, a chain of dependent LDS reads, so rows are spread over as
// many threads as possible (at most kPsumBlocks blocks of kPsumThreads).
// Measured on MI355X: 3968 rows over 32 experts 2.6 us, 80000 rows over 256
// experts 3.0 us, against 3.9 and 5.0 us with 1024-thread blocks of four
// rows per thread.
constexpr int kPsumThreads = 256;
constexpr int64_t kPsumBlocks = 1024;

__global__ __launch_bounds__(kPsumThreads) void m_indices_from_psum_kernel(
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

// Small slabs (at most 4M 16-byte vectors) with at most 64 experts take the
// unit kernels below, whose grid holds at most kSmallBlocks blocks, fewer
// when the slab holds fewer units.
constexpr int kUnitVec = 256;  // 16-byte vectors per unit of work
constexpr int kUnitPerLane = kUnitVec / 64;
constexpr int kSmallBlocks = 256;
constexpr int kSmallThreads = 256;
constexpr int kSmallExperts = 64;  // one per lane of a wavefront

inline bool use_small_copy(int32_t E, int32_t max_m, int64_t vec_per_row) {
  const int64_t v = vec_per_row > 0 ? vec_per_row : 1;
  return E <= kSmallExperts && (int64_t)E * max_m * v <= ((int64_t)4 << 20);
}

inline unsigned small_blocks(int32_t E, int32_t max_m, int64_t vec_per_row) {
  const int64_t upr = vec_per_row > 0 ? ceil_div(vec_per_row, kUnitVec) : 1;
  int64_t b = ceil_div((int64_t)E * max_m * upr, kSmallThreads / 64);
  if (b > kSmallBlocks) b = kSmallBlocks;
  return (unsigned)(b < 1 ? 1 : b);
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

// Small slabs with at most 64 experts: a fixed grid that does not grow with
// E * max_m.  Lane e of every wavefront holds expert e's row range
// (start_e, clipped count c_e) and the inclusive prefix of the counts, so
// real row i (in expert order) belongs to expert e = #{prefix <= i}, one
// ballot.  Work comes in units of (real row, chunk of kUnitVec 16-byte
// vectors); unit u goes to wavefront u mod W of the W in the grid, numbered
// across blocks first so that consecutive units land on different CUs.  A
// wavefront issues the kUnitVec / 64 loads of a unit before its stores.

struct LaneRange {
  int64_t start;  // first source (expanded) row of expert `lane`
  int c;          // clipped row count of expert `lane` (0 past E)
  int incl;       // inclusive prefix of c over experts <= lane
};

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

// Expert and position of real row i: returns e and sets j (row within e).
__device__ __forceinline__ int row_owner(const LaneRange& r, int E, int i,
                                         int& j) {
  const int lane = threadIdx.x & 63;
  const int e = __popcll(__ballot(lane < E && r.incl <= i));
  j = i - (__builtin_amdgcn_readlane(r.incl, e) -
           __builtin_amdgcn_readlane(r.c, e));
  return e;
}

__global__ __launch_bounds__(kSmallThreads) void expand_to_slab_small_kernel(
    const uint8_t* __restrict__ x, int64_t ld_x, int64_t src_rows,
    int64_t row_bytes, const uint8_t* __restrict__ xs, int64_t xs_rs,
    int64_t xs_cs, int32_t s_cols, int32_t s_elem,
    const int32_t* __restrict__ psum, int32_t E, int32_t align, int32_t max_m,
    uint8_t* __restrict__ slab, int64_t ld_slab, uint8_t* __restrict__ ss,
    int64_t ss_rs, int64_t ss_cs, int32_t* __restrict__ masked_m,
    int32_t* __restrict__ flags) {
  const int lane = threadIdx.x & 63;
  const int el = min(lane, E - 1);
  const int64_t p_cur = psum[el];
  const int64_t p_prev = el == 0 ? 0 : (int64_t)psum[el - 1];
  const int64_t pp = p_prev < 0 ? 0 : p_prev;
  LaneRange r;
  r.start = (pp + align - 1) / align * align;
  int64_t c = p_cur - r.start;
  c = c > 0 ? c : 0;
  int f = 0;
  if (c > max_m) { f |= 1; c = max_m; }
  if (r.start + c > src_rows) {
    f |= 2;
    c = src_rows > r.start ? src_rows - r.start : 0;
  }
  if (lane >= E) { c = 0; f = 0; }
  r.c = (int)c;
  r.incl = wave_incl_scan(r.c);
  if (blockIdx.x == 0 && threadIdx.x < 64) {  // one writer of the outputs
    if (lane < E) masked_m[lane] = r.c;
    const bool any1 = __ballot(f & 1) != 0, any2 = __ballot(f & 2) != 0;
    if (lane == 0) *flags = (any1 ? 1 : 0) | (any2 ? 2 : 0);
  }
  const int total = __builtin_amdgcn_readlane(r.incl, 63);
  const int nvec = (int)(row_bytes / 16);
  // at least one unit per row: the first unit of a row also copies its
  // scales (rows of zero bytes still have them)
  const int upr = nvec > 0 ? (nvec + kUnitVec - 1) / kUnitVec : 1;
  const int64_t units = (int64_t)total * upr;
  const int64_t W = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t gw = (int64_t)(threadIdx.x >> 6) * gridDim.x + blockIdx.x;
  for (int64_t u = gw; u < units; u += W) {
    const int i = (int)(u / upr);
    const int k = (int)(u - (int64_t)i * upr);
    int j;
    const int e = row_owner(r, E, i, j);
    const int64_t st = ((int64_t)__builtin_amdgcn_readlane(
                            (int)(r.start >> 32), e) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)r.start, e);
    const int64_t src_row = st + j;
    const int64_t dst_row = (int64_t)e * max_m + j;
    const uint8_t* src = x + src_row * ld_x;
    uint8_t* dst = slab + dst_row * ld_slab;
    if (nvec > 0) {
      u32x4 v[kUnitPerLane];
#pragma unroll
      for (int w = 0; w < kUnitPerLane; ++w) {
        const int vi = k * kUnitVec + w * 64 + lane;
        // index clamped to the row's last vector: every load is issued
        v[w] = load16(src + (int64_t)min(vi, nvec - 1) * 16);
      }
#pragma unroll
      for (int w = 0; w < kUnitPerLane; ++w) {
        const int vi = k * kUnitVec + w * 64 + lane;
        if (vi < nvec) store16(dst + (int64_t)vi * 16, v[w]);
      }
    }
    if (k == 0 && xs != nullptr) {
      for (int g = lane; g < s_cols; g += 64) {
        const uint8_t* sp = xs + src_row * xs_rs + g * xs_cs;
        uint8_t* dp = ss + dst_row * ss_rs + g * ss_cs;
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
}

template <bool WEIGHTED>
__global__ __launch_bounds__(kSmallThreads) void slab_to_expand_small_kernel(
    const uint16_t* __restrict__ slab, int64_t ld_slab, int32_t H,
    const int32_t* __restrict__ masked_m, const int32_t* __restrict__ psum,
    int32_t E, int32_t align, int32_t max_m, const float* __restrict__ wts,
    uint16_t* __restrict__ out, int64_t ld_out, int64_t out_rows) {
  const int lane = threadIdx.x & 63;
  const int el = min(lane, E - 1);
  const int64_t p_prev = el == 0 ? 0 : (int64_t)psum[el - 1];
  int64_t c = masked_m[el];
  const int64_t pp = p_prev < 0 ? 0 : p_prev;
  LaneRange r;
  r.start = (pp + align - 1) / align * align;
  if (c > max_m) c = max_m;
  if (r.start + c > out_rows) c = out_rows > r.start ? out_rows - r.start : 0;
  if (c < 0 || lane >= E) c = 0;
  r.c = (int)c;
  r.incl = wave_incl_scan(r.c);
  const int total = __builtin_amdgcn_readlane(r.incl, 63);
  const int nvec = H / 8;
  const int upr = (nvec + kUnitVec - 1) / kUnitVec;
  const int64_t units = (int64_t)total * upr;
  const int64_t W = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t gw = (int64_t)(threadIdx.x >> 6) * gridDim.x + blockIdx.x;
  for (int64_t u = gw; u < units; u += W) {
    const int i = (int)(u / upr);
    const int k = (int)(u - (int64_t)i * upr);
    int j;
    const int e = row_owner(r, E, i, j);
    const int64_t st = ((int64_t)__builtin_amdgcn_readlane(
                            (int)(r.start >> 32), e) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)r.start, e);
    const int64_t orow = st + j;
    const uint16_t* src = slab + ((int64_t)e * max_m + j) * ld_slab;
    uint16_t* dst = out + orow * ld_out;
    const float wv = WEIGHTED ? wts[orow] : 1.0f;
    u32x4 v[kUnitPerLane];
#pragma unroll
    for (int w = 0; w < kUnitPerLane; ++w) {
      const int vi = k * kUnitVec + w * 64 + lane;
      v[w] = load16(src + (int64_t)min(vi, nvec - 1) * 8);
    }
#pragma unroll
    for (int w = 0; w < kUnitPerLane; ++w) {
      const int vi = k * kUnitVec + w * 64 + lane;
      if (vi >= nvec) continue;
      u32x4 o = v[w];
      if (WEIGHTED) {
        o.x = scale_bf16x2(o.x, wv);
        o.y = scale_bf16x2(o.y, wv);
        o.z = scale_bf16x2(o.z, wv);
        o.w = scale_bf16x2(o.w, wv);
      }
      store16(dst + (int64_t)vi * 8, o);
    }
  }
}

// One block per token.  Lane j of every wavefront loads destination j (K <= 64)
// in one vector load; a token without a valid destination ends there, so its
// row is never read.  The row passes through LDS in chunks of at most
// kRowsChunk bytes: the block loads a chunk (one 16-byte vector per thread
// and pass), then wavefront j writes it to destination j with streaming
// stores, 1 KB per instruction.  Lane g keeps scale entry g (g < 64) from
// the start; a writing wavefront copies the entries through their strides.
// Measured on MI355X with the 8192 x 7168 prefill rows (56 UE8M0 bytes each,
// graph-timed): 32 of 256 experts local, 19.6 us against 22.3 us for the
// layout before (one 448-thread block per token whose every thread stored
// its vector to each destination, rows of tokens without a destination
// read as well); all 256 local, 90.8 against 91.1 us.  Wavefronts of
// 1024-thread blocks fetching future tokens' rows cut the all-local call
// from 110 to 101 us with the MALL flushed, but took the 32-expert slice to
// 31 us; one wavefront of the 512-thread block doing it was within noise.
constexpr int kRowsThreads = 512;
constexpr int64_t kRowsChunk = 32768;

__device__ __forceinline__ uint32_t load_entry(const uint8_t* p, int elem) {
  uint32_t w = 0;
  if (elem == 4)
    __builtin_memcpy(&w, p, 4);
  else
    w = *p;
  return w;
}

__global__ __launch_bounds__(kRowsThreads) void scatter_rows_kernel(
    const uint8_t* __restrict__ x, int64_t ld_x, int64_t row_bytes,
    const uint8_t* __restrict__ xs, int64_t xs_rs, int64_t xs_cs,
    int32_t s_cols, int32_t s_elem, const int32_t* __restrict__ src2dst,
    int32_t K, int64_t num_rows, uint8_t* __restrict__ out, int64_t ld_out,
    uint8_t* __restrict__ os, int64_t os_rs, int64_t os_cs) {
  extern __shared__ __align__(16) uint8_t chunk[];
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int32_t d_lane = src2dst[t * K + min(lane, K - 1)];
  const bool valid = lane < K && d_lane >= 0 && (int64_t)d_lane < num_rows;
  if (__ballot(valid) == 0) return;  // the same in every wavefront
  const uint8_t* xsr = xs != nullptr ? xs + t * xs_rs : nullptr;
  const uint32_t s_own =
      (xsr != nullptr && lane < s_cols)
          ? load_entry(xsr + (int64_t)lane * xs_cs, s_elem)
          : 0;
  const uint8_t* src = x + t * ld_x;
  for (int64_t c0 = 0; c0 < row_bytes; c0 += kRowsChunk) {
    const int nv = (int)(min(row_bytes - c0, kRowsChunk) / 16);
    for (int v = threadIdx.x; v < nv; v += kRowsThreads)
      *reinterpret_cast<u32x4*>(chunk + v * 16) = load16(src + c0 + v * 16);
    __syncthreads();
    for (int j = wave; j < K; j += kRowsThreads / 64) {
      const int64_t d = __builtin_amdgcn_readlane(d_lane, j);
      if (d < 0 || d >= num_rows) continue;
      uint8_t* o = out + d * ld_out + c0;
      for (int v = lane; v < nv; v += 64)
        store16_nt(o + v * 16, *reinterpret_cast<const u32x4*>(chunk + v * 16));
    }
    __syncthreads();
  }
  if (xsr == nullptr) return;
  for (int j = wave; j < K; j += kRowsThreads / 64) {
    const int64_t d = __builtin_amdgcn_readlane(d_lane, j);
    if (d < 0 || d >= num_rows) continue;
    for (int g = lane; g < s_cols; g += 64) {
      const uint32_t w =
          g < 64 ? s_own : load_entry(xsr + (int64_t)g * xs_cs, s_elem);
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
  const size_t lds = (size_t)(row_bytes < kRowsChunk ? row_bytes : kRowsChunk);
  scatter_rows_kernel<<<(unsigned)T, kRowsThreads, lds, as_stream(stream)>>>(
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
  int64_t blocks = ceil_div(num_rows, kPsumThreads);
  if (blocks > kPsumBlocks) blocks = kPsumBlocks;
  m_indices_from_psum_kernel<<<(unsigned)blocks, kPsumThreads,
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
  if (use_small_copy(E, max_m, row_bytes / 16)) {
    expand_to_slab_small_kernel<<<small_blocks(E, max_m, row_bytes / 16),
                                  kSmallThreads, 0, as_stream(stream)>>>(
        static_cast<const uint8_t*>(x), ld_x, src_rows, row_bytes,
        static_cast<const uint8_t*>(x_scales), xs_row_stride, xs_col_stride,
        scale_cols, scale_elem_bytes, psum, E, align, max_m,
        static_cast<uint8_t*>(slab), ld_slab,
        static_cast<uint8_t*>(slab_scales), ss_row_stride, ss_col_stride,
        masked_m, flags);
    return launch_status();
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
  const uint16_t* sl = static_cast<const uint16_t*>(slab_bf16);
  uint16_t* o = static_cast<uint16_t*>(out_bf16);
  if (use_small_copy(E, max_m, H / 8)) {
    const unsigned blocks = small_blocks(E, max_m, H / 8);
    if (weights != nullptr)
      slab_to_expand_small_kernel<true><<<blocks, kSmallThreads, 0,
                                          as_stream(stream)>>>(
          sl, ld_slab, H, masked_m, psum, E, align, max_m, weights, o, ld_out,
          out_rows);
    else
      slab_to_expand_small_kernel<false><<<blocks, kSmallThreads, 0,
                                           as_stream(stream)>>>(
          sl, ld_slab, H, masked_m, psum, E, align, max_m, nullptr, o, ld_out,
          out_rows);
    return launch_status();
  }
  const CopyShape cs = copy_shape(E, max_m, H / 8);
  const int64_t rpb = cs.rows_per_block;
  const int64_t blocks = (int64_t)E * ceil_div(max_m, rpb);
  if (blocks > INT32_MAX || rpb * (H / 8) > (int64_t)INT32_MAX / 2)
    return MXQ_ERR_UNSUPPORTED;
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
