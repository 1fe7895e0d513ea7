// moe_layout: top-k routing -> expert-grouped layout (compact or masked slab).
//
// What is computed follows the standard-dispatch compact layout of sglang
// PR #33128 (implementation breakdown items 2-3: block-aligned per-expert
// regions, -1 expert index on padding rows, static row bound) and the masked
// slab of sglang PR #29525 (implementation breakdown items 2-3: [E, max_m]
// slots with masked_m, overflow fails fast).  Slots inside an expert follow
// ascending flat assignment index t*K + j.
//
// Two launches whose grids depend only on T, K, E and num_rows; one launch
// when T*K <= 4096 (one block per token for up to 2048 tokens,
// layout_token_kernel; otherwise the assign kernel alone, every block
// ranking the whole routing) or when T*K <= 2^14 with at most 256 experts
// (the assign kernel alone, every block counting the whole routing into LDS
// in place of the histogram launch):
//   layout_hist_kernel    one block per chunk of assignments: LDS histogram
//                         of the chunk's local experts -> cnt[chunk][E].
//   layout_assign_kernel  one block of 16 wavefronts per chunk, plus enough
//                         blocks for the m_indices fill:
//     A  every block sums the chunk counts it needs (the totals c_e and the
//        counts of earlier chunks), with a batch of loads in flight;
//     B  a block-wide scan of the padded sizes gives the region starts;
//        block 0 publishes counts, region starts, masked_m and the flag;
//     C  each wavefront ranks its own steps of 64 assignments: lanes with the
//        same expert are found with one ballot per key bit (a bit-sliced
//        multi-split) and a lane's rank among them is the popcount of the
//        matching lower lanes.  Per-wavefront expert counts are then
//        prefix-summed across the block, so slots follow flat order without
//        atomics and without a serial walk over the chunk.
//     D  rows are mapped to experts through an LDS table with one entry per
//        block_e rows (regions start on multiples of block_e), or a binary
//        search over the region starts when that table would not fit in the
//        LDS left over (63 KB per block in all).
#include <mutex>

#include "layout_device.hpp"
#include "mxq_host.hpp"

// Per-chunk expert counts of moe_layout_noalloc: a static device array in
// place of the caller's workspace.  Each device holds its own copy at its
// own address; host code uses that address (looked up once per device with
// hipGetSymbolAddress), never this name.
static __device__ __align__(256) int32_t
    scratch[MXQ_LAYOUT_NOALLOC_SCRATCH_BYTES / sizeof(int32_t)];

namespace {

using namespace mxq;

constexpr int kScanBatch = 16;
constexpr int kAssignWaves = 16;
constexpr int kMaxStepsPerWave = kChunkMax / (64 * kAssignWaves);
constexpr int kAssignLds = 64512;  // dynamic LDS bytes of the assign kernel

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi(
      (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__global__ __launch_bounds__(256) void layout_hist_kernel(
    const int32_t* __restrict__ ids, int64_t A, int32_t begin, int32_t E,
    int32_t chunk, int32_t* __restrict__ cnt) {
  extern __shared__ int32_t hist[];
  for (int i = threadIdx.x; i < E; i += 256) hist[i] = 0;
  __syncthreads();
  const int64_t a0 = (int64_t)blockIdx.x * chunk;
  const int64_t a1 = min(a0 + (int64_t)chunk, A);
  for (int64_t a = a0 + threadIdx.x; a < a1; a += 256) {
    const int64_t e = (int64_t)ids[a] - begin;
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += 256)
    cnt[(int64_t)blockIdx.x * E + i] = hist[i];
}

// Slots: one block of kAssignWaves wavefronts per chunk.  Each wavefront
// owns a contiguous run of whole 64-assignment steps; it ranks its lanes
// within each step (ballot multi-split) and among its own earlier steps, and
// publishes its per-expert counts to LDS.  After a barrier the counts are
// prefix-summed over the wavefronts, so a lane's slot is
// chunk base + count of the same expert in earlier wavefronts + its rank in
// its wavefront: flat order, no atomics, no serial chain across wavefronts.
//
// MODE kFromChunks: the totals and this chunk's first slots come from the
// histogram launch's per-chunk counts.
// MODE kSingle: all assignments form one chunk (T*K <= kSingleMax) and no
// histogram pass runs.  Every block ranks that chunk (C1), takes the totals
// from the per-wavefront counts (C2) and then scans the regions (B); block 0
// alone writes src2dst.
// MODE kInBlock: no histogram launch either; every block counts the whole
// routing itself (A'), wavefront w adding each local id of its share to its
// private LDS count of ids before the block's chunk or from it on.
enum AssignMode { kFromChunks = 0, kSingle = 1, kInBlock = 2 };

template <int MODE>
__global__ __launch_bounds__(1024) void layout_assign_kernel(
    const int32_t* __restrict__ ids, int64_t A, int32_t begin, int32_t E,
    int32_t nbits, int32_t kind, int32_t block_e, int32_t cap,
    int64_t num_rows, int32_t chunk, int32_t nc, int32_t steps_per_wave,
    int32_t tbl_cap, const int32_t* __restrict__ chunk_cnt,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ masked_m, int32_t* __restrict__ overflow,
    int32_t* __restrict__ m_indices, int32_t* __restrict__ src2dst) {
  extern __shared__ int32_t sm[];
  __shared__ int32_t wsum[16];
  int32_t* tot = sm;                   // [E]
  int32_t* off = sm + E;               // [E + 1]
  int32_t* cbase = sm + 2 * E + 1;     // [E] first slot of this chunk
  int32_t* tbl = sm + 3 * E + 1;       // [tbl_cap] expert per block_e rows
  // [kAssignWaves][E] per-wavefront counts, then their prefixes (< chunk)
  uint16_t* cnt = reinterpret_cast<uint16_t*>(tbl + tbl_cap);
  // phase A's partial sums live in the row-table space, which is only used
  // in phase D (tbl_cap >= 2048 for every E)
  int32_t* part_all = tbl;         // [nparts][E], nparts * E <= 1024
  int32_t* part_pre = tbl + 1024;  // [nparts][E]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  constexpr bool SINGLE = MODE == kSingle;
  const int c = SINGLE ? 0 : (int)blockIdx.x;
  const bool has_chunk = c < nc;
  const bool writer = SINGLE ? blockIdx.x == 0 : has_chunk;
  const int64_t c_begin = (int64_t)c * chunk;
  const int64_t c_end = has_chunk ? min(c_begin + (int64_t)chunk, A) : c_begin;
  const int64_t w_begin = c_begin + (int64_t)wv * steps_per_wave * 64;
  const int64_t w_end = min(w_begin + (int64_t)steps_per_wave * 64, c_end);

  // this wavefront's ids, fetched before anything waits.  Each load reads
  // an index clamped to the wavefront's last assignment (no branch, so all
  // are in flight together; steps past the end re-read a line already
  // fetched); which entries count is decided where they are used.
  int32_t idb[kMaxStepsPerWave];
  if (A > 0) {
    const int64_t a_last = w_end > w_begin ? w_end - 1 : A - 1;
#pragma unroll
    for (int st = 0; st < kMaxStepsPerWave; ++st)
      idb[st] = ids[min(w_begin + st * 64 + lane, a_last)];
  } else {
#pragma unroll
    for (int st = 0; st < kMaxStepsPerWave; ++st) idb[st] = 0;
  }

  // A': totals and this chunk's first slots counted here.  Wavefront w takes
  // a contiguous share of the ids, 64 * kScanBatch at a time (indices
  // clamped so that a batch's loads are in flight together), and adds each
  // local one to its private count: hist[0][w] for ids before this block's
  // chunk, hist[1][w] for the others.  The counts live in the row-table
  // space, which is only used in phase D (the host checks that 2 * 16 * E
  // entries fit).
  if constexpr (MODE == kInBlock) {
    int32_t* hist = tbl;  // [2][kAssignWaves][E]
    for (int i = tid; i < 2 * kAssignWaves * E; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    const int64_t per = (A + 64 * kAssignWaves - 1) / (64 * kAssignWaves) * 64;
    const int64_t a0 = (int64_t)wv * per;
    const int64_t a1 = min(A, a0 + per);
    int32_t* h_lo = hist + wv * E;
    int32_t* h_hi = hist + (kAssignWaves + wv) * E;
    for (int64_t ab = a0; ab < a1; ab += 64 * kScanBatch) {
      int32_t v[kScanBatch];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u)
        v[u] = ids[min(ab + u * 64 + lane, a1 - 1)];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) {
        const int64_t a = ab + u * 64 + lane;
        const int64_t e = (int64_t)v[u] - begin;
        if (a < a1 && e >= 0 && e < E)
          atomicAdd((a < c_begin ? h_lo : h_hi) + e, 1);
      }
    }
    __syncthreads();
    int total = 0, first = 0;
    if (tid < E) {
#pragma unroll 4
      for (int w = 0; w < kAssignWaves; ++w) {
        const int lo = hist[w * E + tid];
        total += lo + hist[(kAssignWaves + w) * E + tid];
        first += lo;
      }
      tot[tid] = total;
      cbase[tid] = first;
    }
    region_scan(total, E, kind, block_e, cap, off, wsum, counts, offsets,
                masked_m, overflow);
  }

  // A: totals and this chunk's first slots from the chunk counts.  Up to
  // four groups of threads per expert split the chunks; each issues its
  // loads a batch at a time.
  if constexpr (MODE == kFromChunks) {
    const int er = (E + 63) / 64 * 64;
    const int nparts = max(1, (int)blockDim.x / er);
    const int part = tid / er;
    const int e = tid - part * er;
    if (part < nparts && e < E) {
      const int per = (nc + nparts - 1) / nparts;
      const int c_lo = part * per;
      const int c_hi = min(nc, c_lo + per);
      int all = 0, pre = 0;
      for (int cb0 = c_lo; cb0 < c_hi; cb0 += kScanBatch) {
        int v[kScanBatch];
#pragma unroll
        for (int i = 0; i < kScanBatch; ++i)
          v[i] = chunk_cnt[(int64_t)min(cb0 + i, c_hi - 1) * E + e];
#pragma unroll
        for (int i = 0; i < kScanBatch; ++i) {
          const int cc = cb0 + i;
          if (cc < c_hi) {
            all += v[i];
            pre += cc < c ? v[i] : 0;
          }
        }
      }
      part_all[part * E + e] = all;
      part_pre[part * E + e] = pre;
    }
    __syncthreads();
    int total = 0, first = 0;
    if (tid < E) {
      for (int p = 0; p < nparts; ++p) {
        total += part_all[p * E + tid];
        first += part_pre[p * E + tid];
      }
      tot[tid] = total;
      cbase[tid] = first;
    }
    region_scan(total, E, kind, block_e, cap, off, wsum, counts, offsets,
                masked_m, overflow);
  }
  __syncthreads();
  for (int i = tid; i < kAssignWaves * E; i += blockDim.x) cnt[i] = 0;
  __syncthreads();

  // C1: ranks inside the wavefront
  int key[kMaxStepsPerWave];
  int rank[kMaxStepsPerWave];
  if (has_chunk) {
    uint16_t* cw = cnt + wv * E;
#pragma unroll
    for (int st = 0; st < kMaxStepsPerWave; ++st) {
      key[st] = -1;
      rank[st] = 0;
      if (st >= steps_per_wave || w_begin + st * 64 >= w_end) continue;
      const int64_t a = w_begin + st * 64 + lane;
      const int64_t e64 = a < w_end ? (int64_t)idb[st] - begin : -1;
      const bool local = e64 >= 0 && e64 < E;
      const int ke = local ? (int)e64 : 0;
      uint64_t m = __ballot(local);
      for (int bit = 0; bit < nbits; ++bit) {
        const bool set = (ke >> bit) & 1;
        const uint64_t bb = __ballot(local && set);
        m &= set ? bb : ~bb;
      }
      const int r = lanes_below(m);
      int prev = 0;
      if (local) prev = cw[ke];
      // every lane has read cw[ke] (same instruction) before the lowest lane
      // of each expert advances it
      if (local && r == 0) cw[ke] = (uint16_t)(prev + (int)__popcll(m));
      key[st] = local ? ke : -1;
      rank[st] = prev + r;
    }
  }
  __syncthreads();
  // C2: exclusive prefix of the per-wavefront counts (within the chunk)
  if (has_chunk) {
    for (int e = tid; e < E; e += blockDim.x) {
      int run = 0;
#pragma unroll
      for (int w = 0; w < kAssignWaves; ++w) {
        const int v = cnt[w * E + e];
        cnt[w * E + e] = (uint16_t)run;
        run += v;
      }
      if (SINGLE) {
        tot[e] = run;
        cbase[e] = 0;
      }
    }
  } else if (SINGLE) {
    for (int e = tid; e < E; e += blockDim.x) {
      tot[e] = 0;
      cbase[e] = 0;
    }
  }
  if constexpr (SINGLE) {
    __syncthreads();
    region_scan(tid < E ? tot[tid] : 0, E, kind, block_e, cap, off, wsum,
                counts, offsets, masked_m, overflow);
  }
  __syncthreads();
  // C3: destinations
  if (has_chunk && writer) {
#pragma unroll
    for (int st = 0; st < kMaxStepsPerWave; ++st) {
      if (st >= steps_per_wave) break;
      const int64_t a = w_begin + st * 64 + lane;
      if (a >= w_end) break;
      const int e = key[st];
      int32_t dst = -1;
      if (e >= 0) {
        const int slot = cbase[e] + (int)cnt[wv * E + e] + rank[st];
        if (kind == 0)
          dst = off[e] + slot;
        else
          dst = slot < cap ? e * cap + slot : -1;
      }
      src2dst[a] = dst;
    }
  }

  // D: m_indices
  if (m_indices == nullptr) return;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t r_first = (int64_t)blockIdx.x * blockDim.x + tid;
  if (kind == 1) {
    for (int64_t r = r_first; r < num_rows; r += stride) {
      const int64_t e = r / cap;
      int32_t v = -1;
      if (e < E && r - e * cap < min(tot[e], cap)) v = (int32_t)e;
      m_indices[r] = v;
    }
    return;
  }
  const int32_t used = off[E];
  const int32_t nblk = (used + block_e - 1) / block_e;
  const bool use_tbl = nblk <= tbl_cap;
  if (use_tbl) {
    for (int i = tid; i < nblk; i += blockDim.x) {
      const int32_t r = i * block_e;
      int lo = 0, hi = E - 1;  // largest e with off[e] <= r
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= r) lo = mid; else hi = mid - 1;
      }
      tbl[i] = lo;
    }
  }
  __syncthreads();
  for (int64_t r = r_first; r < num_rows; r += stride) {
    int32_t v = -1;
    if (r < used) {
      int e;
      if (use_tbl) {
        e = tbl[(int32_t)r / block_e];
      } else {
        int lo = 0, hi = E - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (off[mid] <= r) lo = mid; else hi = mid - 1;
        }
        e = lo;
      }
      if (r - off[e] < tot[e]) v = e;
    }
    m_indices[r] = v;
  }
}

// Decode-sized routings (at most kSingleMax assignments over at most
// kTokenMaxTokens tokens): one block per token.  Every block loads the whole
// routing (at most 4096 ids, from L2 after the first blocks) and its own
// token's ids, counts in LDS each local expert's total and its assignments
// in earlier tokens, scans the regions (block 0 publishes counts, region
// starts, masked_m and the flag), and gives its own assignments their slots:
//   slot(t, j) = #{assignments of e before token t} + #{j' < j with e},
// the ascending flat-order slot.  All blocks share the m_indices fill.  No
// ranking and no serial phase over the routing: measured on MI355X
// (graph-timed, against the single-block slot kernel): 128 tokens x 8
// over 32 masked experts 4.1 against 6.2 us, over 256 compact experts 4.8
// against 7.4 us; 512 x 8 4.6-4.9 against 8.3-9.2 us; 1024 x 4 5.4 against
// 10.1 us; 2048 x 2 7.5 against 10.1 us; but 4096 x 1 12.4 against 8.9 us,
// where 4096 blocks each count the whole routing.  Each thread loads PER ids,
// the power of two that covers the routing with NT threads (loads past the
// routing would only repeat its last id): with 512 threads up to 512 tokens
// (the block scan needs at least E threads, 512 up to 512 experts) and 256
// above, 128 x 8 over 32 masked experts took 3.6 against 4.15 us with 256
// threads of 16 loads, over 256 compact experts 4.2 against 4.85 us, 512 x 8
// 4.3 against 4.8 us; at 2048 x 2, 512 threads took 8.9 against 7.6 us.
template <int NT, int PER>
__global__ __launch_bounds__(NT) void layout_token_kernel(
    const int32_t* __restrict__ ids, int32_t K, int32_t A, int32_t begin,
    int32_t E, int32_t kind, int32_t block_e, int32_t cap, int64_t num_rows,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ m_indices, int32_t* __restrict__ masked_m,
    int32_t* __restrict__ src2dst, int32_t* __restrict__ overflow) {
  extern __shared__ int32_t sm[];
  __shared__ int32_t wsum[16];
  __shared__ int32_t tok_e[MXQ_MAX_TOPK];  // local expert of (t, j), or -1
  int32_t* all = sm;          // [E] totals
  int32_t* before = sm + E;   // [E] assignments of earlier tokens
  int32_t* off = sm + 2 * E;  // [E + 1] region starts
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  const int a0 = (int)t * K;
  constexpr int kPer = PER;
  // every id and this token's own ids, all in flight together (indices
  // clamped, no branch)
  int idv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) idv[i] = ids[min(tid + NT * i, A - 1)];
  const int own = ids[a0 + min(tid, K - 1)];
  for (int e = tid; e < E; e += NT) {
    all[e] = 0;
    before[e] = 0;
  }
  if (tid < K) {
    const int e = own - begin;
    tok_e[tid] = (e >= 0 && e < E) ? e : -1;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int a = tid + NT * i;
    const int e = idv[i] - begin;
    if (a < A && e >= 0 && e < E) {
      atomicAdd(&all[e], 1);
      if (a < a0) atomicAdd(&before[e], 1);
    }
  }
  __syncthreads();
  region_scan(tid < E ? all[tid] : 0, E, kind, block_e, cap, off, wsum,
              counts, offsets, masked_m, overflow);
  __syncthreads();
  if (tid < K) {
    const int e = tok_e[tid];
    int32_t d = -1;
    if (e >= 0) {
      int slot = before[e];
      for (int j = 0; j < tid; ++j) slot += tok_e[j] == e ? 1 : 0;
      d = kind == 0 ? off[e] + slot : (slot < cap ? e * cap + slot : -1);
    }
    src2dst[a0 + tid] = d;
  }
  if (m_indices == nullptr) return;
  const int64_t stride = (int64_t)gridDim.x * NT;
  for (int64_t r = (int64_t)blockIdx.x * NT + tid; r < num_rows; r += stride) {
    int32_t v = -1;
    if (kind == 1) {
      const int64_t e = r / cap;
      if (e < E && r - e * cap < min(all[e], cap)) v = (int32_t)e;
    } else if (r < off[E]) {
      int lo = 0, hi = E - 1;  // largest e with off[e] <= r
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= r) lo = mid; else hi = mid - 1;
      }
      if (r - off[lo] < all[lo]) v = lo;
    }
    m_indices[r] = v;
  }
}

}  // namespace

namespace {

// Host checks of moe_layout's arguments other than the workspace.
mxq_status layout_args_ok(const int32_t* topk_ids, int64_t T, int32_t K,
                          int32_t E, mxq_layout_kind kind, int32_t block_e,
                          int32_t capacity, int64_t num_rows,
                          const int32_t* counts, const int32_t* expert_offsets,
                          const int32_t* src2dst,
                          const int32_t* overflow_flag) {
  if (T < 0 || K < 1 || K > MXQ_MAX_TOPK || E < 1 ||
      E > MXQ_MAX_LOCAL_EXPERTS)
    return MXQ_ERR_INVALID_ARGUMENT;
  const int64_t A = T * (int64_t)K;
  if (num_rows < 0 || num_rows > INT32_MAX) return MXQ_ERR_INVALID_ARGUMENT;
  if (A > MXQ_MAX_ASSIGNMENTS) return MXQ_ERR_UNSUPPORTED;
  if (kind == MXQ_LAYOUT_COMPACT) {
    if (block_e < 1) return MXQ_ERR_INVALID_ARGUMENT;
    if (num_rows < moe_compact_row_bound(A, E, block_e))
      return MXQ_ERR_INVALID_ARGUMENT;
  } else if (kind == MXQ_LAYOUT_MASKED) {
    if (capacity < 1 || (int64_t)E * capacity > num_rows)
      return MXQ_ERR_INVALID_ARGUMENT;
  } else {
    return MXQ_ERR_UNSUPPORTED;
  }
  if (counts == nullptr || expert_offsets == nullptr || overflow_flag == nullptr)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (A > 0 && (topk_ids == nullptr || src2dst == nullptr))
    return MXQ_ERR_INVALID_ARGUMENT;
  return MXQ_OK;
}

// The launches of moe_layout once its arguments have been checked;
// chunk_cnt holds at least layout_workspace_bytes(T*K, E) bytes.
mxq_status layout_launch(const int32_t* topk_ids, int64_t T, int32_t K,
                         int32_t expert_begin, int32_t E, mxq_layout_kind kind,
                         int32_t block_e, int32_t capacity, int64_t num_rows,
                         int32_t* counts, int32_t* expert_offsets,
                         int32_t* m_indices, int32_t* masked_m,
                         int32_t* src2dst, int32_t* overflow_flag,
                         int32_t* chunk_cnt, void* stream) {
  const int64_t A = T * (int64_t)K;
  const LayoutGeom g = layout_geom(A);
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  hipStream_t s = as_stream(stream);
  const int32_t cap = kind == MXQ_LAYOUT_MASKED ? capacity : 0;
  if (layout_per_token(A, T, E)) {
    const size_t lds = (size_t)(3 * E + 1) * sizeof(int32_t);
    const int nt = E > 512 ? 1024 : (E > 256 || T <= 512 ? 512 : 256);
    int per = 1;
    while ((int64_t)nt * per < A) per *= 2;  // A <= kSingleMax
    auto launch = [&](auto kernel) {
      kernel<<<(unsigned)T, nt, lds, s>>>(
          topk_ids, K, (int32_t)A, expert_begin, E, (int32_t)kind, block_e,
          cap, num_rows, counts, expert_offsets, m_indices, masked_m, src2dst,
          overflow_flag);
    };
    if (nt == 256) {
      if (per <= 4) launch(layout_token_kernel<256, 4>);
      else if (per == 8) launch(layout_token_kernel<256, 8>);
      else launch(layout_token_kernel<256, 16>);
    } else if (nt == 512) {
      if (per <= 2) launch(layout_token_kernel<512, 2>);
      else if (per == 4) launch(layout_token_kernel<512, 4>);
      else launch(layout_token_kernel<512, 8>);
    } else {
      if (per <= 2) launch(layout_token_kernel<1024, 2>);
      else launch(layout_token_kernel<1024, 4>);
    }
    return launch_status();
  }
  const bool single = A <= kSingleMax;
  const size_t fixed = (size_t)(3 * E + 1) * sizeof(int32_t) +
                       (size_t)kAssignWaves * E * sizeof(uint16_t);
  const int32_t tbl_cap = (int32_t)((kAssignLds - fixed) / sizeof(int32_t));
  const bool in_block = layout_in_block(A, E);
  if (in_block && tbl_cap < 2 * kAssignWaves * E) return MXQ_ERR_UNSUPPORTED;
  if (g.nc > 0 && !single && !in_block) {
    layout_hist_kernel<<<g.nc, 256, (size_t)E * sizeof(int32_t), s>>>(
        topk_ids, A, expert_begin, E, g.chunk, chunk_cnt);
    if (launch_status() != MXQ_OK) return MXQ_ERR_HIP;
  }
  // a single chunk holds every assignment (whole 1024-assignment groups)
  const int32_t chunk = single ? (int32_t)(ceil_div(A > 0 ? A : 1, kChunkMin) *
                                           kChunkMin)
                               : g.chunk;
  const int32_t nc = single ? (A > 0 ? 1 : 0) : g.nc;
  // One block per chunk (at least one: block 0 publishes the per-expert
  // outputs); more blocks (up to 64) if the m_indices fill needs them.
  // Each of the 16 wavefronts of a block takes steps_per_wave steps.
  const int32_t steps_per_wave =
      (int32_t)ceil_div(ceil_div(chunk, 64), kAssignWaves);
  int64_t blocks = nc > 0 ? nc : 1;
  if (m_indices != nullptr) {
    int64_t fill_blocks = ceil_div(num_rows, 4096);
    if (fill_blocks > 64) fill_blocks = 64;
    if (fill_blocks > blocks) blocks = fill_blocks;
  }
  if (single)
    layout_assign_kernel<kSingle><<<(unsigned)blocks, 1024, kAssignLds, s>>>(
        topk_ids, A, expert_begin, E, nbits, (int32_t)kind, block_e, cap,
        num_rows, chunk, nc, steps_per_wave, tbl_cap, nullptr, counts,
        expert_offsets, masked_m, overflow_flag, m_indices, src2dst);
  else if (in_block)
    layout_assign_kernel<kInBlock><<<(unsigned)blocks, 1024, kAssignLds, s>>>(
        topk_ids, A, expert_begin, E, nbits, (int32_t)kind, block_e, cap,
        num_rows, chunk, nc, steps_per_wave, tbl_cap, nullptr, counts,
        expert_offsets, masked_m, overflow_flag, m_indices, src2dst);
  else
    layout_assign_kernel<kFromChunks><<<(unsigned)blocks, 1024, kAssignLds,
                                        s>>>(
        topk_ids, A, expert_begin, E, nbits, (int32_t)kind, block_e, cap,
        num_rows, chunk, nc, steps_per_wave, tbl_cap, chunk_cnt, counts,
        expert_offsets, masked_m, overflow_flag, m_indices, src2dst);
  return launch_status();
}

// Address of this library's scratch array on `dev`, looked up once per
// device with that device current (each device has its own copy).
mxq_status scratch_on_device(int dev, int32_t** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (dev < 0 || dev >= kMaxDevices) return MXQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return MXQ_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return MXQ_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return MXQ_ERR_HIP;
    if (e != hipSuccess || p == nullptr) return MXQ_ERR_HIP;
    addr[dev] = p;
  }
  *out = static_cast<int32_t*>(addr[dev]);
  return MXQ_OK;
}

}  // namespace

extern "C" mxq_status moe_layout(
    const int32_t* topk_ids, int64_t T, int32_t K, int32_t expert_begin,
    int32_t num_local_experts, mxq_layout_kind kind, int32_t block_e,
    int32_t capacity, int64_t num_rows, int32_t* counts,
    int32_t* expert_offsets, int32_t* m_indices, int32_t* masked_m,
    int32_t* src2dst, int32_t* overflow_flag, void* workspace,
    size_t workspace_bytes, void* stream) {
  const int32_t E = num_local_experts;
  const mxq_status st =
      layout_args_ok(topk_ids, T, K, E, kind, block_e, capacity, num_rows,
                     counts, expert_offsets, src2dst, overflow_flag);
  if (st != MXQ_OK) return st;
  const size_t need = layout_workspace_bytes(T * (int64_t)K, E);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return MXQ_ERR_WORKSPACE;
  return layout_launch(topk_ids, T, K, expert_begin, E, kind, block_e,
                       capacity, num_rows, counts, expert_offsets, m_indices,
                       masked_m, src2dst, overflow_flag,
                       static_cast<int32_t*>(workspace), stream);
}

extern "C" mxq_status moe_layout_noalloc(
    const int32_t* topk_ids, int64_t T, int32_t K, int32_t expert_begin,
    int32_t num_local_experts, mxq_layout_kind kind, int32_t block_e,
    int32_t capacity, int64_t num_rows, int32_t* counts,
    int32_t* expert_offsets, int32_t* m_indices, int32_t* masked_m,
    int32_t* src2dst, int32_t* overflow_flag, void* stream) {
  const int32_t E = num_local_experts;
  const mxq_status st =
      layout_args_ok(topk_ids, T, K, E, kind, block_e, capacity, num_rows,
                     counts, expert_offsets, src2dst, overflow_flag);
  if (st != MXQ_OK) return st;
  const size_t need = layout_workspace_bytes(T * (int64_t)K, E);
  if (need > MXQ_LAYOUT_NOALLOC_SCRATCH_BYTES) return MXQ_ERR_SCRATCH_LIMIT;
  int32_t* chunk_cnt = nullptr;
  if (need > 0) {
    // the stream's device (the current one for the null stream)
    int dev = -1;
    hipStream_t s = as_stream(stream);
    if (s == nullptr) {
      if (hipGetDevice(&dev) != hipSuccess) return MXQ_ERR_HIP;
    } else if (hipStreamGetDevice(s, &dev) != hipSuccess) {
      return MXQ_ERR_HIP;
    }
    const mxq_status ss = scratch_on_device(dev, &chunk_cnt);
    if (ss != MXQ_OK) return ss;
  }
  return layout_launch(topk_ids, T, K, expert_begin, E, kind, block_e,
                       capacity, num_rows, counts, expert_offsets, m_indices,
                       masked_m, src2dst, overflow_flag, chunk_cnt, stream);
}
