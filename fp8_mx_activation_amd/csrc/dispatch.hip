// moe_layout_scatter_quant: moe_layout followed by moe_scatter_quant in one
// launch, for routings of at most 4096 assignments (decode batches).
//
// At that size the two calls are dependent launches whose cost is mostly
// latency (the low-latency decode dispatch of sglang PR #14162, and the
// fused quant + scatter of sglang PR #33128, implementation breakdown item
// 3).  Here one block per token does both.  It loads every id of the routing
// (from L2) together with its own token row, and builds in LDS the
// per-expert totals and the counts of assignments that belong to earlier
// tokens.  The slot of assignment (t, j) of local expert e is
//   #{assignments of e in tokens before t} + #{j' < j with expert e},
// the ascending flat-order slot that moe_layout assigns, and the region
// starts come from the same block-wide scan of the padded totals
// (region_scan).  The block then quantizes its row once and writes it to its
// destinations as scatter_quant_kernel does.  Block 0 publishes counts,
// region starts, masked_m and the overflow flag; all blocks share the
// m_indices fill.  Every output equals that of the two calls.
//
// The scan gives one thread to each expert, so a block has at least E
// threads: 512 up to 512 local experts, else 1024.  At 68 VGPRs a 1024-thread
// block is the only one on its CU, while three 512-thread blocks fit; on
// MI355X the 512-thread block took 5.3 us instead of 5.6 us for T=128 top-8
// over 32 experts, and 6.1 us instead of 9.4 us for T=512 top-8.  Each
// thread loads PER ids of the routing, the power of two that covers it
// (loads past the routing would only repeat its last id).
#include "layout_device.hpp"
#include "mxq_host.hpp"

namespace {

using namespace mxq;

constexpr int kFusedMaxAssignments = 4096;

// LDS ints before the staged row: totals [E], earlier counts [E], region
// starts [E + 1], rounded up to 16 bytes.
__host__ __device__ inline int fused_lds_ints(int E) {
  return (3 * E + 1 + 3) & ~3;
}

template <int G, int NT, int PER>
__global__ __launch_bounds__(NT) void layout_scatter_quant_kernel(
    const int32_t* __restrict__ ids, int32_t K, int32_t A, int32_t begin,
    int32_t E, int32_t kind, int32_t block_e, int32_t cap, int64_t num_rows,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ m_indices, int32_t* __restrict__ masked_m,
    int32_t* __restrict__ src2dst, int32_t* __restrict__ overflow,
    const uint16_t* __restrict__ x, int64_t ld_x, int32_t H,
    uint8_t* __restrict__ q, int64_t ld_q, uint8_t* __restrict__ s,
    int64_t ld_s) {
  constexpr int kIdsPerThread = PER;
  extern __shared__ __align__(16) int32_t sm[];
  __shared__ int32_t wsum[16];
  __shared__ int32_t tok_e[MXQ_MAX_TOPK];  // local expert of (t, j), or -1
  __shared__ int32_t dst_l[MXQ_MAX_TOPK];
  int32_t* all = sm;          // [E] totals
  int32_t* before = sm + E;   // [E] assignments of earlier tokens
  int32_t* off = sm + 2 * E;  // [E + 1] region starts
  // [H] fp8 bytes, then [H / G] scale bytes
  uint8_t* row = reinterpret_cast<uint8_t*>(sm + fused_lds_ints(E));
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  const int a0 = (int)t * K;

  // Every load first, all in flight together: the routing's ids (indices
  // clamped, no branch), this token's own ids, and the first 16 channels of
  // the row this lane quantizes (read even if the token turns out to have
  // no local expert).
  int idv[kIdsPerThread];
#pragma unroll
  for (int i = 0; i < kIdsPerThread; ++i)
    idv[i] = ids[min(tid + NT * i, A - 1)];
  const int own = ids[a0 + min(tid, K - 1)];
  const uint16_t* xr = x + t * ld_x;
  const int col0 = tid * 16;
  const int c0 = col0 < H ? col0 : 0;
  const u32x4 xa = load16(xr + c0);
  const u32x4 xb = load16(xr + c0 + 8);

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
  for (int i = 0; i < kIdsPerThread; ++i) {
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

  // destinations of this token's assignments
  if (tid < K) {
    const int e = tok_e[tid];
    int32_t d = -1;
    if (e >= 0) {
      int slot = before[e];
      for (int j = 0; j < tid; ++j) slot += tok_e[j] == e ? 1 : 0;
      if (kind == 0)
        d = off[e] + slot;
      else
        d = slot < cap ? e * cap + slot : -1;
    }
    src2dst[a0 + tid] = d;
    dst_l[tid] = d;
  }

  // m_indices, rows dealt over the whole grid
  if (m_indices != nullptr) {
    const int64_t stride = (int64_t)gridDim.x * NT;
    for (int64_t r = (int64_t)blockIdx.x * NT + tid; r < num_rows;
         r += stride) {
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
  __syncthreads();
  bool any = false;
  for (int j = 0; j < K; ++j) any |= dst_l[j] >= 0;
  if (!any) return;  // block-uniform

  // quantize the row once, stage it in LDS, write it to every destination
  const bool lead = (tid & (G / 16 - 1)) == 0;
  for (int col = col0; col < H; col += NT * 16) {
    u32x4 a = xa, b = xb;
    if (col != col0) {
      a = load16(xr + col);
      b = load16(xr + col + 8);
    }
    int e;
    const u32x4 v = quant16<G>(a, b, e);
    *reinterpret_cast<u32x4*>(row + col) = v;
    if (lead) row[H + col / G] = (uint8_t)(e + 127);
  }
  __syncthreads();
  const int lane = tid & 63;
  const int ng = H / G;
  for (int j = tid >> 6; j < K; j += NT / 64) {
    const int64_t d = dst_l[j];
    if (d < 0) continue;
    uint8_t* qr = q + d * ld_q;
    for (int c = lane * 16; c < H; c += 64 * 16)
      store16_nt(qr + c, *reinterpret_cast<const u32x4*>(row + c));
    for (int g = lane; g < ng; g += 64) s[d * ld_s + g] = row[H + g];
  }
}

}  // namespace

extern "C" mxq_status moe_layout_scatter_quant(
    const int32_t* topk_ids, int64_t T, int32_t K, int32_t expert_begin,
    int32_t num_local_experts, mxq_layout_kind kind, int32_t block_e,
    int32_t capacity, int64_t num_rows, int32_t* counts,
    int32_t* expert_offsets, int32_t* m_indices, int32_t* masked_m,
    int32_t* src2dst, int32_t* overflow_flag, const void* x_bf16,
    int64_t ld_x, int32_t H, mxq_scale_fmt fmt, void* q_fp8, int64_t ld_q,
    uint8_t* scales, int64_t ld_s, void* stream) {
  const int32_t E = num_local_experts;
  const int G = group_of(fmt);
  if (G == 0) return MXQ_ERR_UNSUPPORTED;
  if (T < 0 || K < 1 || K > MXQ_MAX_TOPK || E < 1 ||
      E > MXQ_MAX_LOCAL_EXPERTS || num_rows < 0 || num_rows > INT32_MAX ||
      H <= 0 || H % G != 0)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (H > MXQ_MAX_HIDDEN) return MXQ_ERR_UNSUPPORTED;
  const int64_t A = T * (int64_t)K;
  if (A > kFusedMaxAssignments) return MXQ_ERR_UNSUPPORTED;
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
  if (A == 0)  // no row to quantize: the layout alone (no workspace needed)
    return moe_layout(topk_ids, T, K, expert_begin, E, kind, block_e,
                      capacity, num_rows, counts, expert_offsets, m_indices,
                      masked_m, src2dst, overflow_flag, nullptr, 0, stream);
  if (topk_ids == nullptr || src2dst == nullptr || x_bf16 == nullptr ||
      q_fp8 == nullptr || scales == nullptr)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (ld_x < H || ld_q < H || ld_s < H / G || !aligned16(x_bf16) ||
      (ld_x * 2) % 16 != 0 || !aligned16(q_fp8) || ld_q % 16 != 0)
    return MXQ_ERR_INVALID_ARGUMENT;

  const size_t lds = (size_t)fused_lds_ints(E) * sizeof(int32_t) +
                     (size_t)H + (size_t)(H / G);
  const int32_t cap = kind == MXQ_LAYOUT_MASKED ? capacity : 0;
  hipStream_t s = as_stream(stream);
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  uint8_t* q = static_cast<uint8_t*>(q_fp8);
  auto launch = [&](auto kernel, int nt) {
    kernel<<<(unsigned)T, nt, lds, s>>>(
        topk_ids, K, (int32_t)A, expert_begin, E, (int32_t)kind, block_e, cap,
        num_rows, counts, expert_offsets, m_indices, masked_m, src2dst,
        overflow_flag, x, ld_x, H, q, ld_q, scales, ld_s);
  };
  const int nt = E <= 512 ? 512 : 1024;
  int per = 1;
  while ((int64_t)nt * per < A) per *= 2;  // A <= kFusedMaxAssignments
  if (nt == 512) {
    if (G == 128) {
      if (per <= 2) launch(layout_scatter_quant_kernel<128, 512, 2>, 512);
      else if (per == 4) launch(layout_scatter_quant_kernel<128, 512, 4>, 512);
      else launch(layout_scatter_quant_kernel<128, 512, 8>, 512);
    } else {
      if (per <= 2) launch(layout_scatter_quant_kernel<32, 512, 2>, 512);
      else if (per == 4) launch(layout_scatter_quant_kernel<32, 512, 4>, 512);
      else launch(layout_scatter_quant_kernel<32, 512, 8>, 512);
    }
  } else {
    if (G == 128) {
      if (per <= 2) launch(layout_scatter_quant_kernel<128, 1024, 2>, 1024);
      else launch(layout_scatter_quant_kernel<128, 1024, 4>, 1024);
    } else {
      if (per <= 2) launch(layout_scatter_quant_kernel<32, 1024, 2>, 1024);
      else launch(layout_scatter_quant_kernel<32, 1024, 4>, 1024);
    }
  }
  return launch_status();
}
