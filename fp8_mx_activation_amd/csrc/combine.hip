// moe_combine: expert-output rows -> tokens, weighted by the top-k weights.
//
// The un-permute through src2dst follows sglang PR #33128 (implementation
// breakdown item 2 and risks item 2: post-permute reads the rows the
// scatter wrote, via src2dst); the weights are applied on real rows only, as
// in the fused top-k weighting of sglang PR #29525 (implementation breakdown
// item 3).  Per element: acc = +0, then acc = fma(w_j, y_j, acc) for
// j = 0..K-1 in order, skipping assignments without a row; the result is
// rounded to bf16 (nearest even) or stored as fp32.
//
// One block per token and slice of channels; a lane owns 8 consecutive
// channels.  A slice is the whole row above 192 tokens; with at most 192
// tokens (fewer than the 256 CUs) each token's row is dealt to blocks of
// 1024 channels (128 threads), so that more CUs issue its loads.  Measured
// on MI355X, hidden 7168, top-8, A/B in one process: all 256 experts local
// T = 16 3.1 against 3.9 us, T = 128 3.6 against 4.2-4.4 us, T = 192 4.5
// against 4.7 us, T = 255 6.0 against 5.5 us (so not there); the decode
// slab (T = 128, 32 of 256 local) 3.2 against 3.5 us; T = 8192 178.6 us
// either way.  The token's
// indices and weights arrive in one vector load each (lane j holds entry j),
// and the K rows are then loaded as independent 16-byte vectors before any
// arithmetic, so each lane has up to eight loads in flight.  Per token the
// kernel reads K valid rows of 2H bytes and writes one row.  Every
// expert-output row is read exactly once, so the loads are non-temporal
// (measured on MI355X: the prefill gather took 183 us instead of 196 us with
// plain loads), and the output row is written with streaming (non-temporal)
// stores so it does not displace cached lines.
#include "mxq_device.hpp"
#include "mxq_host.hpp"

namespace {

using namespace mxq;

__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  const uint32_t a = __builtin_bit_cast(uint16_t, (__bf16)lo);
  const uint32_t b = __builtin_bit_cast(uint16_t, (__bf16)hi);
  return a | (b << 16);
}

template <bool F32_OUT>
__global__ __launch_bounds__(1024) void combine_kernel(
    const uint16_t* __restrict__ y, int64_t ld_y, int64_t num_rows,
    const int32_t* __restrict__ src2dst, const float* __restrict__ w,
    int32_t K, int32_t H, int32_t slice, void* __restrict__ out,
    int64_t ld_out) {
  const int64_t t = blockIdx.x;
  const int c_lo = (int)blockIdx.y * slice;
  const int c_hi = min(H, c_lo + slice);
  // lane j of every wavefront loads index and weight j (K <= 64) in one
  // vector load each; readlane then gives them to the whole wavefront, so
  // the row loads wait for one round trip, not one per assignment
  const int lane = threadIdx.x & 63;
  const int jl = min(lane, K - 1);
  const int32_t d_lane = K > 0 ? src2dst[t * K + jl] : -1;
  const int32_t w_lane = K > 0 ? __float_as_int(w[t * K + jl]) : 0;
  for (int col = c_lo + (int)threadIdx.x * 8; col < c_hi;
       col += blockDim.x * 8) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int j0 = 0; j0 < K; j0 += 8) {
      u32x4 v[8];
      float wt[8];
      bool ok[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u;
        const int64_t d =
            j < K ? (int64_t)__builtin_amdgcn_readlane(d_lane, j) : -1;
        ok[u] = d >= 0 && d < num_rows;
        wt[u] = ok[u] ? __int_as_float(__builtin_amdgcn_readlane(w_lane, j))
                      : 0.0f;
        v[u] = ok[u] ? load16_nt(y + d * ld_y + col) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (!ok[u]) continue;
        acc[0] = fmaf(wt[u], bf16_lo(v[u].x), acc[0]);
        acc[1] = fmaf(wt[u], bf16_hi(v[u].x), acc[1]);
        acc[2] = fmaf(wt[u], bf16_lo(v[u].y), acc[2]);
        acc[3] = fmaf(wt[u], bf16_hi(v[u].y), acc[3]);
        acc[4] = fmaf(wt[u], bf16_lo(v[u].z), acc[4]);
        acc[5] = fmaf(wt[u], bf16_hi(v[u].z), acc[5]);
        acc[6] = fmaf(wt[u], bf16_lo(v[u].w), acc[6]);
        acc[7] = fmaf(wt[u], bf16_hi(v[u].w), acc[7]);
      }
    }
    if constexpr (F32_OUT) {
      float* o = static_cast<float*>(out) + t * ld_out + col;
      store16_nt(o, u32x4{__float_as_uint(acc[0]), __float_as_uint(acc[1]),
                          __float_as_uint(acc[2]), __float_as_uint(acc[3])});
      store16_nt(o + 4, u32x4{__float_as_uint(acc[4]), __float_as_uint(acc[5]),
                              __float_as_uint(acc[6]), __float_as_uint(acc[7])});
    } else {
      uint16_t* o = static_cast<uint16_t*>(out) + t * ld_out + col;
      store16_nt(o, u32x4{bf16x2_rne(acc[0], acc[1]), bf16x2_rne(acc[2], acc[3]),
                          bf16x2_rne(acc[4], acc[5]), bf16x2_rne(acc[6], acc[7])});
    }
  }
}

// Up to this many tokens a row is split into slices of kCombineSlice
// channels, one block each.
constexpr int64_t kCombineSliceMaxTokens = 192;
constexpr int32_t kCombineSlice = 1024;

}  // namespace

extern "C" mxq_status moe_combine(const void* y_bf16, int64_t ld_y,
                                  int64_t num_rows, const int32_t* src2dst,
                                  const float* topk_weights, int64_t T,
                                  int32_t K, int32_t H, void* out,
                                  int64_t ld_out, mxq_out_dtype out_dtype,
                                  void* stream) {
  if (out_dtype != MXQ_OUT_BF16 && out_dtype != MXQ_OUT_F32)
    return MXQ_ERR_UNSUPPORTED;
  if (T < 0 || T > INT32_MAX || K < 0 || K > MXQ_MAX_TOPK || H <= 0 ||
      H % 8 != 0 || num_rows < 0 || num_rows > INT32_MAX)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (T == 0) return MXQ_OK;
  if (out == nullptr || ld_out < H) return MXQ_ERR_INVALID_ARGUMENT;
  if (K > 0 && (src2dst == nullptr || topk_weights == nullptr))
    return MXQ_ERR_INVALID_ARGUMENT;
  if (num_rows > 0 && (y_bf16 == nullptr || ld_y < H || !aligned16(y_bf16) ||
                       (ld_y * 2) % 16 != 0))
    return MXQ_ERR_INVALID_ARGUMENT;
  const int64_t esz = out_dtype == MXQ_OUT_F32 ? 4 : 2;
  if (!aligned16(out) || (ld_out * esz) % 16 != 0)
    return MXQ_ERR_INVALID_ARGUMENT;

  const int32_t slice = T <= kCombineSliceMaxTokens && H > kCombineSlice
                            ? kCombineSlice
                            : H;
  const dim3 grid((unsigned)T, (unsigned)ceil_div(H, slice));
  const int threads = row_block_threads(slice, 8);
  hipStream_t s = as_stream(stream);
  const uint16_t* y = static_cast<const uint16_t*>(y_bf16);
  if (out_dtype == MXQ_OUT_F32)
    combine_kernel<true><<<grid, threads, 0, s>>>(
        y, ld_y, num_rows, src2dst, topk_weights, K, H, slice, out, ld_out);
  else
    combine_kernel<false><<<grid, threads, 0, s>>>(
        y, ld_y, num_rows, src2dst, topk_weights, K, H, slice, out, ld_out);
  return launch_status();
}
