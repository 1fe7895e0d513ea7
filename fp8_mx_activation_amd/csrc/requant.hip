// requant_per_token_to_per_tensor: fp8 rows with one fp32 scale per token ->
// fp8 rows with one fp32 scale for the whole tensor, so a low-latency
// dispatch can move fp8 instead of bf16 (sglang PR #14162, implementation
// breakdown items 1-2).
//
// Two launches with static grids:
//   requant_amax_kernel   one wavefront per block, owning a contiguous run of
//                         rows.  No e4m3 magnitude exceeds 448, so row t's
//                         value fl(dec(max|q_t|) * s_t) is at most
//                         bound_t = fl(448 * s_t) (rounding is monotone).
//                         The wavefront reads the scales of its rows, then
//                         reads rows in full in descending order of bound
//                         (four at a time) until no row left has a bound above
//                         the maximum found.  Every skipped row has
//                         bound_t <= that maximum, so the maximum is exact.
//                         A row holding +-448 (what a per-token absmax
//                         quantizer produces) attains its bound, so one row
//                         read settles a run; rows below their bounds are read
//                         until the bounds fall under the maximum, every row
//                         in the worst case.  Each block writes its maximum
//                         (fp32 bits of a non-negative float order like
//                         unsigned integers) to workspace.
//   requant_apply_kernel  every block reduces the partials (a few KB from
//                         L2), forms S = amax / 448 and 1 / S with IEEE
//                         division, then rewrites its rows, one per
//                         wavefront at a time:
//                         q' = e4m3((dec(q) * s_t) * (1 / S)), written with
//                         streaming stores.
#include "mxq_device.hpp"
#include "mxq_host.hpp"

namespace {

using namespace mxq;

constexpr int kPartials = 1024;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Largest magnitude byte (sign bit cleared) of 16 e4m3 bytes.
__device__ __forceinline__ uint32_t mag_max16(const u32x4& v) {
  u16x2 m = {0, 0};
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u16x2 ev = __builtin_bit_cast(u16x2, w[i] & 0x007F007Fu);
    const u16x2 od = __builtin_bit_cast(u16x2, (w[i] >> 8) & 0x007F007Fu);
    m = __builtin_elementwise_max(m, __builtin_elementwise_max(ev, od));
  }
  return max((uint32_t)m.x, (uint32_t)m.y);
}

__device__ __forceinline__ uint32_t requant4(uint32_t w, float st, float inv) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  return pack4_e4m3((lo[0] * st) * inv, (lo[1] * st) * inv,
                    (hi[0] * st) * inv, (hi[1] * st) * inv);
}

// Rows of the max pass read together by one wavefront.
constexpr int kRowsPerWave = 4;

// Rows a block of the max pass owns at least.
constexpr int64_t kAmaxMinRows = 16;

// Largest fl(dec(max|q_r|) * s_r), as fp32 bits, over the rows row[0..NR)
// (NR = 1 or kRowsPerWave; s_r from lane r_lane[u] of `s`).  Every lane
// takes 16-byte columns lane*16, lane*16 + 1024, ... of each row, so the
// NR rows' loads of four column steps are in flight together.
template <int NR>
__device__ __forceinline__ uint32_t rows_value_max(
    const uint8_t* __restrict__ q, int64_t ld, int32_t H, const int64_t* row,
    const int* r_lane, float s) {
  const int lane = threadIdx.x & 63;
  const int64_t H16 = (int64_t)(H / 16) * 16;
  uint32_t m[NR];
#pragma unroll
  for (int u = 0; u < NR; ++u) m[u] = 0;
#pragma unroll 4
  for (int64_t col = lane * 16; col < H16; col += 64 * 16) {
    u32x4 v[NR];
#pragma unroll
    for (int u = 0; u < NR; ++u) v[u] = load16(q + row[u] * ld + col);
#pragma unroll
    for (int u = 0; u < NR; ++u) m[u] = max(m[u], mag_max16(v[u]));
  }
  uint32_t best = 0;
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    const uint8_t* r = q + row[u] * ld;
    for (int64_t col = H16 + lane; col < H; col += 64)
      m[u] = max(m[u], (uint32_t)(r[col] & 0x7F));
    const uint32_t mm = wave_max(m[u]);
    const float su = __int_as_float(
        __builtin_amdgcn_readlane(__float_as_int(s), r_lane[u]));
    const float rq = __builtin_amdgcn_cvt_f32_fp8((int)mm, 0) * su;
    best = max(best, __float_as_uint(rq));
  }
  return best;
}

// One wavefront per block, owning rows [b * rows_per_block, ...).  For each
// run of 64 rows, lane i holds row i's scale and bound fl(448 * s).  Rows
// are then read in descending order of their bound, up to four at a time,
// until no row left has a bound above the maximum found: a row with
// bound <= that maximum cannot raise it.  Rows produced by a per-token
// absmax quantizer hold +-448, so their value equals their bound and the
// first row read settles its run.
__global__ __launch_bounds__(64) void requant_amax_kernel(
    const uint8_t* __restrict__ q, int64_t ld, const float* __restrict__ sc,
    int64_t T, int32_t H, int64_t rows_per_block,
    uint32_t* __restrict__ partial) {
  const int lane = threadIdx.x;
  const int64_t r_begin = (int64_t)blockIdx.x * rows_per_block;
  const int64_t r_end = min(T, r_begin + rows_per_block);
  uint32_t L = 0;  // the block's maximum so far (wave-uniform)
  for (int64_t c0 = r_begin; c0 < r_end; c0 += 64) {
    const int n = (int)min((int64_t)64, r_end - c0);
    // index clamped to the run's last row, so the load is unconditional
    const float s = sc[c0 + min(lane, n - 1)];
    const uint32_t bnd = lane < n ? __float_as_uint(448.0f * s) : 0u;
    uint64_t cand = __ballot(bnd > L);
    while (cand != 0) {
      const uint32_t Bc = __builtin_amdgcn_readfirstlane(
          wave_max(((cand >> lane) & 1) ? bnd : 0u));
      if (Bc <= L) break;
      uint64_t top = cand & __ballot(bnd == Bc);
      int64_t row[kRowsPerWave];
      int r_lane[kRowsPerWave] = {};
      int nr = 0;
#pragma unroll
      for (int u = 0; u < kRowsPerWave; ++u) {
        const int i = top ? __builtin_ctzll(top) : r_lane[0];
        if (top) {
          top &= top - 1;
          cand &= ~(1ull << i);
          ++nr;
        }
        r_lane[u] = i;  // past the last taken row: repeats the first
        row[u] = c0 + i;
      }
      const uint32_t v = nr == 1
                             ? rows_value_max<1>(q, ld, H, row, r_lane, s)
                             : rows_value_max<kRowsPerWave>(q, ld, H, row,
                                                            r_lane, s);
      L = max(L, v);
      cand &= __ballot(bnd > L);
    }
  }
  if (lane == 0) partial[blockIdx.x] = L;
}

// A wavefront takes one row at a time (rows w, w + S, ... with S = number
// of wavefronts), in batches of up to four 16-byte chunks per lane (4 KB of
// the row).  The next batch's loads (the next row's first batch at the end of
// a row) are issued before the current batch is converted and stored, so a
// wavefront keeps one batch in flight while it writes the other.  Measured
// on MI355X at 16384 x 4096 (one batch per row): 24.4 us per call warm
// against 25.3 us when each row's loads waited for the previous row's stores;
// four rows per wavefront in flight had been slower from HBM (30.7 against
// 24.6 us for the pass).  The first batch's loads also go out before the
// partial maxima are reduced.
// q_in and q_out may be the same buffer: positions are disjoint and every
// byte is read before the same lane writes it.
constexpr int kApplyBatch = 4;
constexpr int64_t kApplyBatchBytes = kApplyBatch * 64 * 16;

__device__ __forceinline__ void load_batch(const uint8_t* src, int64_t c0,
                                           int64_t H16,
                                           u32x4 (&v)[kApplyBatch]) {
#pragma unroll
  for (int b = 0; b < kApplyBatch; ++b) {
    const int64_t col = c0 + b * 64 * 16;
    v[b] = col < H16 ? load16(src + col) : u32x4{0, 0, 0, 0};
  }
}

__global__ __launch_bounds__(256) void requant_apply_kernel(
    const uint8_t* q_in, int64_t ld_in, const float* __restrict__ sc,
    int64_t T, int32_t H, uint8_t* q_out, int64_t ld_out,
    const uint32_t* __restrict__ partial, int32_t np,
    float* __restrict__ tensor_scale) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  __shared__ uint32_t red[4];
  const int64_t H16 = (int64_t)(H / 16) * 16;
  const int nb = (int)((H16 + kApplyBatchBytes - 1) / kApplyBatchBytes);
  const int64_t S = (int64_t)gridDim.x * 4;
  int64_t row = (int64_t)blockIdx.x * 4 + wv;
  // first batch of this wavefront's first row, in flight during the
  // reduction below
  u32x4 v[kApplyBatch];
  float st = 0.0f;
  if (row < T) {
    st = sc[row];
    load_batch(q_in + row * ld_in, lane * 16, H16, v);
  }
  // the partials four per thread and round, loaded unconditionally (index
  // clamped to the last one; a repeated partial leaves the maximum as it
  // is) so that they are in flight together
  uint32_t m = 0;
  for (int i0 = 0; i0 < np; i0 += 4 * 256) {
    uint32_t pv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      pv[u] = partial[min(i0 + (int)threadIdx.x + 256 * u, np - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) m = max(m, pv[u]);
  }
  m = wave_max(m);
  if (lane == 0) red[wv] = m;
  __syncthreads();
  const float amax = __uint_as_float(max(max(red[0], red[1]), max(red[2], red[3])));
  const float S_t = amax > 0.0f ? amax / 448.0f : 1.0f;
  const float inv = 1.0f / S_t;
  if (blockIdx.x == 0 && threadIdx.x == 0) *tensor_scale = S_t;

  if (nb == 0) {  // rows shorter than 16 bytes: byte loop only
    for (; row < T; row += S) {
      const float sr = sc[row];
      const uint8_t* src = q_in + row * ld_in;
      uint8_t* dst = q_out + row * ld_out;
      for (int64_t col = lane; col < H; col += 64)
        dst[col] = (uint8_t)requant4(src[col], sr, inv);
    }
    return;
  }
  int kb = 0;  // batch of `row` that v holds
  while (row < T) {
    int64_t nrow = row;
    int nkb = kb + 1;
    if (nkb == nb) {
      nkb = 0;
      nrow = row + S;
    }
    u32x4 nv[kApplyBatch];
    float nst = st;
    if (nrow < T) {
      if (nrow != row) nst = sc[nrow];
      load_batch(q_in + nrow * ld_in, lane * 16 + nkb * kApplyBatchBytes, H16,
                 nv);
    }
    const int64_t c0 = lane * 16 + kb * kApplyBatchBytes;
    uint8_t* dst = q_out + row * ld_out;
#pragma unroll
    for (int b = 0; b < kApplyBatch; ++b) {
      const int64_t col = c0 + b * 64 * 16;
      if (col >= H16) break;
      u32x4 o;
      o.x = requant4(v[b].x, st, inv);
      o.y = requant4(v[b].y, st, inv);
      o.z = requant4(v[b].z, st, inv);
      o.w = requant4(v[b].w, st, inv);
      store16_nt(dst + col, o);
    }
    if (kb == nb - 1) {  // bytes past the last whole 16-byte chunk
      const uint8_t* src = q_in + row * ld_in;
      for (int64_t col = H16 + lane; col < H; col += 64)
        dst[col] = (uint8_t)requant4(src[col], st, inv);
    }
    row = nrow;
    kb = nkb;
    st = nst;
    if (row < T) {
#pragma unroll
      for (int b = 0; b < kApplyBatch; ++b) v[b] = nv[b];
    }
  }
}

}  // namespace

extern "C" size_t requant_workspace_bytes(int64_t T, int32_t H) {
  (void)T;
  (void)H;
  return kPartials * sizeof(uint32_t);
}

extern "C" mxq_status requant_per_token_to_per_tensor(
    const void* q_in_fp8, int64_t ld_in, const float* token_scales, int64_t T,
    int32_t H, void* q_out_fp8, int64_t ld_out, float* tensor_scale,
    void* workspace, size_t workspace_bytes, void* stream) {
  if (T < 0 || H <= 0 || tensor_scale == nullptr)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (T > 0) {
    if (q_in_fp8 == nullptr || q_out_fp8 == nullptr || token_scales == nullptr)
      return MXQ_ERR_INVALID_ARGUMENT;
    if (ld_in < H || ld_out < H) return MXQ_ERR_INVALID_ARGUMENT;
    if (!aligned16(q_in_fp8) || ld_in % 16 != 0 || !aligned16(q_out_fp8) ||
        ld_out % 16 != 0)
      return MXQ_ERR_INVALID_ARGUMENT;
    if (q_in_fp8 == q_out_fp8 && ld_in != ld_out)
      return MXQ_ERR_INVALID_ARGUMENT;
  }
  if (workspace == nullptr || workspace_bytes < requant_workspace_bytes(T, H))
    return MXQ_ERR_WORKSPACE;

  hipStream_t s = as_stream(stream);
  uint32_t* partial = static_cast<uint32_t*>(workspace);
  int64_t rows_per_block = ceil_div(T, (int64_t)kPartials);
  if (rows_per_block < kAmaxMinRows) rows_per_block = kAmaxMinRows;
  const int64_t np = ceil_div(T, rows_per_block);
  if (np > 0) {
    requant_amax_kernel<<<(unsigned)np, 64, 0, s>>>(
        static_cast<const uint8_t*>(q_in_fp8), ld_in, token_scales, T, H,
        rows_per_block, partial);
    if (launch_status() != MXQ_OK) return MXQ_ERR_HIP;
  }
  int64_t blocks = ceil_div(T, 4);
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  requant_apply_kernel<<<(unsigned)blocks, 256, 0, s>>>(
      static_cast<const uint8_t*>(q_in_fp8), ld_in, token_scales, T, H,
      static_cast<uint8_t*>(q_out_fp8), ld_out, partial, (int32_t)np,
      tensor_scale);
  return launch_status();
}
