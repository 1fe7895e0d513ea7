// Receive-side upscale (fp8 + group fp32 scales -> bf16) and weight-side
// UE8M0 block requant (block-scaled fp8 weights -> bf16 -> fp8 with one
// power-of-two scale per 128 x 128 block).
//
// Both round the product of an e4m3 value and an fp32 scale to bf16 exactly
// once.  That product needs up to 28 significant bits, so the fp32 product
// alone could land on a bf16 rounding midpoint that the exact product is not
// on.  mul_round_bf16 keeps the fp32 product's rounding error (one fmaf,
// exact when the scale is at least 2^-90), folds it in as a sticky bit (round
// to odd) and then rounds to bf16 with nearest-even; smaller scales take an
// exact double-precision path, chosen once per scale.
//
//   upscale_kernel         one block per row, one lane per 16 bytes (16
//                          channels) of the row: a 16-byte load, one scale per
//                          lane, two 16-byte stores.  HBM-bound: 3 bytes per
//                          channel plus the scales.
//   weight_requant_kernel  one 512-thread block per 128 x 512 tile (four
//                          128 x 128 scale blocks): each thread loads eight
//                          16-byte chunks of one column (the block reads 16
//                          runs of 512 B per instruction), dequantizes them
//                          to bf16 in registers, the block reduces each scale
//                          block's largest magnitude, and the same threads
//                          requantize and store.  All reads precede the
//                          reduction barrier, so the output may be the input
//                          itself.  The weights are read once, with
//                          non-temporal loads.
#include "mxq_device.hpp"
#include "mxq_host.hpp"

namespace {

using namespace mxq;

// bf16 bits (low 16 bits) of x, given its fp32 rounding p and the exact
// remainder err = x - p: round to odd (truncate toward zero and set the last
// bit when inexact), then to bf16 with nearest-even.  Rounding to odd first
// keeps the second rounding exact, since bf16 drops 16 bits.  NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t round_bf16_sticky(float p, float err) {
  uint32_t pb = __float_as_uint(p);
  const uint32_t odd = (pb - ((__float_as_uint(err) ^ pb) >> 31)) | 1u;
  pb = err != 0.0f ? odd : pb;
  const uint32_t r = (pb + 0x7FFFu + ((pb >> 16) & 1u)) >> 16;
  return p != p ? 0x7FC0u : r;
}

// Exactly rounded a * b for an e4m3 value a and a scale |b| >= 2^-90: every
// nonzero product is then at least 2^-99, where the fmaf remainder is exact
// (no underflow), and a zero product has a zero remainder.
__device__ __forceinline__ uint32_t mul_round_bf16(float a, float b) {
  const float p = a * b;
  return round_bf16_sticky(p, __builtin_fmaf(a, b, -p));
}

// The same for any scale, through an exact double product (4 + 24
// significant bits) whose fp32 rounding is corrected to odd by comparison.
__device__ __forceinline__ uint32_t mul_round_bf16_small(float a, float b) {
  const double x = (double)a * (double)b;
  const float f = (float)x;
  uint32_t fb = __float_as_uint(f);
  const double fd = (double)f;
  if (fd != x) {
    if (__builtin_fabs(fd) > __builtin_fabs(x)) fb -= 1u;
    fb |= 1u;
  }
  const uint32_t r = (fb + 0x7FFFu + ((fb >> 16) & 1u)) >> 16;
  return x != x ? 0x7FC0u : r;
}

__device__ __forceinline__ bool fast_scale(float b) {
  return !(__builtin_fabsf(b) < 0x1p-90f);  // NaN takes the fast path too
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 (nearest even) with v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const bf16x2_t h = __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}

// Nonzero when some byte of w is an e4m3 NaN (S.1111.111).
__device__ __forceinline__ uint32_t nan_byte_bits(uint32_t w) {
  const uint32_t x = ~(w | 0x80808080u);  // a NaN byte becomes 0x00
  return (x - 0x01010101u) & ~x & 0x80808080u;
}

// Sixteen e4m3 bytes times b -> sixteen bf16 (o0: channels 0-7, o1: 8-15),
// each the exactly rounded product.  Fast path: the fp32 product rounded by
// v_cvt_pk_bf16_f32.  That equals the exact rounding unless the fp32 product
// sits exactly on a bf16 rounding midpoint (low 16 bits 0x8000, about one
// product in 65536), so a lane holding such a product, an unusual scale
// (below 2^-90 or not finite) or, when CHECK_NAN, a NaN byte recomputes its
// sixteen products with the exact routines above.
template <bool CHECK_NAN>
__device__ __forceinline__ void upscale16(const u32x4& v, float b, u32x4& o0,
                                          u32x4& o1) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float p[16];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);
    const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);
    p[4 * k] = f01[0] * b;
    p[4 * k + 1] = f01[1] * b;
    p[4 * k + 2] = f23[0] * b;
    p[4 * k + 3] = f23[1] * b;
  }
  // zero exactly when some product's low 16 bits are 0x8000
  uint32_t mid = 0xFFFFu;
#pragma unroll
  for (int k = 0; k < 16; ++k)
    mid = min(mid, (__float_as_uint(p[k]) ^ 0x8000u) & 0xFFFFu);
  bool slow = !fast_scale(b) | (mid == 0u);  // this lane takes the exact path
  if (CHECK_NAN)
    slow = slow | !__builtin_isfinite(b) |
           ((nan_byte_bits(w[0]) | nan_byte_bits(w[1]) | nan_byte_bits(w[2]) |
             nan_byte_bits(w[3])) != 0u);
  uint32_t r[8];
  if (!slow) {
#pragma unroll
    for (int k = 0; k < 8; ++k) r[k] = cvt_pk_bf16(p[2 * k], p[2 * k + 1]);
  } else if (fast_scale(b)) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);
      const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);
      r[2 * k] = mul_round_bf16(f01[0], b) | (mul_round_bf16(f01[1], b) << 16);
      r[2 * k + 1] =
          mul_round_bf16(f23[0], b) | (mul_round_bf16(f23[1], b) << 16);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);
      const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);
      r[2 * k] = mul_round_bf16_small(f01[0], b) |
                 (mul_round_bf16_small(f01[1], b) << 16);
      r[2 * k + 1] = mul_round_bf16_small(f23[0], b) |
                     (mul_round_bf16_small(f23[1], b) << 16);
    }
  }
  o0 = u32x4{r[0], r[1], r[2], r[3]};
  o1 = u32x4{r[4], r[5], r[6], r[7]};
}

template <int G>
__global__ __launch_bounds__(1024) void upscale_kernel(
    const uint8_t* __restrict__ q, int64_t ld_q, const float* __restrict__ s,
    int64_t s_rs, int64_t s_cs, int32_t H, uint16_t* __restrict__ out,
    int64_t ld_out) {
  const int64_t r = blockIdx.x;
  const uint8_t* qr = q + r * ld_q;
  const float* sr = s + r * s_rs;
  uint16_t* orow = out + r * ld_out;
  for (int32_t col = threadIdx.x * 16; col < H; col += blockDim.x * 16) {
    const u32x4 v = load16(qr + col);
    const float b = sr[(int64_t)(col / G) * s_cs];
    u32x4 o0, o1;
    upscale16<true>(v, b, o0, o1);
    store16(orow + col, o0);
    store16(orow + col + 8, o1);
  }
}

constexpr int kWBlock = 128;      // scale block: 128 x 128 weights
constexpr int kWRowsPerPass = 16;  // rows one instruction of a block reads
constexpr int kWChunks = kWBlock / kWRowsPerPass;  // 8 per thread

// One block of TK threads per tile of 128 rows x TK columns (TK / 128 scale
// blocks): thread t owns the 16-byte column chunk c = t % (TK / 16) of rows
// t / (TK / 16) + 16 u, u < 8, so one instruction of the block reads 16 runs
// of TK bytes and every value a thread holds belongs to scale block c / 8.
// The block maximum is reduced over the 8 adjacent lanes of a scale block,
// then over the 16 rows of a pass in LDS.
template <int TK, bool FULL>
__device__ __forceinline__ void weight_tile(
    const uint8_t* qb, int64_t ld, float si, int32_t N, int32_t r0, int32_t cc,
    bool col_ok, u32x4 (&w0)[kWChunks], u32x4 (&w1)[kWChunks], uint32_t& m) {
  const int r = threadIdx.x / (TK / 16);
  // every load is issued before the first dequantization (whose exact
  // rounding branches would otherwise make each load wait for the last)
  u32x4 raw[kWChunks];
#pragma unroll
  for (int u = 0; u < kWChunks; ++u) {
    const int32_t rr = r0 + r + u * kWRowsPerPass;
    raw[u] = (FULL || (col_ok && rr < N))
                 ? load16_nt(qb + (int64_t)rr * ld + cc)
                 : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int u = 0; u < kWChunks; ++u) {
    const int32_t rr = r0 + r + u * kWRowsPerPass;
    if (FULL || (col_ok && rr < N)) {
      upscale16<false>(raw[u], si, w0[u], w1[u]);
      m = max(m, max(max(bf16x2_absmax_bits(w0[u].x), bf16x2_absmax_bits(w0[u].y)),
                     max(bf16x2_absmax_bits(w0[u].z), bf16x2_absmax_bits(w0[u].w))));
      m = max(m, max(max(bf16x2_absmax_bits(w1[u].x), bf16x2_absmax_bits(w1[u].y)),
                     max(bf16x2_absmax_bits(w1[u].z), bf16x2_absmax_bits(w1[u].w))));
    }
  }
}

template <int TK>
__global__ __launch_bounds__(TK) void weight_requant_kernel(
    const uint8_t* q, int64_t ld, int64_t q_bs, const float* __restrict__ s_inv,
    int64_t s_ld, int64_t s_bs, int32_t N, int32_t K, int32_t nbn,
    int32_t ntk, uint8_t* q_out, uint8_t* __restrict__ s_out, int64_t o_ld,
    int64_t o_bs) {
  constexpr int CPR = TK / 16;  // chunks per tile row
  __shared__ uint32_t rmax[kWRowsPerPass][TK / kWBlock];
  // consecutive blocks take consecutive 128-row blocks of one column tile
  // (measured on MI355X at [32, 4096, 7168]: 324.9-329.6 us against
  // 331.3-335.4 us with the column tiles of one row block consecutive)
  const int64_t blk = blockIdx.x;
  const int32_t i = (int32_t)(blk % nbn);
  const int64_t t = blk / nbn;
  const int32_t jt = (int32_t)(t % ntk);
  const int64_t b = t / ntk;
  const int c = threadIdx.x % CPR;
  const int r = threadIdx.x / CPR;
  const int kb = c >> 3;                           // scale block in the tile
  const int32_t j = jt * (TK / kWBlock) + kb;      // scale block in the row
  const int32_t r0 = i * kWBlock;
  const int32_t cc = jt * TK + c * 16;
  const bool col_ok = cc < K;
  const float si = col_ok ? s_inv[b * s_bs + (int64_t)i * s_ld + j] : 0.0f;
  const uint8_t* qb = q + b * q_bs;
  const bool full = r0 + kWBlock <= N && (jt + 1) * TK <= K;

  u32x4 w0[kWChunks], w1[kWChunks];  // 16 bf16 per chunk
  uint32_t m = 0;
  if (full)
    weight_tile<TK, true>(qb, ld, si, N, r0, cc, col_ok, w0, w1, m);
  else
    weight_tile<TK, false>(qb, ld, si, N, r0, cc, col_ok, w0, w1, m);
  m = group_max<8>(m);
  if ((c & 7) == 0) rmax[r][kb] = m;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kWRowsPerPass; ++w) m = max(m, rmax[w][kb]);
  const int e = pow2_exponent(m);
  const float f = pow2_neg(e);

  uint8_t* ob = q_out + b * q_bs;
#pragma unroll
  for (int u = 0; u < kWChunks; ++u) {
    const int32_t rr = r0 + r + u * kWRowsPerPass;
    if (full || (col_ok && rr < N)) {
      u32x4 o;
      quant8<kNoClip>(w0[u], f, o.x, o.y);
      quant8<kNoClip>(w1[u], f, o.z, o.w);
      store16_nt(ob + (int64_t)rr * ld + cc, o);
    }
  }
  if (r == 0 && (c & 7) == 0 && col_ok)
    s_out[b * o_bs + (int64_t)i * o_ld + j] = (uint8_t)(e + 127);
}

// Tile width: 512 columns (512 B runs, two 512-thread blocks per CU at the
// kernel's 112 VGPRs).  Measured on MI355X for the [32, 4096, 7168] gate/up
// set: 332 us, against 356 us with 256, 380 us with 1024 and 370 us with one
// block per 128 x 128 scale block.
constexpr int kWTileK = 512;

}  // namespace

extern "C" mxq_status upscale_fp8_to_bf16(const void* q_fp8, int64_t ld_q,
                                          const float* scales,
                                          int64_t scale_row_stride,
                                          int64_t scale_col_stride,
                                          int64_t num_rows, int32_t H,
                                          int32_t group, void* out_bf16,
                                          int64_t ld_out, void* stream) {
  if (group != 32 && group != 128) return MXQ_ERR_UNSUPPORTED;
  if (num_rows < 0 || num_rows > INT32_MAX || H <= 0 || H % group != 0 ||
      scale_row_stride < 0 || scale_col_stride < 0)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (num_rows == 0) return MXQ_OK;
  if (q_fp8 == nullptr || scales == nullptr || out_bf16 == nullptr)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (ld_q < H || ld_out < H || ld_q % 16 != 0 || ld_out % 8 != 0 ||
      !aligned16(q_fp8) || !aligned16(out_bf16))
    return MXQ_ERR_INVALID_ARGUMENT;
  const int threads = row_block_threads(H, 16);
  hipStream_t s = as_stream(stream);
  const uint8_t* q = static_cast<const uint8_t*>(q_fp8);
  uint16_t* o = static_cast<uint16_t*>(out_bf16);
  if (group == 128)
    upscale_kernel<128><<<(unsigned)num_rows, threads, 0, s>>>(
        q, ld_q, scales, scale_row_stride, scale_col_stride, H, o, ld_out);
  else
    upscale_kernel<32><<<(unsigned)num_rows, threads, 0, s>>>(
        q, ld_q, scales, scale_row_stride, scale_col_stride, H, o, ld_out);
  return launch_status();
}

extern "C" mxq_status requant_weight_block_ue8m0(
    const void* q_fp8, int64_t ld, int64_t matrix_stride, const float* s_inv,
    int64_t s_ld, int64_t s_matrix_stride, int32_t num_matrices, int32_t N,
    int32_t K, int32_t block_n, int32_t block_k, void* q_out,
    uint8_t* scales_out, int64_t o_ld, int64_t o_matrix_stride,
    void* stream) {
  if (block_n != kWBlock || block_k != kWBlock) return MXQ_ERR_UNSUPPORTED;
  if (num_matrices < 0 || N < 0 || K < 0) return MXQ_ERR_INVALID_ARGUMENT;
  if (num_matrices == 0 || N == 0 || K == 0) return MXQ_OK;
  const int64_t nbn = ceil_div(N, kWBlock), nbk = ceil_div(K, kWBlock);
  if (q_fp8 == nullptr || s_inv == nullptr || q_out == nullptr ||
      scales_out == nullptr)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (K % 16 != 0 || ld < K || ld % 16 != 0 || !aligned16(q_fp8) ||
      !aligned16(q_out))
    return MXQ_ERR_INVALID_ARGUMENT;
  const int64_t span = (int64_t)(N - 1) * ld + K;  // bytes of one matrix
  if (num_matrices > 1 && (matrix_stride < span || matrix_stride % 16 != 0))
    return MXQ_ERR_INVALID_ARGUMENT;
  if (s_ld < nbk || (num_matrices > 1 &&
                     s_matrix_stride < (nbn - 1) * s_ld + nbk))
    return MXQ_ERR_INVALID_ARGUMENT;
  if (o_ld < nbk || (num_matrices > 1 &&
                     o_matrix_stride < (nbn - 1) * o_ld + nbk))
    return MXQ_ERR_INVALID_ARGUMENT;
  const int64_t ntk = ceil_div(K, kWTileK);
  const int64_t blocks = (int64_t)num_matrices * nbn * ntk;
  if (blocks > INT32_MAX) return MXQ_ERR_INVALID_ARGUMENT;
  weight_requant_kernel<kWTileK><<<(unsigned)blocks, kWTileK, 0,
                                   as_stream(stream)>>>(
      static_cast<const uint8_t*>(q_fp8), ld, matrix_stride, s_inv, s_ld,
      s_matrix_stride, N, K, (int32_t)nbn, (int32_t)ntk,
      static_cast<uint8_t*>(q_out), scales_out, o_ld, o_matrix_stride);
  return launch_status();
}
