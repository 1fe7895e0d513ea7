// Test instrument, not part of the library: a consumer of quantized rows
// whose scales sit in the block-scaled MFMA placement.  It multiplies the
// fp8 rows (operand A, with their e8m0 scales) by an identity matrix
// (operand B: e4m3 1.0 on the diagonal, scale byte 127) with gfx950's
// v_mfma_scale_f32_32x32x64_f8f6f4 (tile_m = 32) or
// v_mfma_scale_f32_16x16x128_f8f6f4 (tile_m = 16).  Each output element then
// has exactly one nonzero term, dec(q[r][c]) * 2^(scale(r, c/32) - 127), so a
// correct placement reproduces the dequantized rows exactly, while a scale
// read from the wrong lane, tile, word group or op_sel byte shows up as a
// wrong power of two.
//
// Operand layout used (one 64-lane wavefront per tm x tm output tile): for
// instruction s over channels [s*KW, (s+1)*KW), KW = 64*32/tm, lane
// l = g*tm + r holds channels s*KW + 16g + [0, 16) in registers 0-3 and
// s*KW + KW/2 + 16g + [0, 16) in registers 4-7, of row r of A and of column
// r of B; the scale of the instruction's 32-channel block b of row r comes
// from lane b*tm + r.  The fp32 accumulator holds column l % tm, rows
// 8*(v/4) + 4*(l/32) + v%4 for v < 16 (tm = 32) or 4*(l/16) + v for v < 4
// (tm = 16).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr uint32_t kOne = 0x38;  // e4m3 1.0

// 16 channels at p0 into registers 0-3 and 16 at p1 into registers 4-7
__device__ __forceinline__ v8i load_pair(const uint8_t* p0,
                                         const uint8_t* p1) {
  const uint4 lo = *reinterpret_cast<const uint4*>(p0);
  const uint4 hi = *reinterpret_cast<const uint4*>(p1);
  v8i v;
  v[0] = (int)lo.x; v[1] = (int)lo.y; v[2] = (int)lo.z; v[3] = (int)lo.w;
  v[4] = (int)hi.x; v[5] = (int)hi.y; v[6] = (int)hi.z; v[7] = (int)hi.w;
  return v;
}

// column n of the identity restricted to channels [k0, k0 + 16) (bytes
// 0-15) and [k1, k1 + 16) (bytes 16-31)
__device__ __forceinline__ v8i identity_column(int n, int k0, int k1) {
  v8i v;
  for (int i = 0; i < 8; ++i) v[i] = 0;
  int d = -1;
  if (n >= k0 && n < k0 + 16) d = n - k0;
  if (n >= k1 && n < k1 + 16) d = 16 + n - k1;
  if (d >= 0) v[d >> 2] = (int)(kOne << (8 * (d & 3)));
  return v;
}

template <typename Acc, int SEL>
__device__ __forceinline__ Acc mfma_step(const v8i& a, const v8i& b, Acc c,
                                         int sa);

template <>
__device__ __forceinline__ v16f mfma_step<v16f, 0>(const v8i& a, const v8i& b,
                                                   v16f c, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa,
                                                         0, 127);
}
template <>
__device__ __forceinline__ v16f mfma_step<v16f, 1>(const v8i& a, const v8i& b,
                                                   v16f c, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 1, sa,
                                                         0, 127);
}
template <>
__device__ __forceinline__ v16f mfma_step<v16f, 2>(const v8i& a, const v8i& b,
                                                   v16f c, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 2, sa,
                                                         0, 127);
}
template <>
__device__ __forceinline__ v16f mfma_step<v16f, 3>(const v8i& a, const v8i& b,
                                                   v16f c, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 3, sa,
                                                         0, 127);
}
template <>
__device__ __forceinline__ v4f mfma_step<v4f, 0>(const v8i& a, const v8i& b,
                                                 v4f c, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0,
                                                          sa, 0, 127);
}
template <>
__device__ __forceinline__ v4f mfma_step<v4f, 1>(const v8i& a, const v8i& b,
                                                 v4f c, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 1,
                                                          sa, 0, 127);
}
template <>
__device__ __forceinline__ v4f mfma_step<v4f, 2>(const v8i& a, const v8i& b,
                                                 v4f c, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 2,
                                                          sa, 0, 127);
}
template <>
__device__ __forceinline__ v4f mfma_step<v4f, 3>(const v8i& a, const v8i& b,
                                                 v4f c, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 3,
                                                          sa, 0, 127);
}

template <int TM, typename Acc, int NACC>
__global__ __launch_bounds__(64) void identity_kernel(
    const uint8_t* __restrict__ q, int64_t ld_q,
    const uint32_t* __restrict__ words, int64_t nkg, int32_t H,
    int32_t tiles_n, float* __restrict__ out, int64_t ld_out) {
  constexpr int KW = 64 * 32 / TM;  // channels per instruction
  const int lane = threadIdx.x;
  const int64_t mt = blockIdx.x / tiles_n;
  const int nt = blockIdx.x % tiles_n;
  const int r = lane % TM;
  const int g = lane / TM;
  const uint8_t* arow = q + (mt * TM + r) * ld_q;
  const int n = nt * TM + r;
  Acc acc;
  for (int i = 0; i < NACC; ++i) acc[i] = 0.0f;
  for (int s = 0; s < H / KW; ++s) {
    const int k0 = s * KW + 16 * g;
    const int k1 = k0 + KW / 2;
    const v8i a = load_pair(arow + k0, arow + k1);
    const v8i b = identity_column(n, k0, k1);
    const int w = (int)words[(mt * nkg + s / 4) * 64 + lane];
    switch (s & 3) {
      case 0: acc = mfma_step<Acc, 0>(a, b, acc, w); break;
      case 1: acc = mfma_step<Acc, 1>(a, b, acc, w); break;
      case 2: acc = mfma_step<Acc, 2>(a, b, acc, w); break;
      default: acc = mfma_step<Acc, 3>(a, b, acc, w); break;
    }
  }
  const int col = nt * TM + lane % TM;
  for (int v = 0; v < NACC; ++v) {
    const int row = TM == 32 ? 8 * (v / 4) + 4 * (lane / 32) + v % 4
                             : 4 * (lane / 16) + v;
    out[(mt * TM + row) * ld_out + col] = acc[v];
  }
}

}  // namespace

// out[r][c] = dec(q[r][c]) * 2^(scale(r, c/32) - 127) for r < rows, c < H,
// computed by the scaled MFMA from q (fp8 rows, ld_q bytes apart, 16-byte
// aligned) and `words` (the MFMA placement of the scales, nkg word groups per
// row tile).  Needs rows % tile_m == 0 and H % (64*32/tile_m) == 0.  Returns
// 0, or -1 on a rejected argument, or -2 if the launch failed.
extern "C" int mfma_identity_dequant(const uint8_t* q, int64_t ld_q,
                                     const uint32_t* words, int64_t nkg,
                                     int64_t rows, int32_t H, int32_t tile_m,
                                     float* out, int64_t ld_out,
                                     void* stream) {
  if ((tile_m != 16 && tile_m != 32) || rows <= 0 || H <= 0 ||
      rows % tile_m != 0 || H % (64 * 32 / tile_m) != 0 || ld_q < H ||
      ld_q % 16 != 0 || ld_out < H || nkg < (H / 32 + 4 * (64 / tile_m) - 1) /
                                               (4 * (64 / tile_m)) ||
      (reinterpret_cast<uintptr_t>(q) & 15) != 0 || q == nullptr ||
      words == nullptr || out == nullptr)
    return -1;
  const int tiles_n = H / tile_m;
  const int64_t blocks = rows / tile_m * tiles_n;
  if (blocks > INT32_MAX) return -1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (tile_m == 32)
    identity_kernel<32, v16f, 16><<<(unsigned)blocks, 64, 0, s>>>(
        q, ld_q, words, nkg, H, tiles_n, out, ld_out);
  else
    identity_kernel<16, v4f, 4><<<(unsigned)blocks, 64, 0, s>>>(
        q, ld_q, words, nkg, H, tiles_n, out, ld_out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
