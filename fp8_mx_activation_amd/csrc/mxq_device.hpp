// Device-side building blocks for the gfx950 kernels of libmxq.
//
// Data are moved as 16-byte vectors; a lane owns 16 consecutive channels of
// a row (32 B of bf16 in, 16 B of fp8 out), so a 128-channel scale group is
// 8 adjacent lanes and a 32-channel group is 2 adjacent lanes.  Group
// reductions therefore stay inside a wavefront (DPP quad permutes plus one
// ds_swizzle), with no LDS traffic and no barrier.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

struct alignas(16) u32x4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Non-temporal 16-byte load (global_load_dwordx4 ... nt) for data read
// once: it does not displace cached lines.  On MI355X a gather of
// read-once rows runs markedly faster with it than with plain loads.
__device__ __forceinline__ u32x4 load16_nt(const void* p) {
  const uint32_t* s = reinterpret_cast<const uint32_t*>(p);
  return u32x4{__builtin_nontemporal_load(s), __builtin_nontemporal_load(s + 1),
               __builtin_nontemporal_load(s + 2),
               __builtin_nontemporal_load(s + 3)};
}

__device__ __forceinline__ void store16(void* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ void store16_nt(void* p, const u32x4& v) {
  uint32_t* d = reinterpret_cast<uint32_t*>(p);
  __builtin_nontemporal_store(v.x, d + 0);
  __builtin_nontemporal_store(v.y, d + 1);
  __builtin_nontemporal_store(v.z, d + 2);
  __builtin_nontemporal_store(v.w, d + 3);
}

// ---------------------------------------------------------- cross-lane max

// Value held by lane (lane ^ MASK); MASK in {1, 2, 4, 8, 16}.  Masks 1 and 2
// are DPP quad permutes; larger ones use ds_swizzle's xor mode (no LDS
// memory is touched).
template <int MASK>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (MASK == 1) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
  } else if constexpr (MASK == 2) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
  } else {
    static_assert(MASK == 4 || MASK == 8 || MASK == 16, "xor mask");
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (MASK << 10) | 0x1F);
  }
}

// Max over groups of LANES adjacent lanes (LANES a power of two <= 32).
template <int LANES>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
  if constexpr (LANES >= 2) v = max(v, lane_xor<1>(v));
  if constexpr (LANES >= 4) v = max(v, lane_xor<2>(v));
  if constexpr (LANES >= 8) v = max(v, lane_xor<4>(v));
  if constexpr (LANES >= 16) v = max(v, lane_xor<8>(v));
  if constexpr (LANES >= 32) v = max(v, lane_xor<16>(v));
  return v;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = group_max<32>(v);
  uint32_t hi = (uint32_t)__shfl_xor((int)v, 32);
  return max(v, hi);
}

// --------------------------------------------------------- number formats

__device__ __forceinline__ float bf16_lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __uint_as_float(w & 0xFFFF0000u);
}

// Largest |x| of the two bf16 halves of w, as magnitude bits (0..0x7FFF).
// Magnitude order of finite bf16 values equals integer order of these bits.
__device__ __forceinline__ uint32_t bf16x2_absmax_bits(uint32_t w) {
  return max(w & 0x7FFFu, (w >> 16) & 0x7FFFu);
}

// Power-of-two scale exponent of a group from the magnitude bits m of its
// largest bf16 element: the smallest e with amax <= 448 * 2^e.  With
// amax = (1 + f/128) * 2^(E-127) and 448 = 1.75 * 2^8 this is
// E - 135, plus one when f/128 > 0.75 (f > 0x60).  Zero and bf16 subnormals
// (E = 0) fall below -127 and are clamped there; the largest finite bf16
// gives 120, so the upper clamp is never reached by finite data.
__device__ __forceinline__ int pow2_exponent(uint32_t m) {
  int ef = (int)(m >> 7);
  int e = ef - 135 + (((m & 0x7Fu) > 0x60u) ? 1 : 0);
  e = e < -127 ? -127 : e;
  return e > 127 ? 127 : e;
}

// OCP Microscaling shared exponent for e4m3 elements (largest element
// exponent 8): floor(log2 amax) - 8, which for a bf16 amax is its exponent
// field minus 135; zero and subnormals clamp to -127.
__device__ __forceinline__ int ocp_floor_exponent(uint32_t m) {
  int e = (int)(m >> 7) - 135;
  e = e < -127 ? -127 : e;
  return e > 127 ? 127 : e;
}

// 2^-e as a float; e in [-127, 126] keeps it a normal number.
__device__ __forceinline__ float pow2_neg(int e) {
  return __uint_as_float((uint32_t)(127 - e) << 23);
}

// Four floats -> four e4m3fn bytes (little-endian order a, b, c, d) with
// gfx950's v_cvt_pk_fp8_f32 (OCP e4m3, round to nearest even).
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c,
                                              float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Exponent rules: the smallest exponent that needs no clipping, or the OCP
// Microscaling floor rule, whose payload can exceed 448 and is clamped to
// +-448 before conversion (the conversion is only relied on below 464).
enum ScaleRule { kNoClip = 0, kOcpFloor = 1 };

template <int RULE>
__device__ __forceinline__ float clip448(float y) {
  if constexpr (RULE == kOcpFloor)
    return __builtin_fminf(__builtin_fmaxf(y, -448.0f), 448.0f);
  return y;
}

// Eight bf16 (one 16-byte vector) * factor -> eight e4m3 bytes.
template <int RULE>
__device__ __forceinline__ void quant8(const u32x4& v, float f, uint32_t& lo,
                                       uint32_t& hi) {
  lo = pack4_e4m3(clip448<RULE>(bf16_lo(v.x) * f),
                  clip448<RULE>(bf16_hi(v.x) * f),
                  clip448<RULE>(bf16_lo(v.y) * f),
                  clip448<RULE>(bf16_hi(v.y) * f));
  hi = pack4_e4m3(clip448<RULE>(bf16_lo(v.z) * f),
                  clip448<RULE>(bf16_hi(v.z) * f),
                  clip448<RULE>(bf16_lo(v.w) * f),
                  clip448<RULE>(bf16_hi(v.w) * f));
}

// Sixteen consecutive bf16 channels held by one lane (two 16-byte vectors)
// and the lanes of its group (G / 16 lanes): returns the 16 e4m3 bytes and
// writes the group exponent.  Every lane of a group must be active.
template <int G, int RULE = kNoClip>
__device__ __forceinline__ u32x4 quant16(const u32x4& a, const u32x4& b,
                                         int& e_out) {
  uint32_t m = max(max(bf16x2_absmax_bits(a.x), bf16x2_absmax_bits(a.y)),
                   max(bf16x2_absmax_bits(a.z), bf16x2_absmax_bits(a.w)));
  m = max(m, max(max(bf16x2_absmax_bits(b.x), bf16x2_absmax_bits(b.y)),
                 max(bf16x2_absmax_bits(b.z), bf16x2_absmax_bits(b.w))));
  m = group_max<G / 16>(m);
  const int e = RULE == kOcpFloor ? ocp_floor_exponent(m) : pow2_exponent(m);
  const float f = pow2_neg(e);
  u32x4 out;
  quant8<RULE>(a, f, out.x, out.y);
  quant8<RULE>(b, f, out.z, out.w);
  e_out = e;
  return out;
}

// Byte offset of scale g of a row: row*rs + (g/4)*c4 + g%4.  rs = row
// stride and c4 = 4 give row-major bytes; rs = 4 and c4 = 4*ld give the
// packed layout with four bytes per 32-bit word and rows contiguous
// (MN-major).
__device__ __forceinline__ int64_t scale_addr(int64_t row, int g, int64_t rs,
                                              int64_t c4) {
  return row * rs + (int64_t)(g >> 2) * c4 + (g & 3);
}

// Byte offset of the scale of 32-channel block kb of a row in the placement
// that gfx950's block-scaled MFMA (v_mfma_scale_f32_{32x32x64,16x16x128}
// _f8f6f4) reads, for tiles of tm = 2^tm_shift rows (32 or 16).  One
// instruction spans 64/tm blocks of K; the scale of its block b of row r is
// read from lane b * tm + r (whatever lanes hold the block's values), as one
// byte of a 32-bit register, the byte (kb / (64/tm)) mod 4 selected by
// op_sel, so one word per lane serves four consecutive instructions.  Words
// are stored per (row tile, group of four instructions) as 64 lanes x 4
// bytes; nkg is the number of such groups per row tile.
__device__ __forceinline__ int64_t mfma_scale_addr(int64_t row, int kb,
                                                   int tm_shift, int64_t nkg) {
  const int hh_shift = 6 - tm_shift;  // log2 of blocks per instruction
  const int lane = ((kb & ((1 << hh_shift) - 1)) << tm_shift) |
                   (int)(row & ((1 << tm_shift) - 1));
  const int64_t word_group = (row >> tm_shift) * nkg + (kb >> (hh_shift + 2));
  return ((word_group << 6) + lane) * 4 + ((kb >> hh_shift) & 3);
}

}  // namespace mxq
