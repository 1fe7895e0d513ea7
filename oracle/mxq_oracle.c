/*
 * CPU oracle for the MoE dispatch-preprocessing path (fp8 e4m3 activations
 * with power-of-two group scales).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
 * GPU library is checked against.  Only the test suite, the package smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header, table or constant generator with the HIP library, and it must never
 * serve as a fallback for it.
 *
 * Sources (the pages are summaries of sglang pull requests):
 *   [P1] sglang PR #33128 page (DeepGEMM standard MoE dispatch, compact layout,
 *        UE8M0 requant)
 *   [P2] sglang PR #14162 page (DeepEP low-latency dispatch in fp8, per-token
 *        to per-tensor requant)
 *   [P3] sglang PR #29525 page (DeepEPv2 ElasticBuffer backend, psum layouts,
 *        masked-slab repack)
 *   [P4] sglang PR #36119 page (MXFP8 MoRI dispatch on MI355X, send-side
 *        group-32 e8m0 quant over live tokens)
 * Format definitions not on the pages: OCP 8-bit floating point (OFP8) E4M3
 * ("e4m3fn": bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN, largest
 * finite 448) and the OCP Microscaling E8M0 scale (one byte, value 2^(b-127)).
 *
 * Readings of points the pages leave open (each is listed in the design notes):
 *   R1  fp8 e4m3 is OCP e4m3fn; encoding rounds to nearest, ties to even, and
 *       saturates to +-448 (never produces NaN from a finite input).
 *   R2  the power-of-two scale exponent of a group is the smallest integer e
 *       with amax <= 448 * 2^e (no clipping), clamped to [-127, 127]; an
 *       all-zero group gets e = -127.  Same rule for group 128 and group 32.
 *   R3  slots inside an expert's region follow ascending flat assignment index
 *       t*K + j (deterministic, stable).
 *   R4  rows past the last expert's padded region, up to the static bound, are
 *       padding rows (m_indices = -1), like the per-expert padding rows.
 *   R5  masked layout: an expert's assignments beyond the slab capacity get no
 *       slot (src2dst = -1) and raise the overflow flag; masked_m is clipped.
 *   R6  per-token -> per-tensor requant: amax over dequantized values
 *       fl32(dec(q) * s_t); S = fl32(amax / 448) (S = 1 when amax = 0);
 *       inv = fl32(1 / S); q' = enc(fl32(fl32(dec(q) * s_t) * inv)).
 *   R7  combine: fp32 accumulator from +0, one fused multiply-add per
 *       assignment in ascending j, non-local assignments skipped, result
 *       rounded to bf16 (nearest, ties to even) or kept as fp32.
 *   R8  the OCP Microscaling rule, offered beside R2: e = floor(log2 amax) - 8
 *       (8 = largest exponent of e4m3), clamped to [-127, 127]; payload
 *       values then reach up to 2^9 and saturate to +-448.
 *   R9  receive-side upscale: out = bf16(dec(q) * s) with the product taken
 *       exactly and rounded once (nearest, ties to even; overflow to inf);
 *       a NaN result is written as 0x7FC0.  Only the first num_local_tokens
 *       rows are written.
 *   R10 weight-side UE8M0 block requant: each [bn, bk] block (128 x 128) is
 *       dequantized to bf16 with R9's rounding using its fp32 inverse scale,
 *       then quantized again with R2 over the whole block, the exponent
 *       stored as one UE8M0 byte per block.  Inputs are finite.
 *
 * Floating-point: built with -ffp-contract=off.  Quantization arithmetic is
 * done in double, where every step is exact (power-of-two scaling of values
 * with at most 24 significant bits); the requant (R6) and combine (R7) steps
 * are fp32 by definition of the readings, and have fp64 companions for the
 * error bounds.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORA_E4M3_MAX 448.0

/* Thread control for timing runs (no arithmetic). */
int32_t ora_max_threads(void) { return omp_get_max_threads(); }
void ora_set_threads(int32_t n) { omp_set_num_threads(n); }

/* ---------------------------------------------------------------- formats */

/* bf16 is the upper half of an IEEE binary32 word. */
static double bf16_to_double(uint16_t h) {
  uint32_t w = (uint32_t)h << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

static float bf16_to_float(uint16_t h) {
  uint32_t w = (uint32_t)h << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return f;
}

/* Decode one e4m3fn byte (OFP8 E4M3: value = (-1)^s * 2^(E-7) * (1 + m/8)
 * for E >= 1, (-1)^s * 2^-6 * (m/8) for E = 0; S.1111.111 is NaN). */
double ora_e4m3_decode(uint8_t b) {
  int s = b >> 7;
  int ef = (b >> 3) & 0xF;
  int m = b & 0x7;
  double mag;
  if (ef == 15 && m == 7) return s ? -NAN : NAN;
  if (ef == 0)
    mag = ldexp((double)m, -9);
  else
    mag = ldexp((double)(8 + m), ef - 10);
  return s ? -mag : mag;
}

/* Encode a real number to e4m3fn (R1).  The grid spacing at |y| is 2^-9 in
 * the subnormal range (|y| < 2^-6) and 2^(floor(log2|y|) - 3) above it.
 * |y| / spacing is exact in double, so the nearest-even choice below is the
 * textbook rule applied to the exact value. */
uint8_t ora_e4m3_encode(double y) {
  uint8_t sign = signbit(y) ? 0x80 : 0x00;
  double a = fabs(y);
  if (isnan(y)) return sign | 0x7F;
  if (isinf(a)) return sign | 0x7E;
  if (a == 0.0) return sign;

  double spacing;
  if (a < ldexp(1.0, -6)) {
    spacing = ldexp(1.0, -9);
  } else {
    int E;
    frexp(a, &E); /* a = f * 2^E with f in [0.5, 1): floor(log2 a) = E - 1 */
    spacing = ldexp(1.0, (E - 1) - 3);
  }
  double n = a / spacing; /* exact: division by a power of two */
  double lo = floor(n);
  double frac = n - lo; /* exact */
  double r;
  if (frac > 0.5)
    r = lo + 1.0;
  else if (frac < 0.5)
    r = lo;
  else
    r = (fmod(lo, 2.0) == 0.0) ? lo : lo + 1.0;
  double v = r * spacing;
  if (v > ORA_E4M3_MAX) v = ORA_E4M3_MAX; /* satfinite */
  if (v == 0.0) return sign;

  if (v < ldexp(1.0, -6)) { /* subnormal: v = m * 2^-9, m in 1..7 */
    int m = (int)(v / ldexp(1.0, -9));
    return sign | (uint8_t)m;
  }
  int E;
  frexp(v, &E);
  int e = E - 1;                                 /* v = 2^e * (1 + m/8) */
  int m = (int)(v / ldexp(1.0, e - 3)) - 8;      /* 0..7 */
  return sign | (uint8_t)(((e + 7) << 3) | m);
}

/* Round a binary32 value to bf16, nearest with ties to even, by comparing the
 * exact distances to the two neighbouring bf16 values. */
uint16_t ora_bf16_round(float x) {
  uint32_t w;
  memcpy(&w, &x, sizeof w);
  uint16_t sign = (uint16_t)((w >> 16) & 0x8000);
  if (isnan(x)) return sign | 0x7FC0;
  if (isinf(x)) return (uint16_t)(w >> 16);
  uint32_t lo_bits = w & 0xFFFF0000u; /* truncation toward zero */
  uint16_t lo_h = (uint16_t)(lo_bits >> 16);
  double a = fabs((double)x);
  double lo = fabs(bf16_to_double(lo_h));
  if (a == lo) return lo_h;
  /* spacing of bf16 at lo: exponent field of lo, 7 fraction bits */
  int ef = (int)((lo_bits >> 23) & 0xFF);
  double spacing = (ef == 0) ? ldexp(1.0, -133) : ldexp(1.0, ef - 127 - 7);
  double hi = lo + spacing;
  double dlo = a - lo, dhi = hi - a;
  uint16_t mag_lo = lo_h & 0x7FFF;
  uint16_t mag;
  if (dlo < dhi)
    mag = mag_lo;
  else if (dhi < dlo)
    mag = (uint16_t)(mag_lo + 1);
  else
    mag = (mag_lo & 1) ? (uint16_t)(mag_lo + 1) : mag_lo;
  return sign | mag;
}

void ora_bf16_round_array(const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = ora_bf16_round(x[i]);
}

/* Round a real number (held exactly in a double) to bf16 once: nearest, ties
 * to even, overflow to infinity; NaN gives 0x7FC0 (R9).  The bf16 grid
 * spacing at |x| is 2^-133 below 2^-126 (subnormals) and 2^(floor(log2|x|) -
 * 7) above it; |x| / spacing is exact, as in the e4m3 encoder. */
uint16_t ora_bf16_round_f64(double x) {
  if (isnan(x)) return 0x7FC0;
  uint16_t sign = signbit(x) ? 0x8000 : 0x0000;
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (a >= ldexp(1.0, 128)) return sign | 0x7F80;
  int E;
  frexp(a, &E); /* floor(log2 a) = E - 1 */
  double spacing = (E - 1 < -126) ? ldexp(1.0, -133) : ldexp(1.0, E - 1 - 7);
  double n = a / spacing;
  double lo = floor(n);
  double frac = n - lo;
  double r;
  if (frac > 0.5)
    r = lo + 1.0;
  else if (frac < 0.5)
    r = lo;
  else
    r = (fmod(lo, 2.0) == 0.0) ? lo : lo + 1.0;
  float v = (float)(r * spacing); /* a bf16 value (or 2^128 -> inf): exact */
  uint32_t w;
  memcpy(&w, &v, sizeof w);
  return sign | (uint16_t)((w >> 16) & 0x7FFF);
}

void ora_bf16_round_f64_array(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = ora_bf16_round_f64(x[i]);
}

void ora_e4m3_encode_array_f32(const float* y, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = ora_e4m3_encode((double)y[i]);
}

void ora_e4m3_decode_array(const uint8_t* b, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = ora_e4m3_decode(b[i]);
}

/* Encode every binary32 bit pattern w in [w0, w0 + n) (used by the exhaustive
 * codec check; the pattern itself is the input). */
void ora_e4m3_encode_bits_range(uint32_t w0, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint32_t w = w0 + (uint32_t)i;
    float f;
    memcpy(&f, &w, sizeof f);
    out[i] = ora_e4m3_encode((double)f);
  }
}

/* --------------------------------------------------- power-of-two scales */

/* R2: smallest integer e with amax <= 448 * 2^e, clamped to [-127, 127]
 * [P1 Implementation breakdown item 3: quantize with a UE8M0 scale directly;
 *  P4 Implementation breakdown item 1: group-32 e8m0 scales, one byte each]. */
int ora_pow2_scale_exponent(double amax) {
  if (!(amax > 0.0)) return -127;
  int e = (int)ceil(log2(amax / ORA_E4M3_MAX));
  while (ldexp(ORA_E4M3_MAX, e) < amax) ++e;
  while (ldexp(ORA_E4M3_MAX, e - 1) >= amax) --e;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

/* R8: the OCP Microscaling shared exponent for e4m3 elements, whose largest
 * exponent is 8: floor(log2 amax) - 8, clamped to [-127, 127]; an all-zero
 * group gets -127 [P3 Implementation breakdown item 3 and P4 Motivation name
 * the formats the consumers read; the rule itself is the OCP MX one]. */
int ora_ocp_mx_exponent(double amax) {
  if (!(amax > 0.0)) return -127;
  int E;
  frexp(amax, &E); /* amax = f * 2^E, f in [0.5, 1): floor(log2 amax) = E-1 */
  int e = (E - 1) - 8;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

/* One row of H bf16 values -> H e4m3 bytes and H/G scale bytes (byte = e+127).
 * rule 0 = R2 (smallest exponent without clipping), rule 1 = R8 (OCP MX).
 * Each group's payload is x * 2^-e, which is exact in double; the encoder
 * saturates what R8 pushes past 448. */
void ora_quant_row_rule(const uint16_t* x, int32_t H, int32_t G, int32_t rule,
                        uint8_t* q, uint8_t* s) {
  for (int32_t g = 0; g < H / G; ++g) {
    double amax = 0.0;
    for (int32_t i = g * G; i < (g + 1) * G; ++i) {
      double v = fabs(bf16_to_double(x[i]));
      if (v > amax) amax = v;
    }
    int e = rule == 1 ? ora_ocp_mx_exponent(amax)
                      : ora_pow2_scale_exponent(amax);
    for (int32_t i = g * G; i < (g + 1) * G; ++i)
      q[i] = ora_e4m3_encode(ldexp(bf16_to_double(x[i]), -e));
    s[g] = (uint8_t)(e + 127);
  }
}

void ora_quant_row(const uint16_t* x, int32_t H, int32_t G, uint8_t* q,
                   uint8_t* s) {
  ora_quant_row_rule(x, H, G, 0, q, s);
}

/* ------------------------------------------------------------- layout */

/* Static compact row bound [P1 Key source snippets, _get_compact_all_tokens]:
 * every non-empty expert takes at least one block, the remaining assignments
 * fill whole blocks: block_e * (n + (A - n) // block_e), n = min(A, E). */
int64_t ora_compact_row_bound(int64_t num_assignments, int32_t num_experts,
                              int32_t block_e) {
  int64_t n = num_assignments < num_experts ? num_assignments : num_experts;
  return (int64_t)block_e * (n + (num_assignments - n) / block_e);
}

/* Layout choice [P1 Key source snippets, _should_use_masked_standard_layout]:
 * masked iff expert parallelism is on (global > local) and local <= 32. */
int32_t ora_should_use_masked(int32_t num_experts, int32_t num_local_experts) {
  return (num_experts > num_local_experts && num_local_experts <= 32) ? 1 : 0;
}

/* Routing -> expert-grouped layout.
 *   kind 0 (compact) [P1 Implementation breakdown items 2-3; P1 Key source
 *     snippets, _fwd_kernel_ep_scatter_1]: expert e owns rows
 *     [offsets[e], offsets[e] + padded_e), padded_e = ceil(c_e/block_e)*block_e;
 *     rows holding an assignment carry m_indices = e, the rest -1 (R4).
 *   kind 1 (masked slab) [P3 Implementation breakdown item 2, Key source
 *     snippets: masked slab [E, max_m, hidden] with masked_m]: expert e owns
 *     rows [e*cap, (e+1)*cap); slots >= cap are dropped and flagged (R5).
 * Slots follow R3.  Returns 0, or 1 if num_rows is too small for the layout
 * (nothing is written then). */
int32_t ora_moe_layout(const int32_t* topk_ids, int64_t T, int32_t K,
                       int32_t expert_begin, int32_t E, int32_t kind,
                       int32_t block_e, int32_t cap, int64_t num_rows,
                       int32_t* counts, int32_t* offsets, int32_t* m_indices,
                       int32_t* masked_m, int32_t* src2dst,
                       int32_t* overflow) {
  int64_t A = T * (int64_t)K;
  int32_t* fill = (int32_t*)calloc((size_t)(E > 0 ? E : 1), sizeof(int32_t));
  int32_t* cnt = (int32_t*)calloc((size_t)(E > 0 ? E : 1), sizeof(int32_t));
  int64_t* off = (int64_t*)calloc((size_t)E + 1, sizeof(int64_t));

  /* a1: histogram of local assignments */
  for (int64_t i = 0; i < A; ++i) {
    int64_t e = (int64_t)topk_ids[i] - expert_begin;
    if (e >= 0 && e < E) cnt[e] += 1;
  }
  /* a2: region starts */
  off[0] = 0;
  for (int32_t e = 0; e < E; ++e) {
    int64_t region;
    if (kind == 0)
      region = ((int64_t)cnt[e] + block_e - 1) / block_e * block_e;
    else
      region = cap;
    off[e + 1] = off[e] + region;
  }
  if (off[E] > num_rows) {
    free(fill); free(cnt); free(off);
    return 1;
  }
  /* a3: stable slots in ascending flat index */
  int32_t ovf = 0;
  for (int64_t i = 0; i < A; ++i) {
    int64_t e = (int64_t)topk_ids[i] - expert_begin;
    if (e < 0 || e >= E) {
      src2dst[i] = -1;
      continue;
    }
    int32_t r = fill[e]++;
    if (kind == 1 && r >= cap) {
      src2dst[i] = -1;
      ovf = 1;
    } else {
      src2dst[i] = (int32_t)(off[e] + r);
    }
  }
  for (int32_t e = 0; e < E; ++e) {
    counts[e] = cnt[e];
    offsets[e] = (int32_t)off[e];
    if (masked_m) masked_m[e] = (kind == 1 && cnt[e] > cap) ? cap : cnt[e];
  }
  offsets[E] = (int32_t)off[E];
  if (m_indices) {
    for (int64_t r = 0; r < num_rows; ++r) m_indices[r] = -1;
    for (int32_t e = 0; e < E; ++e) {
      int32_t live = (kind == 1 && cnt[e] > cap) ? cap : cnt[e];
      for (int32_t r = 0; r < live; ++r) m_indices[off[e] + r] = e;
    }
  }
  *overflow = ovf;
  free(fill); free(cnt); free(off);
  return 0;
}

/* ---------------------------------------------------- scatter + quant */

/* Every token row is quantized once and its bytes are copied to each of its
 * destination rows [P1 Implementation breakdown item 3: fused quant+scatter
 * with UE8M0 scales].  Rows that are no destination are not touched. */
void ora_scatter_quant(const uint16_t* x, int64_t ld_x, int64_t T, int32_t H,
                       const int32_t* src2dst, int32_t K, int32_t G,
                       uint8_t* q, int64_t ld_q, uint8_t* s, int64_t ld_s) {
#pragma omp parallel
  {
    uint8_t* rq = (uint8_t*)malloc((size_t)H);
    uint8_t* rs = (uint8_t*)malloc((size_t)(H / G));
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      int any = 0;
      for (int32_t j = 0; j < K; ++j) any |= src2dst[t * K + j] >= 0;
      if (!any) continue;
      ora_quant_row(x + t * ld_x, H, G, rq, rs);
      for (int32_t j = 0; j < K; ++j) {
        int64_t d = src2dst[t * K + j];
        if (d < 0) continue;
        memcpy(q + d * ld_q, rq, (size_t)H);
        memcpy(s + d * ld_s, rs, (size_t)(H / G));
      }
    }
    free(rq);
    free(rs);
  }
}

/* The same scatter with a choice of exponent rule and of scale placement:
 * scale byte g of row d goes to byte d*s_rs + (g/4)*s_c4 + g%4.  Row-major
 * bytes are s_rs = ld_s, s_c4 = 4; the packed layout with four bytes per
 * 32-bit word and rows contiguous inside each word column (MN-major) is
 * s_rs = 4, s_c4 = 4 * ld_mn [P3 Implementation breakdown item 3 and Review
 * highlights item 3: column-major packed UE8M0 scales]. */
void ora_scatter_quant_ex(const uint16_t* x, int64_t ld_x, int64_t T,
                          int32_t H, const int32_t* src2dst, int32_t K,
                          int32_t G, int32_t rule, uint8_t* q, int64_t ld_q,
                          uint8_t* s, int64_t s_rs, int64_t s_c4) {
#pragma omp parallel
  {
    uint8_t* rq = (uint8_t*)malloc((size_t)H);
    uint8_t* rs = (uint8_t*)malloc((size_t)(H / G));
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      int any = 0;
      for (int32_t j = 0; j < K; ++j) any |= src2dst[t * K + j] >= 0;
      if (!any) continue;
      ora_quant_row_rule(x + t * ld_x, H, G, rule, rq, rs);
      for (int32_t j = 0; j < K; ++j) {
        int64_t d = src2dst[t * K + j];
        if (d < 0) continue;
        memcpy(q + d * ld_q, rq, (size_t)H);
        for (int32_t g = 0; g < H / G; ++g)
          s[d * s_rs + (g / 4) * s_c4 + g % 4] = rs[g];
      }
    }
    free(rq);
    free(rs);
  }
}

/* Send-side quant over live rows only [P4 Features & motivation;
 * Implementation breakdown item 1]: segment g holds rows
 * [g*rows_per_segment, (g+1)*rows_per_segment); its first live[g] rows are
 * quantized, the others are not touched. */
void ora_mx_quant_live_rows(const uint16_t* x, int64_t ld_x,
                            int32_t num_segments, int64_t rows_per_segment,
                            const int32_t* live, int32_t H, int32_t G,
                            uint8_t* q, int64_t ld_q, uint8_t* s,
                            int64_t ld_s) {
  for (int32_t g = 0; g < num_segments; ++g) {
    int64_t n = live[g];
    if (n > rows_per_segment) n = rows_per_segment;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
      int64_t row = (int64_t)g * rows_per_segment + r;
      ora_quant_row(x + row * ld_x, H, G, q + row * ld_q, s + row * ld_s);
    }
  }
}

/* ------------------------------------------------------------- requant */

/* Per-token scaled fp8 -> one per-tensor scale [P2 Implementation breakdown
 * items 1-2], reading R6.  Input scales are per token, fp32, positive. */
void ora_requant_per_token_to_per_tensor(const uint8_t* q_in, int64_t ld_in,
                                         const float* token_scales, int64_t T,
                                         int32_t H, uint8_t* q_out,
                                         int64_t ld_out, float* tensor_scale) {
  float amax = 0.0f;
  for (int64_t t = 0; t < T; ++t) {
    double row = 0.0;
    for (int32_t j = 0; j < H; ++j) {
      double v = fabs(ora_e4m3_decode(q_in[t * ld_in + j]));
      if (v > row) row = v;
    }
    float rq = (float)row * token_scales[t];
    if (rq > amax) amax = rq;
  }
  float S = (amax > 0.0f) ? amax / 448.0f : 1.0f;
  float inv = 1.0f / S;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t j = 0; j < H; ++j) {
      float v = (float)ora_e4m3_decode(q_in[t * ld_in + j]);
      float deq = v * token_scales[t];
      float y = deq * inv;
      q_out[t * ld_out + j] = ora_e4m3_encode((double)y);
    }
  }
  *tensor_scale = S;
}

/* ------------------------------------------------------------- combine */

/* Un-permute with top-k weights [P1 Implementation breakdown item 2 and
 * Risks item 2 (post-permute through src2dst); P3 Implementation breakdown
 * item 3 (top-k weights applied on real rows only)], reading R7.
 * acc_out receives the fp32 accumulator per element. */
void ora_combine_f32(const uint16_t* y, int64_t ld_y, const int32_t* src2dst,
                     const float* w, int64_t T, int32_t K, int32_t H,
                     float* acc_out, int64_t ld_out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t h = 0; h < H; ++h) {
      float acc = 0.0f;
      for (int32_t j = 0; j < K; ++j) {
        int64_t d = src2dst[t * K + j];
        if (d < 0) continue;
        acc = fmaf(w[t * K + j], bf16_to_float(y[d * ld_y + h]), acc);
      }
      acc_out[t * ld_out + h] = acc;
    }
  }
}

/* The same sum in double (exact products, one rounding per addition); the
 * reference for the error bound of the fp32 combine. */
void ora_combine_f64(const uint16_t* y, int64_t ld_y, const int32_t* src2dst,
                     const float* w, int64_t T, int32_t K, int32_t H,
                     double* out, double* abs_sum, int64_t ld_out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t h = 0; h < H; ++h) {
      double acc = 0.0, mag = 0.0;
      for (int32_t j = 0; j < K; ++j) {
        int64_t d = src2dst[t * K + j];
        if (d < 0) continue;
        double p = (double)w[t * K + j] * bf16_to_double(y[d * ld_y + h]);
        acc += p;
        mag += fabs(p);
      }
      out[t * ld_out + h] = acc;
      abs_sum[t * ld_out + h] = mag;
    }
  }
}

/* ------------------------------------------- psum (expanded) layout repack */

/* Expanded layout of a dispatcher [P3 Key source snippets, _build_layout]:
 * expert e owns rows [start_e, psum[e]) with start_e = align(psum[e-1]) and
 * psum[-1] = 0.  A psum entry below its start gives an empty expert. */
static int64_t psum_start(const int32_t* psum, int32_t e, int32_t align) {
  int64_t prev = e == 0 ? 0 : psum[e - 1];
  if (prev < 0) prev = 0;
  return (prev + align - 1) / align * align;
}

static int64_t psum_count(const int32_t* psum, int32_t e, int32_t align) {
  int64_t c = (int64_t)psum[e] - psum_start(psum, e, align);
  return c > 0 ? c : 0;
}

/* m_indices of the contiguous GEMM rebuilt from psum [P3 Implementation
 * breakdown item 3 (m_indices from psum with a static grid); Review
 * highlights item 1 (the tail of each expert's range is masked, so a row
 * past psum[e] never gets e)]: m[r] = e on real rows, -1 elsewhere. */
void ora_m_indices_from_psum(const int32_t* psum, int32_t E, int32_t align,
                             int64_t num_rows, int32_t* m_indices) {
  for (int64_t r = 0; r < num_rows; ++r) m_indices[r] = -1;
  for (int32_t e = 0; e < E; ++e) {
    int64_t s = psum_start(psum, e, align), c = psum_count(psum, e, align);
    for (int64_t j = 0; j < c && s + j < num_rows; ++j) m_indices[s + j] = e;
  }
}

/* Expanded -> masked slab [P3 Implementation breakdown item 3; Key source
 * snippets (_check_expand_roundtrip: masked_m equals the counts, slab row j
 * of expert e equals expanded row start_e + j); Review highlights (overflow
 * fails fast)].  Rows are opaque byte strings of row_bytes; scale entries
 * (elem bytes each, s_cols per row) are addressed with explicit row and
 * column strides on both sides, so column-major packed sources work.
 * Copies min(count, max_m) rows of each expert whose source rows exist;
 * masked_m[e] = that number; returns flags: 1 = some count > max_m,
 * 2 = some real row lies past src_rows. */
int32_t ora_expand_to_masked_slab(
    const uint8_t* x, int64_t ld_x, int64_t src_rows, int64_t row_bytes,
    const uint8_t* xs, int64_t xs_rs, int64_t xs_cs, int32_t s_cols,
    int32_t s_elem, const int32_t* psum, int32_t E, int32_t align,
    int32_t max_m, uint8_t* slab, int64_t ld_slab, uint8_t* slab_s,
    int64_t ss_rs, int64_t ss_cs, int32_t* masked_m) {
  int32_t flags = 0;
  for (int32_t e = 0; e < E; ++e) {
    int64_t s = psum_start(psum, e, align), c = psum_count(psum, e, align);
    if (c > max_m) { flags |= 1; c = max_m; }
    if (s + c > src_rows) { flags |= 2; c = src_rows > s ? src_rows - s : 0; }
    masked_m[e] = (int32_t)c;
    for (int64_t j = 0; j < c; ++j) {
      int64_t dr = (int64_t)e * max_m + j;
      memcpy(slab + dr * ld_slab, x + (s + j) * ld_x, (size_t)row_bytes);
      if (xs && slab_s)
        for (int32_t g = 0; g < s_cols; ++g)
          memcpy(slab_s + dr * ss_rs + g * ss_cs,
                 xs + (s + j) * xs_rs + g * xs_cs, (size_t)s_elem);
    }
  }
  return flags;
}

/* Masked slab -> expanded with the top-k weights fused on real rows only
 * [P3 Implementation breakdown item 3; Key source snippets
 * (_check_expand_roundtrip)]: out[start_e + j] = bf16(w[start_e + j] *
 * slab[e][j]) (one fp32 product, nearest-even rounding; w = NULL copies the
 * row) for j < masked_m[e]; every other expanded row is left untouched. */
void ora_masked_slab_to_expand(const uint16_t* slab, int64_t ld_slab,
                               int32_t H, const int32_t* masked_m,
                               const int32_t* psum, int32_t E, int32_t align,
                               int32_t max_m, const float* w, uint16_t* out,
                               int64_t ld_out, int64_t out_rows) {
  for (int32_t e = 0; e < E; ++e) {
    int64_t s = psum_start(psum, e, align);
    int64_t c = masked_m[e];
    if (c > max_m) c = max_m;
    for (int64_t j = 0; j < c && s + j < out_rows; ++j) {
      const uint16_t* src = slab + ((int64_t)e * max_m + j) * ld_slab;
      uint16_t* dst = out + (s + j) * ld_out;
      for (int32_t h = 0; h < H; ++h) {
        if (w) {
          float v = bf16_to_float(src[h]) * w[s + j];
          dst[h] = ora_bf16_round(v);
        } else {
          dst[h] = src[h];
        }
      }
    }
  }
}

/* ---------------------------------------------- scatter of quantized rows */

/* Rows already quantized by the sender (fp8 payload plus scales) copied to
 * their destination rows [P3 Implementation breakdown item 3 and the
 * deep_gemm.py snippet: on the prefill path the dispatcher's rows are written
 * into the contiguous layout at the offsets its psum gives, with the scales
 * copied through their own strides].  For each (t, j) with 0 <= d =
 * src2dst[t*K + j] < num_rows: row d of out takes row t of x (row_bytes
 * bytes) and, if scales are given, scale entry (d, g) takes entry (t, g) for
 * g < scale_cols (entries of elem bytes at row/column strides in bytes). */
void ora_scatter_rows(const uint8_t* x, int64_t ld_x, int64_t T,
                      int64_t row_bytes, const uint8_t* xs, int64_t xs_rs,
                      int64_t xs_cs, int32_t scale_cols, int32_t elem,
                      const int32_t* src2dst, int32_t K, int64_t num_rows,
                      uint8_t* out, int64_t ld_out, uint8_t* os, int64_t os_rs,
                      int64_t os_cs) {
  for (int64_t t = 0; t < T; ++t)
    for (int32_t j = 0; j < K; ++j) {
      const int64_t d = src2dst[t * K + j];
      if (d < 0 || d >= num_rows) continue;
      memcpy(out + d * ld_out, x + t * ld_x, (size_t)row_bytes);
      if (xs == NULL) continue;
      for (int32_t g = 0; g < scale_cols; ++g)
        memcpy(os + d * os_rs + (int64_t)g * os_cs,
               xs + t * xs_rs + (int64_t)g * xs_cs, (size_t)elem);
    }
}

/* ------------------------------------------------------ receive-side upscale */

/* fp8 payload with group-G fp32 scales -> bf16, over the first `rows` rows
 * [P4 Implementation breakdown item 3 and the aiter.py snippet: an fp8
 * dispatch carries group-128 fp32 scales, and the receiver turns it back into
 * bf16 for the first num_local_tokens rows before a kernel that wants bf16].
 * Scale of (r, channel h) at scales[r * s_rs + (h / G) * s_cs] (R9). */
void ora_upscale_fp8(const uint8_t* q, int64_t ld_q, const float* scales,
                     int64_t s_rs, int64_t s_cs, int64_t rows, int32_t H,
                     int32_t G, uint16_t* out, int64_t ld_out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int32_t h = 0; h < H; ++h) {
      double s = (double)scales[r * s_rs + (int64_t)(h / G) * s_cs];
      out[r * ld_out + h] = ora_bf16_round_f64(ora_e4m3_decode(q[r * ld_q + h]) * s);
    }
}

/* ------------------------------------------------ weight-side block requant */

/* UE8M0 block requant of block-scaled fp8 weights (R10) [P1 Implementation
 * breakdown item 1 and the fp8.py snippet: the gate/up and down expert
 * weights of a standard MoE layer are requantized to UE8M0 block scales at
 * load time, with bf16 as the dequantized type].  B matrices of [N, K] e4m3
 * (row stride ld, matrix stride q_bs); inverse scales s_inv [B, ceil(N/bn),
 * ceil(K/bk)] fp32 (row stride s_ld, matrix stride s_bs): weight = dec(q) *
 * s_inv of its block.  Writes q_out (same strides as q; may be q itself) and
 * one scale byte per block to s_out (row stride o_ld, matrix stride o_bs). */
void ora_requant_weight_block_ue8m0(const uint8_t* q, int64_t ld, int64_t q_bs,
                                    const float* s_inv, int64_t s_ld,
                                    int64_t s_bs, int32_t B, int32_t N,
                                    int32_t K, int32_t bn, int32_t bk,
                                    uint8_t* q_out, uint8_t* s_out,
                                    int64_t o_ld, int64_t o_bs) {
  const int32_t nbn = (N + bn - 1) / bn, nbk = (K + bk - 1) / bk;
#pragma omp parallel
  {
    uint16_t* w = (uint16_t*)malloc((size_t)bn * (size_t)bk * sizeof(uint16_t));
#pragma omp for collapse(3) schedule(static)
    for (int32_t b = 0; b < B; ++b)
      for (int32_t i = 0; i < nbn; ++i)
        for (int32_t j = 0; j < nbk; ++j) {
          const int32_t r0 = i * bn, c0 = j * bk;
          const int32_t nr = (N - r0 < bn) ? N - r0 : bn;
          const int32_t nc = (K - c0 < bk) ? K - c0 : bk;
          const double si = (double)s_inv[b * s_bs + (int64_t)i * s_ld + j];
          double amax = 0.0;
          for (int32_t r = 0; r < nr; ++r)
            for (int32_t c = 0; c < nc; ++c) {
              const uint8_t v = q[b * q_bs + (int64_t)(r0 + r) * ld + c0 + c];
              const uint16_t h = ora_bf16_round_f64(ora_e4m3_decode(v) * si);
              w[r * bk + c] = h;
              const double m = fabs(bf16_to_double(h));
              if (m > amax) amax = m;
            }
          const int e = ora_pow2_scale_exponent(amax);
          for (int32_t r = 0; r < nr; ++r)
            for (int32_t c = 0; c < nc; ++c)
              q_out[b * q_bs + (int64_t)(r0 + r) * ld + c0 + c] =
                  ora_e4m3_encode(ldexp(bf16_to_double(w[r * bk + c]), -e));
          s_out[b * o_bs + (int64_t)i * o_ld + j] = (uint8_t)(e + 127);
        }
    free(w);
  }
}
