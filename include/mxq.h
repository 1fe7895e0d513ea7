/*
 * mxq.h - MoE expert-dispatch preprocessing with fp8 e4m3 activations and
 * power-of-two group scales, for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libmxq.so.  Every entry point takes plain pointers and sizes.
 *
 * Sources (summaries of sglang pull requests):
 *   [P1] sglang PR #33128 page - DeepGEMM under the standard MoE dispatcher:
 *        compact layout with a static row bound, -1 expert index on padding
 *        rows, direct UE8M0 activation quant.
 *   [P2] sglang PR #14162 page - DeepEP low-latency dispatch in fp8: a
 *        per-token -> per-tensor fp8 requant step.
 *   [P3] sglang PR #29525 page - DeepEPv2 backend: psum (block-aligned)
 *        layout, masked slab [E, max_m, hidden] with masked_m, fused top-k
 *        weights on real rows only, fail-fast overflow.
 *   [P4] sglang PR #36119 page - MXFP8 dispatch on MI355X: send-side quant
 *        over live tokens, one e8m0 byte per 32 channels (224 at hidden 7168).
 *
 * Conventions shared by every call:
 *   - Device pointers are HIP device memory; "host" marks the exceptions.
 *     The caller owns every buffer.  The library allocates nothing and keeps
 *     no state between calls, so calls are re-entrant.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on it and returns without waiting, except
 *     moe_read_overflow, which waits for the stream.
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     failed check returns MXQ_ERR_INVALID_ARGUMENT (or MXQ_ERR_UNSUPPORTED
 *     for a format or size the library does not implement, MXQ_ERR_WORKSPACE
 *     for a short workspace) and enqueues nothing.  MXQ_ERR_HIP means a kernel
 *     launch was rejected by the runtime.
 *   - Launch geometry depends only on the host arguments, never on device
 *     data, so every call can be captured in a hipGraph and replayed.
 *   - Row offsets are 64-bit internally; row indices stored in int32 arrays
 *     limit a layout to 2^31 - 1 rows.
 *   - bf16 = bfloat16 (upper half of an IEEE binary32).  fp8 = OCP e4m3fn
 *     (bias 7, largest finite 448, no infinities).  A scale byte b means the
 *     factor 2^(b - 127) (UE8M0 / e8m0).
 *   - Vector rows: bf16 and fp8 row starts must be 16-byte aligned (base
 *     pointer 16-byte aligned, row stride a multiple of 16 bytes).
 *   - Inputs are finite; NaN or infinite activations give unspecified bytes.
 */
#ifndef MXQ_H
#define MXQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXQ_ABI_VERSION 1
#define MXQ_MAX_LOCAL_EXPERTS 1024
#define MXQ_MAX_TOPK 64
#define MXQ_MAX_ASSIGNMENTS (1 << 24) /* T*K limit of moe_layout */
#define MXQ_MAX_HIDDEN 32768 /* moe_scatter_quant stages one row in LDS */
/* Static device scratch of moe_layout_noalloc, per device (1 MiB). */
#define MXQ_LAYOUT_NOALLOC_SCRATCH_BYTES (1u << 20)

typedef enum {
  MXQ_OK = 0,
  MXQ_ERR_INVALID_ARGUMENT = 1,
  MXQ_ERR_UNSUPPORTED = 2,
  MXQ_ERR_CAPACITY_OVERFLOW = 3,
  MXQ_ERR_WORKSPACE = 4,
  MXQ_ERR_HIP = 5,
  MXQ_ERR_SCRATCH_LIMIT = 6 /* beyond the library's static scratch */
} mxq_status;

typedef enum { MXQ_LAYOUT_COMPACT = 0, MXQ_LAYOUT_MASKED = 1 } mxq_layout_kind;

/* Both formats store one byte per group meaning 2^(b-127); the exponent is
 * the smallest e with amax(group) <= 448 * 2^e, clamped to [-127, 127]. */
typedef enum {
  MXQ_SCALE_UE8M0_G128 = 0, /* 128 channels per scale [P1 impl. item 3] */
  MXQ_SCALE_E8M0_G32 = 1    /* 32 channels per scale  [P4 impl. item 1] */
} mxq_scale_fmt;

/* Exponent rule for the *_ex quantizers.  MXQ_RULE_NO_CLIP is the rule
 * above.  MXQ_RULE_OCP_FLOOR is the OCP Microscaling shared exponent
 * floor(log2 amax) - 8 (8 = largest e4m3 exponent), clamped to [-127, 127]:
 * payload values then reach up to 2^9 and are clamped to +-448 before
 * conversion. */
typedef enum { MXQ_RULE_NO_CLIP = 0, MXQ_RULE_OCP_FLOOR = 1 } mxq_scale_rule;

typedef enum { MXQ_OUT_BF16 = 0, MXQ_OUT_F32 = 1 } mxq_out_dtype;

/* ------------------------------------------------------------ host-only */

/* Static row count of the compact layout that no routing can exceed
 * [P1 Key source snippets, _get_compact_all_tokens]:
 *   block_e * (n + (A - n) / block_e), n = min(A, E):
 * each non-empty expert takes one block for its first assignment, so the
 * worst case has min(A, E) non-empty experts and every other assignment
 * packed into whole blocks.
 * Pure host function.  Returns -1 if an argument is negative or block_e < 1. */
int64_t moe_compact_row_bound(int64_t num_assignments,
                              int32_t num_local_experts, int32_t block_e);

/* Layout choice [P1 Key source snippets, _should_use_masked_standard_layout]:
 * 1 (masked slab) iff num_experts > num_local_experts and
 * num_local_experts <= 32, else 0 (compact).  Pure host function. */
int32_t moe_should_use_masked(int32_t num_experts, int32_t num_local_experts);

/* Workspace bytes moe_layout needs for T tokens, top-K, E local experts: 0
 * when T*K <= 4096, or T*K <= 2^14 with E <= 256 (the layout then runs as
 * one launch that counts the whole routing in every block), else the
 * per-chunk expert counts of its histogram launch. */
size_t moe_layout_workspace_bytes(int64_t T, int32_t K, int32_t E);

/* Workspace bytes requant_per_token_to_per_tensor needs. */
size_t requant_workspace_bytes(int64_t T, int32_t H);

/* ----------------------------------------------------------------- layout */

/* Lay top-k routing out by expert [P1 impl. items 2-3 and Key source snippets
 * (_fwd_kernel_ep_scatter_1); P3 impl. items 2-3 (masked slab, masked_m)].
 *
 *   topk_ids      int32 [T, K] row-major, global expert ids.  Assignment
 *                 (t, j) is local iff e = topk_ids[t*K+j] - expert_begin lies
 *                 in [0, num_local_experts).
 *   kind          MXQ_LAYOUT_COMPACT: expert e owns rows
 *                   [expert_offsets[e], expert_offsets[e+1]) whose length is
 *                   ceil(c_e / block_e) * block_e (0 for an empty expert),
 *                   regions in ascending e.  num_rows must be at least
 *                   moe_compact_row_bound(T*K, E, block_e).
 *                 MXQ_LAYOUT_MASKED: expert e owns rows [e*capacity,
 *                   (e+1)*capacity); num_rows must be >= E*capacity.
 *   Slots: the i-th local assignment of expert e in ascending flat index
 *   t*K+j gets row expert_offsets[e] + i (deterministic).
 *
 * Outputs (all written by every call; no prior clearing needed):
 *   counts         int32 [E]    c_e, the local assignments of expert e.
 *   expert_offsets int32 [E+1]  region starts; [E] = end of the last region.
 *   m_indices      int32 [num_rows] or NULL: e on rows holding an assignment
 *                  of e, -1 on every other row (padding and tail rows).
 *   masked_m       int32 [E] or NULL: min(c_e, capacity) (masked) or c_e.
 *   src2dst        int32 [T, K]: destination row, -1 for a non-local
 *                  assignment or (masked) a slot >= capacity.
 *   overflow_flag  int32 [1]: 1 if some expert exceeded the slab capacity
 *                  (masked), else 0.  Overflowing assignments are dropped,
 *                  never written out of bounds; read with moe_read_overflow.
 *   workspace      >= moe_layout_workspace_bytes(T, K, E) bytes, device.
 * Limits: 1 <= E <= MXQ_MAX_LOCAL_EXPERTS, 1 <= K <= MXQ_MAX_TOPK,
 * num_rows < 2^31 (else MXQ_ERR_INVALID_ARGUMENT), T*K <= MXQ_MAX_ASSIGNMENTS
 * (else MXQ_ERR_UNSUPPORTED).  T = 0 is valid (regions empty, m_indices all
 * -1). */
mxq_status moe_layout(const int32_t* topk_ids, int64_t T, int32_t K,
                      int32_t expert_begin, int32_t num_local_experts,
                      mxq_layout_kind kind, int32_t block_e, int32_t capacity,
                      int64_t num_rows, int32_t* counts,
                      int32_t* expert_offsets, int32_t* m_indices,
                      int32_t* masked_m, int32_t* src2dst,
                      int32_t* overflow_flag, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Host read of the overflow flag written by moe_layout.  Waits for `stream`.
 * host_value (host) receives the flag; returns MXQ_ERR_CAPACITY_OVERFLOW if
 * it is set, MXQ_OK otherwise [P3 Review highlights: overflow fails fast]. */
mxq_status moe_read_overflow(const int32_t* overflow_flag, int32_t* host_value,
                             void* stream);

/* moe_layout without a workspace argument, for callers that cannot allocate
 * device memory (code under hipGraph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Arguments, outputs and results are those of
 * moe_layout; the per-chunk counts that moe_layout keeps in the caller's
 * workspace live instead in a static device array of the library,
 * MXQ_LAYOUT_NOALLOC_SCRATCH_BYTES per device, held until the process ends.
 * A routing whose moe_layout_workspace_bytes(T, K, E) exceeds that returns
 * MXQ_ERR_SCRATCH_LIMIT and enqueues nothing (8192 tokens, top-8 over 384
 * experts need 96 KiB; routings for which moe_layout needs no workspace use
 * none of it).  The call allocates nothing.  Its first call on a device
 * looks up that device's copy of the array (a host query, no allocation);
 * make it outside graph capture.  Every call on one device shares the array:
 * calls that overlap on one device (e.g. on two streams) race and must be
 * ordered by the caller.  The array needs no clearing: each call overwrites
 * what it reads.  The stream's device is the one used. */
mxq_status moe_layout_noalloc(const int32_t* topk_ids, int64_t T, int32_t K,
                              int32_t expert_begin, int32_t num_local_experts,
                              mxq_layout_kind kind, int32_t block_e,
                              int32_t capacity, int64_t num_rows,
                              int32_t* counts, int32_t* expert_offsets,
                              int32_t* m_indices, int32_t* masked_m,
                              int32_t* src2dst, int32_t* overflow_flag,
                              void* stream);

/* ---------------------------------------------------------- scatter + quant */

/* Quantize each token row once and scatter it to its destination rows
 * [P1 impl. item 3: fused quant + scatter with UE8M0 scales computed
 * directly; P1 Key source snippets].
 *
 *   x        bf16 [T, ld_x] device, the first H columns of each row are used.
 *   src2dst  int32 [T, K] from moe_layout (either kind); entries < 0 or
 *            >= num_rows are skipped.
 *   fmt      group size and scale format.  H must be a multiple of the group.
 *   q        fp8 [num_rows, ld_q]; for every destination row d of token t the
 *            first H bytes become e4m3(x[t, i] * 2^-e_g).
 *   scales   uint8 [num_rows, ld_s]; byte g of row d becomes e_g + 127,
 *            ld_s >= H / G (any stride, padded strides allowed).
 * Rows that are no destination are not written (padding keeps whatever the
 * caller left there; consumers skip them through m_indices = -1).
 * H <= MXQ_MAX_HIDDEN, else MXQ_ERR_UNSUPPORTED. */
mxq_status moe_scatter_quant(const void* x_bf16, int64_t ld_x, int64_t T,
                             int32_t H, const int32_t* src2dst, int32_t K,
                             mxq_scale_fmt fmt, void* q_fp8, int64_t ld_q,
                             uint8_t* scales, int64_t ld_s, int64_t num_rows,
                             void* stream);

/* moe_layout followed by moe_scatter_quant in one launch, for routings of
 * at most 4096 assignments (decode batches) [P2 impl. items 1-2: the
 * low-latency decode dispatch; P1 impl. item 3: quant fused with the
 * scatter].  One block per token ranks its own assignments from per-expert
 * counts of the whole routing, so no separate layout launch is needed.
 *
 * Arguments are those of moe_layout (no workspace) followed by those of
 * moe_scatter_quant (x_bf16 [T, ld_x], H, fmt, q_fp8 [num_rows, ld_q],
 * scales [num_rows, ld_s], row-major scale bytes, exponent rule of
 * moe_scatter_quant).  Every output (counts, expert_offsets, m_indices,
 * masked_m, src2dst, overflow_flag, q, scales) is byte-identical to the two
 * calls; rows that are no destination are not written.  A token's row may be
 * read even when none of its experts is local.
 * Errors: those of the two calls; T*K > 4096 is MXQ_ERR_UNSUPPORTED (use the
 * two calls).  T = 0 runs the layout alone. */
mxq_status moe_layout_scatter_quant(
    const int32_t* topk_ids, int64_t T, int32_t K, int32_t expert_begin,
    int32_t num_local_experts, mxq_layout_kind kind, int32_t block_e,
    int32_t capacity, int64_t num_rows, int32_t* counts,
    int32_t* expert_offsets, int32_t* m_indices, int32_t* masked_m,
    int32_t* src2dst, int32_t* overflow_flag, const void* x_bf16,
    int64_t ld_x, int32_t H, mxq_scale_fmt fmt, void* q_fp8, int64_t ld_q,
    uint8_t* scales, int64_t ld_s, void* stream);

/* moe_scatter_quant with a choice of exponent rule and of scale placement
 * [P3 impl. item 3 and Review highlights item 3: consumers read scales
 * column-major with four UE8M0 bytes packed per 32-bit word].  Scale byte g
 * of row d is written to scales + d*scale_row_stride +
 * (g/4)*scale_quad_stride + g%4.  Two placements are accepted:
 *   row-major bytes:  scale_quad_stride = 4, scale_row_stride >= H/G;
 *   packed MN-major:  scale_row_stride = 4, scale_quad_stride a multiple of
 *                     4 and >= 4*num_rows (int32 [ceil(H/G/4), ld], rows
 *                     contiguous, ld = scale_quad_stride / 4).
 * moe_scatter_quant(..., ld_s, ...) is this call with MXQ_RULE_NO_CLIP,
 * scale_row_stride = ld_s and scale_quad_stride = 4. */
mxq_status moe_scatter_quant_ex(const void* x_bf16, int64_t ld_x, int64_t T,
                                int32_t H, const int32_t* src2dst, int32_t K,
                                mxq_scale_fmt fmt, mxq_scale_rule rule,
                                void* q_fp8, int64_t ld_q, void* scales,
                                int64_t scale_row_stride,
                                int64_t scale_quad_stride, int64_t num_rows,
                                void* stream);

/* Scale placement read directly by gfx950's block-scaled MFMA
 * (v_mfma_scale_f32_32x32x64_f8f6f4 with tile_m = 32, or
 * v_mfma_scale_f32_16x16x128_f8f6f4 with tile_m = 16) when the quantized
 * rows are its A operand [P3 Review highlights item 3 and P4 impl.
 * item 1: scales are stored the way the consuming GEMM reads them].  One
 * instruction covers a tile of tile_m rows by 64*32/tile_m channels; the
 * scale of its 32-channel block h (h < 64/tile_m) of row r is read from lane
 * l = h*tile_m + r as one byte of a 32-bit register, selected by op_sel, so
 * one register serves four consecutive instructions.  Byte
 * offset of the scale of 32-channel block kb of row d:
 *     ((d / tile_m) * nkg + kb / (4 * 64/tile_m)) * 256
 *   + ((kb % (64/tile_m)) * tile_m + d % tile_m) * 4
 *   + (kb / (64/tile_m)) % 4,
 * nkg = ceil((H/32) / (4 * 64/tile_m)): per row tile, nkg runs of 64 words,
 * one word per lane.  With group 128 each scale byte is written to its four
 * 32-channel blocks (the instruction's block is 32 channels).  Bytes of rows
 * past the last row and of blocks past H/32 are never written.
 *
 * Size of that placement for `rows` rows (rounded up to whole tiles) of H
 * channels: ceil(rows / tile_m) * nkg * 256 bytes.  Returns -1 unless
 * rows >= 0, H > 0, H % 32 == 0 and tile_m is 16 or 32.  Pure host function. */
int64_t mxq_mfma_scale_bytes(int64_t rows, int32_t H, int32_t tile_m);

/* moe_scatter_quant_ex with the scales in the block-scaled MFMA placement
 * above: `scales` holds mxq_mfma_scale_bytes(num_rows, H, tile_m) bytes and
 * is 4-byte aligned (whole 32-bit words are written).  Errors as
 * moe_scatter_quant_ex; tile_m other than 16 or 32, or an unaligned
 * `scales`, is MXQ_ERR_INVALID_ARGUMENT. */
mxq_status moe_scatter_quant_mfma(const void* x_bf16, int64_t ld_x, int64_t T,
                                  int32_t H, const int32_t* src2dst,
                                  int32_t K, mxq_scale_fmt fmt,
                                  mxq_scale_rule rule, void* q_fp8,
                                  int64_t ld_q, void* scales, int32_t tile_m,
                                  int64_t num_rows, void* stream);

/* Send-side quant over live rows only [P4 Features & motivation and impl.
 * item 1: quantize on the sender over the live tokens, not the padded
 * receive buffer; 224 one-byte scales per 7168-wide row].
 *
 *   x            bf16 [num_segments * rows_per_segment, ld_x].
 *   live_counts  int32 [num_segments] device: segment g's live rows are
 *                [g*rows_per_segment, g*rows_per_segment + live_counts[g]);
 *                counts are clipped to [0, rows_per_segment].
 *   q, scales    same layout as the input rows; only live rows are written.
 * The grid is sized from the host arguments; blocks beyond the live rows
 * return at once. */
mxq_status mx_quant_live_rows(const void* x_bf16, int64_t ld_x,
                              int32_t num_segments, int64_t rows_per_segment,
                              const int32_t* live_counts, int32_t H,
                              mxq_scale_fmt fmt, void* q_fp8, int64_t ld_q,
                              uint8_t* scales, int64_t ld_s, void* stream);

/* mx_quant_live_rows with an exponent rule and a scale placement, as in
 * moe_scatter_quant_ex (the packed placement needs scale_quad_stride >= 4 *
 * num_segments * rows_per_segment). */
mxq_status mx_quant_live_rows_ex(const void* x_bf16, int64_t ld_x,
                                 int32_t num_segments, int64_t rows_per_segment,
                                 const int32_t* live_counts, int32_t H,
                                 mxq_scale_fmt fmt, mxq_scale_rule rule,
                                 void* q_fp8, int64_t ld_q, void* scales,
                                 int64_t scale_row_stride,
                                 int64_t scale_quad_stride, void* stream);

/* mx_quant_live_rows_ex with the scales in the block-scaled MFMA placement
 * (see mxq_mfma_scale_bytes): `scales` holds
 * mxq_mfma_scale_bytes(num_segments * rows_per_segment, H, tile_m) bytes and
 * only the bytes of live rows are written. */
mxq_status mx_quant_live_rows_mfma(const void* x_bf16, int64_t ld_x,
                                   int32_t num_segments,
                                   int64_t rows_per_segment,
                                   const int32_t* live_counts, int32_t H,
                                   mxq_scale_fmt fmt, mxq_scale_rule rule,
                                   void* q_fp8, int64_t ld_q, void* scales,
                                   int32_t tile_m, void* stream);

/* --------------------------------------------------------- diagnostics */

/* Bandwidth reference, not a step of the path: copies `bytes` (a multiple of
 * 16) from src to dst (both device, 16-byte aligned, not overlapping) with
 * 16-byte vector loads and stores, four loads in flight per lane.
 * `nontemporal` bit 0 makes the stores non-temporal, bit 1 the loads (values
 * 0-3; others: MXQ_ERR_INVALID_ARGUMENT).  Timing it beside the path's
 * kernels gives the box's achievable copy rate. */
mxq_status mxq_copy16(const void* src, void* dst, int64_t bytes,
                      int32_t nontemporal, void* stream);

/* Bandwidth reference, not a step of the path: the combine's reads alone.
 * Block g (g < groups) reads rows idx[g*group + j], j < group (entries
 * outside [0, num_rows) are skipped), row_bytes bytes each (a multiple of
 * 16) at row stride ld (bytes, a multiple of 16; rows 16-byte aligned),
 * with the combine's pattern: a lane loads 16 bytes of each of the group's
 * rows, all in flight, non-temporal.  sink[g] (device uint32 [groups])
 * receives the XOR of the 32-bit words the block read.  1 <= group <= 64. */
mxq_status mxq_gather_read16(const void* rows, int64_t ld, int64_t num_rows,
                             const int32_t* idx, int64_t groups, int32_t group,
                             int64_t row_bytes, uint32_t* sink, void* stream);

/* Bandwidth reference, not a step of the path: the combine's writes alone.
 * Writes `pattern` to every 32-bit word of rows [0, rows) of dst (row_bytes
 * each, a multiple of 16, at row stride ld bytes; 16-byte aligned), one
 * block per row, 16-byte streaming stores. */
mxq_status mxq_fill_rows16(void* dst, int64_t ld, int64_t rows,
                           int64_t row_bytes, uint32_t pattern, void* stream);

/* ------------------------------------------------------------- requant */

/* Per-token scaled fp8 -> one per-tensor scale [P2 impl. items 1-2].
 *
 *   q_in          fp8 [T, ld_in]; token_scales fp32 [T] (positive, finite).
 *   q_out         fp8 [T, ld_out]; may equal q_in when ld_out == ld_in.
 *   tensor_scale  fp32 [1] device: S = fl(amax / 448) where
 *                 amax = max_t fl(max_i |dec(q_in[t,i])| * s_t); S = 1 when
 *                 amax = 0.  q_out = e4m3(fl(fl(dec(q_in) * s_t) * fl(1/S))).
 *   workspace     >= requant_workspace_bytes(T, H) bytes, device.
 * Two kernels: a max pass, then the requant pass.  The max pass skips rows
 * whose bound fl(448 * s_t) cannot raise the maximum (the result is the
 * same); NaN codes in q_in are outside this contract and give an
 * unspecified S. */
mxq_status requant_per_token_to_per_tensor(
    const void* q_in_fp8, int64_t ld_in, const float* token_scales, int64_t T,
    int32_t H, void* q_out_fp8, int64_t ld_out, float* tensor_scale,
    void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------- combine */

/* Un-permute expert outputs to tokens with the top-k weights [P1 impl. item 2
 * and Risks item 2 (post-permute through src2dst); P3 impl. item 3 (top-k
 * weights fused on real rows only)].
 *
 *   y             bf16 [num_rows, ld_y] expert outputs in layout order.
 *   src2dst       int32 [T, K]; entries < 0 or >= num_rows are skipped, so
 *                 padding rows are never read.
 *   topk_weights  fp32 [T, K].
 *   out           [T, ld_out], bf16 or fp32 per out_dtype:
 *                 acc = +0; for j = 0..K-1 with a valid row:
 *                 acc = fma(w[t,j], y[row, i], acc); out = acc rounded to
 *                 nearest-even bf16, or acc itself for fp32.
 * H must be a multiple of 8. */
mxq_status moe_combine(const void* y_bf16, int64_t ld_y, int64_t num_rows,
                       const int32_t* src2dst, const float* topk_weights,
                       int64_t T, int32_t K, int32_t H, void* out,
                       int64_t ld_out, mxq_out_dtype out_dtype, void* stream);

/* ------------------------------------------------ psum (expanded) layout */

/* The expanded layout a dispatcher hands over [P3 Key source snippets,
 * _build_layout]: expert e owns rows [start_e, psum[e]) with
 * start_e = align(psum[e-1]), psum[-1] = 0; psum (device, int32 [E]) must be
 * non-decreasing (other values give unspecified but in-bounds results). */

/* m_indices of the contiguous grouped GEMM from psum [P3 impl. item 3
 * (m_indices from psum, static grid); Review highlights item 1 (each range's
 * tail is masked)]: m_indices[r] = e for r in [start_e, psum[e]), -1 for
 * every other r < num_rows.  m_indices int32 [num_rows], device. */
mxq_status moe_m_indices_from_psum(const int32_t* psum, int32_t E,
                                   int32_t align, int64_t num_rows,
                                   int32_t* m_indices, void* stream);

/* Expanded rows -> masked slab [P3 impl. item 3 (scales copied by the
 * source's pack-dim stride); Key source snippets (masked_m equals the
 * counts; slab row j of expert e is expanded row start_e + j); Review
 * highlights (over-capacity must fail fast, never truncate silently)].
 *
 *   x            src_rows rows of row_bytes bytes, row stride ld_x bytes
 *                (any payload: fp8, bf16, ...); row_bytes % 16 == 0.
 *   x_scales     optional: scale_cols entries of scale_elem_bytes (1 or 4)
 *                per row, entry (r, g) at r*xs_row_stride + g*xs_col_stride
 *                bytes (row- or column-major sources alike).
 *   slab         [E * max_m] rows, stride ld_slab bytes; slab_scales entry
 *                (row, g) at row*ss_row_stride + g*ss_col_stride bytes.
 *   masked_m     int32 [E]: rows copied for expert e, min(count, max_m),
 *                also limited to rows that exist in the source.
 *   flags        int32 [1]: bit 0 = some count > max_m, bit 1 = some range
 *                reaches past src_rows; read with moe_read_overflow.
 * Only rows [0, masked_m[e]) of each expert's slab are written. */
mxq_status moe_expand_to_masked_slab(
    const void* x, int64_t ld_x, int64_t src_rows, int64_t row_bytes,
    const void* x_scales, int64_t xs_row_stride, int64_t xs_col_stride,
    int32_t scale_cols, int32_t scale_elem_bytes, const int32_t* psum,
    int32_t E, int32_t align, int32_t max_m, void* slab, int64_t ld_slab,
    void* slab_scales, int64_t ss_row_stride, int64_t ss_col_stride,
    int32_t* masked_m, int32_t* flags, void* stream);

/* Masked slab -> expanded rows with the top-k weights applied on real rows
 * only [P3 impl. item 3 (top-k weights fused in the kernel); Key source
 * snippets (round trip expanded <-> slab)].  For j < min(masked_m[e], max_m)
 * and start_e + j < out_rows: out[start_e + j] = bf16(w[start_e + j] *
 * slab[e*max_m + j]) (fp32 product, one nearest-even rounding), or a plain
 * copy when weights is NULL.  Every other output row is left untouched.
 * masked_m[e] must not reach past the expert's region (start_{e+1} -
 * start_e rows), which holds for the values moe_expand_to_masked_slab
 * writes; a larger value gives unspecified but in-bounds results.
 *   slab_bf16 [E * max_m, ld_slab], out_bf16 [out_rows, ld_out] (elements),
 *   weights fp32 [out_rows] or NULL; H % 8 == 0. */
mxq_status moe_masked_slab_to_expand(
    const void* slab_bf16, int64_t ld_slab, int32_t H, const int32_t* masked_m,
    const int32_t* psum, int32_t E, int32_t align, int32_t max_m,
    const float* weights, void* out_bf16, int64_t ld_out, int64_t out_rows,
    void* stream);

/* ------------------------------------------- receive-side upscale (fp8) */

/* fp8 payload with fp32 group scales -> bf16, over the first num_rows rows
 * [P4 impl. item 3 and the aiter.py snippet: an fp8 dispatch carries
 * group-128 fp32 scales and is turned back into bf16 for the live rows
 * (num_local_tokens) before a kernel that consumes bf16].
 *
 *   q_fp8    e4m3 [num_rows, ld_q] bytes, ld_q % 16 == 0, 16-byte aligned.
 *   scales   fp32; scale of (row r, channel c) at
 *            scales[r*scale_row_stride + (c/group)*scale_col_stride]
 *            (row-major [rows, H/group]: strides (H/group, 1); MN-major
 *            [H/group, rows]: strides (1, rows)).
 *   out      bf16 [num_rows, ld_out], ld_out % 8 == 0, 16-byte aligned:
 *            out = bf16(dec(q) * s), the exact product rounded once to
 *            nearest-even (overflow to inf); a NaN result is 0x7FC0.
 *   group    32 or 128 (others: MXQ_ERR_UNSUPPORTED); H % group == 0.
 * Rows at or past num_rows are not touched. */
mxq_status upscale_fp8_to_bf16(const void* q_fp8, int64_t ld_q,
                               const float* scales, int64_t scale_row_stride,
                               int64_t scale_col_stride, int64_t num_rows,
                               int32_t H, int32_t group, void* out_bf16,
                               int64_t ld_out, void* stream);

/* ------------------------------------------ weight-side UE8M0 requant */

/* Block-scaled fp8 weights -> fp8 with one UE8M0 (power-of-two) scale per
 * 128 x 128 block [P1 impl. item 1 and the fp8.py snippet: the gate/up and
 * down expert weights of a standard MoE layer are requantized to UE8M0
 * block scales at load time, with bf16 as the dequantized type].
 *
 *   q_fp8      num_matrices matrices of e4m3 [N, K]: element (m, n, k) at
 *              m*matrix_stride + n*ld + k bytes; K % 16 == 0, ld % 16 == 0,
 *              16-byte aligned.
 *   s_inv      fp32 inverse scales [m][ceil(N/128)][ceil(K/128)] at
 *              m*s_matrix_stride + i*s_ld + j: weight = dec(q) * s_inv.
 *   q_out      same geometry as q_fp8; may be q_fp8 itself (in place), must
 *              not overlap it otherwise.
 *   scales_out one byte per block at m*o_matrix_stride + i*o_ld + j:
 *              e + 127, where w = bf16(dec(q) * s_inv) (exact product, one
 *              rounding), e is the smallest integer with max|w| over the
 *              block <= 448 * 2^e (clamped to [-127, 127]), and
 *              q_out = e4m3(w * 2^-e) (nearest-even).
 *   block_n, block_k must be 128 (others: MXQ_ERR_UNSUPPORTED).
 * Inputs must be finite (no NaN bytes, finite products). */
mxq_status requant_weight_block_ue8m0(
    const void* q_fp8, int64_t ld, int64_t matrix_stride, const float* s_inv,
    int64_t s_ld, int64_t s_matrix_stride, int32_t num_matrices, int32_t N,
    int32_t K, int32_t block_n, int32_t block_k, void* q_out,
    uint8_t* scales_out, int64_t o_ld, int64_t o_matrix_stride, void* stream);

/* Already-quantized rows (and their scales) written to their destination
 * rows [P3 impl. item 3 and the deep_gemm.py snippet: on the prefill path
 * the dispatcher's fp8 rows go into the contiguous layout at its psum
 * offsets, scales copied through their own strides].  The psum geometry is
 * the compact layout's (regions start at align(psum[e-1])), so moe_layout
 * with block_e = the alignment gives the destinations in src2dst.
 *
 *   x            T rows of row_bytes bytes (row_bytes % 16 == 0), row stride
 *                ld_x bytes, 16-byte aligned.
 *   x_scales     optional: scale_cols entries of scale_elem_bytes (1 or 4)
 *                per row, entry (t, g) at t*xs_row_stride + g*xs_col_stride
 *                bytes; out_scales entry (d, g) at d*os_row_stride +
 *                g*os_col_stride bytes (row- or column-major alike).
 *   src2dst      int32 [T, K]; entries outside [0, num_rows) are skipped.
 *   out          num_rows rows, stride ld_out bytes (% 16), 16-byte aligned.
 * For each (t, j) with a valid destination d, row d of out (and its scale
 * entries) takes row t of x.  Rows that are no destination are untouched. */
mxq_status moe_scatter_rows(const void* x, int64_t ld_x, int64_t T,
                            int64_t row_bytes, const void* x_scales,
                            int64_t xs_row_stride, int64_t xs_col_stride,
                            int32_t scale_cols, int32_t scale_elem_bytes,
                            const int32_t* src2dst, int32_t K,
                            int64_t num_rows, void* out, int64_t ld_out,
                            void* out_scales, int64_t os_row_stride,
                            int64_t os_col_stride, void* stream);

/* ---------------------------------------------------------- diagnostics */

/* The fp32 -> e4m3fn conversion every kernel above uses, exposed so it can
 * be checked value by value (OCP e4m3fn, nearest-even).  Defined for
 * |x| < 464; larger inputs are outside the contract of the quant kernels,
 * which never produce them.  in fp32 [n], out uint8 [n], device. */
mxq_status mxq_e4m3_encode_f32(const float* in, int64_t n, uint8_t* out,
                               void* stream);

const char* mxq_status_string(mxq_status s);
int32_t mxq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H */
