// moe_scatter_quant, mx_quant_live_rows and the e4m3 codec check.
//
// Quantization follows sglang PR #33128 (implementation breakdown item 3:
// quantize activations with a UE8M0 scale computed directly, fused with the
// scatter) and sglang PR #36119 (implementation breakdown item 1: one e8m0
// byte per 32 channels, quantized on the sender over live rows only).
//
// Work split: one block per token row (scatter); on the send side one
// wavefront per (live row, 1024-channel chunk) over a grid of about one
// block per CU.  A lane owns 16 consecutive channels, so a row is read once
// with 16-byte loads and its group exponents come from in-wavefront max
// reductions.  The
// scatter path is bandwidth-bound: per token it reads 2H bytes and writes
// K*(H + H/G) bytes.
#include "mxq_device.hpp"
#include "mxq_host.hpp"

namespace {

using namespace mxq;

// Scale placement of the quantizers: strided (row-major bytes or packed
// MN-major words: s_rs, s_c4 as in scale_addr) or the block-scaled MFMA
// operand order (s_rs = log2 of the tile rows, s_c4 = word groups per row
// tile, as in mfma_scale_addr; each 32-channel block gets its own byte).
enum Placement { kStrided = 0, kMfma = 1 };

// One block per token, in two phases.  Phase 1: the block reads the token
// row once (16-byte loads, a lane owns 16 channels), quantizes it and stages
// the fp8 row and its scale bytes in LDS.  Phase 2: wavefront w writes
// destinations j = w, w + nw, ...; each destination row is written by one
// wavefront as a contiguous run of 1 KB streaming (non-temporal) stores,
// followed by its scale bytes.  Writing whole rows per wavefront and
// bypassing cache allocation for the write-once payload keeps the HBM write
// stream sequential; the scale bytes use ordinary stores so partial lines
// merge in L2.  Destinations come from src2dst in one vector load per
// wavefront (lane j holds destination j, handed out with readlane); a token
// without a destination in [0, num_rows) is skipped before its row is
// read.
//
// MFMA placement.  A row's scale bytes go to one 32-bit word per (group of
// four instructions, block within the instruction), words that the other
// rows of its tile share lines with.  Those rows are consecutive slots of
// one expert, i.e. tokens in ascending order.  Blocks are dealt to the 8
// XCDs round-robin, so with block b taking token b a tile's lines were
// written partly from several L2s; here the blocks of one XCD (b mod 8) take
// one contiguous eighth of the tokens instead, so most tiles are written
// from a single L2 and leave it as whole lines.  Measured on MI355X at the
// prefill shape (8192 x 7168, 98048 rows, group 128): tiles of 32 rows
// 109.8 -> 93.1 us and 566 -> 508 MB written (tiles of 16: 105.8 -> 91.2
// us), with the word stores below; the row-major placement keeps token
// order (87.0 us against 92.3 us with the contiguous ranges).
//
// Lookahead.  Phase 1 reads with H / 16 lanes; the wavefronts after them
// have nothing to read, so they fetch one word per 128 bytes (one L2 line)
// of the rows of the tokens that blocks blockIdx.x + kAhead,
// blockIdx.x + 2 * kAhead, ... take, if those tokens have a destination
// (the same test as below): two wavefronts per row at H = 7168.  Those
// blocks run on the same XCD (kAhead is a multiple of 8) one, two, ...
// microseconds later and find their rows' lines in flight or in L2, so
// reads from HBM keep more requests in flight without more destination
// rows open for writing.  The depth follows the rows the block writes,
// which set how long it stays resident: none below kAheadMinRows (the two
// round trips, the token's destinations and then its row, must end before
// the block's own writes do), two rows ahead from kAheadMinRows, four from
// kAheadDeepRows.  The fetched words are folded into a value stored only
// where `sink` is non-null (the launch passes null); the compiler cannot
// know that, so the loads stay.  Measured on MI355X (graph-timed; MALL
// flushed before each call, write-back charged, in brackets), prefill
// shape (eight rows per token): 86.6-86.7 us [107.0-107.9] against 87.1 us
// [108.7-109.1] with two rows ahead for every block of four or more rows,
// 87.6 us [110.4-111.7] with one row ahead at one word per 64 bytes and
// 87.3 us [112.0-112.7] without lookahead.  Four rows ahead from six rows
// gained 0.5 us more there but cost a slice with 192 of 256 experts local
// (six rows per token on average) 2 us from HBM; from seven rows that
// slice takes 91.6-92.0 against 90.7-91.1 us with two rows ahead.  Four
// rows ahead from four rows cost a slice with 128 local 2 us (67.1 against
// 65.0 us).  With 32 of 256 experts local (about one row per token) the
// kernel takes 23.0-23.1 us against 22.2 us without any lookahead code and
// 23.9 us for the kernel before it.  Smaller blocks (more tokens in flight
// per CU) and one block per CU were measured too: the first slower
// everywhere (121 us from HBM), the second 108 us from HBM with one row
// ahead but 30.5 against 22.4 us with 32 experts local.
constexpr int kAhead = 96;
constexpr int kAheadRows = 2;
constexpr int kAheadRowsDeep = 4;
constexpr int kAheadStride = 128;
constexpr int kAheadMinRows = 4;
constexpr int kAheadDeepRows = 7;

template <int PLACE>
__device__ __forceinline__ int64_t token_of_block(int64_t b, int64_t nblocks) {
  if constexpr (PLACE == kMfma)  // nblocks is a multiple of 8
    return (b & 7) * (nblocks >> 3) + (b >> 3);
  return b;
}

// At most 64 VGPRs (eight waves per SIMD), so that two blocks fit on a CU
// (one block per CU made a slice with 32 of 256 experts local 36 % slower).
template <int G, int RULE, int PLACE>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(8)))
void scatter_quant_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, int32_t H, int64_t T,
    const int32_t* __restrict__ src2dst, int32_t K, uint8_t* __restrict__ q,
    int64_t ld_q, uint8_t* __restrict__ s, int64_t s_rs, int64_t s_c4,
    int64_t num_rows, uint32_t* __restrict__ sink) {
  extern __shared__ __align__(16) uint8_t row[];  // [H] fp8, then [H/G] scales
  const int64_t t = token_of_block<PLACE>(blockIdx.x, gridDim.x);
  if constexpr (PLACE == kMfma) {
    if (t >= T) return;
  }
  // lane j of every wavefront loads destination j (K <= 64) in one vector
  // load; a ballot tells whether the token has any, and readlane hands each
  // writing wavefront its row, so the row loads wait for one round trip
  const int lane = threadIdx.x & 63;
  const int32_t d_lane = src2dst[t * K + min(lane, K - 1)];
  const bool valid = lane < K && d_lane >= 0 && (int64_t)d_lane < num_rows;
  const uint64_t has = __ballot(valid);
  if (has == 0) return;  // the same in every wavefront
  // lookahead by the wavefronts with no channels in phase 1: wpr of them
  // per row ahead, two or four rows
  const int p0 = ((H / 16 + 63) / 64) * 64;
  uint32_t pf = 0;
  const int nrows = __popcll(has);
  if ((int)threadIdx.x >= p0 && nrows >= kAheadMinRows) {
    const int wi = ((int)threadIdx.x - p0) >> 6;
    const int wpr = (H * 2 / kAheadStride + 63) / 64;
    const int rows_ahead = nrows >= kAheadDeepRows ? kAheadRowsDeep
                                                   : kAheadRows;
    const int which = wpr > 0 ? wi / wpr : rows_ahead;
    const int64_t b2 = (int64_t)blockIdx.x + (int64_t)kAhead * (which + 1);
    if (which < rows_ahead && b2 < (int64_t)gridDim.x) {
      const int64_t t2 = token_of_block<PLACE>(b2, gridDim.x);
      if (t2 < T) {
        const int32_t d2 = src2dst[t2 * K + min(lane, K - 1)];
        if (__ballot(lane < K && d2 >= 0 && (int64_t)d2 < num_rows) != 0) {
          const int64_t off =
              (int64_t)((wi - which * wpr) * 64 + lane) * kAheadStride;
          if (off + 4 <= (int64_t)H * 2)
            pf = *reinterpret_cast<const uint32_t*>(
                reinterpret_cast<const uint8_t*>(x + t2 * ld_x) + off);
        }
      }
    }
  }
  const uint16_t* xr = x + t * ld_x;
  const bool lead = (threadIdx.x & (G / 16 - 1)) == 0;
  for (int col = threadIdx.x * 16; col < H; col += blockDim.x * 16) {
    const u32x4 a = load16(xr + col);
    const u32x4 b = load16(xr + col + 8);
    int e;
    const u32x4 v = quant16<G, RULE>(a, b, e);
    *reinterpret_cast<u32x4*>(row + col) = v;
    if (lead) row[H + col / G] = (uint8_t)(e + 127);
  }
  __syncthreads();
  const int nw = blockDim.x >> 6;
  const int ng = H / G;
  for (int j = threadIdx.x >> 6; j < K; j += nw) {
    const int64_t d = __builtin_amdgcn_readlane(d_lane, j);
    if (d < 0 || d >= num_rows) continue;
    uint8_t* qr = q + d * ld_q;
    for (int c = lane * 16; c < H; c += 64 * 16)
      store16_nt(qr + c, *reinterpret_cast<const u32x4*>(row + c));
    if constexpr (PLACE == kMfma) {
      // word (g4, h) of row d holds blocks kb0 + b * hh, b = 0..3, with
      // kb0 = g4 * 4 * hh + h (hh = 64 / tm blocks per instruction); words
      // whose last block is past H / 32 are written byte by byte
      const int tm_shift = (int)s_rs;
      const int hh_shift = 6 - tm_shift;
      const int hh = 1 << hh_shift;
      const int nb = H >> 5;
      const int words = (int)s_c4 << hh_shift;
      for (int wi = lane; wi < words; wi += 64) {
        const int kb0 = ((wi >> hh_shift) << (hh_shift + 2)) + (wi & (hh - 1));
        const int64_t wa = mfma_scale_addr(d, kb0, tm_shift, s_c4);
        if (kb0 + 3 * hh < nb) {
          uint32_t w = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b)
            w |= (uint32_t)row[H + (kb0 + b * hh) * 32 / G] << (8 * b);
          *reinterpret_cast<uint32_t*>(s + wa) = w;
        } else {
          for (int b = 0; b < 4; ++b)
            if (kb0 + b * hh < nb) s[wa + b] = row[H + (kb0 + b * hh) * 32 / G];
        }
      }
    } else {
      // not unrolled: unrolled, its 64-bit addresses pushed the kernel past
      // 64 VGPRs
#pragma unroll 1
      for (int g = lane; g < ng; g += 64)
        s[scale_addr(d, g, s_rs, s_c4)] = row[H + g];
    }
  }
  if (sink != nullptr) sink[threadIdx.x] = pf;
}

// Send-side quant for more than 64 segments.  Segment g owns blocks
// [g*bps, (g+1)*bps); block i of a segment handles its live rows i, i + bps,
// ...  The grid depends only on the host arguments; blocks past the live
// count return at once.  The fp8 rows
// are written once, with streaming stores (all 24576 rows of the padded
// buffer live: 101.6 us instead of 108 us with plain stores on MI355X).
template <int G, int RULE, int PLACE>
__global__ __launch_bounds__(1024) void live_rows_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, int64_t rps, int32_t bps,
    const int32_t* __restrict__ live, int32_t H, uint8_t* __restrict__ q,
    int64_t ld_q, uint8_t* __restrict__ s, int64_t s_rs, int64_t s_c4) {
  const int32_t g = blockIdx.x / bps;
  const int32_t i = blockIdx.x - g * bps;
  int64_t n = live[g];
  n = n < 0 ? 0 : (n > rps ? rps : n);
  const bool lead = (threadIdx.x & (G / 16 - 1)) == 0;
  for (int64_t r = i; r < n; r += bps) {
    const int64_t row = (int64_t)g * rps + r;
    const uint16_t* xr = x + row * ld_x;
    for (int col = threadIdx.x * 16; col < H; col += blockDim.x * 16) {
      const u32x4 a = load16(xr + col);
      const u32x4 b = load16(xr + col + 8);
      int e;
      const u32x4 v = quant16<G, RULE>(a, b, e);
      store16_nt(q + row * ld_q + col, v);
      if (lead) {
        const uint8_t sb = (uint8_t)(e + 127);
        if constexpr (PLACE == kMfma) {
#pragma unroll
          for (int u = 0; u < G / 32; ++u)
            s[mfma_scale_addr(row, col / 32 + u, (int)s_rs, s_c4)] = sb;
        } else {
          s[scale_addr(row, col / G, s_rs, s_c4)] = sb;
        }
      }
    }
  }
}

// Send-side quant for up to 64 segments, with a grid of 4096 wavefronts
// that does not grow with the padded buffer.  Lane g of every
// wavefront holds segment g's live count (clipped to [0, rps]) and their
// inclusive prefix, so live row i (in segment order) lies in segment
// g = #{segments whose prefix <= i}, one ballot.  Work comes in units of
// (live row, chunk of 1024 channels); unit u goes to wavefront u mod W of
// the W in the grid, numbered across blocks first so that consecutive
// units land on different CUs.  Only the counts are read before a
// wavefront with no unit exits.  Measured on MI355X (24576 x 7168 padded,
// group 32, graph-timed): 112 live rows 2.9 us (3.7 us with a block per
// padded row group), all rows live 97.6 us (102.1 us); two or four units
// per wavefront and round were slower with many rows live (103.3 and
// 108.0 us).  The 4096 wavefronts come in blocks of two: 14 x 8 live rows
// 2.65 us, empty 2.16 us, all live 97.0 us, against 2.81 / 2.14 / 97.0 us
// in blocks of 16 (256 x 1024), 2.75 / 2.06 / 96.1 us in blocks of 4 and
// 2.81 / 2.55 / 97.8 us in blocks of one; with half as many wavefronts all
// live took 100-104 us.  The launch alone costs about 2.1 us per call
// here (an empty kernel measured the same), which is what an all-empty
// batch costs.
constexpr int kLiveChunk = 1024;  // channels of one unit (64 lanes x 16)
constexpr int kLiveThreads = 128;

template <int G, int RULE, int PLACE>
__global__ __launch_bounds__(kLiveThreads) void live_units_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, int64_t rps, int32_t nseg,
    const int32_t* __restrict__ live, int32_t H, int32_t upr,
    uint8_t* __restrict__ q, int64_t ld_q, uint8_t* __restrict__ s,
    int64_t s_rs, int64_t s_c4) {
  const int lane = threadIdx.x & 63;
  int c = live[min(lane, nseg - 1)];
  c = lane < nseg ? (c < 0 ? 0 : (int64_t)c > rps ? (int)rps : c) : 0;
  int incl = c;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  const int total = __builtin_amdgcn_readlane(incl, 63);
  const int64_t units = (int64_t)total * upr;
  const int64_t W = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t gw = (int64_t)(threadIdx.x >> 6) * gridDim.x + blockIdx.x;
  const bool lead = (lane & (G / 16 - 1)) == 0;
  for (int64_t u = gw; u < units; u += W) {
    const int i = (int)(u / upr);
    const int ch = (int)(u - (int64_t)i * upr);
    const int g = __popcll(__ballot(lane < nseg && incl <= i));
    const int excl = __builtin_amdgcn_readlane(incl, g) -
                     __builtin_amdgcn_readlane(c, g);
    const int64_t row = (int64_t)g * rps + (i - excl);
    const int col = ch * kLiveChunk + lane * 16;
    if (col >= H) continue;
    const uint16_t* xr = x + row * ld_x + col;
    const u32x4 a = load16(xr);
    const u32x4 b = load16(xr + 8);
    int e;
    const u32x4 v = quant16<G, RULE>(a, b, e);
    store16_nt(q + row * ld_q + col, v);
    if (lead) {
      const uint8_t sb = (uint8_t)(e + 127);
      if constexpr (PLACE == kMfma) {
#pragma unroll
        for (int w = 0; w < G / 32; ++w)
          s[mfma_scale_addr(row, col / 32 + w, (int)s_rs, s_c4)] = sb;
      } else {
        s[scale_addr(row, col / G, s_rs, s_c4)] = sb;
      }
    }
  }
}

__global__ __launch_bounds__(256) void encode_e4m3_kernel(
    const float* __restrict__ in, int64_t n, uint8_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n;
       i += stride) {
    if (i + 4 <= n) {
      const uint32_t w = pack4_e4m3(in[i], in[i + 1], in[i + 2], in[i + 3]);
      out[i] = (uint8_t)w;
      out[i + 1] = (uint8_t)(w >> 8);
      out[i + 2] = (uint8_t)(w >> 16);
      out[i + 3] = (uint8_t)(w >> 24);
    } else {
      for (int64_t k = i; k < n; ++k)
        out[k] = (uint8_t)pack4_e4m3(in[k], 0.f, 0.f, 0.f);
    }
  }
}

bool rows_ok_bf16(const void* p, int64_t ld) {
  return aligned16(p) && (ld * 2) % 16 == 0;
}
bool rows_ok_u8(const void* p, int64_t ld) {
  return aligned16(p) && ld % 16 == 0;
}

// Scale placement check: row-major bytes (c4 == 4, rs >= groups) or packed
// words with rows contiguous (rs == 4, c4 >= 4 * rows); both keep every
// (row, group) at its own byte.
bool scale_place_ok(int64_t rs, int64_t c4, int64_t groups, int64_t rows) {
  if (c4 == 4) return rs >= groups;
  if (rs == 4) return c4 % 4 == 0 && c4 >= 4 * rows;
  return false;
}

template <int G, int PLACE>
void launch_scatter(int rule, unsigned T, int threads, size_t lds,
                    hipStream_t s, const uint16_t* x, int64_t ld_x, int32_t H,
                    const int32_t* src2dst, int32_t K, uint8_t* q,
                    int64_t ld_q, uint8_t* sc, int64_t rs, int64_t c4,
                    int64_t num_rows) {
  // the MFMA placement's token ranges per XCD need a multiple of 8 blocks
  const unsigned grid = PLACE == kMfma ? (T + 7) / 8 * 8 : T;
  if (rule == MXQ_RULE_OCP_FLOOR)
    scatter_quant_kernel<G, kOcpFloor, PLACE><<<grid, threads, lds, s>>>(
        x, ld_x, H, T, src2dst, K, q, ld_q, sc, rs, c4, num_rows, nullptr);
  else
    scatter_quant_kernel<G, kNoClip, PLACE><<<grid, threads, lds, s>>>(
        x, ld_x, H, T, src2dst, K, q, ld_q, sc, rs, c4, num_rows, nullptr);
}

// Launch of the send-side quant: up to 64 segments the unit kernel with a
// grid of at most kLiveBlocks blocks of kLiveThreads threads, fewer when
// the padded buffer holds fewer units; above 64 segments the row kernel
// with about 1024 blocks over the segments.
constexpr int kLiveBlocks = 2048;
constexpr int kLiveUnitSegments = 64;

template <int G, int RULE, int PLACE>
void launch_live_rule(hipStream_t s, const uint16_t* x, int64_t ld_x,
                      int32_t nseg, int64_t rps, const int32_t* live,
                      int32_t H, uint8_t* q, int64_t ld_q, uint8_t* sc,
                      int64_t rs, int64_t c4) {
  if (nseg <= kLiveUnitSegments) {
    const int32_t upr = (int32_t)ceil_div(H, kLiveChunk);
    const int64_t max_units = (int64_t)nseg * rps * upr;
    int64_t blocks = ceil_div(max_units, kLiveThreads / 64);
    if (blocks > kLiveBlocks) blocks = kLiveBlocks;
    live_units_kernel<G, RULE, PLACE><<<(unsigned)blocks, kLiveThreads, 0,
                                        s>>>(
        x, ld_x, rps, nseg, live, H, upr, q, ld_q, sc, rs, c4);
    return;
  }
  // About 1024 blocks in all, at most one per padded row of a segment.
  int64_t bps = ceil_div(1024, nseg);
  if (bps > rps) bps = rps;
  if (bps < 1) bps = 1;
  const int64_t blocks = bps * nseg;
  live_rows_kernel<G, RULE, PLACE><<<(unsigned)blocks,
                                     row_block_threads(H, 16), 0, s>>>(
      x, ld_x, rps, (int32_t)bps, live, H, q, ld_q, sc, rs, c4);
}

template <int G, int PLACE>
void launch_live(int rule, hipStream_t s, const uint16_t* x, int64_t ld_x,
                 int32_t nseg, int64_t rps, const int32_t* live, int32_t H,
                 uint8_t* q, int64_t ld_q, uint8_t* sc, int64_t rs,
                 int64_t c4) {
  if (rule == MXQ_RULE_OCP_FLOOR)
    launch_live_rule<G, kOcpFloor, PLACE>(s, x, ld_x, nseg, rps, live, H, q,
                                          ld_q, sc, rs, c4);
  else
    launch_live_rule<G, kNoClip, PLACE>(s, x, ld_x, nseg, rps, live, H, q,
                                        ld_q, sc, rs, c4);
}

// Word groups per row tile of the MFMA placement: one group holds the scales
// of four instructions, each spanning 64/tm blocks of 32 channels.
int64_t mfma_word_groups(int32_t H, int32_t tile_m) {
  return ceil_div(H / 32, 4 * (64 / tile_m));
}

int mfma_tile_shift(int32_t tile_m) {
  return tile_m == 32 ? 5 : (tile_m == 16 ? 4 : -1);
}

// Shared body of the scatter entry points; `place` selects the scale
// placement, whose own arguments (rs, c4) the caller has checked.
mxq_status scatter_quant_impl(const void* x_bf16, int64_t ld_x, int64_t T,
                              int32_t H, const int32_t* src2dst, int32_t K,
                              mxq_scale_fmt fmt, mxq_scale_rule rule,
                              void* q_fp8, int64_t ld_q, void* scales,
                              int place, int64_t rs, int64_t c4,
                              int64_t num_rows, void* stream) {
  const int G = group_of(fmt);
  if (T == 0 || K == 0 || num_rows == 0) return MXQ_OK;

  // 1024 threads: at most two tokens in flight per CU, which keeps the
  // number of concurrent destination-row write streams low.
  const int threads = 1024;
  const size_t lds = (size_t)H + (size_t)(H / G);
  hipStream_t s = as_stream(stream);
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  uint8_t* q = static_cast<uint8_t*>(q_fp8);
  uint8_t* sc = static_cast<uint8_t*>(scales);
  if (place == kMfma) {
    if (G == 128)
      launch_scatter<128, kMfma>(rule, (unsigned)T, threads, lds, s, x, ld_x,
                                 H, src2dst, K, q, ld_q, sc, rs, c4, num_rows);
    else
      launch_scatter<32, kMfma>(rule, (unsigned)T, threads, lds, s, x, ld_x,
                                H, src2dst, K, q, ld_q, sc, rs, c4, num_rows);
  } else {
    if (G == 128)
      launch_scatter<128, kStrided>(rule, (unsigned)T, threads, lds, s, x,
                                    ld_x, H, src2dst, K, q, ld_q, sc, rs, c4,
                                    num_rows);
    else
      launch_scatter<32, kStrided>(rule, (unsigned)T, threads, lds, s, x,
                                   ld_x, H, src2dst, K, q, ld_q, sc, rs, c4,
                                   num_rows);
  }
  return launch_status();
}

// Checks shared by the scatter entry points (everything but the scale
// placement).  Returns MXQ_OK when the call may go on.
mxq_status scatter_args_ok(const void* x_bf16, int64_t ld_x, int64_t T,
                           int32_t H, const int32_t* src2dst, int32_t K,
                           mxq_scale_fmt fmt, mxq_scale_rule rule,
                           const void* q_fp8, int64_t ld_q,
                           const void* scales, int64_t num_rows) {
  const int G = group_of(fmt);
  if (G == 0 || (rule != MXQ_RULE_NO_CLIP && rule != MXQ_RULE_OCP_FLOOR))
    return MXQ_ERR_UNSUPPORTED;
  if (T < 0 || T > INT32_MAX || H <= 0 || H % G != 0 || K < 0 ||
      K > MXQ_MAX_TOPK || num_rows < 0 || num_rows > INT32_MAX)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (H > MXQ_MAX_HIDDEN) return MXQ_ERR_UNSUPPORTED;
  if (T == 0 || K == 0) return MXQ_OK;
  if (x_bf16 == nullptr || src2dst == nullptr || ld_x < H)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (num_rows > 0 && (q_fp8 == nullptr || scales == nullptr))
    return MXQ_ERR_INVALID_ARGUMENT;
  if (ld_q < H) return MXQ_ERR_INVALID_ARGUMENT;
  if (!rows_ok_bf16(x_bf16, ld_x) || (num_rows > 0 && !rows_ok_u8(q_fp8, ld_q)))
    return MXQ_ERR_INVALID_ARGUMENT;
  return MXQ_OK;
}

// Shared body of the live-row entry points, as scatter_quant_impl.
mxq_status live_rows_impl(const void* x_bf16, int64_t ld_x,
                          int32_t num_segments, int64_t rows_per_segment,
                          const int32_t* live_counts, int32_t H,
                          mxq_scale_fmt fmt, mxq_scale_rule rule, void* q_fp8,
                          int64_t ld_q, void* scales, int place, int64_t rs,
                          int64_t c4, void* stream) {
  const int G = group_of(fmt);
  hipStream_t s = as_stream(stream);
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  uint8_t* q = static_cast<uint8_t*>(q_fp8);
  uint8_t* sc = static_cast<uint8_t*>(scales);
  if (place == kMfma) {
    if (G == 32)
      launch_live<32, kMfma>(rule, s, x, ld_x, num_segments, rows_per_segment,
                             live_counts, H, q, ld_q, sc, rs, c4);
    else
      launch_live<128, kMfma>(rule, s, x, ld_x, num_segments,
                              rows_per_segment, live_counts, H, q, ld_q, sc,
                              rs, c4);
  } else {
    if (G == 32)
      launch_live<32, kStrided>(rule, s, x, ld_x, num_segments,
                                rows_per_segment, live_counts, H, q, ld_q, sc,
                                rs, c4);
    else
      launch_live<128, kStrided>(rule, s, x, ld_x, num_segments,
                                 rows_per_segment, live_counts, H, q, ld_q,
                                 sc, rs, c4);
  }
  return launch_status();
}

// Checks shared by the live-row entry points except the scale placement.
// Sets *rows to the padded row count.  Returns MXQ_OK when the call may go
// on and there is work (*rows > 0), or an error, or MXQ_OK with *rows = 0.
mxq_status live_args_ok(const void* x_bf16, int64_t ld_x,
                        int32_t num_segments, int64_t rows_per_segment,
                        const int32_t* live_counts, int32_t H,
                        mxq_scale_fmt fmt, mxq_scale_rule rule,
                        const void* q_fp8, int64_t ld_q, const void* scales,
                        int64_t* rows) {
  *rows = 0;
  const int G = group_of(fmt);
  if (G == 0 || (rule != MXQ_RULE_NO_CLIP && rule != MXQ_RULE_OCP_FLOOR))
    return MXQ_ERR_UNSUPPORTED;
  if (num_segments < 0 || rows_per_segment < 0 || H <= 0 || H % G != 0)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (num_segments == 0 || rows_per_segment == 0) return MXQ_OK;
  const int64_t n = (int64_t)num_segments * rows_per_segment;
  if (n > INT32_MAX) return MXQ_ERR_INVALID_ARGUMENT;
  if (x_bf16 == nullptr || live_counts == nullptr || q_fp8 == nullptr ||
      scales == nullptr)
    return MXQ_ERR_INVALID_ARGUMENT;
  if (ld_x < H || ld_q < H) return MXQ_ERR_INVALID_ARGUMENT;
  if (!rows_ok_bf16(x_bf16, ld_x) || !rows_ok_u8(q_fp8, ld_q))
    return MXQ_ERR_INVALID_ARGUMENT;
  *rows = n;
  return MXQ_OK;
}

}  // namespace

extern "C" mxq_status moe_scatter_quant_ex(
    const void* x_bf16, int64_t ld_x, int64_t T, int32_t H,
    const int32_t* src2dst, int32_t K, mxq_scale_fmt fmt, mxq_scale_rule rule,
    void* q_fp8, int64_t ld_q, void* scales, int64_t scale_row_stride,
    int64_t scale_quad_stride, int64_t num_rows, void* stream) {
  const mxq_status st = scatter_args_ok(x_bf16, ld_x, T, H, src2dst, K, fmt,
                                        rule, q_fp8, ld_q, scales, num_rows);
  if (st != MXQ_OK) return st;
  if (T == 0 || K == 0) return MXQ_OK;
  if (!scale_place_ok(scale_row_stride, scale_quad_stride,
                      H / group_of(fmt), num_rows))
    return MXQ_ERR_INVALID_ARGUMENT;
  return scatter_quant_impl(x_bf16, ld_x, T, H, src2dst, K, fmt, rule, q_fp8,
                            ld_q, scales, kStrided, scale_row_stride,
                            scale_quad_stride, num_rows, stream);
}

extern "C" mxq_status moe_scatter_quant(const void* x_bf16, int64_t ld_x,
                                        int64_t T, int32_t H,
                                        const int32_t* src2dst, int32_t K,
                                        mxq_scale_fmt fmt, void* q_fp8,
                                        int64_t ld_q, uint8_t* scales,
                                        int64_t ld_s, int64_t num_rows,
                                        void* stream) {
  return moe_scatter_quant_ex(x_bf16, ld_x, T, H, src2dst, K, fmt,
                              MXQ_RULE_NO_CLIP, q_fp8, ld_q, scales, ld_s, 4,
                              num_rows, stream);
}

extern "C" int64_t mxq_mfma_scale_bytes(int64_t rows, int32_t H,
                                        int32_t tile_m) {
  if (rows < 0 || H <= 0 || H % 32 != 0 || mfma_tile_shift(tile_m) < 0)
    return -1;
  return ceil_div(rows, tile_m) * mfma_word_groups(H, tile_m) * 256;
}

extern "C" mxq_status moe_scatter_quant_mfma(
    const void* x_bf16, int64_t ld_x, int64_t T, int32_t H,
    const int32_t* src2dst, int32_t K, mxq_scale_fmt fmt, mxq_scale_rule rule,
    void* q_fp8, int64_t ld_q, void* scales, int32_t tile_m, int64_t num_rows,
    void* stream) {
  const mxq_status st = scatter_args_ok(x_bf16, ld_x, T, H, src2dst, K, fmt,
                                        rule, q_fp8, ld_q, scales, num_rows);
  if (st != MXQ_OK) return st;
  const int shift = mfma_tile_shift(tile_m);
  if (shift < 0) return MXQ_ERR_INVALID_ARGUMENT;
  // the scales are written as 32-bit words
  if ((reinterpret_cast<uintptr_t>(scales) & 3) != 0)
    return MXQ_ERR_INVALID_ARGUMENT;
  return scatter_quant_impl(x_bf16, ld_x, T, H, src2dst, K, fmt, rule, q_fp8,
                            ld_q, scales, kMfma, shift,
                            mfma_word_groups(H, tile_m), num_rows, stream);
}

extern "C" mxq_status mx_quant_live_rows_ex(
    const void* x_bf16, int64_t ld_x, int32_t num_segments,
    int64_t rows_per_segment, const int32_t* live_counts, int32_t H,
    mxq_scale_fmt fmt, mxq_scale_rule rule, void* q_fp8, int64_t ld_q,
    void* scales, int64_t scale_row_stride, int64_t scale_quad_stride,
    void* stream) {
  int64_t rows = 0;
  const mxq_status st =
      live_args_ok(x_bf16, ld_x, num_segments, rows_per_segment, live_counts,
                   H, fmt, rule, q_fp8, ld_q, scales, &rows);
  if (st != MXQ_OK || rows == 0) return st;
  if (!scale_place_ok(scale_row_stride, scale_quad_stride,
                      H / group_of(fmt), rows))
    return MXQ_ERR_INVALID_ARGUMENT;
  return live_rows_impl(x_bf16, ld_x, num_segments, rows_per_segment,
                        live_counts, H, fmt, rule, q_fp8, ld_q, scales,
                        kStrided, scale_row_stride, scale_quad_stride, stream);
}

extern "C" mxq_status mx_quant_live_rows(const void* x_bf16, int64_t ld_x,
                                         int32_t num_segments,
                                         int64_t rows_per_segment,
                                         const int32_t* live_counts, int32_t H,
                                         mxq_scale_fmt fmt, void* q_fp8,
                                         int64_t ld_q, uint8_t* scales,
                                         int64_t ld_s, void* stream) {
  return mx_quant_live_rows_ex(x_bf16, ld_x, num_segments, rows_per_segment,
                               live_counts, H, fmt, MXQ_RULE_NO_CLIP, q_fp8,
                               ld_q, scales, ld_s, 4, stream);
}

extern "C" mxq_status mx_quant_live_rows_mfma(
    const void* x_bf16, int64_t ld_x, int32_t num_segments,
    int64_t rows_per_segment, const int32_t* live_counts, int32_t H,
    mxq_scale_fmt fmt, mxq_scale_rule rule, void* q_fp8, int64_t ld_q,
    void* scales, int32_t tile_m, void* stream) {
  int64_t rows = 0;
  const mxq_status st =
      live_args_ok(x_bf16, ld_x, num_segments, rows_per_segment, live_counts,
                   H, fmt, rule, q_fp8, ld_q, scales, &rows);
  if (st != MXQ_OK) return st;
  const int shift = mfma_tile_shift(tile_m);
  if (shift < 0) return MXQ_ERR_INVALID_ARGUMENT;
  if (rows == 0) return MXQ_OK;
  return live_rows_impl(x_bf16, ld_x, num_segments, rows_per_segment,
                        live_counts, H, fmt, rule, q_fp8, ld_q, scales, kMfma,
                        shift, mfma_word_groups(H, tile_m), stream);
}

extern "C" mxq_status mxq_e4m3_encode_f32(const float* in, int64_t n,
                                          uint8_t* out, void* stream) {
  if (n < 0) return MXQ_ERR_INVALID_ARGUMENT;
  if (n == 0) return MXQ_OK;
  if (in == nullptr || out == nullptr) return MXQ_ERR_INVALID_ARGUMENT;
  int64_t blocks = ceil_div(ceil_div(n, 4), 256);
  if (blocks > 16384) blocks = 16384;
  encode_e4m3_kernel<<<(unsigned)blocks, 256, 0, as_stream(stream)>>>(in, n,
                                                                       out);
  return launch_status();
}
