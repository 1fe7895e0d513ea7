// Host-side helpers shared by the entry points of libmxq: argument checks
// and launch-error mapping.  Every check runs before any work is enqueued.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq.h"

namespace mxq {

inline bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Launch status of the kernel just enqueued.
inline mxq_status launch_status() {
  return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

inline int group_of(mxq_scale_fmt fmt) {
  switch (fmt) {
    case MXQ_SCALE_UE8M0_G128:
      return 128;
    case MXQ_SCALE_E8M0_G32:
      return 32;
  }
  return 0;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Threads per block for a row split in chunks of `per_lane` channels: a
// whole number of 64-lane wavefronts, at most 1024.
inline int row_block_threads(int64_t H, int per_lane) {
  int64_t lanes = ceil_div(H, per_lane);
  int64_t t = ceil_div(lanes, 64) * 64;
  if (t < 64) t = 64;
  if (t > 1024) t = 1024;
  return (int)t;
}

}  // namespace mxq

namespace mxq {

// Layout work split: the T*K assignments are cut into chunks of a whole
// number of 1024-assignment groups (at least 1024, at most 8192, aiming at
// 64 chunks); one block of 16 wavefronts owns a chunk.  The split depends
// only on T*K, so the grid is static.
constexpr int kChunkMin = 1024;
constexpr int kChunkMax = 8192;
constexpr int kChunksTarget = 64;

struct LayoutGeom {
  int32_t nc;     // number of chunks (0 when there are no assignments)
  int32_t chunk;  // assignments per chunk
};

inline LayoutGeom layout_geom(int64_t A) {
  LayoutGeom g{0, kChunkMin};
  if (A <= 0) return g;
  int64_t chunk = ceil_div(ceil_div(A, kChunksTarget), kChunkMin) * kChunkMin;
  if (chunk > kChunkMax) chunk = kChunkMax;
  g.chunk = (int32_t)chunk;
  g.nc = (int32_t)ceil_div(A, chunk);
  return g;
}

// Up to this many assignments the layout runs as one launch in which every
// block ranks the whole routing (at most four 64-assignment steps per
// wavefront); above it the histogram + slots pair over chunks is faster.
constexpr int64_t kSingleMax = 4096;

// Within kSingleMax, up to this many tokens the layout takes one block per
// token instead (each block counts the whole routing and places its own
// assignments): up to 2048 tokens with blocks of 256 threads (at most 256
// local experts), up to 1024 with blocks of 1024 (more experts, which the
// region scan spreads one per thread).
constexpr int64_t kTokenMaxTokens = 2048;
constexpr int64_t kTokenMaxTokensWide = 1024;

inline bool layout_per_token(int64_t A, int64_t T, int32_t E) {
  return A > 0 && A <= kSingleMax &&
         T <= (E <= 256 ? kTokenMaxTokens : kTokenMaxTokensWide);
}

// Above kSingleMax and up to these sizes the slot kernel still runs alone:
// each of its blocks counts the whole routing into LDS itself (its 16
// wavefronts keep private counts), so the histogram launch and its per-chunk
// workspace go away.  Every block reads and counts all ids, so this pays
// only for mid-sized routings: measured on MI355X (Zipf top-8 over 256
// experts, graph-timed) 10.1 against 11.2-11.4 us for 5120 to 16384
// assignments, but 12.1 against 11.0 us at 32768 and 16.9 against 12.2 us
// at 65536, where the LDS atomics of every block on the hot experts cost
// more than the launch they save.
constexpr int64_t kInBlockMaxAssign = (int64_t)1 << 14;
constexpr int32_t kInBlockMaxExperts = 256;

inline bool layout_in_block(int64_t A, int32_t E) {
  return A > kSingleMax && A <= kInBlockMaxAssign && E <= kInBlockMaxExperts;
}

// Workspace: per-chunk expert counts [nc][E]; none when the layout runs as
// one launch (A <= kSingleMax, or counted in every block).
inline size_t layout_workspace_bytes(int64_t A, int32_t E) {
  if (A <= kSingleMax || layout_in_block(A, E)) return 0;
  LayoutGeom g = layout_geom(A);
  return (size_t)g.nc * (size_t)(E > 0 ? E : 0) * sizeof(int32_t);
}

}  // namespace mxq
