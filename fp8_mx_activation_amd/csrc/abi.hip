// Host-only entry points of libmxq: the static layout helpers, workspace
// queries, the overflow read-back and status strings.
#include "mxq_host.hpp"

extern "C" int64_t moe_compact_row_bound(int64_t num_assignments,
                                         int32_t num_local_experts,
                                         int32_t block_e) {
  // The largest padded row count any routing of A assignments over E
  // experts can need (the static bound of sglang PR #33128 page, Key source
  // snippets).  An expert with c > 0 assignments takes ceil(c / b) blocks:
  // one block for its first assignment and floor((c - 1) / b) for the rest.
  // With m non-empty experts the blocks therefore number at most
  // m + floor((A - m) / b); raising m by one adds a block and removes at
  // most one, so the worst case has as many non-empty experts as possible,
  // m = min(A, E), and packs every remaining assignment into whole blocks.
  if (num_assignments < 0 || num_local_experts < 0 || block_e < 1) return -1;
  const int64_t A = num_assignments;
  const int64_t first_blocks = A < num_local_experts ? A : num_local_experts;
  const int64_t rest_blocks = (A - first_blocks) / block_e;
  return (int64_t)block_e * (first_blocks + rest_blocks);
}

extern "C" int32_t moe_should_use_masked(int32_t num_experts,
                                         int32_t num_local_experts) {
  // Layout choice of sglang PR #33128 page, Key source snippets: the masked
  // slab is chosen when experts are split across ranks (this rank holds a
  // proper subset) and it holds at most 32 of them; otherwise compact.
  const bool experts_split = num_experts > num_local_experts;
  const bool few_local = num_local_experts <= 32;
  return (experts_split && few_local) ? 1 : 0;
}

extern "C" size_t moe_layout_workspace_bytes(int64_t T, int32_t K, int32_t E) {
  if (T < 0 || K < 1 || E < 1) return 0;
  return mxq::layout_workspace_bytes(T * (int64_t)K, E);
}

extern "C" mxq_status moe_read_overflow(const int32_t* overflow_flag,
                                        int32_t* host_value, void* stream) {
  if (overflow_flag == nullptr || host_value == nullptr)
    return MXQ_ERR_INVALID_ARGUMENT;
  hipStream_t s = mxq::as_stream(stream);
  if (hipMemcpyAsync(host_value, overflow_flag, sizeof(int32_t),
                     hipMemcpyDeviceToHost, s) != hipSuccess)
    return MXQ_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return MXQ_ERR_HIP;
  return *host_value ? MXQ_ERR_CAPACITY_OVERFLOW : MXQ_OK;
}

extern "C" const char* mxq_status_string(mxq_status s) {
  switch (s) {
    case MXQ_OK:
      return "ok";
    case MXQ_ERR_INVALID_ARGUMENT:
      return "invalid argument";
    case MXQ_ERR_UNSUPPORTED:
      return "unsupported format or size";
    case MXQ_ERR_CAPACITY_OVERFLOW:
      return "masked slab capacity exceeded";
    case MXQ_ERR_WORKSPACE:
      return "workspace missing or too small";
    case MXQ_ERR_HIP:
      return "HIP runtime error";
    case MXQ_ERR_SCRATCH_LIMIT:
      return "size exceeds the library's static scratch";
  }
  return "unknown status";
}

extern "C" int32_t mxq_abi_version(void) { return MXQ_ABI_VERSION; }
