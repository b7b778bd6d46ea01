// Internal helpers shared by the library's translation units (not ABI).
#pragma once

#include <cstddef>
#include <cstdint>

#include "pkv.h"

namespace pkv {
// Record the hipError_t behind a PKV_ERR_HIP for pkv_last_hip_error (per thread).
void set_hip_error(int e);

// pkv_decode (fused), or pkv_decode_splits then pkv_merge (not fused), with
// optional events ev0 / ev1 (hipEvent_t) that take the decode kernel's own
// start timestamp and the step's last kernel's own end timestamp
// (hipExtLaunchKernel).  Used by the step runner.
int decode_timed(const void* q, const void* k_pool, const void* v_pool, int64_t num_pages,
                 const int32_t* block_table, int32_t max_pages_per_row, const int32_t* seq_lens,
                 const int32_t* tasks, int64_t num_tasks, const int32_t* split_offsets,
                 int64_t num_partial_slots, int32_t B, int32_t Hq, int32_t Hkv, int32_t head_dim,
                 int32_t page_size, int32_t dtype, float scale, float k_scale, float v_scale,
                 void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream,
                 bool fused, void* ev0, void* ev1);

// The head_dim to give the scheduling policy for pools of `dtype`.  Its time
// model counts a page tile at 2-byte elements, and an fp8 pool is priced the
// same: the decode kernel moves an fp8 page in the same number of loads,
// conversions and MFMAs per token, so a workgroup's pages per second barely
// change with the element size (judged on fp8 runs of every trace: held-out
// regret 1.012 mean, 1.052 max, against 1.048 and 1.211 when the model was
// given the fp8 tile's bytes, which let it pick too few splits for one long
// row).
inline int policy_head_dim(int head_dim, int dtype) {
  (void)dtype;
  return head_dim;
}
}  // namespace pkv
