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

// The head_dim to give the scheduling policy for pools of `dtype`: its time
// model counts 2-byte elements, so an fp8 pool (one byte) moves the bytes of
// a 2-byte pool of half the head dimension.
inline int policy_head_dim(int head_dim, int dtype) {
  return (dtype == PKV_DTYPE_F16_KV_FP8 || dtype == PKV_DTYPE_BF16_KV_FP8) ? head_dim / 2
                                                                          : head_dim;
}
}  // namespace pkv
