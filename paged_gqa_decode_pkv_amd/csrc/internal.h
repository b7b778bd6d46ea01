// Internal helpers shared by the library's translation units (not ABI).
#pragma once

#include "pkv.h"

namespace pkv {
// Record the hipError_t behind a PKV_ERR_HIP for pkv_last_hip_error (per thread).
void set_hip_error(int e);

// The head_dim to give the scheduling policy for pools of `dtype`: its time
// model counts 2-byte elements, so an fp8 pool (one byte) moves the bytes of
// a 2-byte pool of half the head dimension.
inline int policy_head_dim(int head_dim, int dtype) {
  return (dtype == PKV_DTYPE_F16_KV_FP8 || dtype == PKV_DTYPE_BF16_KV_FP8) ? head_dim / 2
                                                                          : head_dim;
}
}  // namespace pkv
