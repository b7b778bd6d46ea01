// Internal helpers shared by the library's translation units (not ABI).
#pragma once

namespace pkv {
// Record the hipError_t behind a PKV_ERR_HIP for pkv_last_hip_error (per thread).
void set_hip_error(int e);
}  // namespace pkv
