// Time model of one candidate plan, used by the scheduling policy on the host
// (pkv_policy) and by the device-side planner (pkv_decode_device_plan).
//
// Source: gist.science explainer, "2. Calibrated Adaptive Policy" (a policy
// calibrated on one seed, judged on held-out seeds) and the fugumt.com (v2)
// abstract ("roofline-style").  include/pkv.h documents the formula; both
// callers evaluate it through this one function, in double precision, with
// floating-point contraction off, so host and device take the same decision.
#pragma once

#include <climits>
#include <cstdint>

#include "pkv.h"

#if defined(__HIP__)
#define PKV_HOST_DEVICE __host__ __device__
#else
#define PKV_HOST_DEVICE
#endif

namespace pkv {

// What the model needs to know about a plan.
struct PlanShape {
  int64_t T = 0;       // tasks
  int64_t P = 0;       // page tiles (page x KV head) in all
  int64_t pmax = 0;    // pages of the largest task
  int64_t maxS = 0;    // splits of the deepest row
  int64_t groups = 0;  // (row, KV head) groups with work
};

PKV_HOST_DEVICE inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// cdiv for 0 <= a and 1 <= b; operands below 2^31 take a 32-bit division
// (the same quotient; a 64-bit division is a long instruction sequence on
// the GPU).
PKV_HOST_DEVICE inline int64_t cdiv_nonneg(int64_t a, int64_t b) {
  if (a <= INT32_MAX && b <= INT32_MAX)
    return static_cast<int64_t>((static_cast<uint32_t>(a) + static_cast<uint32_t>(b) - 1u) /
                                static_cast<uint32_t>(b));
  return cdiv(a, b);
}

// Add row b (n pages) to the shape of the plan (mode, param).
PKV_HOST_DEVICE inline void shape_add_row(PlanShape& f, int64_t n, int32_t Hkv, int32_t mode,
                                          int64_t param) {
  if (n <= 0) return;
  const int64_t c = mode == PKV_MODE_SPLIT ? cdiv(n, param) : param;
  const int64_t S = cdiv(n, c);
  f.T += Hkv * S;
  f.P += Hkv * n;
  f.groups += Hkv;
  const int64_t largest = c < n ? c : n;
  if (largest > f.pmax) f.pmax = largest;
  if (S > f.maxS) f.maxS = S;
}

// The launch form of a plan of shape f: two launches (decode kernel, then
// merge kernel) when its deepest row has more than fuse_max_splits splits
// and its groups times those splits exceed fuse_max_group_splits.
PKV_HOST_DEVICE inline bool two_launch_form(const pkv_policy_params& p, int64_t maxS,
                                            int64_t groups) {
  return maxS > p.fuse_max_splits && groups * maxS > p.fuse_max_group_splits;
}

// Model time (microseconds) of one step of a plan of shape f.  `two`: the
// two-launch form (decode kernel, then merge kernel) instead of the fused one.
PKV_HOST_DEVICE inline double model_us(const pkv_policy_params& p, const PlanShape& f,
                                       int32_t num_cus, int32_t head_dim, int32_t page_size,
                                       bool two) {
#pragma clang fp contract(off)
  if (f.T == 0) return p.t0_us;
  const int64_t cus = num_cus;
  const int64_t W = f.T < 2 * cus ? f.T : 2 * cus;   // decode grid
  const int64_t A = W < cus ? W : cus;               // CUs in use
  const double share = p.hbm_gbps / static_cast<double>(A);
  const double rho = share < p.cu_gbps ? share : p.cu_gbps;
  double load;
  if (f.T <= W) {
    load = static_cast<double>(cdiv_nonneg(f.T, A) * f.pmax);
  } else {
    load = static_cast<double>(f.P) / static_cast<double>(A) +
           p.alpha * static_cast<double>(f.pmax);
  }
  const double tile = 2.0 * page_size * head_dim * 2.0;
  double t = p.t0_us + p.t_round_us * static_cast<double>(cdiv_nonneg(f.T, W)) +
             load * tile / (rho * 1e3);
  if (two) {
    t = t + p.t_two_us + p.t_two_split_us * static_cast<double>(f.maxS);
  } else {
    t = t + p.t_fused_split_us * static_cast<double>(f.maxS);
  }
  return t;
}

}  // namespace pkv
