// Host side of libpkv: status strings, the scheduling policy and the task
// planner.  Pure C++: nothing here touches the device, so it runs and is
// tested on machines without a GPU.
//
// Source: PersistentKV (arXiv 2606.26666), gist.science explainer,
// "Technische Samenvatting" > Methodologie, items "Row-Local Bounds" and
// "Compact Workqueue", and "2. Calibrated Adaptive Policy".

#include "pkv.h"
#include "internal.h"
#include "policy_model.h"

#include <cstdint>
#include <cstring>

namespace {

constexpr int32_t kPageSize = 16;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

thread_local int g_last_hip_error = 0;

}  // namespace

namespace pkv {
void set_hip_error(int e) { g_last_hip_error = e; }
}  // namespace pkv

extern "C" {

int pkv_abi_version(void) { return PKV_ABI_VERSION; }

int pkv_last_hip_error(void) { return g_last_hip_error; }

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported shape (head_dim, page_size or GQA ratio)";
    case PKV_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case PKV_ERR_BAD_INDEX: return "block-table entry outside the page pool";
    case PKV_ERR_HIP: return "HIP runtime error";
    case PKV_ERR_SCRATCH_TOO_SMALL:
      return "step larger than the static workspace of pkv_decode_static (16 MiB)";
    default: return "unknown status";
  }
}

int pkv_policy_defaults(pkv_policy_params* p) {
  if (!p) return PKV_ERR_INVALID_ARG;
  p->split_max = 256;
  p->chunk_min = 4;
  p->chunk_max = 256;
  p->fuse_max_splits = 16;
  p->fuse_max_group_splits = 256;
  // Fitted on the calibration seed (paged_gqa_decode_pkv_amd/calibration/
  // mi355x_fit.json, written by policy_fit.py from calibrate.py's runs).
  p->t0_us = 2.309;
  p->t_round_us = 4.153;
  p->alpha = 1.145;
  p->cu_gbps = 46.34;
  p->hbm_gbps = 8667.0;
  p->t_two_us = 6.018;
  p->t_two_split_us = 0.0436;
  p->t_fused_split_us = 0.2422;
  return PKV_OK;
}

}  // extern "C"

namespace {

using pkv::PlanShape;

PlanShape plan_shape(const int32_t* seq_lens, int32_t B, int32_t Hkv, int32_t page_size,
                     int32_t mode, int64_t param) {
  PlanShape f;
  for (int32_t b = 0; b < B; ++b)
    pkv::shape_add_row(f, ceil_div(seq_lens[b], page_size), Hkv, mode, param);
  return f;
}

using pkv::model_us;

int check_policy_args(const int32_t* seq_lens, int32_t B, int32_t Hkv, int32_t head_dim,
                      int32_t page_size, int32_t num_cus, const pkv_policy_params& p) {
  if (B < 0 || (B > 0 && !seq_lens) || Hkv < 1 || head_dim < 1 || page_size < 1 || num_cus < 1)
    return PKV_ERR_INVALID_ARG;
  if (p.split_max < 1 || p.chunk_min < 1 || p.chunk_max < p.chunk_min || p.fuse_max_splits < 0 ||
      p.fuse_max_group_splits < 0)
    return PKV_ERR_INVALID_ARG;
  if (!(p.cu_gbps > 0.0) || !(p.hbm_gbps > 0.0) || !(p.t0_us >= 0.0) ||
      !(p.t_round_us >= 0.0) || !(p.alpha >= 0.0) || !(p.t_two_us >= 0.0) ||
      !(p.t_two_split_us >= 0.0) || !(p.t_fused_split_us >= 0.0))
    return PKV_ERR_INVALID_ARG;
  for (int32_t b = 0; b < B; ++b)
    if (seq_lens[b] < 0) return PKV_ERR_INVALID_ARG;
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_policy_predict(const int32_t* seq_lens, int32_t B, int32_t Hkv, int32_t head_dim,
                       int32_t page_size, int32_t num_cus, const pkv_policy_params* params,
                       int32_t mode, int32_t param, int32_t two_launch, double* us) {
  pkv_policy_params p;
  if (params) {
    p = *params;
  } else {
    pkv_policy_defaults(&p);
  }
  if (!us || (mode != PKV_MODE_SPLIT && mode != PKV_MODE_WORKQUEUE) || param < 1)
    return PKV_ERR_INVALID_ARG;
  const int st = check_policy_args(seq_lens, B, Hkv, head_dim, page_size, num_cus, p);
  if (st != PKV_OK) return st;
  const PlanShape f = plan_shape(seq_lens, B, Hkv, page_size, mode, param);
  const bool two = two_launch < 0 ? pkv::two_launch_form(p, f.maxS, f.groups) : two_launch != 0;
  *us = model_us(p, f, num_cus, head_dim, page_size, two);
  return PKV_OK;
}

// "2. Calibrated Adaptive Policy": the fastest candidate under the fitted
// roofline-style model (include/pkv.h documents the model).
int pkv_policy(const int32_t* seq_lens, int32_t B, int32_t Hkv, int32_t head_dim,
               int32_t page_size, int32_t num_cus, const pkv_policy_params* params,
               int32_t* mode, int32_t* param) {
  if (!mode || !param) return PKV_ERR_INVALID_ARG;
  pkv_policy_params p;
  if (params) {
    p = *params;
  } else {
    pkv_policy_defaults(&p);
  }
  const int st = check_policy_args(seq_lens, B, Hkv, head_dim, page_size, num_cus, p);
  if (st != PKV_OK) return st;
  int64_t active = 0;
  for (int32_t b = 0; b < B; ++b)
    if (seq_lens[b] > 0) ++active;
  if (active == 0) {
    *mode = PKV_MODE_SPLIT;
    *param = 1;
    return PKV_OK;
  }
  bool have = false;
  double best = 0.0;
  auto consider = [&](int32_t m, int64_t v) {
    const PlanShape f = plan_shape(seq_lens, B, Hkv, page_size, m, v);
    const double t =
        model_us(p, f, num_cus, head_dim, page_size, pkv::two_launch_form(p, f.maxS, f.groups));
    if (!have || t < best) {
      have = true;
      best = t;
      *mode = m;
      *param = static_cast<int32_t>(v);
    }
  };
  // The mode follows the explainer's rule: a single long row is split along
  // the sequence, a batch of rows goes through the compact workqueue.  The
  // fitted model picks the split count or the chunk.
  if (active == 1) {
    for (int64_t S = 1; S <= p.split_max; S *= 2) consider(PKV_MODE_SPLIT, S);
  } else {
    for (int64_t c = p.chunk_min; c <= p.chunk_max; c *= 2) consider(PKV_MODE_WORKQUEUE, c);
  }
  return PKV_OK;
}

// "Row-Local Bounds" + "Compact Workqueue": per-row chunking from the true
// length, one record per non-empty (row, KV head, split).
int pkv_plan(const int32_t* seq_lens, int32_t B, int32_t Hkv, int32_t page_size,
             int32_t max_pages_per_row, const int32_t* block_table, int64_t num_pages,
             int32_t mode, int32_t param, int32_t* tasks, int64_t task_cap,
             int32_t* split_offsets, int64_t* num_tasks, int64_t* num_partial_slots) {
  if (!num_tasks || !num_partial_slots || B < 0 || (B > 0 && !seq_lens) || Hkv < 1 ||
      max_pages_per_row < 0 || param < 1 || task_cap < 0)
    return PKV_ERR_INVALID_ARG;
  if (page_size != kPageSize) return PKV_ERR_INVALID_ARG;
  if (mode != PKV_MODE_SPLIT && mode != PKV_MODE_WORKQUEUE) return PKV_ERR_INVALID_ARG;

  // Pass 1: per-row split counts, validation, totals.
  int64_t slots = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t N = seq_lens[b];
    if (N < 0) return PKV_ERR_INVALID_ARG;
    const int64_t n = ceil_div(N, page_size);
    if (n > max_pages_per_row) return PKV_ERR_INVALID_ARG;
    if (n == 0) continue;
    const int64_t c = (mode == PKV_MODE_SPLIT) ? ceil_div(n, param) : param;
    slots += ceil_div(n, c);
    if (block_table) {
      if (num_pages < 0) return PKV_ERR_INVALID_ARG;
      const int32_t* row = block_table + static_cast<int64_t>(b) * max_pages_per_row;
      for (int64_t p = 0; p < n; ++p)
        if (row[p] < 0 || row[p] >= num_pages) return PKV_ERR_BAD_INDEX;
    }
  }
  const int64_t T = slots * Hkv;
  if (T > INT32_MAX || slots > INT32_MAX) return PKV_ERR_INVALID_ARG;
  *num_tasks = T;
  *num_partial_slots = slots;
  if (tasks && task_cap < T) return PKV_ERR_BUFFER_TOO_SMALL;

  // Pass 2: offsets and records in (row, KV head, split) order.
  int64_t off = 0, t = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t n = ceil_div(seq_lens[b], page_size);
    const int64_t c = n == 0 ? 1 : (mode == PKV_MODE_SPLIT ? ceil_div(n, param) : param);
    const int64_t S = n == 0 ? 0 : ceil_div(n, c);
    if (split_offsets) split_offsets[b] = static_cast<int32_t>(off);
    off += S;
    if (!tasks) continue;
    for (int32_t g = 0; g < Hkv; ++g) {
      for (int64_t s = 0; s < S; ++s, ++t) {
        int32_t* r = tasks + 4 * t;
        r[0] = b;
        r[1] = g;
        r[2] = static_cast<int32_t>(s);
        r[3] = static_cast<int32_t>(c);
      }
    }
  }
  if (split_offsets) split_offsets[B] = static_cast<int32_t>(off);
  return PKV_OK;
}

int pkv_workspace_size(int64_t num_partial_slots, int32_t Hq, int32_t head_dim,
                       size_t* bytes) {
  if (!bytes || num_partial_slots < 0 || Hq < 0 || head_dim < 0) return PKV_ERR_INVALID_ARG;
  const uint64_t per_slot = static_cast<uint64_t>(Hq) * (static_cast<uint64_t>(head_dim) + 2) * 4;
  uint64_t total = PKV_WORKSPACE_HEADER_BYTES + static_cast<uint64_t>(num_partial_slots) * per_slot;
  total = (total + 255) & ~static_cast<uint64_t>(255);
  *bytes = static_cast<size_t>(total);
  return PKV_OK;
}

}  // extern "C"
