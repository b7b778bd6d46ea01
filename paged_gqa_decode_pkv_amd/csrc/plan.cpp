// Host side of libpkv: status strings, the scheduling policy and the task
// planner.  Pure C++: nothing here touches the device, so it runs and is
// tested on machines without a GPU.
//
// Source: PersistentKV (arXiv 2606.26666), gist.science explainer,
// "Technische Samenvatting" > Methodologie, items "Row-Local Bounds" and
// "Compact Workqueue", and "2. Calibrated Adaptive Policy".

#include "pkv.h"
#include "internal.h"

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
    default: return "unknown status";
  }
}

int pkv_policy_defaults(pkv_policy_params* p) {
  if (!p) return PKV_ERR_INVALID_ARG;
  p->tasks_per_cu = 0.75f;
  p->chunk_min = 4;
  p->chunk_max = 256;
  p->split_max = 256;
  p->uniform_ratio = 1.25f;
  p->fuse_max_splits = 16;
  return PKV_OK;
}

// "2. Calibrated Adaptive Policy": split for one long row, workqueue for a
// ragged batch.  The thresholds are this library's own.
int pkv_policy(const int32_t* seq_lens, int32_t B, int32_t Hkv, int32_t page_size,
               int32_t num_cus, const pkv_policy_params* params, int32_t* mode,
               int32_t* param) {
  if (!mode || !param || B < 0 || (B > 0 && !seq_lens) || Hkv < 1 || page_size < 1 ||
      num_cus < 1)
    return PKV_ERR_INVALID_ARG;
  pkv_policy_params p;
  if (params) {
    p = *params;
  } else {
    pkv_policy_defaults(&p);
  }
  if (!(p.tasks_per_cu > 0.0f) || p.chunk_min < 1 || p.chunk_max < p.chunk_min ||
      p.split_max < 1 || !(p.uniform_ratio >= 1.0f) || p.fuse_max_splits < 0)
    return PKV_ERR_INVALID_ARG;

  int64_t active = 0, total = 0, nmin = INT64_MAX, nmax = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (seq_lens[b] < 0) return PKV_ERR_INVALID_ARG;
    const int64_t n = ceil_div(seq_lens[b], page_size);
    if (n == 0) continue;
    ++active;
    total += n;
    if (n < nmin) nmin = n;
    if (n > nmax) nmax = n;
  }
  if (active == 0) {
    *mode = PKV_MODE_SPLIT;
    *param = 1;
    return PKV_OK;
  }
  const double target = static_cast<double>(p.tasks_per_cu) * num_cus;
  if (active == 1 ||
      static_cast<double>(nmax) <= static_cast<double>(p.uniform_ratio) * nmin) {
    const double want = target / static_cast<double>(active * Hkv);
    int64_t S = 1;
    while (S < want && S < p.split_max) S *= 2;
    if (S > p.split_max) S = p.split_max;
    *mode = PKV_MODE_SPLIT;
    *param = static_cast<int32_t>(S);
    return PKV_OK;
  }
  const double per = static_cast<double>(Hkv) * static_cast<double>(total) / target;
  int64_t c = 1;
  while (static_cast<double>(c * 2) <= per) c *= 2;
  if (c < p.chunk_min) c = p.chunk_min;
  if (c > p.chunk_max) c = p.chunk_max;
  *mode = PKV_MODE_WORKQUEUE;
  *param = static_cast<int32_t>(c);
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
