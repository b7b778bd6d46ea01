// Native step runner: one call runs the whole hot path of a decode step.
// It chooses the policy, plans on the host, hands the plan to the kernels
// (pinned memory for a new plan, a device copy for a repeated one), and
// enqueues the decode kernel (and the merge kernel in the two-launch form).
//
// Source: PersistentKV (arXiv 2606.26666), gist.science explainer,
// "Technische Samenvatting" > "2. Calibrated Adaptive Policy" and
// Methodologie ("Row-Local Bounds", "Compact Workqueue").  Host planning is
// part of the step, and the "Evaluatieprotocol" wall timing includes it.
//
// The runner owns a ring of pinned plan buffers, each guarded by a HIP event,
// so a slot is rewritten only after the kernels that read it have completed.
// A step whose plan differs from the previous one is read by its kernels in
// place from pinned host memory (16 bytes per task); the plan is also copied,
// on a side stream, into the tail of the caller's workspace.  Later steps
// with the same plan (the steady state of decoding, where a row's task
// records only change when it crosses a chunk boundary) read that device
// copy, which removes a host-memory round trip from the start of every
// workgroup.  The runner allocates no device memory: every device buffer
// (inputs, outputs, workspace with the plan copy) belongs to the caller.

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "pkv.h"
#include "internal.h"
#include "policy_model.h"

namespace {

struct Slot {
  int32_t* host = nullptr;   // pinned: split_offsets (padded) then tasks
  int32_t* dev = nullptr;    // the same memory as seen by the device
  size_t bytes = 0;
  hipEvent_t done = nullptr; // recorded after the kernels that read it
  bool armed = false;
  int32_t B = 0;
  int64_t T = 0;
};

inline size_t pad4(int64_t n) { return static_cast<size_t>((n + 3) & ~int64_t(3)); }

// Capacity for a plan buffer that must hold `bytes`: at least 64 KiB (about
// 4000 tasks), else the next power of two, so that growing plans reallocate
// (and, for pinned memory, re-pin) only a few times.
inline size_t grown_size(size_t bytes) {
  size_t n = size_t(1) << 16;
  while (n < bytes) n <<= 1;
  return n;
}

}  // namespace

struct pkv_runner {
  int32_t num_cus = 0;
  pkv_policy_params params{};
  std::vector<Slot> ring;
  size_t next = 0;
  Slot* last = nullptr;
  // device copy of the last distinct plan, in the tail of the caller's
  // workspace (dplan_ws, dplan_ws_bytes identify the workspace)
  int device = -1;                 // device the runner was created on
  hipStream_t side = nullptr;      // stream of the uploads
  int32_t* dplan = nullptr;
  const void* dplan_ws = nullptr;
  size_t dplan_ws_bytes = 0;
  std::vector<int32_t> shadow;     // what dplan holds (or will hold)
  bool shadow_valid = false;
  Slot* upload_src = nullptr;      // slot the pending upload reads
  hipEvent_t uploaded = nullptr;   // recorded on `side` after the upload
  uint64_t upload_seq = 0;         // uploads started so far
  uint64_t waited_seq = 0;         // upload that `waited_stream` has waited for
  hipStream_t waited_stream = nullptr;
  hipStream_t reader_stream = nullptr;  // stream of the last kernels that read dplan
  bool have_reader = false;
  hipEvent_t readers_done = nullptr;    // recorded on reader_stream before an upload
};

namespace {

int hip_fail(hipError_t e) {
  pkv::set_hip_error(static_cast<int>(e));
  return PKV_ERR_HIP;
}

// Start copying the plan in `s` (words int32) to `dst` (in the caller's
// workspace) on the side stream, after every kernel enqueued so far on the
// stream that last read the old copy.
int upload_plan(pkv_runner* r, Slot& s, size_t words, int32_t* dst, const void* ws,
                size_t ws_bytes) {
  const size_t bytes = words * sizeof(int32_t);
  hipError_t e = hipSuccess;
  r->shadow_valid = false;
  if (r->have_reader) {
    e = hipEventRecord(r->readers_done, r->reader_stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(r->side, r->readers_done, 0);
    if (e != hipSuccess) return hip_fail(e);
    r->have_reader = false;
  }
  e = hipMemcpyAsync(dst, s.host, bytes, hipMemcpyHostToDevice, r->side);
  if (e == hipSuccess) e = hipEventRecord(r->uploaded, r->side);
  if (e != hipSuccess) return hip_fail(e);
  r->dplan = dst;
  r->dplan_ws = ws;
  r->dplan_ws_bytes = ws_bytes;
  r->shadow.assign(s.host, s.host + words);
  r->shadow_valid = true;
  r->upload_src = &s;
  ++r->upload_seq;
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_runner_create(int32_t num_cus, const pkv_policy_params* params, int32_t ring_depth,
                      pkv_runner** runner) {
  if (!runner || ring_depth < 1 || ring_depth > 1024 || num_cus < 0) return PKV_ERR_INVALID_ARG;
  *runner = nullptr;
  if (num_cus == 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || num_cus <= 0) {
      pkv::set_hip_error(static_cast<int>(e));
      return PKV_ERR_HIP;
    }
  }
  pkv_runner* r = new (std::nothrow) pkv_runner();
  if (!r) return PKV_ERR_INVALID_ARG;
  r->num_cus = num_cus;
  if (params) {
    r->params = *params;
  } else {
    pkv_policy_defaults(&r->params);
  }
  r->ring.resize(static_cast<size_t>(ring_depth));
  {
    hipError_t e = hipGetDevice(&r->device);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&r->side, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&r->uploaded, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&r->readers_done, hipEventDisableTiming);
    if (e != hipSuccess) {
      pkv::set_hip_error(static_cast<int>(e));
      pkv_runner_destroy(r);
      return PKV_ERR_HIP;
    }
  }
  // Buffers of the initial capacity up front, so that the first steps do
  // not pin memory.
  for (Slot& s : r->ring) {
    hipError_t e = hipEventCreateWithFlags(&s.done, hipEventDisableTiming);
    if (e == hipSuccess)
      e = hipHostMalloc(reinterpret_cast<void**>(&s.host), grown_size(0), hipHostMallocDefault);
    if (e == hipSuccess) e = hipHostGetDevicePointer(reinterpret_cast<void**>(&s.dev), s.host, 0);
    if (e != hipSuccess) {
      pkv::set_hip_error(static_cast<int>(e));
      pkv_runner_destroy(r);
      return PKV_ERR_HIP;
    }
    s.bytes = grown_size(0);
  }
  *runner = r;
  return PKV_OK;
}

int pkv_runner_destroy(pkv_runner* r) {
  if (!r) return PKV_OK;
  int st = PKV_OK;
  if (r->readers_done) {
    if (r->have_reader && hipEventRecord(r->readers_done, r->reader_stream) == hipSuccess)
      hipEventSynchronize(r->readers_done);
    hipEventDestroy(r->readers_done);
  }
  if (r->side) {
    hipStreamSynchronize(r->side);
    hipStreamDestroy(r->side);
  }
  if (r->uploaded) hipEventDestroy(r->uploaded);
  for (Slot& s : r->ring) {
    if (s.done) {
      if (s.armed) hipEventSynchronize(s.done);
      hipEventDestroy(s.done);
    }
    if (s.host && hipHostFree(s.host) != hipSuccess) st = PKV_ERR_HIP;
  }
  delete r;
  return st;
}

int pkv_runner_step(pkv_runner* r, pkv_step_args* a) {
  if (!r || !a) return PKV_ERR_INVALID_ARG;
  if (a->B < 0 || (a->B > 0 && !a->seq_lens_host)) return PKV_ERR_INVALID_ARG;

  // policy ("2. Calibrated Adaptive Policy")
  int32_t mode = a->mode, param = a->param;
  if (mode < 0) {
    int st = pkv_policy(a->seq_lens_host, a->B, a->Hkv, pkv::policy_head_dim(a->head_dim, a->dtype),
                        a->page_size, r->num_cus, &r->params, &mode, &param);
    if (st != PKV_OK) return st;
  }
  a->chosen_mode = mode;
  a->chosen_param = param;

  // plan sizes and buffer checks
  int64_t T = 0, slots = 0;
  int st = pkv_plan(a->seq_lens_host, a->B, a->Hkv, a->page_size, a->max_pages_per_row, nullptr,
                    0, mode, param, nullptr, 0, nullptr, &T, &slots);
  if (st != PKV_OK) return st;
  a->num_tasks = T;
  a->num_partial_slots = slots;
  const size_t off_words = pad4(static_cast<int64_t>(a->B) + 1);
  const size_t plan_bytes = (off_words + 4 * static_cast<size_t>(T)) * sizeof(int32_t);
  size_t ws_bytes = 0;
  pkv_workspace_size(slots, a->Hq, a->head_dim, &ws_bytes);
  // the device copy of the plan sits in the last plan_area bytes of the
  // workspace, behind the partial states
  const size_t plan_area = (plan_bytes + 255) & ~size_t(255);
  a->workspace_bytes_needed = ws_bytes + plan_area;
  if (!a->workspace) return PKV_ERR_INVALID_ARG;
  if (a->workspace_bytes < ws_bytes + plan_area) return PKV_ERR_BUFFER_TOO_SMALL;
  int32_t* plan_dst = reinterpret_cast<int32_t*>(
      static_cast<char*>(a->workspace) + ((a->workspace_bytes - plan_area) & ~size_t(255)));

  // a plan slot whose previous readers have finished
  Slot& s = r->ring[r->next];
  r->next = (r->next + 1) % r->ring.size();
  hipStream_t stream = static_cast<hipStream_t>(a->stream);
  hipError_t e = hipSuccess;
  if (s.armed) {
    e = hipEventSynchronize(s.done);
    s.armed = false;
    if (e != hipSuccess) {
      pkv::set_hip_error(static_cast<int>(e));
      return PKV_ERR_HIP;
    }
  }
  if (r->upload_src == &s) {
    // the pending upload reads this slot
    e = hipEventSynchronize(r->uploaded);
    r->upload_src = nullptr;
    if (e != hipSuccess) return hip_fail(e);
  }
  if (s.bytes < plan_bytes) {
    if (s.host) hipHostFree(s.host);
    s.host = s.dev = nullptr;
    s.bytes = 0;
    const size_t want = grown_size(plan_bytes);
    e = hipHostMalloc(reinterpret_cast<void**>(&s.host), want, hipHostMallocDefault);
    if (e == hipSuccess) e = hipHostGetDevicePointer(reinterpret_cast<void**>(&s.dev), s.host, 0);
    if (e != hipSuccess) {
      if (s.host) hipHostFree(s.host);
      s.host = s.dev = nullptr;
      pkv::set_hip_error(static_cast<int>(e));
      return PKV_ERR_HIP;
    }
    s.bytes = want;
  }
  int32_t* offs_h = s.host;
  int32_t* tasks_h = s.host + off_words;
  st = pkv_plan(a->seq_lens_host, a->B, a->Hkv, a->page_size, a->max_pages_per_row, nullptr, 0,
                mode, param, tasks_h, T, offs_h, &T, &slots);
  if (st != PKV_OK) return st;
  for (size_t i = static_cast<size_t>(a->B) + 1; i < off_words; ++i) offs_h[i] = 0;
  int32_t max_splits = 0;
  int64_t active_groups = 0;
  for (int32_t b = 0; b < a->B; ++b) {
    const int32_t sb = offs_h[b + 1] - offs_h[b];
    if (sb > max_splits) max_splits = sb;
    if (sb > 0) active_groups += a->Hkv;
  }
  a->max_splits = max_splits;
  const bool two = a->two_launch < 0 ? pkv::two_launch_form(r->params, max_splits, active_groups)
                                     : (a->two_launch != 0);
  a->chosen_two_launch = two ? 1 : 0;
  s.B = a->B;
  s.T = T;
  r->last = &s;
  const int32_t* offs_d = s.dev;
  const int32_t* tasks_d = s.dev + off_words;

  // The device copy serves this step if it holds the same plan; otherwise
  // the kernels read the pinned slot and the new plan is uploaded for the
  // steps after this one.
  const size_t words = off_words + 4 * static_cast<size_t>(T);
  int dev = -1;
  bool use_dev = false;
  if (hipGetDevice(&dev) == hipSuccess && dev == r->device) {
    if (r->shadow_valid && r->dplan_ws == a->workspace &&
        r->dplan_ws_bytes == a->workspace_bytes && r->dplan == plan_dst &&
        r->shadow.size() == words &&
        std::memcmp(r->shadow.data(), s.host, words * sizeof(int32_t)) == 0) {
      if (r->waited_seq != r->upload_seq || r->waited_stream != stream) {
        e = hipStreamWaitEvent(stream, r->uploaded, 0);
        if (e != hipSuccess) return hip_fail(e);
        r->waited_seq = r->upload_seq;
        r->waited_stream = stream;
      }
      use_dev = true;
      offs_d = r->dplan;
      tasks_d = r->dplan + off_words;
    }
  }
  // Readers of the device copy on another stream go first: the next upload
  // is ordered only after the last reader stream, so a change of stream
  // orders the new one behind the old one's readers.
  if (use_dev && r->have_reader && r->reader_stream != stream) {
    e = hipEventRecord(r->readers_done, r->reader_stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, r->readers_done, 0);
    if (e != hipSuccess) return hip_fail(e);
  }

  // the decode kernel (merge fused in), or decode then merge kernel; the
  // events, if any, take the decode kernel's own start and the last
  // kernel's own end timestamps
  st = pkv::decode_timed(a->q, a->k_pool, a->v_pool, a->num_pages, a->block_table,
                         a->max_pages_per_row, a->seq_lens, tasks_d, T, offs_d, slots, a->B,
                         a->Hq, a->Hkv, a->head_dim, a->page_size, a->dtype, a->scale,
                         a->k_scale, a->v_scale, a->out, a->lse, a->workspace,
                         a->workspace_bytes, a->stream, !two, a->event_before_decode,
                         a->event_after_decode);
  if (st != PKV_OK) return st;
  // A slot the kernels read is free once everything enqueued so far has run.
  // A step served by the device copy leaves its slot unread, and records
  // nothing: an event between two steps costs the stream several
  // microseconds of idle time, and in the steady state every step is such a
  // step.
  if (!use_dev) {
    e = hipEventRecord(s.done, stream);
    if (e != hipSuccess) {
      pkv::set_hip_error(static_cast<int>(e));
      return PKV_ERR_HIP;
    }
    s.armed = true;
  }
  if (use_dev) {
    r->reader_stream = stream;
    r->have_reader = true;
  } else if (st == PKV_OK && dev == r->device) {
    st = upload_plan(r, s, words, plan_dst, a->workspace, a->workspace_bytes);
  }
  return st;
}

int pkv_runner_last_plan(const pkv_runner* r, const int32_t** split_offsets,
                         const int32_t** tasks, int64_t* num_tasks, int32_t* B) {
  if (!r || !split_offsets || !tasks || !num_tasks || !B) return PKV_ERR_INVALID_ARG;
  if (!r->last) return PKV_ERR_INVALID_ARG;
  const Slot& s = *r->last;
  *split_offsets = s.host;
  *tasks = s.host + pad4(static_cast<int64_t>(s.B) + 1);
  *num_tasks = s.T;
  *B = s.B;
  return PKV_OK;
}

}  // extern "C"
