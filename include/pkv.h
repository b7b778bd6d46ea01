/*
 * pkv.h -- C ABI of libpkv.so: paged grouped-query-attention decode for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (PersistentKV, arXiv 2606.26666):
 *   single-query (decode) attention for grouped-query attention.  G = Hq/Hkv
 *   query heads share one KV head (gist.science explainer, "Technische
 *   Samenvatting" > Methodologie > "1. Native Block-Table Decode Engine").  It
 *   runs in place over a paged KV cache through a block table, without
 *   repacking pages (same section, item "Layout").  Work is mapped by
 *   (batch row, KV head, sequence split), so one K/V page tile serves all G
 *   query heads of its group (Lattice and fugumt.com abstracts).  Long rows
 *   are split into disjoint ranges whose partial online-softmax states a
 *   separate merge combines exactly (item "Sequentie Splitting").  Ranges
 *   follow each row's true length (item "Row-Local Bounds").  Only non-empty
 *   (row, KV head, split) tasks are emitted, as a 1-D list (item "Compact
 *   Workqueue").
 *
 * For row b and query head h, with g = floor(h / G) and N_b = seq_lens[b]:
 *   s_t = scale * <q[b,h,:], K[page(b,t), g, t%16, :]>     t in [0, N_b)
 *   out[b,h,:] = sum_t softmax(s)_t * V[page(b,t), g, t%16, :]
 *   lse[b,h]   = log sum_t exp(s_t)
 *   with page(b,t) = block_table[b, t/16].
 * A row with N_b = 0 gets out = 0 and lse = -inf.
 *
 * Conventions
 *   - Every call returns an int status (pkv_status).  No exception crosses
 *     the ABI.  The one-shot entry points allocate no device memory and keep
 *     no per-call state; the caller owns every buffer.  (A step runner owns
 *     its plan buffers; see pkv_runner_create.)
 *   - "stream" is a hipStream_t passed as void* (NULL = the null stream).
 *     Device work is enqueued asynchronously and never synchronised.
 *   - Supported shapes: page_size = 16, head_dim in {64, 128, 256},
 *     G = Hq/Hkv in {1, 2, 4, 8, 16}.  Others return
 *     PKV_ERR_UNSUPPORTED.
 *   - Data types: q and out are fp16 or bf16; the K and V pools are the same
 *     type or fp8 E4M3 with per-tensor dequantisation scales (pkv_dtype).
 *     lse and the partial states are fp32.  Indices are int32.
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 6

/* Fixed-size head of every workspace: control words (task counter, exit
 * counter, error word) and the per-(row, KV head) arrival counters of the
 * fused merge.  pkv_workspace_init zeroes it.  Every launch leaves it zeroed
 * again, except the sticky error word. */
#define PKV_WORKSPACE_HEADER_BYTES 65536
/* Largest B * Hkv the single-launch (fused-merge) decode serves.  Larger
 * batches fall back to the two-launch form. */
#define PKV_MAX_FUSED_GROUPS ((PKV_WORKSPACE_HEADER_BYTES - 256) / 4)

/* Status codes. */
enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,      /* null pointer, negative size, inconsistent shapes */
  PKV_ERR_UNSUPPORTED = 2,      /* head_dim, page_size or G outside the supported set */
  PKV_ERR_BUFFER_TOO_SMALL = 3, /* caller buffer too small; size outputs hold the need */
  PKV_ERR_BAD_INDEX = 4,        /* block-table entry outside [0, num_pages) */
  PKV_ERR_HIP = 5,              /* a HIP runtime call failed; see pkv_last_hip_error */
  PKV_ERR_SCRATCH_TOO_SMALL = 6 /* pkv_decode_static: the step needs more than its static
                                   workspace (PKV_STATIC_SCRATCH_BYTES) */
};

/* Element types of q and out (E) and of the K and V pools.  Scores, softmax
 * state and accumulators are fp32 in every case; lse is fp32.  The fp8 pools
 * hold OCP 8-bit floating point E4M3 codes ("e4m3fn": bias 7, no
 * infinities, S.1111.111 is NaN; OCP 8-bit Floating Point Specification
 * (OFP8)), each exactly representable in E; their dequantised value is
 * k_scale * code (K) and v_scale * code (V), per-tensor scales that the
 * decode entry points take. */
enum pkv_dtype {
  PKV_DTYPE_F16 = 0,          /* q, K, V, out: IEEE half */
  PKV_DTYPE_BF16 = 1,         /* q, K, V, out: bfloat16 */
  PKV_DTYPE_F16_KV_FP8 = 2,   /* q, out: IEEE half; K, V: fp8 E4M3 */
  PKV_DTYPE_BF16_KV_FP8 = 3   /* q, out: bfloat16; K, V: fp8 E4M3 */
};

/* Scheduling modes of the task list (gist.science explainer, "2. Calibrated
 * Adaptive Policy": sequence splitting for one long row, the compact
 * workqueue for batches of 8 or more long rows). */
enum pkv_mode {
  PKV_MODE_SPLIT = 0,     /* param = S: every row is cut into at most S splits */
  PKV_MODE_WORKQUEUE = 1  /* param = c: every split holds c pages (the last may hold fewer) */
};

/* Bits of the device error word that pkv_decode's kernels set (sticky until
 * pkv_workspace_init).  A flagged task or page is skipped, never read. */
enum pkv_device_error {
  PKV_DEVERR_TASK = 1u,        /* task record out of range for B, Hkv or the row length */
  PKV_DEVERR_PAGE = 2u,        /* block-table entry outside [0, num_pages) */
  PKV_DEVERR_ROW = 4u,         /* seq_lens[b] < 0 or above max_pages_per_row * 16 */
  PKV_DEVERR_SLOT = 8u         /* split_offsets points outside the partial-state slots */
};

/* Policy constants: the candidate sets and the cost model (see pkv_policy).
 * The pages print no thresholds.  The defaults are this library's own fit on
 * the calibration seed (see pkv_policy_defaults). */
typedef struct pkv_policy_params {
  int32_t split_max;        /* split candidates S = 1, 2, 4, ... <= split_max */
  int32_t chunk_min;        /* workqueue candidates c = chunk_min, 2 chunk_min, ... */
  int32_t chunk_max;        /*   ... <= chunk_max, in pages */
  int32_t fuse_max_splits;  /* the fused single launch when no row has more
                               splits than this, ... */
  int32_t fuse_max_group_splits; /* ... or when (row, KV head) groups x the deepest
                               row's splits is at most this; else the two-launch
                               form (the fused merge runs at the tail of a split
                               group, one group per workgroup, so many long
                               groups favour the separate merge kernel) */
  /* cost model of one step (microseconds, GB/s) */
  double t0_us;             /* fixed time of a step */
  double t_round_us;        /* per round of tasks, ceil(T / W) */
  double alpha;             /* dynamic-queue imbalance, in largest tasks */
  double cu_gbps;           /* streaming rate of one CU */
  double hbm_gbps;          /* streaming rate of the chip */
  double t_two_us;          /* extra fixed time of the two-launch form */
  double t_two_split_us;    /* two-launch: per split of the deepest row */
  double t_fused_split_us;  /* fused merge: per split of the deepest row */
} pkv_policy_params;

/* ABI version (PKV_ABI_VERSION of the built library). */
int pkv_abi_version(void);

/*
 * Cache policy the decode kernel gives its K/V page loads for a plan (a
 * performance choice of the library; results do not depend on it):
 *   0  default for K and V (2-byte pools at head_dim 256);
 *   1  non-temporal (streaming) V loads: every other plan, except
 *   2  non-temporal K and V loads: 2-byte pools whose plan has more than
 *      2 * num_cus tasks.
 * num_tasks < 0 asks for a self-planned step (pkv_decode_device_plan).
 * Host only; no device is touched.  PKV_ERR_INVALID_ARG for a NULL `mode`,
 * num_cus < 1 or an unknown dtype, PKV_ERR_UNSUPPORTED for a head_dim outside
 * {64, 128, 256}.
 */
int pkv_page_load_mode(int32_t head_dim, int32_t dtype, int64_t num_tasks, int32_t num_cus,
                       int32_t* mode);

/* Static, human-readable text of a status code.  Never NULL. */
const char* pkv_status_string(int status);

/* hipError_t of the last PKV_ERR_HIP returned on this thread (0 if none). */
int pkv_last_hip_error(void);

/* Fill *params with the default policy constants: split_max 256, chunks
 * 4..256, fuse_max_splits 16, fuse_max_group_splits 256, and the cost model fitted on seed 20260622 of
 * the calibration traces on one MI355X (256 CUs): every candidate schedule of
 * eight trace families (B = 1 fixed and bucketed, 4, 8 bimodal / Zipf /
 * uniform, 32, 64) timed on the GPU, least squares on log time.  Returns
 * PKV_ERR_INVALID_ARG if params is NULL. */
int pkv_policy_defaults(pkv_policy_params* params);

/*
 * pkv_policy -- choose the scheduling mode and its parameter for one step.
 * Host only and deterministic.  The device is not touched.
 *
 * Source: gist.science explainer, "2. Calibrated Adaptive Policy": a single
 * long row uses sequence splitting to open enough parallel work; a batch of
 * 8 or more long rows uses the compact workqueue, which amortises the
 * split+merge overhead; the thresholds are calibrated on one seed and judged
 * on held-out seeds ("Resultaten").  The fugumt.com (v2) abstract calls the
 * policy "roofline-style".  The branches that hand work to another library
 * are outside this library.
 *
 * The mode follows the explainer's rule: a batch with one active row (N_b >
 * 0) is split along the sequence, a batch with two or more active rows goes
 * through the workqueue.  Within the mode, the policy predicts the time of
 * every candidate plan with a roofline-style model and returns the fastest.
 * Candidates, in this order (ties keep the earlier one): one active row,
 * SPLIT with S = 1, 2, 4, ... <= split_max; otherwise WORKQUEUE with
 * c = chunk_min, 2 chunk_min, ... <= chunk_max.  For a candidate, with
 * n_b = ceil(N_b / page_size), c_b the chunk of row b (SPLIT: ceil(n_b/S);
 * WORKQUEUE: c) and S_b = ceil(n_b / c_b) over rows with n_b > 0:
 *   T = Hkv sum S_b tasks, P = Hkv sum n_b page tiles,
 *   pmax = max min(c_b, n_b), maxS = max S_b,
 *   W = min(T, 2 num_cus) workgroups (the decode grid), A = min(W, num_cus),
 *   rho = min(cu_gbps, hbm_gbps / A)                 per-CU rate,
 *   load = ceil(T / A) pmax              if T <= W   (every task static)
 *        = P / A + alpha pmax            otherwise   (dynamic queue),
 *   tile = 2 * page_size * head_dim * 2 bytes (K and V of one page of one
 *          KV head at 2-byte elements; fp8 pools are priced the same, since
 *          the kernel streams their pages at about the same pages per
 *          second),
 *   two = maxS > fuse_max_splits and Gr maxS > fuse_max_group_splits, with
 *         Gr = Hkv x (rows with n_b > 0) the (row, KV head) groups,
 *   t = t0_us + t_round_us ceil(T / W) + load tile / (rho 1e3)
 *       + (two ? t_two_us + t_two_split_us maxS : t_fused_split_us maxS).
 * All in double precision, in this order of operations (pkv_policy_predict
 * returns t).  No active row gives (SPLIT, 1).
 *
 * seq_lens: host int32 [B].  params: NULL selects the defaults.
 * Outputs *mode (pkv_mode) and *param.
 * Errors: PKV_ERR_INVALID_ARG for a NULL pointer, B < 0, Hkv < 1,
 * head_dim < 1, page_size < 1, num_cus < 1, a negative length or parameters
 * outside their domain (split_max < 1, chunk_min < 1, chunk_max < chunk_min,
 * fuse_max_splits < 0, fuse_max_group_splits < 0, a rate <= 0, a negative
 * time or alpha).
 */
int pkv_policy(const int32_t* seq_lens, int32_t B, int32_t Hkv, int32_t head_dim,
               int32_t page_size, int32_t num_cus, const pkv_policy_params* params,
               int32_t* mode, int32_t* param);

/* The model time t (microseconds) of one candidate (mode, param) of
 * pkv_policy, for tools and tests.  two_launch < 0 applies the policy's
 * launch-form rule (`two` above); 0 / 1 force the fused / two-launch term.  Same
 * arguments and errors as pkv_policy, plus PKV_ERR_INVALID_ARG for an unknown
 * mode or param < 1. */
int pkv_policy_predict(const int32_t* seq_lens, int32_t B, int32_t Hkv, int32_t head_dim,
                       int32_t page_size, int32_t num_cus, const pkv_policy_params* params,
                       int32_t mode, int32_t param, int32_t two_launch, double* us);

/*
 * pkv_plan -- build the compact task list and the per-row split offsets.
 * Host only and deterministic.
 *
 * Source: gist.science explainer, Methodologie, items "Row-Local Bounds" and
 * "Compact Workqueue".  Tile counts and split ranges follow each row's true
 * length, and only non-empty (row, KV head, split) intervals become tasks.
 * The Lattice and fugumt.com abstracts say the same.
 *
 * With n_b = ceil(N_b / page_size):
 *   chunk c_b = ceil(n_b / param)   in PKV_MODE_SPLIT
 *             = param               in PKV_MODE_WORKQUEUE
 *   S_b = ceil(n_b / c_b), or 0 when N_b = 0.
 *   Task record = int32[4] {row b, kv_head g, split s, c_b}, ordered by b,
 *   then g, then s.  Split s covers pages [s*c_b, min((s+1)*c_b, n_b)), that
 *   is tokens [s*c_b*16, min((s+1)*c_b*16, N_b)).
 *   num_tasks = Hkv * sum_b S_b.
 *   split_offsets[0..B] = the exclusive prefix sum of S_b.
 *   num_partial_slots = split_offsets[B].  Split s of row b owns slot
 *   split_offsets[b] + s.
 *
 * Arguments:
 *   seq_lens          host int32 [B]
 *   max_pages_per_row row stride of block_table.  Every n_b must be <= it.
 *   block_table       host int32 [B, max_pages_per_row], or NULL.  If given,
 *                     every entry a task will read (p < n_b) must lie in
 *                     [0, num_pages).  Otherwise PKV_ERR_BAD_INDEX.
 *   num_pages         pool size in pages.  Checked only when block_table != NULL.
 *   tasks             host int32 [task_cap][4], or NULL for a size query
 *   split_offsets     host int32 [B+1], or NULL
 *   num_tasks, num_partial_slots  outputs, always written on PKV_OK and on
 *                     PKV_ERR_BUFFER_TOO_SMALL
 * Errors: PKV_ERR_INVALID_ARG (NULL seq_lens / outputs, negative length,
 * n_b > max_pages_per_row, unknown mode, param < 1, page_size != 16,
 * more than 2^31-1 tasks); PKV_ERR_BAD_INDEX; PKV_ERR_BUFFER_TOO_SMALL when
 * tasks != NULL and task_cap < num_tasks.
 */
int pkv_plan(const int32_t* seq_lens, int32_t B, int32_t Hkv, int32_t page_size,
             int32_t max_pages_per_row, const int32_t* block_table, int64_t num_pages,
             int32_t mode, int32_t param, int32_t* tasks, int64_t task_cap,
             int32_t* split_offsets, int64_t* num_tasks, int64_t* num_partial_slots);

/*
 * pkv_workspace_size -- device workspace bytes that pkv_decode needs.
 * Layout: the PKV_WORKSPACE_HEADER_BYTES header (a 256-byte control block:
 * task counter, exit counter, error word; then uint32 arrival counters of
 * the fused merge, one per (row, KV head)), then the fp32 partial outputs
 * [num_partial_slots][Hq][head_dim], then the fp32 (max, sum) pairs
 * [num_partial_slots][Hq][2].  The total is rounded up to 256 bytes.
 * Errors: PKV_ERR_INVALID_ARG for NULL bytes or a negative size.
 */
int pkv_workspace_size(int64_t num_partial_slots, int32_t Hq, int32_t head_dim,
                       size_t* bytes);

/*
 * pkv_workspace_init -- zero the workspace header on `stream`.  Call it
 * once after allocating a workspace.  It also clears the device error word.
 * Every decode leaves the counters at zero when it completes, so one init
 * serves any number of later decodes on that workspace.
 * Errors: PKV_ERR_INVALID_ARG (NULL or smaller than the header), PKV_ERR_HIP.
 */
int pkv_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_workspace_error_flags -- copy the device error word (pkv_device_error
 * bits) to *flags.  This synchronises `stream`, so it is for tests and
 * debugging, not the hot path.
 */
int pkv_workspace_error_flags(const void* workspace, uint32_t* flags, void* stream);

/*
 * pkv_decode -- run one decode step in ONE launch: the persistent decode
 * kernel over the task list, with the split merge fused into it.
 *
 * Source: gist.science explainer, Methodologie, item "Sequentie Splitting".
 * Each split computes a partial online-softmax state, and the states are
 * combined exactly.  Item "Compact Workqueue": one 1-D grid runs the task
 * list.  The pages run the combination as a separate merge kernel, 2
 * launches per step (fugumt.com abstract).  That form is
 * pkv_decode_splits followed by pkv_merge.  Here the workgroup that finishes
 * the last split of a (row, KV head) merges that group instead.  It finds
 * out through a device-scope arrival counter, which every workgroup bumps
 * for its splits once its write-through partial stores are acknowledged.
 * The arithmetic is that of pkv_merge.  A row with a single split
 * writes its output directly.  A row with N_b = 0 gets out = 0 and
 * lse = -inf.  With B * Hkv > PKV_MAX_FUSED_GROUPS, or no task at all, the
 * call falls back to the two-launch form.
 *
 * All pointers are device pointers.  Tensors are contiguous, row-major; E is
 * the q / out element type of `dtype` (pkv_dtype: fp16 or bf16):
 *   q            E     [B, Hq, head_dim]
 *   k_pool       KV    [num_pages, Hkv, page_size, head_dim]
 *   v_pool       KV    [num_pages, Hkv, page_size, head_dim]
 *                (KV = E, or fp8 E4M3 codes for the *_KV_FP8 types)
 *   block_table  int32 [B, max_pages_per_row]
 *   seq_lens     int32 [B]
 *   tasks        int32 [num_tasks][4] and split_offsets int32 [B+1], as
 *                written by pkv_plan for the same seq_lens, Hkv and
 *                page_size.  Device memory or device-mapped pinned host
 *                memory (the runner uses the latter).
 *   out          E     [B, Hq, head_dim], rounded to nearest even
 *   lse          fp32  [B, Hq] natural-log log-sum-exp, or NULL
 *   workspace    >= pkv_workspace_size(num_partial_slots, Hq, head_dim)
 *                bytes, 256-byte aligned, initialised once by
 *                pkv_workspace_init.  Calls that share a workspace must be
 *                ordered on one stream.  Concurrent calls need separate
 *                workspaces.
 * scale is the softmax scale (1/sqrt(head_dim) for standard attention).
 * k_scale and v_scale dequantise the pools: attention runs over
 * k_scale * K and v_scale * V (pass 1 and 1 for fp16 / bf16 pools; with 1
 * the result is bit for bit the unscaled one).  Both must be finite and > 0.
 * q, k_pool, v_pool and out must be 16-byte aligned.
 *
 * Validation: scalar arguments and the alignment are checked on the host.
 * Device data is checked by the kernels.  A bad task record, block-table
 * entry, row length or slot is skipped and flagged in the device error word
 * (pkv_workspace_error_flags).  It is never dereferenced.
 * Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_BUFFER_TOO_SMALL
 * (workspace), PKV_ERR_HIP (launch failure).
 */
int pkv_decode(const void* q, const void* k_pool, const void* v_pool, int64_t num_pages,
               const int32_t* block_table, int32_t max_pages_per_row,
               const int32_t* seq_lens, const int32_t* tasks, int64_t num_tasks,
               const int32_t* split_offsets, int64_t num_partial_slots, int32_t B,
               int32_t Hq, int32_t Hkv, int32_t head_dim, int32_t page_size, int32_t dtype,
               float scale, float k_scale, float v_scale, void* out, float* lse,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_decode_static -- pkv_decode without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.
 *
 * The step's workspace is a static device array of PKV_STATIC_SCRATCH_BYTES
 * (16 MiB) in the library, one per GPU, held from the library's first use
 * on that GPU until the process ends; its address is looked up once per
 * device (the first call on it, with that device current).  Nothing is
 * allocated or freed, here or later.  Every call first zeroes the array's
 * control block and this step's arrival counters with a small kernel on
 * `stream` (no memset), then runs pkv_decode's kernels on it.  Every call on
 * one GPU shares that GPU's array, and the array keeps the last call's
 * contents: calls that overlap on one GPU (other streams, other threads)
 * race, so they must be ordered.  The device error word of the array is
 * cleared by each call and not reported; check the block table on the host
 * (pkv_plan with block_table) beforehand.
 * Arguments, layouts and results: those of pkv_decode without workspace and
 * workspace_bytes; the results are bit for bit pkv_decode's.
 * Errors: those of pkv_decode, and PKV_ERR_SCRATCH_TOO_SMALL when
 * pkv_workspace_size(num_partial_slots, Hq, head_dim) exceeds
 * PKV_STATIC_SCRATCH_BYTES (checked on the host before anything is
 * launched).
 */
#define PKV_STATIC_SCRATCH_BYTES (16u << 20)
int pkv_decode_static(const void* q, const void* k_pool, const void* v_pool, int64_t num_pages,
                      const int32_t* block_table, int32_t max_pages_per_row,
                      const int32_t* seq_lens, const int32_t* tasks, int64_t num_tasks,
                      const int32_t* split_offsets, int64_t num_partial_slots, int32_t B,
                      int32_t Hq, int32_t Hkv, int32_t head_dim, int32_t page_size,
                      int32_t dtype, float scale, float k_scale, float v_scale, void* out,
                      float* lse, void* stream);

/*
 * pkv_decode_splits -- the first of pkv_decode's two launches: the persistent
 * decode kernel alone.  It takes the same arguments and has the same rules.
 * Rows with one split get their final out (and lse).  Rows with several
 * splits get partial states in the workspace, which pkv_merge then combines.
 * Source: as for pkv_decode.  The split state items are "Sequentie
 * Splitting" and "Row-Local Bounds".
 */
int pkv_decode_splits(const void* q, const void* k_pool, const void* v_pool, int64_t num_pages,
                      const int32_t* block_table, int32_t max_pages_per_row,
                      const int32_t* seq_lens, const int32_t* tasks, int64_t num_tasks,
                      const int32_t* split_offsets, int64_t num_partial_slots, int32_t B,
                      int32_t Hq, int32_t Hkv, int32_t head_dim, int32_t page_size,
                      int32_t dtype, float scale, float k_scale, float v_scale, void* out,
                      float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_merge -- the second launch: the exact log-sum-exp merge (gist.science
 * explainer, Methodologie, "Sequentie Splitting": a separate merge kernel
 * combines the split states exactly).  For every row b with S_b =
 * split_offsets[b+1] - split_offsets[b] != 1 and every query head h:
 *   M = max_s m_s,  w_s = 2^(m_s - M),
 *   out[b,h] = sum_s w_s o_s / sum_s w_s l_s   (dtype E),
 *   lse[b,h] = (M + log2 sum_s w_s l_s) * ln 2.
 * Here (m_s, l_s, o_s) are the base-2 partial states that pkv_decode_splits
 * left in the workspace.  S_b = 0 (an empty row) writes out = 0 and lse =
 * -inf.  Rows with S_b = 1 are not touched.
 * Pointers are device pointers, laid out as for pkv_decode.  One
 * workgroup merges the G = Hq/Hkv heads of one (row, KV head).
 * Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED (head_dim or G),
 * PKV_ERR_BUFFER_TOO_SMALL, PKV_ERR_HIP.
 */
int pkv_merge(const int32_t* split_offsets, int64_t num_partial_slots, int32_t B, int32_t Hq,
              int32_t Hkv, int32_t head_dim, int32_t dtype, void* out, float* lse,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Device-side planning -- one decode step whose plan is built on the device
 * from the row lengths in device memory: no host copy of the lengths, no
 * host planning, nothing the host must wait for.  (The pages plan on the
 * host and count it in the step's wall time; this entry point moves that
 * step onto the GPU.)
 *
 * Source: gist.science explainer, "Row-Local Bounds", "Compact Workqueue" and
 * "2. Calibrated Adaptive Policy".  The plan: with mode = -1, (mode, param)
 * exactly as pkv_policy would pick them with `policy` limited to the capacity
 * (split_max <= max_splits; workqueue chunks c with ceil(max_pages_per_row /
 * c) <= max_splits; a batch of several rows for which the capacity leaves no
 * workqueue candidate takes the split candidates); then the same
 * split_offsets and task records as pkv_plan, and a header.  Launches on
 * `stream`:
 *   B <= 1024: the persistent decode kernel (num_cus workgroups), every
 *      workgroup planning for itself from the lengths it stages (workgroup 0
 *      writes the plan out for pkv_device_plan_read);
 *   B > 1024: a one-workgroup planner kernel, then the decode kernel reading
 *      the task count from the header;
 *   nothing else when B * Hkv <= PKV_MAX_FUSED_GROUPS: the step is always
 *      the fused single launch, and the policy times every candidate in
 *      that form (its launch-form rule is not applied: a second launch in a
 *      captured step costs more than the separate merge saves);
 *   with more groups, the merge kernel (the two-launch form).
 * The plan therefore equals pkv_policy's with fuse_max_splits raised to
 * INT32_MAX when B * Hkv <= PKV_MAX_FUSED_GROUPS.
 * Arguments as for pkv_decode, except:
 *   seq_lens     device int32 [B]; a row with N_b < 0 or needing more than
 *                max_pages_per_row pages is planned as empty (out = 0,
 *                lse = -inf) and flagged with PKV_DEVERR_ROW
 *   mode, param  -1 (any param): the policy on the device; else an explicit
 *                schedule, which must fit the capacity
 *   max_splits   capacity: the most splits any row may get (>= 1)
 *   policy       candidate sets and model constants; NULL = the defaults
 *   num_cus      CUs of the device for the model and the grid; 0 = query
 *   workspace    >= pkv_workspace_size_device_plan(B, Hq, Hkv, head_dim,
 *                max_splits) bytes, 256-byte aligned, initialised once by
 *                pkv_workspace_init.  Layout: the pkv_decode workspace for
 *                B * max_splits partial slots, then the plan area: header
 *                (16 int32), split_offsets (B+1, padded to 16 B), records.
 *                Header words 8..11 keep the last policy decision made on
 *                the device (with B <= 1024), keyed by a hash of the rows'
 *                page counts, the shape, num_cus and `policy`: a later step
 *                with the same key takes it instead of searching the
 *                candidates.  An entry that fails its check word or is not
 *                a candidate of the step is ignored, so a stale or
 *                overwritten entry costs one search, never a wrong plan.
 * Errors: those of pkv_decode; PKV_ERR_INVALID_ARG for mode outside
 * {-1, 0, 1}, max_splits < 1, an explicit schedule that could exceed
 * max_splits for some row of up to max_pages_per_row pages, or invalid
 * policy constants.
 */
int pkv_workspace_size_device_plan(int32_t B, int32_t Hq, int32_t Hkv, int32_t head_dim,
                                   int32_t max_splits, size_t* bytes);

int pkv_decode_device_plan(const void* q, const void* k_pool, const void* v_pool,
                           int64_t num_pages, const int32_t* block_table,
                           int32_t max_pages_per_row, const int32_t* seq_lens, int32_t B,
                           int32_t Hq, int32_t Hkv, int32_t head_dim, int32_t page_size,
                           int32_t dtype, float scale, float k_scale, float v_scale,
                           int32_t mode, int32_t param, int32_t max_splits,
                           const pkv_policy_params* policy, int32_t num_cus,
                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Read back the plan the last pkv_decode_device_plan on this workspace built
 * (after synchronizing `stream`): header[8] = {tasks, fused (1) or
 * two-launch (0), mode, param, partial slots, deepest row's splits, 1 if a
 * row was flagged, 0}; split_offsets [B+1] and tasks [header[0]][4] are
 * optional (NULL skips them; task_capacity is the record capacity of
 * `tasks`).  For tests and tools.  Errors: PKV_ERR_INVALID_ARG,
 * PKV_ERR_BUFFER_TOO_SMALL (workspace or task_capacity), PKV_ERR_HIP. */
int pkv_device_plan_read(const void* workspace, size_t workspace_bytes, int32_t B, int32_t Hq,
                         int32_t Hkv, int32_t head_dim, int32_t max_splits, int32_t* header,
                         int32_t* split_offsets, int32_t* tasks, int64_t task_capacity,
                         void* stream);

/*
 * Step runner -- the whole hot path of one decode step in one call:
 * policy, host plan, then the decode kernel and the merge kernel on the
 * caller's stream.
 *
 * Source: gist.science explainer, "2. Calibrated Adaptive Policy" and
 * Methodologie ("Row-Local Bounds", "Compact Workqueue").  "Evaluatieprotocol"
 * counts host planning in the synchronized wall time of a step.
 *
 * A runner owns a ring of pinned host plan buffers, each guarded by a HIP
 * event recorded after the merge kernel, so it never rewrites a plan that
 * enqueued kernels still read, and a side stream (default priority).  It
 * allocates no device memory.  When a step's plan differs from the previous
 * distinct plan, its kernels read it in place from pinned host memory (16
 * bytes per task) and the plan is uploaded on the side stream into the tail
 * of the caller's workspace; a later step with the same plan and the same
 * workspace reads that device copy (the caller's stream waits for the
 * upload).  The workspace of a step must therefore hold the partial states
 * and the plan: workspace_bytes_needed = pkv_workspace_size(num_partial_slots,
 * Hq, head_dim) + the plan's size (4 (pad4(B + 1) + 4 num_tasks) bytes)
 * rounded up to 256; the copy sits in the last such bytes of the workspace.
 * Steps may move between streams: a step that reads the device copy on a new
 * stream first waits for the readers on the previous one, and an upload
 * waits for the readers of the old copy.  One runner serves one thread at a
 * time and the device that was current when it was created (on another
 * device it always reads the pinned plan).  A stream passed to a step must
 * stay valid until pkv_runner_destroy returns.
 */
typedef struct pkv_runner pkv_runner;

typedef struct pkv_step_args {
  /* host input */
  const int32_t* seq_lens_host;  /* int32 [B], the same lengths as seq_lens */
  int32_t B;
  int32_t mode;                  /* pkv_mode, or -1 to let pkv_policy choose */
  int32_t param;                 /* S or c for an explicit mode */
  int32_t two_launch;            /* 0: pkv_decode (one launch, merge fused);
                                    1: pkv_decode_splits then pkv_merge;
                                    -1: the policy's rule (fuse_max_splits,
                                        fuse_max_group_splits) */
  /* device inputs, laid out as for pkv_decode */
  const void* q;
  const void* k_pool;
  const void* v_pool;
  int64_t num_pages;
  const int32_t* block_table;
  int32_t max_pages_per_row;
  const int32_t* seq_lens;
  int32_t Hq;
  int32_t Hkv;
  int32_t head_dim;
  int32_t page_size;
  int32_t dtype;                 /* pkv_dtype of q, the pools and out */
  float scale;
  float k_scale;                 /* dequantisation scales of the pools (1 for */
  float v_scale;                 /* fp16 / bf16 pools), as for pkv_decode */
  /* device outputs and scratch */
  void* out;                     /* E [B, Hq, head_dim] */
  float* lse;                    /* fp32 [B, Hq] or NULL */
  void* workspace;               /* as for pkv_decode */
  size_t workspace_bytes;
  void* stream;                  /* hipStream_t */
  void* event_before_decode;     /* optional hipEvent_t pair (created by the caller)
                                    that takes the decode kernel's own start ... */
  void* event_after_decode;      /* ... and the end timestamp of the step's last kernel
                                    (hipExtLaunchKernel): the decode kernel, or the
                                    merge kernel in the two-launch form, so the pair
                                    spans the whole step on the GPU.  Either may be
                                    NULL.  A step without tasks records them where
                                    the decode kernel would have run. */
  /* outputs */
  int32_t chosen_mode;
  int32_t chosen_param;
  int32_t chosen_two_launch;     /* the launch form actually used */
  int32_t max_splits;            /* max over rows of S_b */
  int64_t num_tasks;
  int64_t num_partial_slots;
  size_t workspace_bytes_needed;
} pkv_step_args;

/* num_cus = 0 queries the current device.  params = NULL selects the
 * defaults.  ring_depth is the number of pinned staging slots (1..1024).
 * Errors: PKV_ERR_INVALID_ARG, PKV_ERR_HIP. */
int pkv_runner_create(int32_t num_cus, const pkv_policy_params* params, int32_t ring_depth,
                      pkv_runner** runner);

/* Enqueue one step.  Fills the output fields of *args.  If the workspace is
 * too small (partial states and the plan copy, see above), nothing is
 * enqueued, workspace_bytes_needed holds the size, and
 * PKV_ERR_BUFFER_TOO_SMALL is returned.  The block table
 * is not checked here: pkv_plan with a host copy of it does that.  Other
 * errors are those of pkv_policy, pkv_plan and pkv_decode, or PKV_ERR_HIP. */
int pkv_runner_step(pkv_runner* runner, pkv_step_args* args);

/* Host view of the plan that the last step's kernels read (valid until that
 * ring slot is reused): split_offsets [B+1], tasks [num_tasks][4].  For
 * tests and debugging. */
int pkv_runner_last_plan(const pkv_runner* runner, const int32_t** split_offsets,
                         const int32_t** tasks, int64_t* num_tasks, int32_t* B);

/* Wait for the kernels and uploads that use the runner's plans, then free
 * its resources.  NULL is a no-op. */
int pkv_runner_destroy(pkv_runner* runner);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
