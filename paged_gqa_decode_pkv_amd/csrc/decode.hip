// Paged GQA decode kernels for gfx950 (MI355X) and the pkv_decode entry point.
//
// Source: PersistentKV (arXiv 2606.26666).  gist.science explainer,
// "Technische Samenvatting" > Methodologie > "1. Native Block-Table Decode
// Engine", items "Layout", "Sequentie Splitting", "Row-Local Bounds" and
// "Compact Workqueue".  Lattice and fugumt.com abstracts: work is mapped by
// KV-head group so K/V tiles are reused across the grouped query heads.
//
// Kernel 1, pkv_decode_kernel (persistent workqueue):
//   A grid of (CUs x 2) workgroups of 4 waves.  A workgroup takes task
//   indices from a device-scope atomic counter.  The next index is fetched
//   while the current task runs.  A task is (row b, KV head g, split s,
//   chunk c).  The 4 waves interleave over the task's pages.  Each wave
//   keeps an online-softmax state for the G query heads.  At task end the
//   4 states are combined in LDS.  The result is written as the final fp16
//   output (rows with one split) or as an fp32 partial state.
//
// Kernel 2, pkv_merge_kernel: the exact log-sum-exp combination of a row's
//   partial states, one workgroup per (row, query head).
//
// One page tile = 16 tokens x head_dim fp16 of one KV head (4 KiB at
// d=128), contiguous in the pool.  Per page and wave:
//   S^T[16 tok x 16 head] = K[16 tok x d] . Q^T[d x 16 head]
//       d/32 MFMA 16x16x32 f16.  A = K rows straight from memory, B = q of
//       the G heads (columns >= G are zero).
//   online softmax in fp32, base 2.  scale*log2(e) is folded into the scores.
//   O^T[d x 16 head] += V^T[d x 16 tok] . P^T[16 tok x 16 head]
//       d/16 MFMA 16x16x16 f16.  The C layout of the score MFMA (lane l holds
//       rows 4*(l/16)+j, column l%16) is exactly the B layout that the
//       16x16x16 MFMA wants, so P feeds straight through in registers.  The
//       A operand gathers 4 tokens of one d column per lane.  Lane l loads
//       16 bytes of each token row 4*(l/16)+j, so each load instruction
//       covers 4 whole rows of 256 B, and the gather is a byte permute.
//
// Numerics: fp16 inputs, fp32 scores / max / sums / accumulators.  The
// probabilities p = 2^(s - m) lie in (0, 1] (unnormalised) and are rounded to
// fp16 for the PV MFMA.  The row sum uses the same rounded values, so the
// normalisation is consistent.  Final division in fp32, output rounded to
// nearest even.  Tokens past the row's length are masked with selects, never
// multiplies, so NaN in unused page slots cannot leak.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "pkv.h"

namespace pkv {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <int N>
using halfN = _Float16 __attribute__((ext_vector_type(N)));

constexpr int kPage = 16;
constexpr int kWaves = 4;             // waves per workgroup (one task at a time)
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxG = 8;
constexpr float kLn2 = 0.69314718055994530942f;

struct DecodeArgs {
  const _Float16* q;
  const _Float16* k;
  const _Float16* v;
  int64_t num_pages;
  const int32_t* block_table;
  int32_t max_pages;
  const int32_t* seq_lens;
  const int32_t* tasks;
  int32_t num_tasks;
  const int32_t* split_offsets;
  int64_t num_slots;
  int32_t B, Hq, Hkv, G;
  float scale_log2;   // softmax scale * log2(e)
  _Float16* out;
  float* lse;
  uint32_t* ctrl;     // [0] task counter, [1] exit counter, [2] error word
  float* part_o;      // [slots][Hq][D]
  float2* part_ml;    // [slots][Hq] (max in log2 units, sum)
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void flag_error(uint32_t* ctrl, uint32_t bits) {
  atomicOr(ctrl + 2, bits);
}

// Per-page registers of one wave: the K operand and the raw V rows.
template <int D>
struct PageRegs {
  static constexpr int KK = D / 32;
  static constexpr int VW = D / 16;
  half8 k[KK];
  halfN<VW> v[4];
};

// K operand of the score MFMA: token row `col`, 8 halves at d-chunk 4*kk+grp
// (d = 32*kk + 8*grp .. +8).  V: token rows 4*grp + j, VW halves starting at
// d = VW*col.  Each load instruction reads whole 64-byte (K) or row-wide (V)
// runs of the contiguous page tile.
template <int D>
__device__ __forceinline__ void load_page(PageRegs<D>& r, const _Float16* __restrict__ kt,
                                          const _Float16* __restrict__ vt, int col, int grp) {
  constexpr int KK = D / 32;
  constexpr int VW = D / 16;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    r.k[kk] = *reinterpret_cast<const half8*>(kt + col * D + 8 * (4 * kk + grp));
#pragma unroll
  for (int j = 0; j < 4; ++j)
    r.v[j] = *reinterpret_cast<const halfN<VW>*>(vt + (4 * grp + j) * D + VW * col);
}

template <int D>
__global__ void __launch_bounds__(kThreads, 2) pkv_decode_kernel(DecodeArgs a) {
  constexpr int KK = D / 32;
  constexpr int VW = D / 16;
  constexpr int LDS_STRIDE = D + 4;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;

  __shared__ int s_task[2];
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  __shared__ float s_o[kWaves][kMaxG][LDS_STRIDE];

  uint32_t next_task = 0;
  if (threadIdx.x == 0) s_task[0] = static_cast<int>(atomicAdd(a.ctrl, 1u));

  const int G = a.G;
  const int64_t tile_elems = static_cast<int64_t>(kPage) * D;

  for (int it = 0;; ++it) {
    __syncthreads();
    const int t = s_task[it & 1];
    if (t >= a.num_tasks) break;
    if (threadIdx.x == 0) next_task = atomicAdd(a.ctrl, 1u);

    // ---- task record and row-local bounds ("Row-Local Bounds")
    const int4 rec = *reinterpret_cast<const int4*>(a.tasks + 4 * static_cast<int64_t>(t));
    const int b = rec.x, g = rec.y, s = rec.z, c = rec.w;
    bool ok = (b >= 0 && b < a.B && g >= 0 && g < a.Hkv && s >= 0 && c >= 1);
    int N = 0, p0 = 0, p1 = 0, Sb = 0;
    int64_t slot = 0;
    if (ok) {
      N = a.seq_lens[b];
      const int npages = (N + kPage - 1) / kPage;
      if (N < 0 || npages > a.max_pages) {
        if (threadIdx.x == 0) flag_error(a.ctrl, PKV_DEVERR_ROW);
        ok = false;
      } else {
        const int64_t q0 = static_cast<int64_t>(s) * c;
        p0 = static_cast<int>(q0 < npages ? q0 : npages);
        const int64_t q1 = q0 + c;
        p1 = static_cast<int>(q1 < npages ? q1 : npages);
        const int o0 = a.split_offsets[b], o1 = a.split_offsets[b + 1];
        Sb = o1 - o0;
        slot = static_cast<int64_t>(o0) + s;
        if (p0 >= p1 || s >= Sb || o0 < 0 || slot >= a.num_slots) {
          if (threadIdx.x == 0) flag_error(a.ctrl, PKV_DEVERR_SLOT);
          ok = false;
        }
      }
    } else if (threadIdx.x == 0) {
      flag_error(a.ctrl, PKV_DEVERR_TASK);
    }
    if (!ok) {
      if (threadIdx.x == 0) s_task[(it + 1) & 1] = static_cast<int>(next_task);
      continue;
    }

    // ---- q operand: B of the score MFMA, column = head within the group
    half8 qf[KK];
    {
      const bool live = col < G;
      const _Float16* qp =
          a.q + (static_cast<int64_t>(b) * a.Hq + static_cast<int64_t>(g) * G + (live ? col : 0)) * D;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        half8 x = *reinterpret_cast<const half8*>(qp + 8 * (4 * kk + grp));
        qf[kk] = live ? x : half8{};
      }
    }

    // ---- per-wave online softmax over pages p0 + wave, p0 + wave + 4, ...
    float m_run = -INFINITY;
    float l_run = 0.f;
    floatx4 acc[VW];
#pragma unroll
    for (int e = 0; e < VW; ++e) acc[e] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int32_t* bt_row = a.block_table + static_cast<int64_t>(b) * a.max_pages;
    const _Float16* kbase = a.k + static_cast<int64_t>(g) * tile_elems;
    const _Float16* vbase = a.v + static_cast<int64_t>(g) * tile_elems;
    const int64_t page_stride = static_cast<int64_t>(a.Hkv) * tile_elems;

    int p = p0 + wave;
    PageRegs<D> cur;
    bool have = false;
    auto fetch = [&](int pg, PageRegs<D>& r) -> bool {
      int phys = bt_row[pg];
      phys = __builtin_amdgcn_readfirstlane(phys);
      if (phys < 0 || phys >= a.num_pages) {
        if (lane == 0) flag_error(a.ctrl, PKV_DEVERR_PAGE);
        return false;
      }
      const int64_t off = static_cast<int64_t>(phys) * page_stride;
      load_page<D>(r, kbase + off, vbase + off, col, grp);
      return true;
    };
    if (p < p1) have = fetch(p, cur);

    while (p < p1) {
      const int pn = p + kWaves;
      PageRegs<D> nxt;
      bool have_n = false;
      if (pn < p1) have_n = fetch(pn, nxt);

      if (have) {
        const int nvalid = N - p * kPage;   // >= 1; >= 16 means a full page
        // scores S^T: lane holds tokens 4*grp + j, head col
        floatx4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur.k[kk], qf[kk], sacc, 0, 0, 0);
        float sc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x = sacc[j] * a.scale_log2;
          sc[j] = (4 * grp + j < nvalid) ? x : -INFINITY;
        }
        if (nvalid < kPage) {
          // zero V rows past the end so 0 * NaN cannot reach the accumulators
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (4 * grp + j >= nvalid) cur.v[j] = halfN<VW>{};
        }
        float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        if (__any(m_new > m_run)) {
          const float alpha = fast_exp2(m_run - m_new);
          l_run *= alpha;
#pragma unroll
          for (int e = 0; e < VW; ++e) acc[e] *= alpha;
          m_run = m_new;
        }
        half4 pb;
#pragma unroll
        for (int j = 0; j < 4; ++j) pb[j] = static_cast<_Float16>(fast_exp2(sc[j] - m_run));
        l_run += (static_cast<float>(pb[0]) + static_cast<float>(pb[1])) +
                 (static_cast<float>(pb[2]) + static_cast<float>(pb[3]));
#pragma unroll
        for (int e = 0; e < VW; ++e) {
          half4 av = {cur.v[0][e], cur.v[1][e], cur.v[2][e], cur.v[3][e]};
          acc[e] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, pb, acc[e], 0, 0, 0);
        }
      }
      cur = nxt;
      have = have_n;
      p = pn;
    }

    // ---- combine the 4 waves' states in LDS
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (col < G) {
      if (grp == 0) {
        s_m[wave][col] = m_run;
        s_l[wave][col] = l_run;
      }
      // acc[e][j] is O[head col][d = VW*(4*grp + j) + e]
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < VW; ++e) s_o[wave][col][VW * (4 * grp + j) + e] = acc[e][j];
    }
    if (threadIdx.x == 0) s_task[(it + 1) & 1] = static_cast<int>(next_task);
    __syncthreads();

    const bool direct = (Sb == 1);
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
      const int h = idx / D;
      const int d = idx - h * D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
      float L = 0.f, O = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = s_m[w][h];
        const float wt = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
        L += wt * s_l[w][h];
        O += wt * s_o[w][h][d];
      }
      const int64_t hq = static_cast<int64_t>(g) * G + h;
      if (direct) {
        a.out[(static_cast<int64_t>(b) * a.Hq + hq) * D + d] = static_cast<_Float16>(O / L);
        if (d == 0 && a.lse) a.lse[static_cast<int64_t>(b) * a.Hq + hq] = (M + __log2f(L)) * kLn2;
      } else {
        a.part_o[(slot * a.Hq + hq) * D + d] = O;
        if (d == 0) a.part_ml[slot * a.Hq + hq] = make_float2(M, L);
      }
    }
  }

  // Last workgroup out resets the counters for the next launch.
  if (threadIdx.x == 0) {
    const uint32_t prev = atomicAdd(a.ctrl + 1, 1u);
    if (prev == gridDim.x - 1) {
      atomicExch(a.ctrl, 0u);
      atomicExch(a.ctrl + 1, 0u);
    }
  }
}

struct MergeArgs {
  const int32_t* split_offsets;
  int64_t num_slots;
  int32_t B, Hq;
  const float* part_o;
  const float2* part_ml;
  _Float16* out;
  float* lse;
  uint32_t* ctrl;
};

// "Sequentie Splitting": the separate merge that combines split states
// exactly.  M = max m_s, w_s = 2^(m_s - M), out = sum w_s o_s / sum w_s l_s.
template <int D>
__global__ void __launch_bounds__(64) pkv_merge_kernel(MergeArgs a) {
  constexpr int PER = D / 64;
  const int b = blockIdx.x / a.Hq;
  const int h = blockIdx.x - b * a.Hq;
  const int o0 = a.split_offsets[b];
  const int S = a.split_offsets[b + 1] - o0;
  if (S == 1) return;   // written directly by the decode kernel
  const int64_t row = static_cast<int64_t>(b) * a.Hq + h;
  if (S <= 0 || o0 < 0 || static_cast<int64_t>(o0) + S > a.num_slots) {
    if (S != 0 && threadIdx.x == 0) flag_error(a.ctrl, PKV_DEVERR_SLOT);
    // empty row: out = 0, lse = -inf
#pragma unroll
    for (int i = 0; i < PER; ++i) a.out[row * D + threadIdx.x * PER + i] = static_cast<_Float16>(0.f);
    if (threadIdx.x == 0 && a.lse) a.lse[row] = -INFINITY;
    return;
  }
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, a.part_ml[(static_cast<int64_t>(o0) + s) * a.Hq + h].x);
  float L = 0.f;
  float O[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) O[i] = 0.f;
  for (int s = 0; s < S; ++s) {
    const int64_t sl = (static_cast<int64_t>(o0) + s) * a.Hq + h;
    const float2 ml = a.part_ml[sl];
    const float w = (ml.x == -INFINITY) ? 0.f : fast_exp2(ml.x - M);
    L += w * ml.y;
    const float* po = a.part_o + sl * D + threadIdx.x * PER;
#pragma unroll
    for (int i = 0; i < PER; ++i) O[i] += w * po[i];
  }
  const float inv = 1.f / L;
#pragma unroll
  for (int i = 0; i < PER; ++i) a.out[row * D + threadIdx.x * PER + i] = static_cast<_Float16>(O[i] * inv);
  if (threadIdx.x == 0 && a.lse) a.lse[row] = (M + __log2f(L)) * kLn2;
}

// ---------------------------------------------------------------------------
// host glue

thread_local int g_last_hip_error = 0;

int num_cus_of_current_device(int* cus) {
  static int cache[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return PKV_ERR_HIP;
  }
  if (dev >= 0 && dev < 64 && cache[dev] > 0) {
    *cus = cache[dev];
    return PKV_OK;
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || n <= 0) {
    g_last_hip_error = static_cast<int>(e);
    return PKV_ERR_HIP;
  }
  if (dev >= 0 && dev < 64) cache[dev] = n;
  *cus = n;
  return PKV_OK;
}

template <int D>
int launch(const DecodeArgs& da, const MergeArgs& ma, int grid, hipStream_t stream) {
  if (da.num_tasks > 0) {
    hipLaunchKernelGGL(pkv_decode_kernel<D>, dim3(grid), dim3(kThreads), 0, stream, da);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
      g_last_hip_error = static_cast<int>(e);
      return PKV_ERR_HIP;
    }
  }
  if (ma.B > 0) {
    hipLaunchKernelGGL(pkv_merge_kernel<D>, dim3(ma.B * ma.Hq), dim3(64), 0, stream, ma);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
      g_last_hip_error = static_cast<int>(e);
      return PKV_ERR_HIP;
    }
  }
  return PKV_OK;
}

}  // namespace pkv

extern "C" {

int pkv_last_hip_error(void) { return pkv::g_last_hip_error; }

int pkv_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || workspace_bytes < 256) return PKV_ERR_INVALID_ARG;
  hipError_t e = hipMemsetAsync(workspace, 0, 256, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    pkv::g_last_hip_error = static_cast<int>(e);
    return PKV_ERR_HIP;
  }
  return PKV_OK;
}

int pkv_workspace_error_flags(const void* workspace, uint32_t* flags, void* stream) {
  if (!workspace || !flags) return PKV_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(st);
  if (e == hipSuccess)
    e = hipMemcpy(flags, static_cast<const uint32_t*>(workspace) + 2, sizeof(uint32_t),
                  hipMemcpyDeviceToHost);
  if (e != hipSuccess) {
    pkv::g_last_hip_error = static_cast<int>(e);
    return PKV_ERR_HIP;
  }
  return PKV_OK;
}

namespace {

// Validate the scalar arguments shared by the decode entry points and fill
// both kernels' argument blocks.  Touches no device state.
int prepare(const void* q, const void* k_pool, const void* v_pool, int64_t num_pages,
            const int32_t* block_table, int32_t max_pages_per_row, const int32_t* seq_lens,
            const int32_t* tasks, int64_t num_tasks, const int32_t* split_offsets,
            int64_t num_partial_slots, int32_t B, int32_t Hq, int32_t Hkv, int32_t head_dim,
            int32_t page_size, float scale, void* out, float* lse, void* workspace,
            size_t workspace_bytes, bool need_decode, pkv::DecodeArgs* da, pkv::MergeArgs* ma) {
  if (B < 0 || Hq < 1 || Hkv < 1 || num_pages < 0 || max_pages_per_row < 0 || num_tasks < 0 ||
      num_tasks > INT32_MAX || num_partial_slots < 0 || !(scale == scale))
    return PKV_ERR_INVALID_ARG;
  if (page_size != pkv::kPage || (head_dim != 64 && head_dim != 128) || Hq % Hkv != 0)
    return PKV_ERR_UNSUPPORTED;
  const int G = Hq / Hkv;
  if (need_decode && G != 1 && G != 2 && G != 4 && G != 8) return PKV_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(B) * Hq > INT32_MAX) return PKV_ERR_INVALID_ARG;
  if (B == 0) return PKV_OK;
  if (!split_offsets || !out || !workspace) return PKV_ERR_INVALID_ARG;
  if (need_decode && (!q || !k_pool || !v_pool || !block_table || !seq_lens ||
                      (num_tasks > 0 && !tasks)))
    return PKV_ERR_INVALID_ARG;
  auto misaligned = [](const void* p, uintptr_t al) {
    return (reinterpret_cast<uintptr_t>(p) & (al - 1)) != 0;
  };
  if (misaligned(q, 16) || misaligned(k_pool, 16) || misaligned(v_pool, 16) ||
      misaligned(out, 16) || misaligned(workspace, 256) || misaligned(tasks, 16))
    return PKV_ERR_INVALID_ARG;
  size_t need = 0;
  pkv_workspace_size(num_partial_slots, Hq, head_dim, &need);
  if (workspace_bytes < need) return PKV_ERR_BUFFER_TOO_SMALL;

  char* ws = static_cast<char*>(workspace);
  float* part_o = reinterpret_cast<float*>(ws + 256);
  float2* part_ml = reinterpret_cast<float2*>(
      ws + 256 + static_cast<size_t>(num_partial_slots) * Hq * head_dim * sizeof(float));
  uint32_t* ctrl = reinterpret_cast<uint32_t*>(ws);

  da->q = static_cast<const _Float16*>(q);
  da->k = static_cast<const _Float16*>(k_pool);
  da->v = static_cast<const _Float16*>(v_pool);
  da->num_pages = num_pages;
  da->block_table = block_table;
  da->max_pages = max_pages_per_row;
  da->seq_lens = seq_lens;
  da->tasks = tasks;
  da->num_tasks = static_cast<int32_t>(num_tasks);
  da->split_offsets = split_offsets;
  da->num_slots = num_partial_slots;
  da->B = B;
  da->Hq = Hq;
  da->Hkv = Hkv;
  da->G = G;
  da->scale_log2 = scale * 1.44269504088896340736f;
  da->out = static_cast<_Float16*>(out);
  da->lse = lse;
  da->ctrl = ctrl;
  da->part_o = part_o;
  da->part_ml = part_ml;

  ma->split_offsets = split_offsets;
  ma->num_slots = num_partial_slots;
  ma->B = B;
  ma->Hq = Hq;
  ma->part_o = part_o;
  ma->part_ml = part_ml;
  ma->out = static_cast<_Float16*>(out);
  ma->lse = lse;
  ma->ctrl = ctrl;
  return PKV_OK;
}

int run(const void* q, const void* k_pool, const void* v_pool, int64_t num_pages,
        const int32_t* block_table, int32_t max_pages_per_row, const int32_t* seq_lens,
        const int32_t* tasks, int64_t num_tasks, const int32_t* split_offsets,
        int64_t num_partial_slots, int32_t B, int32_t Hq, int32_t Hkv, int32_t head_dim,
        int32_t page_size, float scale, void* out, float* lse, void* workspace,
        size_t workspace_bytes, void* stream, bool do_decode, bool do_merge) {
  pkv::DecodeArgs da{};
  pkv::MergeArgs ma{};
  int st = prepare(q, k_pool, v_pool, num_pages, block_table, max_pages_per_row, seq_lens, tasks,
                   num_tasks, split_offsets, num_partial_slots, B, Hq, Hkv, head_dim, page_size,
                   scale, out, lse, workspace, workspace_bytes, do_decode, &da, &ma);
  if (st != PKV_OK || B == 0) return st;
  int grid = 1;
  if (do_decode) {
    int cus = 0;
    st = pkv::num_cus_of_current_device(&cus);
    if (st != PKV_OK) return st;
    int64_t g = static_cast<int64_t>(cus) * 2;
    if (g > num_tasks) g = num_tasks;
    grid = static_cast<int>(g < 1 ? 1 : g);
  } else {
    da.num_tasks = 0;
  }
  if (!do_merge) ma.B = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return head_dim == 128 ? pkv::launch<128>(da, ma, grid, s) : pkv::launch<64>(da, ma, grid, s);
}

}  // namespace

int pkv_decode(const void* q, const void* k_pool, const void* v_pool, int64_t num_pages,
               const int32_t* block_table, int32_t max_pages_per_row,
               const int32_t* seq_lens, const int32_t* tasks, int64_t num_tasks,
               const int32_t* split_offsets, int64_t num_partial_slots, int32_t B,
               int32_t Hq, int32_t Hkv, int32_t head_dim, int32_t page_size, float scale,
               void* out, float* lse, void* workspace, size_t workspace_bytes,
               void* stream) {
  return run(q, k_pool, v_pool, num_pages, block_table, max_pages_per_row, seq_lens, tasks,
             num_tasks, split_offsets, num_partial_slots, B, Hq, Hkv, head_dim, page_size, scale,
             out, lse, workspace, workspace_bytes, stream, true, true);
}

int pkv_decode_splits(const void* q, const void* k_pool, const void* v_pool, int64_t num_pages,
                      const int32_t* block_table, int32_t max_pages_per_row,
                      const int32_t* seq_lens, const int32_t* tasks, int64_t num_tasks,
                      const int32_t* split_offsets, int64_t num_partial_slots, int32_t B,
                      int32_t Hq, int32_t Hkv, int32_t head_dim, int32_t page_size,
                      float scale, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return run(q, k_pool, v_pool, num_pages, block_table, max_pages_per_row, seq_lens, tasks,
             num_tasks, split_offsets, num_partial_slots, B, Hq, Hkv, head_dim, page_size, scale,
             out, lse, workspace, workspace_bytes, stream, true, false);
}

int pkv_merge(const int32_t* split_offsets, int64_t num_partial_slots, int32_t B, int32_t Hq,
              int32_t head_dim, void* out, float* lse, void* workspace, size_t workspace_bytes,
              void* stream) {
  return run(nullptr, nullptr, nullptr, 0, nullptr, 0, nullptr, nullptr, 0, split_offsets,
             num_partial_slots, B, Hq, 1, head_dim, pkv::kPage, 1.0f, out, lse, workspace,
             workspace_bytes, stream, false, true);
}

}  // extern "C"
