// Paged GQA decode kernels for gfx950 (MI355X) and the pkv_decode entry point.
//
// Source: PersistentKV (arXiv 2606.26666).  gist.science explainer,
// "Technische Samenvatting" > Methodologie > "1. Native Block-Table Decode
// Engine", items "Layout", "Sequentie Splitting", "Row-Local Bounds" and
// "Compact Workqueue".  Lattice and fugumt.com abstracts: work is mapped by
// KV-head group so K/V tiles are reused across the grouped query heads.
//
// Kernel 1, pkv_decode_kernel (persistent workqueue):
//   min(T, 2 x CUs) workgroups of 4 waves (one per CU at d = 256).  A
//   workgroup's first two tasks are static (blockIdx.x, blockIdx.x +
//   gridDim.x); later indices come from a device-scope atomic counter, fetched
//   two tasks ahead.  A task is (row b, KV head g, split s, chunk c).  The 4
//   waves interleave over the task's pages, each keeping an online-softmax
//   state for the G query heads; at task end the 4 states are combined in LDS
//   and written as the final output (rows with one split) or as an fp32
//   partial state.  In the fused form the workgroup that brings a group's
//   arrival count to its split count merges the group (merge_group).  The
//   kSelfPlan instance plans the step itself from the row lengths (policy,
//   split offsets, task records), for the device-planned step.
//
// Kernel 2, pkv_merge_kernel: the exact log-sum-exp combination of a row's
//   partial states in the two-launch form, (G*D/4 R)/64 64-thread workgroups
//   per (row, KV head), folding every column as the fused merge does.
//
// Kernel 3, pkv_plan_kernel: the device-planned step's plan for batches too
//   large to stage in LDS (one workgroup).
//
// One page tile = 16 tokens x head_dim elements of one KV head (4 KiB at
// d=128 in fp16), contiguous in the pool.  Per page and wave:
//   S^T[16 tok x 16 head] = K[16 tok x d] . Q^T[d x 16 head]
//       d/32 MFMA 16x16x32 (f16 or bf16).  A = K rows straight from memory
//       (fp8 codes converted in registers), B = q of the G heads (columns
//       >= G are zero).
//   online softmax in fp32, base 2.  scale*log2(e) is folded into the scores.
//   O^T[d x 16 head] += V^T[d x 16 tok] . P^T[16 tok x 16 head]
//       d/16 MFMA 16x16x16.  The C layout of the score MFMA (lane l holds
//       rows 4*(l/16)+j, column l%16) is exactly the B layout that the
//       16x16x16 MFMA wants, so P feeds straight through in registers.  The
//       A operand gathers 4 tokens of one d column per lane: lane l loads
//       its slice of each token row 4*(l/16)+j, so each load instruction
//       covers 4 whole rows, and the gather is a byte permute.
//
// Numerics: fp16 / bf16 inputs (fp8 E4M3 pools decode exactly into q's
// type), fp32 scores / max / sums / accumulators.  The probabilities
// p = 2^(s - m) lie in (0, 2^8] (lazy maximum) and are rounded to q's type
// for the PV MFMA.  The row sum uses the same rounded values, so the
// normalisation is consistent.  Final division in fp32, output rounded to
// nearest even.  Tokens past the row's length are masked with selects, never
// multiplies, so NaN in unused page slots cannot leak.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "pkv.h"
#include "policy_model.h"
#include "internal.h"

namespace pkv {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned uint2x __attribute__((ext_vector_type(2)));
typedef short shortx4 __attribute__((ext_vector_type(4)));

// Vectors of the element type E of q, K, V and out: _Float16 or __bf16.
template <class E, int N>
using vecE = E __attribute__((ext_vector_type(N)));

// The two MFMA shapes for each element type (fp32 accumulate):
//   k32: 16x16x32, A and B are 8 elements per lane;
//   k16: 16x16x16, A and B are 4 elements per lane.
template <class E>
struct Mfma;
template <>
struct Mfma<_Float16> {
  static __device__ __forceinline__ floatx4 k32(vecE<_Float16, 8> a, vecE<_Float16, 8> b,
                                                floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ floatx4 k16(vecE<_Float16, 4> a, vecE<_Float16, 4> b,
                                                floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Mfma<__bf16> {
  static __device__ __forceinline__ floatx4 k32(vecE<__bf16, 8> a, vecE<__bf16, 8> b,
                                                floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ floatx4 k16(vecE<__bf16, 4> a, vecE<__bf16, 4> b,
                                                floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(shortx4, a),
                                                     __builtin_bit_cast(shortx4, b), c, 0, 0, 0);
  }
};

// KV pool element types.  A 2-byte pool holds E itself.  An fp8 pool holds
// OCP E4M3 codes ("e4m3fn": sign, 4 exponent bits with bias 7, 3 mantissa
// bits; no infinities; S.1111.111 is NaN), which every E represents exactly,
// so the kernel converts them to E in registers and keeps E's MFMA path.
struct Fp8E4M3 {};
template <class KV>
constexpr int kv_bytes() {
  return 2;
}
template <>
constexpr int kv_bytes<Fp8E4M3>() {
  return 1;
}

typedef unsigned uint4x __attribute__((ext_vector_type(4)));

// Two codes (bytes 2*kHi, 2*kHi+1 of w) to E, exact: the hardware converter
// with a unit scale.
template <class E, bool kHi>
__device__ __forceinline__ vecE<E, 2> fp8x2(uint32_t w);
template <>
__device__ __forceinline__ vecE<_Float16, 2> fp8x2<_Float16, false>(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
}
template <>
__device__ __forceinline__ vecE<_Float16, 2> fp8x2<_Float16, true>(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
}
template <>
__device__ __forceinline__ vecE<__bf16, 2> fp8x2<__bf16, false>(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
}
template <>
__device__ __forceinline__ vecE<__bf16, 2> fp8x2<__bf16, true>(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
}
// Four codes (the bytes of w, lowest first) to E.
template <class E>
__device__ __forceinline__ vecE<E, 4> fp8x4(uint32_t w) {
  const vecE<E, 2> lo = fp8x2<E, false>(w);
  const vecE<E, 2> hi = fp8x2<E, true>(w);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
}
template <class E>
__device__ __forceinline__ vecE<E, 8> fp8x8(uint2x w) {
  const vecE<E, 4> a = fp8x4<E>(w[0]);
  const vecE<E, 4> b = fp8x4<E>(w[1]);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

constexpr int kPage = 16;
constexpr int kWaves = 4;             // waves per workgroup (one task at a time)
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxG = 16;
constexpr float kLn2 = 0.69314718055994530942f;

struct DecodeArgs {
  const void* q;      // E [B, Hq, D]
  const void* k;      // E [pages, Hkv, 16, D]
  const void* v;
  int64_t num_pages;
  const int32_t* block_table;
  int32_t max_pages;
  const int32_t* seq_lens;
  const int32_t* tasks;
  int32_t num_tasks;  // tasks of a host plan
  int32_t task_cap;   // records readable at `tasks` (>= 1)
  const int32_t* plan_hdr;  // device plan: [0] tasks, [1] fuse; NULL for a host plan
  const int32_t* split_offsets;
  int64_t num_slots;
  int32_t B, Hq, Hkv, G;
  float scale_log2;   // softmax scale * K's dequantisation scale * log2(e)
  float v_scale;      // V's dequantisation scale
  void* out;          // E [B, Hq, D]
  float* lse;
  uint32_t* ctrl;     // [0] task counter, [1] exit counter, [2] error word
  uint32_t* arrive;   // [B*Hkv] arrival counters of the fused merge
  int32_t fuse;       // 1: the last split of a (row, KV head) merges it
  float* part_o;      // [slots][Hq][D]
  float2* part_ml;    // [slots][Hq] (max in log2 units, sum)
  // Self-planned step (pkv_decode_device_plan, B <= kRowStage): every
  // workgroup derives the plan from the staged lengths; workgroup 0 writes
  // the header and the offsets, each task's record is written by the
  // workgroup that runs it.
  int32_t plan_mode, plan_param;   // mode < 0: the policy chooses
  int32_t plan_num_cus, plan_head_dim, plan_groups_fit;
  pkv_policy_params plan_pol;      // candidate sets limited to the capacity
  int32_t* plan_out;               // header [kPlanHdrInts]; NULL: not self-planned
  int32_t* plan_offs_out;          // [B + 1]
  int4* plan_tasks_out;            // [tasks]
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void flag_error(uint32_t* ctrl, uint32_t bits) {
  atomicOr(ctrl + 2, bits);
}

// Per-page registers of one wave: the K operand and the raw V rows.
template <int D, class E, class KV>
struct PageRegs {
  static constexpr int KK = D / 32;
  static constexpr int VW = D / 16;
  vecE<E, 8> k[KK];
  vecE<E, VW> v[4];
};

// N fp8 codes in one, two or four dwords.
template <int N>
struct CodeVec;
template <>
struct CodeVec<4> {
  using T = uint32_t;
};
template <>
struct CodeVec<8> {
  using T = uint2x;
};
template <>
struct CodeVec<16> {
  using T = uint4x;
};

// An fp8 pool keeps the codes as loaded (half the registers of a 2-byte
// page); process_page converts them.
template <int D, class E>
struct PageRegs<D, E, Fp8E4M3> {
  static constexpr int KK = D / 32;
  static constexpr int VW = D / 16;
  uint2x k[KK];                    // the 8 codes of the K operand of MFMA step kk
  typename CodeVec<VW>::T v[4];    // VW codes of token row 4*grp + j
};

template <class E, int N>
__device__ __forceinline__ vecE<E, N> fp8_row(typename CodeVec<N>::T c) {
  if constexpr (N == 4) {
    return fp8x4<E>(c);
  } else if constexpr (N == 8) {
    return fp8x8<E>(c);
  } else {
    const vecE<E, 8> a = fp8x8<E>(uint2x{c[0], c[1]});
    const vecE<E, 8> b = fp8x8<E>(uint2x{c[2], c[3]});
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
  }
}

// Buffer resource for raw buffer loads (gfx9 dword3).  Loads at offsets
// >= num_records return zero without touching memory.  This gives the
// streaming loop unconditional loads: a page outside the wave's range, or one
// whose block-table entry is out of bounds, is loaded with num_records = 0.
constexpr int kRsrcDword3 = 0x00020000;

// Cache policy of the partial states: system-scope (sc0 sc1) stores write
// through the per-XCD L2s, and loads with the same bits bypass them.  Split
// states then reach other workgroups, on any XCD, without a fence that would
// write back or invalidate a whole L2.
constexpr int kCoherent = 17;   // sc0 | sc1

// Cache policy of the page loads.  A step reads every K/V tile exactly once,
// and the nt (non-temporal, streaming) bit makes the V loads faster on every
// plan measured: with it, B8 bimodal at d = 128 takes 47.5 instead of 51 us,
// B8 Zipf at c = 256 (208 tasks) 70 instead of 75 us.  On the K loads it
// pays only where a 2-byte pool's plan runs more than two tasks per CU (fp16
// B32: 408 against 428 us with V alone) and costs elsewhere (B8 uniform: 82
// against 77 us).  2-byte pools at d = 256 (one workgroup per CU, 8 KiB
// tiles) stream about 7% slower with the bit.  The modes (kLoadMode):
//   0  default policy for K and V: 2-byte pools at d = 256;
//   1  nt on the V loads: every other plan, except
//   2  nt on K and V: 2-byte pools whose plan has more tasks than twice the
//      CUs.
// The loads must be wide: fp8 K rows read in 8-byte pieces streamed far
// slower with the bit (B64: 833 -> 1066 us), hence the 16-byte K loads of
// load_page.
constexpr int kStream = 2;   // nt
constexpr int kDefault = 0;

// num_tasks < 0: not known on the host (a self-planned step).
inline int load_mode(int head_dim, int dtype, int64_t num_tasks, int num_cus) {
  const bool fp8 = dtype == PKV_DTYPE_F16_KV_FP8 || dtype == PKV_DTYPE_BF16_KV_FP8;
  if (head_dim == 256 && !fp8) return 0;
  return (!fp8 && num_tasks > 2 * static_cast<int64_t>(num_cus)) ? 2 : 1;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kRsrcDword3);
}

// d-chunk (8 elements) of the score MFMA's step kk for lane group grp.
template <class KV>
__device__ __forceinline__ constexpr int k_chunk(int kk, int grp) {
  return kv_bytes<KV>() == 1 ? 8 * (kk >> 1) + 2 * grp + (kk & 1) : 4 * kk + grp;
}

// K operand of the score MFMA: token row `col`, 8 elements at d-chunk
// k_chunk(kk, grp) (8 elements per chunk).  2-byte pools: chunk 4*kk+grp,
// byte offset koff + 64*kk with koff = 2*(col*D + 8*grp); fp8 pools: chunks
// 8*(kk/2) + 2*grp + kk%2, so one 16-byte load at koff + 64*(kk/2) with
// koff = col*D + 16*grp brings the codes of kk and kk+1.  Either way each K
// instruction reads 16 runs of 64 contiguous bytes; q takes the same chunk
// map, and the score sums over all chunks.  V: token rows 4*grp + j, VW
// elements at d = VW*col (byte offset voff + e*D*j with voff =
// e*(4*grp*D + VW*col), e bytes per element): each V instruction reads 4
// whole rows of the contiguous page tile.
template <int D, class E, class KV, int kKCpol, int kVCpol>
__device__ __forceinline__ void load_page(PageRegs<D, E, KV>& r, __amdgpu_buffer_rsrc_t kr,
                                          __amdgpu_buffer_rsrc_t vr, int koff, int voff) {
  constexpr int KK = D / 32;
  constexpr int VW = D / 16;
  if constexpr (kv_bytes<KV>() == 1) {
    // the same lanes and rows, at one byte per element
#pragma unroll
    for (int kk = 0; kk < KK; kk += 2) {
      const uint4x w = __builtin_bit_cast(
          uint4x, __builtin_amdgcn_raw_buffer_load_b128(kr, koff + 32 * kk, 0, kKCpol));
      r.k[kk] = uint2x{w[0], w[1]};
      r.k[kk + 1] = uint2x{w[2], w[3]};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (VW == 16)
        r.v[j] = __builtin_bit_cast(
            uint4x, __builtin_amdgcn_raw_buffer_load_b128(vr, voff + D * j, 0, kVCpol));
      else if constexpr (VW == 8)
        r.v[j] = __builtin_bit_cast(
            uint2x, __builtin_amdgcn_raw_buffer_load_b64(vr, voff + D * j, 0, kVCpol));
      else
        r.v[j] = __builtin_amdgcn_raw_buffer_load_b32(vr, voff + D * j, 0, kVCpol);
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      r.k[kk] = __builtin_bit_cast(
          vecE<E, 8>, __builtin_amdgcn_raw_buffer_load_b128(kr, koff + 64 * kk, 0, kKCpol));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (VW == 16) {
        const vecE<E, 8> lo = __builtin_bit_cast(
            vecE<E, 8>, __builtin_amdgcn_raw_buffer_load_b128(vr, voff + 2 * D * j, 0, kVCpol));
        const vecE<E, 8> hi = __builtin_bit_cast(
            vecE<E, 8>,
            __builtin_amdgcn_raw_buffer_load_b128(vr, voff + 2 * D * j + 16, 0, kVCpol));
        r.v[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13,
                                         14, 15);
      } else if constexpr (VW == 8) {
        r.v[j] = __builtin_bit_cast(
            vecE<E, VW>, __builtin_amdgcn_raw_buffer_load_b128(vr, voff + 2 * D * j, 0, kVCpol));
      } else {
        r.v[j] = __builtin_bit_cast(
            vecE<E, VW>, __builtin_amdgcn_raw_buffer_load_b64(vr, voff + 2 * D * j, 0, kVCpol));
      }
    }
  }
}

// Online-softmax state of one wave for the G heads of its task, and the
// per-page update.  Scores are kept in base-2 units (scale*log2(e) folded in).
//
// Lazy maximum: the reference m only moves when some score exceeds it by
// more than kLazy (base 2).  Any reference value gives the same normalised
// result, since 2^-m cancels between numerator and denominator, and keeping
// p <= 2^kLazy stays far inside fp16 and fp32 range.  In the common case a
// page costs no cross-lane traffic and no rescale of the accumulators.
constexpr float kLazy = 8.0f;

template <int D>
struct WaveState {
  static constexpr int VW = D / 16;
  float m;              // reference max (base 2), same in all 4 lane groups
  float l;              // this lane's share of sum p (tokens 4*grp+j of each page)
  floatx4 acc[VW];      // O^T block e: lane holds O[head col][VW*(4*grp+j)+e]
};

template <int D, class E, class KV>
__device__ __forceinline__ void process_page(WaveState<D>& st, PageRegs<D, E, KV>& pg,
                                             const vecE<E, 8>* __restrict__ qf_lds, int nvalid,
                                             float scale_log2, int lane) {
  constexpr int KK = D / 32;
  constexpr int VW = D / 16;
  constexpr bool kFp8 = kv_bytes<KV>() == 1;
  const int grp = lane >> 4;
  // S^T = K . Q^T: lane holds the raw scores of tokens 4*grp+j for head col.
  // The q operand is re-read from LDS for each page (saves 16 VGPRs).
  floatx4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    vecE<E, 8> kop;
    if constexpr (kFp8)
      kop = fp8x8<E>(pg.k[kk]);
    else
      kop = pg.k[kk];
    sacc = Mfma<E>::k32(kop, qf_lds[kk * 64 + lane], sacc);
  }
  float sc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) sc[j] = sacc[j] * scale_log2;
  if (nvalid < kPage) {   // last page of the row: mask the tail with selects
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool live = 4 * grp + j < nvalid;
      sc[j] = live ? sc[j] : -INFINITY;
      if (!live) pg.v[j] = {};   // E zeros, or fp8 code 0 (+0)
    }
  }
  const float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  if (__builtin_amdgcn_ballot_w64(mx > st.m + kLazy) != 0) {
    // a score escaped the window: exact max over the 16 tokens, rescale
    float mg = fmaxf(mx, __shfl_xor(mx, 16));
    mg = fmaxf(mg, __shfl_xor(mg, 32));
    const float m_new = fmaxf(st.m, mg);
    const float alpha = fast_exp2(st.m - m_new);   // 0 on the first page (m = -inf)
    st.l *= alpha;
#pragma unroll
    for (int e = 0; e < VW; ++e) st.acc[e] *= alpha;
    st.m = m_new;
  }
  vecE<E, 4> pb;
#pragma unroll
  for (int j = 0; j < 4; ++j) pb[j] = static_cast<E>(fast_exp2(sc[j] - st.m));
  st.l += (static_cast<float>(pb[0]) + static_cast<float>(pb[1])) +
          (static_cast<float>(pb[2]) + static_cast<float>(pb[3]));
  // V rows in E (converted from the codes for an fp8 pool)
  vecE<E, VW> vr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (kFp8)
      vr[j] = fp8_row<E, VW>(pg.v[j]);
    else
      vr[j] = pg.v[j];
  }
  // O^T += V^T . P^T, one 16x16x16 MFMA per 16 output columns
#pragma unroll
  for (int e = 0; e < VW; ++e) {
    const vecE<E, 4> av = {vr[0][e], vr[1][e], vr[2][e], vr[3][e]};
    st.acc[e] = Mfma<E>::k16(av, pb, st.acc[e]);
  }
}

struct MergeArgs {
  const int32_t* split_offsets;
  int64_t num_slots;
  int32_t B, Hq, Hkv, G;
  const int32_t* plan_hdr;   // device plan: [1] != 0 means the decode kernel merged
  const float* part_o;
  const float2* part_ml;
  void* out;          // E [B, Hq, D]
  float* lse;
  uint32_t* ctrl;
};

// "Sequentie Splitting": the exact combination of the split states.  For
// query head h of row b, with base-2 states (m_s, l_s, o_s):
//   M = max_s m_s,  w_s = 2^(m_s - M),
//   out = sum_s w_s o_s / sum_s w_s l_s,  lse = (M + log2 sum_s w_s l_s) ln 2.
// One workgroup merges the G heads of one (row, KV head), whose partial
// outputs are contiguous (G*D floats per slot), over slots o0 .. o0+S-1.
// A float4 column of the group (C = G*D/4 of them) folds slots r, r+R,
// r+2R, ... into a running (max, sum, vector) state kB slots at a time, so
// kB loads per thread are in flight together (fold_column).  With C <= 256,
// thread t owns column t % C and r = t / C, R = 256 / C, and the R states of
// a column are combined in LDS.  A wider group (G * D > 1024) takes
// ceil(C / 256) passes of one column per thread over all the slots (R = 1).
// The result is the same maximum and the same sums as the two-pass form, up
// to the order of the additions.
// Slots in flight per thread in the merge.  Every merge (fused or not) uses
// the same value, so both forms add the states in the same order.
constexpr int kMergeBatch = 8;

template <int D>
constexpr int merge_lds_floats() {
  return kThreads * 6;
}

template <int D, int kB>
__device__ __forceinline__ void fold_column(__amdgpu_buffer_rsrc_t ml_rsrc,
                                            __amdgpu_buffer_rsrc_t o_rsrc, int Hq, int ml_off,
                                            int o_off, int r, int R, int S, float& M, float& L,
                                            floatx4& O) {
  M = -INFINITY;
  L = 0.f;
  O = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int base = r; base < S; base += R * kB) {
    float2 ml[kB];
    floatx4 o[kB];
    // Slot indices are clamped so every load is unconditional; clamped
    // slots get weight 0 below.
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      const int sl = min(base + R * k, S - 1);
      ml[k] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(
          ml_rsrc, 8 * sl * Hq + ml_off, 0, kCoherent));
      o[k] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(
          o_rsrc, 4 * sl * Hq * D + o_off, 0, kCoherent));
    }
    __builtin_amdgcn_sched_barrier(0);   // all 2*kB loads issue before the first wait
    float Mn = M;
#pragma unroll
    for (int k = 0; k < kB; ++k)
      if (base + R * k < S) Mn = fmaxf(Mn, ml[k].x);
    const float f = (M == -INFINITY) ? 0.f : fast_exp2(M - Mn);
    O *= f;
    L *= f;
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      const bool live = base + R * k < S && ml[k].x != -INFINITY;
      const float w = live ? fast_exp2(ml[k].x - Mn) : 0.f;
      O += w * o[k];
      L += w * ml[k].y;
    }
    M = Mn;
  }
}

template <int D, int kB, class E>
__device__ void merge_group(const MergeArgs& a, int b, int g, int o0, int S, float* lds) {
  const int tid = threadIdx.x;
  const int G = a.G;
  const int cols = G * (D / 4);
  const int64_t head0 = static_cast<int64_t>(b) * a.Hq + static_cast<int64_t>(g) * G;
  // Coherent (L2-bypassing) loads: the states may come from other XCDs.
  const __amdgpu_buffer_rsrc_t ml_rsrc = make_rsrc(
      a.part_ml + static_cast<int64_t>(o0) * a.Hq, static_cast<uint32_t>(S) * a.Hq * 8u);
  const __amdgpu_buffer_rsrc_t o_rsrc = make_rsrc(
      a.part_o + static_cast<int64_t>(o0) * a.Hq * D, static_cast<uint32_t>(S) * a.Hq * D * 4u);
  auto write = [&](int c, float Mt, float Lt, floatx4 Ot) {
    const int h = (4 * c) / D;
    const float inv = 1.f / Lt;
    E* dst = static_cast<E*>(a.out) + head0 * D + 4 * c;
    dst[0] = static_cast<E>(Ot[0] * inv);
    dst[1] = static_cast<E>(Ot[1] * inv);
    dst[2] = static_cast<E>(Ot[2] * inv);
    dst[3] = static_cast<E>(Ot[3] * inv);
    if ((4 * c) % D == 0 && a.lse) a.lse[head0 + h] = (Mt + __log2f(Lt)) * kLn2;
  };

  if (cols > kThreads) {
    for (int c = tid; c < cols; c += kThreads) {
      const int h = (4 * c) / D;
      float M, L;
      floatx4 O;
      fold_column<D, kB>(ml_rsrc, o_rsrc, a.Hq, 8 * (g * G + h), 4 * (g * G * D + 4 * c), 0, 1,
                         S, M, L, O);
      write(c, M, L, O);
    }
    return;
  }

  const int R = kThreads / cols;
  const int r = tid / cols;
  const int c = tid - r * cols;
  const int h = (4 * c) / D;
  float* s_M = lds;
  float* s_L = lds + kThreads;
  floatx4* s_O = reinterpret_cast<floatx4*>(lds + 2 * kThreads);
  float M = -INFINITY, L = 0.f;
  floatx4 O = floatx4{0.f, 0.f, 0.f, 0.f};
  if (r < R)
    fold_column<D, kB>(ml_rsrc, o_rsrc, a.Hq, 8 * (g * G + h), 4 * (g * G * D + 4 * c), r, R, S,
                       M, L, O);
  s_M[tid] = M;
  s_L[tid] = L;
  s_O[tid] = O;
  __syncthreads();

  if (tid < cols) {
    float Mt = -INFINITY;
    for (int j = 0; j < R; ++j) Mt = fmaxf(Mt, s_M[tid + j * cols]);
    float Lt = 0.f;
    floatx4 Ot = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < R; ++j) {
      const float mj = s_M[tid + j * cols];
      const float w = (mj == -INFINITY) ? 0.f : fast_exp2(mj - Mt);
      Lt += w * s_L[tid + j * cols];
      Ot += w * s_O[tid + j * cols];
    }
    write(tid, Mt, Lt, Ot);
  }
}

// Output of an empty row (N_b = 0): out = 0, lse = -inf, for the G heads of
// KV head g.
template <int D, class E>
__device__ __forceinline__ void write_empty_group(const MergeArgs& a, int b, int g) {
  const int64_t head0 = static_cast<int64_t>(b) * a.Hq + static_cast<int64_t>(g) * a.G;
  for (int i = threadIdx.x; i < a.G * D; i += kThreads)
    static_cast<E*>(a.out)[head0 * D + i] = static_cast<E>(0.f);
  if (static_cast<int>(threadIdx.x) < a.G && a.lse) a.lse[head0 + threadIdx.x] = -INFINITY;
}

// Batches up to kRowStage rows get their lengths and split offsets staged in
// LDS once per workgroup.  Larger batches read them with scalar loads.
constexpr int kRowStage = 1024;
// Page tiles in flight per wave (one "round").  Plans of at most two tasks
// per CU (load modes 0 and 1): about 16 KiB of K and V per wave.  A 2-byte
// page at d = 128 holds 8 KiB, so 2; at d = 64 and for fp8 pools at d = 128
// a page holds 4 KiB, so 4 (the most the task rounds use).  At d = 256 a
// 2-byte page holds 16 KiB and a wave keeps 2, so that it still has a page in
// flight while it consumes one.  Plans of more tasks (load mode 2, two
// workgroups per CU that stream for hundreds of microseconds) keep 4 at
// d = 128.  Measured with 2-byte pools at d = 128: 16 KiB per wave instead of
// 32 made the short steps 0.3-0.9 us faster (B1, B1 bucketed, B4 and B8;
// the extra bytes in flight only lengthen every load's wait in the memory
// queues) and the long ones 0.7-2.2% slower (B64, B32); for fp8 pools twice
// the depth was 3 us slower on the short steps.
template <int D, class KV, int kLoadMode>
constexpr int ring_depth() {
  if constexpr (D == 256) return 2;
  return (D == 128 && kv_bytes<KV>() == 2 && kLoadMode != 2) ? 2 : 4;
}

// Split tasks of a workgroup whose arrival is deferred: they are counted in
// together when the workgroup runs out of tasks or holds kMaxDone of them.
constexpr int kMaxDone = 64;

// Per-workgroup timeline, in a profiling build only (compiled with
// -DPKV_TIMELINE: build.py --timeline, read back by timeline.py).  Each
// workgroup keeps the realtime counter (100 MHz) at fixed points of its run
// in registers and stores them once, at its exit, into a device array; the
// product build compiles every mark away.  Marks: 0 entry, 1 device plan
// done (self-planned step), 2 first page loads issued, 3 prologue barrier
// passed, 4 first round of the first task consumed, 5 last round of the
// latest task consumed, 6 task loop left, 7 final arrivals and merges done,
// 8 exit; slot 9 holds the XCD, slot 10 the tasks run; for the latest task,
// 11 the last of the four waves' last rounds consumed, 12 the wave states in
// LDS (barrier passed), 13 the combined state written.
#ifdef PKV_TIMELINE
constexpr int kTimelineSlots = 16;
constexpr int kTimelineWorkgroups = 4096;
__device__ unsigned long long timeline[kTimelineWorkgroups * kTimelineSlots];
#define PKV_TL_DECL unsigned long long tl_[14] = {}; unsigned tl_tasks_ = 0
#define PKV_TL_MARK(i) (tl_[i] = __builtin_amdgcn_s_memrealtime())
#define PKV_TL_TASK() (++tl_tasks_)
#define PKV_TL_STORE()                                                                     \
  do {                                                                                    \
    if (threadIdx.x == 0 && blockIdx.x < kTimelineWorkgroups) {                           \
      unsigned xcc;                                                                       \
      asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));                  \
      unsigned long long* o = timeline + static_cast<size_t>(blockIdx.x) * kTimelineSlots; \
      for (int k_ = 0; k_ < 8; ++k_) o[k_] = tl_[k_];                                     \
      o[8] = __builtin_amdgcn_s_memrealtime();                                            \
      o[9] = xcc;                                                                         \
      o[10] = tl_tasks_;                                                                  \
      for (int k_ = 11; k_ < 14; ++k_) o[k_] = tl_[k_];                                   \
    }                                                                                     \
  } while (0)
#else
#define PKV_TL_DECL
#define PKV_TL_MARK(i) ((void)0)
#define PKV_TL_TASK() ((void)0)
#define PKV_TL_STORE() ((void)0)
#endif

struct PlanArgs {
  const int32_t* seq_lens;
  int32_t B, Hkv, head_dim, page_size, num_cus;
  int32_t max_pages;
  int32_t mode, param;      // mode < 0: the policy chooses
  int32_t groups_fit;       // B * Hkv fits the fused merge's arrival counters
  pkv_policy_params pol;    // candidate sets already limited to the capacity
  int32_t* hdr;             // [kPlanHdrInts]
  int32_t* offs;            // [B + 1]
  int4* tasks;              // capacity Hkv * B * max_splits
  uint32_t* ctrl;
};

constexpr int kPlanHdrInts = 16;
constexpr int kPlanStage = 4096;   // rows whose page counts the planner keeps in LDS
constexpr int kCandBatch = kThreads / 16;   // policy candidates evaluated together

__device__ __forceinline__ uint32_t cdiv32(uint32_t a, uint32_t b) { return (a + b - 1) / b; }

// Pages of row b, or -1 for a row to flag (N_b < 0 or more than max_pages
// pages).  Read from global memory; the planner stages the first kPlanStage.
__device__ __forceinline__ int32_t plan_row_pages_global(const PlanArgs& a, int b) {
  const int32_t N = a.seq_lens[b];
  if (N < 0) return -1;
  const int64_t n = (static_cast<int64_t>(N) + a.page_size - 1) / a.page_size;
  return n > a.max_pages ? -1 : static_cast<int32_t>(n);
}

__device__ __forceinline__ int64_t wave_max64(int64_t v) {
  for (int off = 32; off >= 1; off >>= 1) {
    const int64_t o = __shfl_xor(v, off);
    v = o > v ? o : v;
  }
  return v;
}

// Exchanges inside 16-lane rows (DPP): lanes i and i^1, i and i^2, then
// lanes i and 7-i of each 8, then i and 15-i of the row.  Applied in that
// order with a commutative operation, every lane ends with the reduction of
// its row (pairs, quads, 8-lane halves, the row).
constexpr int kDppSwap1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int kDppSwap2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;   // row_half_mirror
constexpr int kDppMirror = 0x140;       // row_mirror

template <int kCtrl>
__device__ __forceinline__ int64_t dpp_xchg64(int64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(v), kCtrl, 0xF, 0xF, false);
  const int hi =
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v >> 32), kCtrl, 0xF, 0xF, false);
  return static_cast<int64_t>((static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                              static_cast<uint32_t>(lo));
}

__device__ __forceinline__ int64_t row16_sum(int64_t v) {
  v += dpp_xchg64<kDppSwap1>(v);
  v += dpp_xchg64<kDppSwap2>(v);
  v += dpp_xchg64<kDppHalfMirror>(v);
  v += dpp_xchg64<kDppMirror>(v);
  return v;
}

__device__ __forceinline__ int row16_max32(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, kDppSwap1, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, kDppSwap2, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, kDppHalfMirror, 0xF, 0xF, false));
  return max(v, __builtin_amdgcn_update_dpp(0, v, kDppMirror, 0xF, 0xF, false));
}

// Maximum over the wave (every lane active): the rows' maxima, then the
// four rows' through scalar reads.
__device__ __forceinline__ int wave_max32(int v) {
  v = row16_max32(v);
  const int a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const int c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(u), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(u >> 32), l);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// LDS of the policy's candidate search: each wave's first fastest candidate
// of a batch, double-buffered over batches.
struct PickLds {
  double t[2][kWaves];
  int i[2][kWaves];
};

// "2. Calibrated Adaptive Policy" on the device: the candidates of pkv_policy
// in its order, each timed by the same model (policy_model.h), the earliest
// fastest kept.  Candidates go 16 at a time, one per 16-lane row: lane r of
// candidate j's row folds rows r, r+16, ... into a plan shape, the row sums
// them with DPP exchanges and every lane of it evaluates the model; each
// wave keeps the first fastest of its four candidates, and after one barrier
// every thread takes the first fastest of the four waves'.  active_rows:
// rows with at least one page; row_n(b): pages of row b (0 for an empty or
// flagged row).  All threads call it and all get the choice.
// The policy decision of a self-planned step is kept in the plan header
// (words 8..11: key, mode, param, check) for the next step on the same
// workspace.  The key hashes everything the decision depends on: the batch
// size, the page count of every row (flagged rows as 0), the shape, the CU
// count and the policy's parameters.  A later step whose key matches takes
// the kept decision instead of searching; a torn or stale entry fails the
// check, the key or the candidate-set test and the step searches.  The
// decision only selects among valid plans, so a kept one can change a step's
// speed, never its result.
__host__ __device__ inline uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

constexpr int kPlanCacheWord = 8;   // plan header words 8..11

__device__ __forceinline__ uint32_t plan_cache_check(uint32_t key, uint32_t mode,
                                                     uint32_t param) {
  return mix32(key ^ mix32(mode * 0x9e3779b1u + 0x632be5abu) ^ mix32(param + 0x85ebca77u));
}

// Key of the policy's inputs other than the rows: shape, CU count, policy
// parameters (their bit patterns).  Computed on the host at launch and passed
// in a preloaded kernel argument: on the device its 64 bytes of parameters
// were an argument-segment load on the prologue's critical path (the
// device-planned step measured 0.3-0.4 us faster without it).
__host__ inline uint32_t plan_cache_config_key(const pkv_policy_params& p, int B,
                                                          int Hkv, int num_cus, int head_dim,
                                                          int max_pages) {
  uint32_t h = mix32(static_cast<uint32_t>(B) + 0x27d4eb2du);
  h = mix32(h ^ static_cast<uint32_t>(Hkv));
  h = mix32(h ^ static_cast<uint32_t>(num_cus));
  h = mix32(h ^ static_cast<uint32_t>(head_dim));
  h = mix32(h ^ static_cast<uint32_t>(max_pages));
  h = mix32(h ^ static_cast<uint32_t>(p.split_max));
  h = mix32(h ^ static_cast<uint32_t>(p.chunk_min));
  h = mix32(h ^ static_cast<uint32_t>(p.chunk_max));
  h = mix32(h ^ static_cast<uint32_t>(p.fuse_max_splits));
  h = mix32(h ^ static_cast<uint32_t>(p.fuse_max_group_splits));
  const double d[8] = {p.t0_us, p.t_round_us, p.alpha, p.cu_gbps,
                       p.hbm_gbps, p.t_two_us, p.t_two_split_us, p.t_fused_split_us};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint64_t u = __builtin_bit_cast(uint64_t, d[i]);
    h = mix32(h ^ static_cast<uint32_t>(u));
    h = mix32(h ^ static_cast<uint32_t>(u >> 32));
  }
  return h;
}

// Whether (mode, param) is one of the candidates the policy would search for
// a batch with `active_rows` rows with pages (the explainer's mode rule).
__device__ __forceinline__ bool plan_cache_candidate(const pkv_policy_params& p,
                                                     int active_rows, uint32_t mode,
                                                     uint32_t param) {
  int nchunk = 0;
  for (int64_t c = p.chunk_min; c <= p.chunk_max; c *= 2) ++nchunk;
  const bool use_split = active_rows <= 1 || nchunk == 0;
  if (active_rows == 0) return mode == PKV_MODE_SPLIT && param == 1;
  if (use_split) {
    return mode == PKV_MODE_SPLIT && param >= 1 && (param & (param - 1)) == 0 &&
           static_cast<int64_t>(param) <= p.split_max;
  }
  if (mode != PKV_MODE_WORKQUEUE || p.chunk_min < 1) return false;
  for (int64_t c = p.chunk_min; c <= p.chunk_max; c *= 2)
    if (c == static_cast<int64_t>(param)) return true;
  return false;
}

template <class RowN>
__device__ void choose_plan(const pkv_policy_params& p, int B, int Hkv, int num_cus,
                            int head_dim, int page_size, RowN row_n, int64_t active_rows,
                            PickLds& L, int& mode, int& param) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int nsplit = 0;
  for (int64_t S = 1; S <= p.split_max; S *= 2) ++nsplit;
  int nchunk = 0;
  for (int64_t c = p.chunk_min; c <= p.chunk_max; c *= 2) ++nchunk;
  const int ncand = nsplit + nchunk;
  // The mode follows the explainer's rule, as pkv_policy: one active row is
  // split along the sequence (candidates [0, nsplit)), several rows go
  // through the workqueue (candidates [nsplit, ncand)); if the capacity left
  // no workqueue candidate, the split candidates serve.
  const bool use_split = active_rows <= 1 || nchunk == 0;
  const int c_lo = use_split ? 0 : nsplit;
  const int c_hi = use_split ? nsplit : ncand;
  const int j = tid >> 4;    // candidate of this thread's row within the batch
  const int r = tid & 15;    // rows r, r + 16, ...
  // page tiles and groups do not depend on the candidate
  int64_t pages = 0;
  for (int b = r; b < B; b += 16) pages += row_n(b);
  const int64_t P = static_cast<int64_t>(Hkv) * row16_sum(pages);
  const int64_t groups = static_cast<int64_t>(Hkv) * active_rows;
  double best_t = 0.0;
  int best_i = -1;
  for (int cb = c_lo, par = 0; cb < c_hi; cb += kCandBatch, par ^= 1) {
    const int i = cb + j;
    int64_t splits = 0;   // sum of the rows' splits
    int pmax = 0, maxS = 0;
    if (i < c_hi) {
      const bool split = i < nsplit;
      const uint32_t v = split ? (1u << i) : static_cast<uint32_t>(p.chunk_min) << (i - nsplit);
      for (int b = r; b < B; b += 16) {
        const uint32_t n = static_cast<uint32_t>(row_n(b));
        if (n == 0) continue;
        const uint32_t c = split ? cdiv32(n, v) : v;
        const uint32_t S = cdiv32(n, c);
        splits += S;
        pmax = max(pmax, static_cast<int>(c < n ? c : n));
        maxS = max(maxS, static_cast<int>(S));
      }
    }
    PlanShape F;
    F.T = static_cast<int64_t>(Hkv) * row16_sum(splits);
    F.P = P;
    F.groups = groups;
    F.pmax = row16_max32(pmax);
    F.maxS = row16_max32(maxS);
    const double t = i < c_hi ? model_us(p, F, num_cus, head_dim, page_size,
                                         two_launch_form(p, F.maxS, F.groups))
                              : 0.0;
    // this wave's candidates cb + 4 wave + k sit in lanes 16 k
    double wt = 0.0;
    int wi = -1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int ik = cb + 4 * wave + k;
      const double tk = readlane_f64(t, 16 * k);
      if (ik < c_hi && (wi < 0 || tk < wt)) {
        wt = tk;
        wi = ik;
      }
    }
    if (lane == 0) {
      L.t[par][wave] = wt;
      L.i[par][wave] = wi;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int iw = L.i[par][w];
      const double tw = L.t[par][w];
      if (iw >= 0 && (best_i < 0 || tw < best_t)) {
        best_t = tw;
        best_i = iw;
      }
    }
  }
  if (active_rows == 0 || best_i < 0) {
    mode = PKV_MODE_SPLIT;
    param = 1;
  } else if (best_i < nsplit) {
    mode = PKV_MODE_SPLIT;
    param = 1 << best_i;
  } else {
    mode = PKV_MODE_WORKQUEUE;
    param = p.chunk_min << (best_i - nsplit);
  }
}

// Everything the workgroup needs to know about one task.  All fields are
// wave-uniform and live in SGPRs.
struct Meta {
  int t;          // task index (>= num_tasks: no task)
  int b, g;
  int N;          // row length in tokens
  int p0, p1;     // page range [p0, p1) of the row
  int Sb;         // splits of the row
  int o0;         // first partial-state slot of the row
  int64_t slot;   // partial-state slot
  int rounds;     // >= 1 rounds of R positions per wave
  bool ok;        // a real task whose checks passed
};

// Task record and row-local bounds ("Row-Local Bounds").  A failed check is
// flagged in the error word and leaves ok = false (all pages disabled).
// The read-only inputs arrive as restrict pointers, so uniform loads from
// them are scalar (SMEM) loads, whose waits never cover vector page loads.
// The record of task t (a scalar load).  The index is clamped to the
// readable records, so the load does not wait for the task count; records
// past the count are never used.
__device__ __forceinline__ int4 load_record(const int4* __restrict__ tasks, int task_cap, int t) {
  return tasks[t < task_cap ? t : task_cap - 1];
}

// v clamped into [0, n) (n >= 1), wave-uniform.
__device__ __forceinline__ int clamp_index(int v, int n) {
  v = __builtin_amdgcn_readfirstlane(v);
  return v < 0 ? 0 : (v >= n ? n - 1 : v);
}

// Task metadata from its record and its row's length and split offsets
// (N = seq_lens[b], o0 = offs[b], o1 = offs[b + 1], read by the caller for
// the record's row clamped into range, so that the reads may leave before
// the record is checked).
template <int R>
__device__ __forceinline__ Meta meta_from_row(const DecodeArgs& a, int num_tasks, int t, int4 rec,
                                              int N, int o0, int o1) {
  Meta m;
  m.t = t;
  m.b = m.g = m.N = m.p0 = m.p1 = m.Sb = m.o0 = 0;
  m.slot = 0;
  m.rounds = 1;
  m.ok = false;
  if (t >= num_tasks) return m;
  const int b = __builtin_amdgcn_readfirstlane(rec.x);
  const int g = __builtin_amdgcn_readfirstlane(rec.y);
  const int s = __builtin_amdgcn_readfirstlane(rec.z);
  const int c = __builtin_amdgcn_readfirstlane(rec.w);
  if (!(b >= 0 && b < a.B && g >= 0 && g < a.Hkv && s >= 0 && c >= 1)) {
    if (threadIdx.x == 0) flag_error(a.ctrl, PKV_DEVERR_TASK);
    return m;
  }
  N = __builtin_amdgcn_readfirstlane(N);
  o0 = __builtin_amdgcn_readfirstlane(o0);
  o1 = __builtin_amdgcn_readfirstlane(o1);
  const int npages = (N + kPage - 1) / kPage;
  if (N < 0 || npages > a.max_pages) {
    if (threadIdx.x == 0) flag_error(a.ctrl, PKV_DEVERR_ROW);
    return m;
  }
  const int64_t q0 = static_cast<int64_t>(s) * c;
  const int64_t q1 = q0 + c;
  const int p0 = static_cast<int>(q0 < npages ? q0 : npages);
  const int p1 = static_cast<int>(q1 < npages ? q1 : npages);
  const int64_t slot = static_cast<int64_t>(o0) + s;
  if (p0 >= p1 || s >= o1 - o0 || o0 < 0 || slot >= a.num_slots) {
    if (threadIdx.x == 0) flag_error(a.ctrl, PKV_DEVERR_SLOT);
    return m;
  }
  m.b = b;
  m.g = g;
  m.N = N;
  m.p0 = p0;
  m.p1 = p1;
  m.Sb = o1 - o0;
  m.o0 = o0;
  m.slot = slot;
  const int per_wave = (p1 - p0 + kWaves - 1) / kWaves;
  m.rounds = (per_wave + R - 1) / R;
  m.ok = true;
  return m;
}

template <bool kStaged, int R>
__device__ __forceinline__ Meta decode_meta(const DecodeArgs& a,
                                            const int32_t* __restrict__ seq_lens,
                                            const int32_t* __restrict__ offs, const int* s_len,
                                            const int* s_off, int num_tasks, int t, int4 rec) {
  // Staging is a compile-time choice.  A runtime select between an LDS and
  // a global pointer would become a flat load, whose wait also drains every
  // page load in flight.
  const int b = clamp_index(rec.x, a.B);
  int N, o0, o1;
  if constexpr (kStaged) {
    N = s_len[b];
    o0 = s_off[b];
    o1 = s_off[b + 1];
  } else {
    N = seq_lens[b];
    o0 = offs[b];
    o1 = offs[b + 1];
  }
  return meta_from_row<R>(a, num_tasks, t, rec, N, o0, o1);
}

template <bool kStaged, int R>
__device__ __forceinline__ Meta load_meta(const DecodeArgs& a, const int4* __restrict__ tasks,
                                          int task_cap, const int32_t* __restrict__ seq_lens,
                                          const int32_t* __restrict__ offs, const int* s_len,
                                          const int* s_off, int num_tasks, int t) {
  return decode_meta<kStaged, R>(a, seq_lens, offs, s_len, s_off, num_tasks, t,
                              load_record(tasks, task_cap, t));
}

// Count in n deferred split tasks (row, KV head, first slot, splits) of this
// workgroup: one wait for all of its write-through partial stores, one
// arrival per task (in parallel), then the workgroup merges, one after
// another, the groups whose last split it holds.  All threads call it.
template <int D, int kB, class E>
__device__ __forceinline__ void flush_done(const DecodeArgs& a, const MergeArgs& ma, int n,
                                        const int4* s_done, int* s_lastf, float* scratch) {
  const int tid = threadIdx.x;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid < n) {
    const int4 d = s_done[tid];
    uint32_t* cnt = a.arrive + static_cast<int64_t>(d.x) * a.Hkv + d.y;
    s_lastf[tid] = (atomicAdd(cnt, 1u) + 1u == static_cast<uint32_t>(d.w)) ? 1 : 0;
  }
  __syncthreads();
  for (int i = 0; i < n; ++i) {
    if (s_lastf[i]) {
      const int4 d = s_done[i];
      merge_group<D, kB, E>(ma, d.x, d.y, d.z, d.w, scratch);
      if (tid == 0) atomicExch(a.arrive + static_cast<int64_t>(d.x) * a.Hkv + d.y, 0u);
      __syncthreads();   // the scratch is reused by the next merge
    }
  }
}

// Block-table entries of round j of task m for this wave: position 4j+r is
// page p0 + wave + 16j + 4r.  Positions past the range read a clamped,
// in-row entry that issue() never uses (it re-checks page < p1); an invalid
// task reads its row's first entry, and a table without columns is not read.
// No select on the loaded values, so the four scalar loads issue back to
// back.
template <int R>
struct Round {
  int e[R];
};

template <int R>
__device__ __forceinline__ Round<R> load_round(const DecodeArgs& a, const int32_t* __restrict__ bt,
                                               const Meta& m, int wave, int j) {
  Round<R> r;
  if (a.max_pages <= 0) {   // a table without columns: no row has a page
#pragma unroll
    for (int i = 0; i < R; ++i) r.e[i] = 0;
    return r;
  }
  const int32_t* row = bt + static_cast<int64_t>(m.b) * a.max_pages;
  const int last = m.ok ? m.p1 - 1 : 0;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int page = m.p0 + wave + kWaves * (R * j + i);
    r.e[i] = row[page < last ? page : last];
  }
  return r;
}

// The first round's block-table entries of the task in record `rec`, for
// this wave, from the record alone (the row's length is not yet known):
// positions p0 + wave + 4i of the chunk [p0, p0 + c), p0 = split * c,
// clamped to the chunk's last position and to the row's last table entry,
// with the row clamped into [0, B).  Every page that issue() loads lies
// below p1 = min(p0 + c, n_b) with n_b <= max_pages, where the clamps change
// nothing: the entries it uses are those of load_round.  A table without
// columns (max_pages = 0: no row has a page) is not read.
template <int R>
__device__ __forceinline__ Round<R> first_round(const DecodeArgs& a,
                                                const int32_t* __restrict__ bt,
                                                const int32_t* __restrict__ spare, int4 rec,
                                                int wave) {
  Round<R> r;
  const int b = clamp_index(rec.x, a.B);
  const int s = __builtin_amdgcn_readfirstlane(rec.z);
  const int c = __builtin_amdgcn_readfirstlane(rec.w);
  const int64_t cc = c < 1 ? 1 : c;
  const int64_t p0 = static_cast<int64_t>(s < 0 ? 0 : s) * cc;
  const int64_t end = p0 + cc < a.max_pages ? p0 + cc : a.max_pages;
  const int64_t last = end - 1 > 0 ? end - 1 : 0;
  // No branch around the loads (a table without columns reads entry 0 of
  // `spare`, a readable array, and the values are dropped), so they issue in
  // the same block as the caller's loads and share one wait.
  const bool cols = a.max_pages > 0;
  const int32_t* row = cols ? bt + static_cast<int64_t>(b) * a.max_pages : spare;
  int e[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int64_t pos = p0 + wave + kWaves * i;
    e[i] = row[cols ? (pos < last ? pos : last) : 0];
  }
#pragma unroll
  for (int i = 0; i < R; ++i) r.e[i] = cols ? e[i] : 0;
  return r;
}

// Two workgroups per CU at d <= 128 (256 VGPRs each); one at d = 256, whose
// larger tiles and accumulators need the AGPR half of the register file.
// The first two arguments are preloaded into SGPRs: the task list and the
// records it holds for a host plan; for a self-planned step (which builds
// its records in the kernel) the second one is the key of the step's shape
// and policy, the rows' part of which the kernel adds.
template <int D, bool kStaged, class E, class KV, bool kSelfPlan, int kLoadMode>
__global__ void __launch_bounds__(kThreads, D == 256 ? 1 : 2)
pkv_decode_kernel(const int4* __restrict__ tasks_in, int32_t task_cap, DecodeArgs a,
                  const int32_t* __restrict__ bt_in, const int32_t* __restrict__ seq_lens_in,
                  const int32_t* __restrict__ offs_in) {
  constexpr int KK = D / 32;
  constexpr int VW = D / 16;
  constexpr int LDS_STRIDE = D + 4;
  constexpr int kKvb = kv_bytes<KV>();
  constexpr uint32_t kTileBytes = static_cast<uint32_t>(kPage * D * kKvb);
  constexpr int kRing = ring_depth<D, KV, kLoadMode>();
  constexpr int kGroup = kMaxG;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int col = lane & 15;
  const int grp = lane >> 4;
  PKV_TL_DECL;
  PKV_TL_MARK(0);
  // Host plan: the first task's record is the kernel's first load.  Its
  // address needs only the first two kernel arguments, which the kernel
  // finds in SGPRs at entry (kernarg preload): no round trip to the
  // argument segment lies before it.
  uint4x rec0v{};
  if constexpr (!kSelfPlan) {
    const int t0 = static_cast<int>(blockIdx.x) < task_cap ? static_cast<int>(blockIdx.x)
                                                           : task_cap - 1;
    // a vector load marked volatile (aux bit 31): the compiler keeps it here
    // instead of sinking it behind the argument loads to its first use
    const uint32_t recs = static_cast<uint32_t>(t0) + 1u;   // records t0 may lie in
    rec0v = __builtin_bit_cast(uint4x, __builtin_amdgcn_raw_buffer_load_b128(
        make_rsrc(tasks_in, recs * 16u), 16 * t0, 0, static_cast<int>(1u << 31)));
    __builtin_amdgcn_sched_barrier(0);
  }

  __shared__ int s_len[kStaged ? kRowStage : 1];
  __shared__ int s_off[kStaged ? kRowStage + 1 : 1];
  __shared__ int s_next[2];
#ifdef PKV_TIMELINE
  __shared__ unsigned long long s_tlw[kWaves];   // each wave's last round of its latest task
#endif
  __shared__ vecE<E, 8> s_q[2][KK * 64];            // q operand of a task, per lane
  __shared__ float s_m[2][kWaves][16];
  __shared__ float s_l[2][kWaves][16];
  // The waves' accumulators, single-buffered (room for G = 16 heads): a
  // barrier after the combine keeps the next task's writes behind its reads.
  __shared__ __attribute__((aligned(16))) float s_o[kWaves][kGroup][LDS_STRIDE];
  __shared__ int4 s_done[kMaxDone];   // (row, KV head, first slot, splits)
  __shared__ int s_lastf[kMaxDone];
  // self-planned step only: the policy's candidate search and the row scan
  __shared__ typename std::conditional<kSelfPlan, PickLds, char>::type s_pick;
  __shared__ int s_plan[kSelfPlan ? 5 * kWaves : 1];
  static_assert(kWaves * kGroup * LDS_STRIDE >= merge_lds_floats<D>(), "merge scratch");
  static_assert(!kSelfPlan || kStaged, "a self-planned step stages its rows");

  const MergeArgs ma{a.split_offsets, a.num_slots, a.B, a.Hq, a.Hkv, a.G, nullptr,
                     a.part_o, a.part_ml, a.out, a.lse, a.ctrl};
  // Task count and merge form: kernel arguments, or the header the
  // device-side planner wrote before this launch.
  int num_tasks = a.num_tasks;
  int fuse = a.fuse;
  if (a.plan_hdr) {
    num_tasks = __builtin_amdgcn_readfirstlane(a.plan_hdr[0]);
    fuse = __builtin_amdgcn_readfirstlane(a.plan_hdr[1]);
  }
  // Self-planned step: "Row-Local Bounds" / "Compact Workqueue" from the
  // staged lengths, as the planner kernel builds them (same policy, same
  // offsets, same records in the same order).
  int plan_mode = 0, plan_param = 1;
  if constexpr (kSelfPlan) {
    constexpr int kPer = (kRowStage + kThreads) / kThreads;
    constexpr int kRows = kRowStage / kThreads;   // rows per thread in the scan
    int lv[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = tid + k * kThreads;
      lv[k] = i < a.B ? seq_lens_in[i] : 0;
    }
    // the decision kept by the previous step on this workspace (coherent
    // load: it may have been written on another XCD)
    const uint4x kept = __builtin_bit_cast(uint4x, __builtin_amdgcn_raw_buffer_load_b128(
        make_rsrc(a.plan_out + kPlanCacheWord, 16u), 0, 0, kCoherent));
    // A row with N < 0 or more than max_pages pages is flagged and planned
    // empty (its length staged as 0).  Rows with pages and flagged rows are
    // counted per wave (ballots) into LDS slots of their own: nothing to
    // clear, one barrier.
    int wact = 0, wbad = 0;
    uint32_t rkey = 0;   // XOR of the rows' (index, page count) hashes
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = tid + k * kThreads;
      const int N = lv[k];
      const bool ok = N >= 0 && (static_cast<int64_t>(N) + kPage - 1) / kPage <= a.max_pages;
      if (i < a.B) {
        s_len[i] = ok ? N : 0;
        const uint32_t n = ok ? static_cast<uint32_t>((N + kPage - 1) / kPage) : 0u;
        rkey ^= mix32(mix32(static_cast<uint32_t>(i) + 0x165667b1u) ^ n);
      }
      wact += __builtin_popcountll(__ballot(i < a.B && ok && N > 0));
      wbad |= __ballot(i < a.B && !ok) != 0 ? 1 : 0;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) rkey ^= __shfl_xor(rkey, off);
    if (lane == 0) {
      s_plan[wave] = wact;
      s_plan[kWaves + wave] = wbad;
      s_plan[4 * kWaves + wave] = static_cast<int>(rkey);
    }
    __syncthreads();
    int active_rows = 0, any_bad = 0;
    // a self-planned step gets its shape and policy key in `task_cap`
    uint32_t key = static_cast<uint32_t>(task_cap);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      active_rows += s_plan[w];
      any_bad |= s_plan[kWaves + w];
      key ^= static_cast<uint32_t>(s_plan[4 * kWaves + w]);
    }
    key = mix32(key);
    auto row_n = [&](int b) -> int32_t { return (s_len[b] + kPage - 1) / kPage; };
    plan_mode = a.plan_mode;
    plan_param = a.plan_param;
    if (plan_mode < 0) {
      const uint32_t kkey = __builtin_amdgcn_readfirstlane(kept[0]);
      const uint32_t kmode = __builtin_amdgcn_readfirstlane(kept[1]);
      const uint32_t kparam = __builtin_amdgcn_readfirstlane(kept[2]);
      const uint32_t kcheck = __builtin_amdgcn_readfirstlane(kept[3]);
      if (kkey == key && kcheck == plan_cache_check(kkey, kmode, kparam) &&
          plan_cache_candidate(a.plan_pol, active_rows, kmode, kparam)) {
        plan_mode = static_cast<int>(kmode);
        plan_param = static_cast<int>(kparam);
      } else {
        choose_plan(a.plan_pol, a.B, a.Hkv, a.plan_num_cus, a.plan_head_dim, kPage, row_n,
                    active_rows, s_pick, plan_mode, plan_param);
        if (blockIdx.x == 0 && tid == 0) {
          const uint32_t m = static_cast<uint32_t>(plan_mode);
          const uint32_t pr = static_cast<uint32_t>(plan_param);
          __builtin_amdgcn_raw_buffer_store_b128(
              uint4x{key, m, pr, plan_cache_check(key, m, pr)},
              make_rsrc(a.plan_out + kPlanCacheWord, 16u), 0, 0, kCoherent);
        }
      }
    }
    // splits per row, then their exclusive prefix: thread t takes rows
    // kRows*t .. kRows*t + kRows-1
    int sv[kRows];
    int sum = 0, mx = 0;
#pragma unroll
    for (int k = 0; k < kRows; ++k) {
      const int b = kRows * tid + k;
      int S = 0;
      if (b < a.B) {
        const uint32_t n = static_cast<uint32_t>(row_n(b));
        if (n > 0) {
          const uint32_t c = plan_mode == PKV_MODE_SPLIT ? cdiv32(n, plan_param)
                                                         : static_cast<uint32_t>(plan_param);
          S = static_cast<int>(cdiv32(n, c));
        }
      }
      sv[k] = S;
      sum += S;
      mx = S > mx ? S : mx;
    }
    int incl = sum;   // inclusive scan over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    const int wmax = wave_max32(mx);
    if (lane == 63) s_plan[2 * kWaves + wave] = incl;
    if (lane == 0) s_plan[3 * kWaves + wave] = wmax;
    __syncthreads();
    int base = incl - sum;
    int total = 0, maxS = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (w < wave) base += s_plan[2 * kWaves + w];
      total += s_plan[2 * kWaves + w];
      maxS = s_plan[3 * kWaves + w] > maxS ? s_plan[3 * kWaves + w] : maxS;
    }
#pragma unroll
    for (int k = 0; k < kRows; ++k) {
      const int b = kRows * tid + k;
      if (b < a.B) s_off[b] = base;
      base += sv[k];
    }
    if (tid == 0) s_off[a.B] = total;
    num_tasks = a.Hkv * total;
    fuse = (num_tasks == 0 ||
            (!two_launch_form(a.plan_pol, maxS, static_cast<int64_t>(a.Hkv) * active_rows) &&
             a.plan_groups_fit))
               ? 1
               : 0;
    __syncthreads();
    if (blockIdx.x == 0) {
      for (int b = tid; b <= a.B; b += kThreads) a.plan_offs_out[b] = s_off[b];
      if (tid == 0) {
        a.plan_out[0] = num_tasks;
        a.plan_out[1] = fuse;
        a.plan_out[2] = plan_mode;
        a.plan_out[3] = plan_param;
        a.plan_out[4] = total;
        a.plan_out[5] = maxS;
        a.plan_out[6] = any_bad ? 1 : 0;
        if (any_bad) flag_error(a.ctrl, PKV_DEVERR_ROW);
      }
    }
  }
  if constexpr (kSelfPlan) PKV_TL_MARK(1);
  // Record of task t of a self-planned step, from the offsets in LDS: the
  // row is the last one whose first task is <= t (rows without tasks share
  // the next row's offset and come before it).  With `publish`, thread 0
  // writes it out for read-back (the workgroup that takes the task does).
  auto self_record = [&](int t, bool publish) -> int4 {
    if (t >= num_tasks) return int4{0, 0, 0, 1};
    int lo = 0, hi = a.B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.Hkv * s_off[mid] <= t) lo = mid;
      else hi = mid;
    }
    const int b = lo;
    const int S = s_off[b + 1] - s_off[b];
    const int r = t - a.Hkv * s_off[b];
    const int g = r / S;
    const uint32_t n = static_cast<uint32_t>((s_len[b] + kPage - 1) / kPage);
    const int c = plan_mode == PKV_MODE_SPLIT ? static_cast<int>(cdiv32(n, plan_param))
                                              : plan_param;
    const int4 rec = int4{b, g, r - g * S, c};
    if (publish && tid == 0) a.plan_tasks_out[t] = rec;
    return rec;
  };
  const int G = a.G;
  const int64_t tile_elems = static_cast<int64_t>(kPage) * D;
  const int64_t stride_bytes = static_cast<int64_t>(a.Hkv) * tile_elems * kKvb;
  const int koff = kKvb == 1 ? col * D + 16 * grp : kKvb * (col * D + 8 * grp);
  const int voff = kKvb * (4 * grp * D + VW * col);
  const char* kpool = reinterpret_cast<const char*>(a.k);
  const char* vpool = reinterpret_cast<const char*>(a.v);

  // Load the page at position `pos` of task m (entry e) into `r`.  A
  // position past the range, an invalid task or an out-of-pool entry loads
  // nothing (num_records = 0) and returns false.
  auto issue = [&](const Meta& m, int pos, int e, PageRegs<D, E, KV>& r) -> bool {
    const int page = m.p0 + wave + kWaves * pos;
    const bool want = m.ok && page < m.p1;
    const bool inr = e >= 0 && static_cast<int64_t>(e) < a.num_pages;
    if (want && !inr && lane == 0) flag_error(a.ctrl, PKV_DEVERR_PAGE);
    const bool live = want && inr;
    const int64_t off = static_cast<int64_t>(m.g) * tile_elems * kKvb +
                        (live ? static_cast<int64_t>(e) * stride_bytes : 0);
    const uint32_t bytes = live ? kTileBytes : 0u;
    load_page<D, E, KV, kLoadMode == 2 ? kStream : kDefault, kLoadMode >= 1 ? kStream : kDefault>(
        r, make_rsrc(kpool + off, bytes), make_rsrc(vpool + off, bytes), koff, voff);
    return live;
  };
  // q of row b, KV head g (B operand of the score MFMA, column = head
  // within the group); ok = false loads column 0 only.  Raw loads; columns
  // >= G, and every column of a task that turns out invalid, are zeroed
  // when stored to LDS, so the loads can stay in flight until then.
  auto load_q = [&](int b, int g, bool ok, vecE<E, 8> (&qf)[KK]) {
    const bool live = ok && col < G;
    const E* qp = static_cast<const E*>(a.q) + (static_cast<int64_t>(b) * a.Hq +
                                static_cast<int64_t>(g) * G + (live ? col : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = *reinterpret_cast<const vecE<E, 8>*>(qp + 8 * k_chunk<KV>(kk, grp));
  };
  auto store_q = [&](const Meta& m, const vecE<E, 8> (&qf)[KK], vecE<E, 8>* dst) {
    const bool live = m.ok && col < G;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) dst[kk * 64 + lane] = live ? qf[kk] : vecE<E, 8>{};
  };

  // ---- prologue: task 0 = blockIdx.x, task 1 = blockIdx.x + gridDim.x
  Meta cur;
  PageRegs<D, E, KV> ring[kRing];
  bool valid[kRing];
  vecE<E, 8> qf[KK];   // wave 0: q of the first task
  if constexpr (kSelfPlan) {
    // the record and the row bounds come from the plan in LDS
    cur = decode_meta<kStaged, kRing>(a, seq_lens_in, offs_in, s_len, s_off, num_tasks,
                                      blockIdx.x, self_record(blockIdx.x, false));
    // q is loaded before the pages: vector loads complete in order, so its
    // wait (and the barrier behind it) does not also wait for the first
    // round of pages, and every wave starts consuming (and refilling) its
    // ring as soon as its first page lands.
    if (wave == 0) load_q(cur.b, cur.g, cur.ok, qf);
    __builtin_amdgcn_sched_barrier(0);
    const Round<kRing> r0 = load_round<kRing>(a, bt_in, cur, wave, 0);
#pragma unroll
    for (int r = 0; r < kRing; ++r) valid[r] = issue(cur, r, r0.e[r], ring[r]);
    PKV_TL_MARK(2);
    // written out for read-back behind the page loads (recomputed, so that
    // nothing is held across them)
    self_record(blockIdx.x, true);
  } else {
    // Host plan.  The first task does not wait for the staging: its record
    // went out at entry, the staging loads go out behind it (vector loads
    // complete in order, so the record's wait does not cover them); from the
    // record alone come the first round's table entries and its row bounds
    // (scalar loads from global memory, not from the staged copy, issued
    // together), then q (vector).  Two round trips lie before the first page
    // load, the record's and the table's; the argument loads and the staging
    // complete in their shadow, and the staging is stored to LDS for the
    // later tasks.  The scheduling barriers keep that order.
    constexpr int kPer = kStaged ? (kRowStage + kThreads) / kThreads : 1;   // B+1 <= kRowStage+1
    int lv[kPer], ov[kPer];
    if constexpr (kStaged) {
      // Buffer loads bounded by the arrays' sizes (entries past them read
      // 0): no branch around them, so the wait for the record below counts
      // exactly the loads issued before it and none of these.
      const __amdgpu_buffer_rsrc_t len_rsrc =
          make_rsrc(seq_lens_in, static_cast<uint32_t>(a.B) * 4u);
      const __amdgpu_buffer_rsrc_t off_rsrc =
          make_rsrc(offs_in, static_cast<uint32_t>(a.B + 1) * 4u);
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int i = tid + k * kThreads;
        lv[k] = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(len_rsrc, 4 * i, 0, 0));
        ov[k] = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(off_rsrc, 4 * i, 0, 0));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    const int4 rec0{static_cast<int>(__builtin_amdgcn_readfirstlane(rec0v[0])),
                    static_cast<int>(__builtin_amdgcn_readfirstlane(rec0v[1])),
                    static_cast<int>(__builtin_amdgcn_readfirstlane(rec0v[2])),
                    static_cast<int>(__builtin_amdgcn_readfirstlane(rec0v[3]))};
    // The first round's table entries and the row's length and split
    // offsets are read together (scalar), for the record's row clamped into
    // range: one round trip after the record's, then the page loads.
    const int rb = clamp_index(rec0.x, a.B);
    const Round<kRing> r0 = first_round<kRing>(a, bt_in, seq_lens_in, rec0, wave);
    const int rN = seq_lens_in[rb];
    const int ro0 = offs_in[rb];
    const int ro1 = offs_in[rb + 1];
    cur = meta_from_row<kRing>(a, num_tasks, blockIdx.x, rec0, rN, ro0, ro1);
    __builtin_amdgcn_sched_barrier(0);
    // q goes out just ahead of the pages, so that its wait covers no page
    if (wave == 0) load_q(rb, clamp_index(rec0.y, a.Hkv), true, qf);
#pragma unroll
    for (int r = 0; r < kRing; ++r) valid[r] = issue(cur, r, r0.e[r], ring[r]);
    PKV_TL_MARK(2);
    if constexpr (kStaged) {
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int i = tid + k * kThreads;
        if (i < a.B) s_len[i] = lv[k];
        if (i <= a.B) s_off[i] = ov[k];
      }
    }
  }
  // store_q zeroes the columns of an invalid first task
  if (wave == 0) store_q(cur, qf, s_q[0]);
  int t_nxt = blockIdx.x + gridDim.x;
  __syncthreads();
  if (fuse) {
    // rows without tasks (N_b = 0): out = 0, lse = -inf
    for (int b = blockIdx.x; b < a.B; b += gridDim.x) {
      const int sb = kStaged ? s_off[b + 1] - s_off[b] : offs_in[b + 1] - offs_in[b];
      if (sb == 0)
        for (int g = 0; g < a.Hkv; ++g) write_empty_group<D, E>(ma, b, g);
    }
  }

  PKV_TL_MARK(3);
  int n_done = 0;   // entries of s_done (workgroup-uniform)
  for (int it = 0; cur.t < num_tasks; ++it) {
    const int par = it & 1;
    // next task's metadata, its first round of table entries and its q;
    // the index of the task after it (counter values start at 2*gridDim.x)
    Meta nxt;
    if constexpr (kSelfPlan)
      nxt = decode_meta<kStaged, kRing>(a, seq_lens_in, offs_in, s_len, s_off, num_tasks, t_nxt,
                                        self_record(t_nxt, true));
    else
      nxt = load_meta<kStaged, kRing>(a, tasks_in, task_cap, seq_lens_in, offs_in, s_len, s_off,
                                      num_tasks, t_nxt);
    const Round<kRing> nr0 = load_round<kRing>(a, bt_in, nxt, wave, 0);
    // Wave 0: the index after next (counter atomic, issued now) and the next
    // task's q (loaded at the start of this task's last round), both stored
    // to LDS at the end of the last round.  Vector loads complete in order,
    // so those waits cover only pages already consumed, never the refills
    // in flight behind them.
    const bool fetch = t_nxt < num_tasks;
    uint32_t raw_nn = 0;
    if (wave == 0 && fetch && lane == 0) raw_nn = atomicAdd(a.ctrl, 1u);

    WaveState<D> st;
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int e = 0; e < VW; ++e) st.acc[e] = floatx4{0.f, 0.f, 0.f, 0.f};

    for (int j = 0; j < cur.rounds; ++j) {
      const bool last = (j + 1 == cur.rounds);
      vecE<E, 8> qn[KK];
      if (last && wave == 0) load_q(nxt.b, nxt.g, nxt.ok, qn);
      const Round<kRing> fr = last ? nr0 : load_round<kRing>(a, bt_in, cur, wave, j + 1);
#pragma unroll
      for (int r = 0; r < kRing; ++r) {
        if (valid[r]) {
          const int page = cur.p0 + wave + kWaves * (kRing * j + r);
          process_page<D, E, KV>(st, ring[r], s_q[par], cur.N - page * kPage, a.scale_log2,
                                 lane);
        }
        // refill the slot with the position one round ahead
        if (last)
          valid[r] = issue(nxt, r, fr.e[r], ring[r]);
        else
          valid[r] = issue(cur, kRing * (j + 1) + r, fr.e[r], ring[r]);
      }
#ifdef PKV_TIMELINE
      if (it == 0 && j == 0) PKV_TL_MARK(4);
      if (last) {
        PKV_TL_MARK(5);
        PKV_TL_TASK();
        if (lane == 0) s_tlw[wave] = __builtin_amdgcn_s_memrealtime();
      }
#endif
      if (last && wave == 0) {
        store_q(nxt, qn, s_q[par ^ 1]);
        if (lane == 0)
          s_next[par] = fetch ? static_cast<int>(2u * gridDim.x + raw_nn) : num_tasks;
      }
    }

    // ---- this wave's state to LDS
    st.l += __shfl_xor(st.l, 16);
    st.l += __shfl_xor(st.l, 32);
    if (col < G) {
      if (grp == 0) {
        s_m[par][wave][col] = st.m;
        s_l[par][wave][col] = st.l;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < VW; ++e) s_o[wave][col][VW * (4 * grp + j) + e] = st.acc[e][j];
    }
    __syncthreads();
#ifdef PKV_TIMELINE
    PKV_TL_MARK(12);
    tl_[11] = s_tlw[0];
    for (int w_ = 1; w_ < kWaves; ++w_) tl_[11] = s_tlw[w_] > tl_[11] ? s_tlw[w_] : tl_[11];
#endif

    // ---- combine the 4 waves' states; write the output or the partial
    if (cur.ok) {
      const bool direct = (cur.Sb == 1);
      for (int idx = tid; idx < G * D; idx += kThreads) {
        const int h = idx / D;
        const int d = idx - h * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[par][w][h]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float mw = s_m[par][w][h];
          const float wt = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
          L += wt * s_l[par][w][h];
          O += wt * s_o[w][h][d];
        }
        O *= a.v_scale;   // V's dequantisation scale (exact for 1)
        const int64_t hq = static_cast<int64_t>(cur.g) * G + h;
        if (direct) {
          static_cast<E*>(a.out)[(static_cast<int64_t>(cur.b) * a.Hq + hq) * D + d] =
              static_cast<E>(O / L);
          if (d == 0 && a.lse)
            a.lse[static_cast<int64_t>(cur.b) * a.Hq + hq] = (M + __log2f(L)) * kLn2;
        } else {
          // write-through (system-scope) stores, read back by the merge
          const __amdgpu_buffer_rsrc_t po = make_rsrc(
              a.part_o + cur.slot * a.Hq * D, static_cast<uint32_t>(a.Hq) * D * 4u);
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, O), po,
                                                4 * (static_cast<int>(hq) * D + d), 0, kCoherent);
          if (d == 0) {
            const __amdgpu_buffer_rsrc_t pm = make_rsrc(
                a.part_ml + cur.slot * a.Hq, static_cast<uint32_t>(a.Hq) * 8u);
            __builtin_amdgcn_raw_buffer_store_b64(
                __builtin_bit_cast(uint2x, make_float2(M, L)), pm, 8 * static_cast<int>(hq), 0,
                kCoherent);
          }
        }
      }
#ifdef PKV_TIMELINE
      PKV_TL_MARK(13);
#endif
      if (fuse && !direct) {
        // Fused merge, deferred: the split is counted in later, so waiting
        // for its stores does not also wait for the page loads of the tasks
        // behind it.
        if (tid == 0) s_done[n_done] = int4{cur.b, cur.g, cur.o0, cur.Sb};
        if (++n_done == kMaxDone) {
          flush_done<D, kMergeBatch, E>(a, ma, n_done, s_done, s_lastf, &s_o[0][0][0]);
          n_done = 0;
        }
      }
    }
    __syncthreads();   // every read of s_o above precedes the next task's writes
    t_nxt = __builtin_amdgcn_readfirstlane(s_next[par]);
    cur = nxt;
  }

  PKV_TL_MARK(6);
  if (n_done > 0) flush_done<D, kMergeBatch, E>(a, ma, n_done, s_done, s_lastf, &s_o[0][0][0]);
  PKV_TL_MARK(7);
  PKV_TL_STORE();

  // Last workgroup out resets the counters for the next launch.  With no
  // more tasks than workgroups every task is static: no workgroup touched
  // the task counter (its next index, blockIdx.x + gridDim.x, is past the
  // list), so there is nothing to reset and no workgroup waits for the exit
  // count (a round trip at the end of the launch, about 0.5 us at B8).
  if (tid == 0 && num_tasks > static_cast<int>(gridDim.x)) {
    const uint32_t prev = atomicAdd(a.ctrl + 1, 1u);
    if (prev == gridDim.x - 1) {
      atomicExch(a.ctrl, 0u);
      atomicExch(a.ctrl + 1, 0u);
    }
  }
}

// Kernel 2 of the two-launch form, 64-thread workgroups.  A group's C =
// G*D/4 float4 columns are folded exactly as merge_group folds them inside
// the decode kernel -- R = 256/C threads per column (1 for C > 256), each
// over slots r, r+R, ..., the R states combined in LDS in the same order --
// so the two launch forms give the same bits; but the columns are spread
// over (C R) / 64 workgroups per group instead of one, so a deep group is
// merged by many CUs at once.
constexpr int kMergeKernelThreads = 64;

template <int D>
__device__ __forceinline__ int merge_threads_per_column(int G) {
  const int cols = G * (D / 4);
  return cols > kThreads ? 1 : kThreads / cols;
}

template <int D>
inline int merge_kernel_blocks(int G) {
  const int cols = G * (D / 4);
  const int R = cols > kThreads ? 1 : kThreads / cols;
  return cols * R / kMergeKernelThreads;
}

template <int D, class E>
__global__ void __launch_bounds__(kMergeKernelThreads) pkv_merge_kernel(MergeArgs a) {
  __shared__ __attribute__((aligned(16))) float lds[kMergeKernelThreads * 6];
  if (a.plan_hdr && a.plan_hdr[1]) return;   // merged inside the decode kernel
  const int G = a.G;
  const int R = merge_threads_per_column<D>(G);
  const int cpw = kMergeKernelThreads / R;         // columns per workgroup
  const int nch = G * (D / 4) / cpw;
  const int bg = blockIdx.x / nch;
  const int chunk = blockIdx.x - bg * nch;
  const int b = bg / a.Hkv;
  const int g = bg - b * a.Hkv;
  const int tid = threadIdx.x;
  const int r = tid / cpw;
  const int c = chunk * cpw + (tid - r * cpw);
  const int h = (4 * c) / D;
  const int64_t head0 = static_cast<int64_t>(b) * a.Hq + static_cast<int64_t>(g) * G;
  const int o0 = __builtin_amdgcn_readfirstlane(a.split_offsets[b]);
  const int S = __builtin_amdgcn_readfirstlane(a.split_offsets[b + 1]) - o0;
  if (S == 1) return;   // written directly by the decode kernel
  auto write = [&](float Mt, float Lt, floatx4 Ot) {
    const float inv = 1.f / Lt;
    E* dst = static_cast<E*>(a.out) + head0 * D + 4 * c;
    dst[0] = static_cast<E>(Ot[0] * inv);
    dst[1] = static_cast<E>(Ot[1] * inv);
    dst[2] = static_cast<E>(Ot[2] * inv);
    dst[3] = static_cast<E>(Ot[3] * inv);
    if ((4 * c) % D == 0 && a.lse) a.lse[head0 + h] = (Mt + __log2f(Lt)) * kLn2;
  };
  if (S <= 0 || o0 < 0 || static_cast<int64_t>(o0) + S > a.num_slots) {
    // an empty row (out = 0, lse = -inf), or a bad offset (flagged)
    if (S != 0 && chunk == 0 && tid == 0) flag_error(a.ctrl, PKV_DEVERR_SLOT);
    if (r == 0) {
      E* dst = static_cast<E*>(a.out) + head0 * D + 4 * c;
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = static_cast<E>(0.f);
      if ((4 * c) % D == 0 && a.lse) a.lse[head0 + h] = -INFINITY;
    }
    return;
  }
  // Coherent (L2-bypassing) loads: the states come from other XCDs.
  const __amdgpu_buffer_rsrc_t ml_rsrc = make_rsrc(
      a.part_ml + static_cast<int64_t>(o0) * a.Hq, static_cast<uint32_t>(S) * a.Hq * 8u);
  const __amdgpu_buffer_rsrc_t o_rsrc = make_rsrc(
      a.part_o + static_cast<int64_t>(o0) * a.Hq * D, static_cast<uint32_t>(S) * a.Hq * D * 4u);
  float M, L;
  floatx4 O;
  fold_column<D, kMergeBatch>(ml_rsrc, o_rsrc, a.Hq, 8 * (g * G + h), 4 * (g * G * D + 4 * c),
                              r, R, S, M, L, O);
  if (R == 1) {
    write(M, L, O);
    return;
  }
  float* s_M = lds;
  float* s_L = lds + kMergeKernelThreads;
  floatx4* s_O = reinterpret_cast<floatx4*>(lds + 2 * kMergeKernelThreads);
  s_M[tid] = M;
  s_L[tid] = L;
  s_O[tid] = O;
  __syncthreads();
  if (tid < cpw) {
    float Mt = -INFINITY;
    for (int j = 0; j < R; ++j) Mt = fmaxf(Mt, s_M[tid + j * cpw]);
    float Lt = 0.f;
    floatx4 Ot = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < R; ++j) {
      const float mj = s_M[tid + j * cpw];
      const float w = (mj == -INFINITY) ? 0.f : fast_exp2(mj - Mt);
      Lt += w * s_L[tid + j * cpw];
      Ot += w * s_O[tid + j * cpw];
    }
    write(Mt, Lt, Ot);
  }
}

// ---------------------------------------------------------------------------
// Device-side planner: the plan (and, if asked, the policy's choice) from the
// row lengths in device memory, so a step needs no host copy of them.
//
// "2. Calibrated Adaptive Policy" / "Row-Local Bounds" / "Compact Workqueue"
// (gist.science explainer): the same candidate search and time model as
// pkv_policy (policy_model.h), and the same records, offsets and order as
// pkv_plan, computed by one workgroup:
//   1. policy (mode < 0): 16 candidates at a time, each over 16 groups of
//      rows in parallel; 16 threads evaluate the model; the earliest fastest
//      candidate wins.
//   2. rows in chunks of 256: S_b per thread, an exclusive scan in LDS gives
//      split_offsets; then, row by row, all threads write the row's records.
//   3. the header: tasks, fused or not, mode, param, slots, deepest row.
// A row with N_b < 0 or more than max_pages pages is flagged
// (PKV_DEVERR_ROW) and planned as empty.

__global__ void __launch_bounds__(kThreads) pkv_plan_kernel(PlanArgs a) {
  __shared__ int32_t s_n[kPlanStage];
  __shared__ PickLds s_pick;
  __shared__ int s_best_i[kWaves];
  __shared__ int s_scan[kThreads];
  __shared__ int s_S[kThreads];
  __shared__ int s_c[kThreads];
  __shared__ int s_bad;
  __shared__ int s_active;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int staged = a.B < kPlanStage ? a.B : kPlanStage;

  // ---- 0. page counts of the rows, once; flagged rows and rows with pages
  int bad = 0, act = 0;
  if (tid == 0) {
    s_bad = 0;
    s_active = 0;
  }
  for (int b = tid; b < staged; b += kThreads) {
    const int32_t n = plan_row_pages_global(a, b);
    bad |= n < 0;
    act += n > 0 ? 1 : 0;
    s_n[b] = n < 0 ? 0 : n;
  }
  for (int b = staged + tid; b < a.B; b += kThreads) {
    const int32_t n = plan_row_pages_global(a, b);
    bad |= n < 0;
    act += n > 0 ? 1 : 0;
  }
  __syncthreads();
  if (bad) s_bad = 1;
  if (act > 0) atomicAdd(&s_active, act);
  __syncthreads();
  const int active_rows = s_active;
  auto row_n = [&](int b) -> int32_t {
    if (b < kPlanStage) return s_n[b];
    const int32_t n = plan_row_pages_global(a, b);
    return n < 0 ? 0 : n;
  };

  // ---- 1. policy
  int mode = a.mode, param = a.param;
  if (mode < 0)
    choose_plan(a.pol, a.B, a.Hkv, a.num_cus, a.head_dim, a.page_size, row_n, active_rows,
                s_pick, mode, param);

  // ---- 2. split offsets and records, 256 rows at a time
  int carry = 0;
  int maxS = 0;
  for (int base = 0; base < a.B; base += kThreads) {
    const int b = base + tid;
    int S = 0, c = 0;
    if (b < a.B) {
      const uint32_t n = static_cast<uint32_t>(row_n(b));
      if (n > 0) {
        c = static_cast<int>(mode == PKV_MODE_SPLIT ? cdiv32(n, param) : param);
        S = static_cast<int>(cdiv32(n, c));
      }
    }
    maxS = S > maxS ? S : maxS;
    s_S[tid] = S;
    s_c[tid] = c;
    s_scan[tid] = S;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {   // inclusive scan
      const int v = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    if (b < a.B) a.offs[b] = carry + s_scan[tid] - S;
    const int rows = a.B - base < kThreads ? a.B - base : kThreads;
    for (int r = 0; r < rows; ++r) {
      const int Sr = s_S[r];
      const int cr = s_c[r];
      const int64_t t0 = static_cast<int64_t>(a.Hkv) * (carry + s_scan[r] - Sr);
      for (int i = tid; i < a.Hkv * Sr; i += kThreads) {
        const int g = i / Sr;
        const int sp = i - g * Sr;
        a.tasks[t0 + i] = int4{base + r, g, sp, cr};
      }
    }
    carry += s_scan[kThreads - 1];
    __syncthreads();   // the chunk's LDS is reused
  }
  if (tid == 0) a.offs[a.B] = carry;

  // ---- 3. header
  const int deep_w = static_cast<int>(wave_max64(maxS));
  if (lane == 0) s_best_i[wave] = deep_w;
  __syncthreads();
  if (tid == 0) {
    int deep = 0;
    for (int w = 0; w < kWaves; ++w) deep = s_best_i[w] > deep ? s_best_i[w] : deep;
    const int T = a.Hkv * carry;
    a.hdr[0] = T;
    const int64_t groups = static_cast<int64_t>(a.Hkv) * active_rows;
    a.hdr[1] = (T == 0 || (!two_launch_form(a.pol, deep, groups) && a.groups_fit)) ? 1 : 0;
    a.hdr[2] = mode;
    a.hdr[3] = param;
    a.hdr[4] = carry;
    a.hdr[5] = deep;
    a.hdr[6] = s_bad;
    if (s_bad) flag_error(a.ctrl, PKV_DEVERR_ROW);
  }
}

// ---------------------------------------------------------------------------
// host glue

int num_cus_of_current_device(int* cus) {
  static int cache[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_hip_error(static_cast<int>(e));
    return PKV_ERR_HIP;
  }
  if (dev >= 0 && dev < 64 && cache[dev] > 0) {
    *cus = cache[dev];
    return PKV_OK;
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || n <= 0) {
    set_hip_error(static_cast<int>(e));
    return PKV_ERR_HIP;
  }
  if (dev >= 0 && dev < 64) cache[dev] = n;
  *cus = n;
  return PKV_OK;
}

// ev0 / ev1 (optional): events that take the decode kernel's own start and
// end timestamps (hipExtLaunchKernel), for timing it without the queue time
// of separately recorded events.
// kMode: cache policy of the page loads (load_mode).
template <int D, class E, class KV, int kMode>
int launch_mode(const DecodeArgs& da, const MergeArgs& ma, int grid, hipStream_t stream,
              bool decode, hipEvent_t ev0, hipEvent_t ev1) {
  // With a merge kernel behind the decode kernel, the end event takes the
  // merge kernel's end: the events then span the whole step.
  const hipEvent_t ev_dec_end = ma.B > 0 ? nullptr : ev1;
  if (decode) {
    const int4* tasks = reinterpret_cast<const int4*>(da.tasks);
    const bool staged = da.B <= kRowStage;
    if (da.plan_out) {   // self-planned step (staged rows only; checked by the caller)
      // (load_mode never gives mode 2 to a self-planned step).  It builds
      // its task list itself and reads no `tasks`: the second (preloaded)
      // argument carries the key of its shape and policy instead.
      const uint32_t key = plan_cache_config_key(da.plan_pol, da.B, da.Hkv, da.plan_num_cus,
                                                 da.plan_head_dim, da.max_pages);
      hipLaunchKernelGGL((pkv_decode_kernel<D, true, E, KV, true, kMode == 2 ? 1 : kMode>),
                         dim3(grid), dim3(kThreads), 0, stream, tasks, static_cast<int32_t>(key),
                         da, da.block_table, da.seq_lens, da.split_offsets);
    } else if (ev0 || ev_dec_end) {
      if (staged)
        hipExtLaunchKernelGGL((pkv_decode_kernel<D, true, E, KV, false, kMode>), dim3(grid),
                              dim3(kThreads), 0, stream, ev0, ev_dec_end, 0, tasks, da.task_cap,
                              da, da.block_table, da.seq_lens, da.split_offsets);
      else
        hipExtLaunchKernelGGL((pkv_decode_kernel<D, false, E, KV, false, kMode>), dim3(grid),
                              dim3(kThreads), 0, stream, ev0, ev_dec_end, 0, tasks, da.task_cap,
                              da, da.block_table, da.seq_lens, da.split_offsets);
    } else if (staged) {
      hipLaunchKernelGGL((pkv_decode_kernel<D, true, E, KV, false, kMode>), dim3(grid),
                         dim3(kThreads), 0, stream, tasks, da.task_cap, da, da.block_table,
                         da.seq_lens, da.split_offsets);
    } else {
      hipLaunchKernelGGL((pkv_decode_kernel<D, false, E, KV, false, kMode>), dim3(grid),
                         dim3(kThreads), 0, stream, tasks, da.task_cap, da, da.block_table,
                         da.seq_lens, da.split_offsets);
    }
  } else {
    // no decode kernel (no tasks): the events still mark this point of the stream
    if (ev0 && hipEventRecord(ev0, stream) != hipSuccess) return PKV_ERR_HIP;
    if (ev_dec_end && hipEventRecord(ev_dec_end, stream) != hipSuccess) return PKV_ERR_HIP;
  }
  if (decode) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
      set_hip_error(static_cast<int>(e));
      return PKV_ERR_HIP;
    }
  }
  if (ma.B > 0) {
    const dim3 mgrid(ma.B * ma.Hkv * merge_kernel_blocks<D>(ma.G));
    if (ev1)
      hipExtLaunchKernelGGL((pkv_merge_kernel<D, E>), mgrid, dim3(kMergeKernelThreads), 0,
                            stream, nullptr, ev1, 0, ma);
    else
      hipLaunchKernelGGL((pkv_merge_kernel<D, E>), mgrid, dim3(kMergeKernelThreads), 0, stream,
                         ma);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
      set_hip_error(static_cast<int>(e));
      return PKV_ERR_HIP;
    }
  }
  return PKV_OK;
}

template <int D, class E, class KV>
int launch(const DecodeArgs& da, const MergeArgs& ma, int grid, hipStream_t stream, bool decode,
           int mode, hipEvent_t ev0, hipEvent_t ev1) {
  // Only the modes load_mode can give this pool type and head dimension are
  // compiled: 0 for 2-byte pools at d = 256, 1 for fp8 pools, 1 or 2 else.
  constexpr bool kFp8 = kv_bytes<KV>() == 1;
  if constexpr (D == 256 && !kFp8) {
    return launch_mode<D, E, KV, 0>(da, ma, grid, stream, decode, ev0, ev1);
  } else if constexpr (kFp8) {
    return launch_mode<D, E, KV, 1>(da, ma, grid, stream, decode, ev0, ev1);
  } else {
    return mode == 2 ? launch_mode<D, E, KV, 2>(da, ma, grid, stream, decode, ev0, ev1)
                     : launch_mode<D, E, KV, 1>(da, ma, grid, stream, decode, ev0, ev1);
  }
}

template <class E, class KV>
int launch_d(int head_dim, const DecodeArgs& da, const MergeArgs& ma, int grid,
             hipStream_t stream, bool decode, int mode, hipEvent_t ev0, hipEvent_t ev1) {
  if (head_dim == 256) return launch<256, E, KV>(da, ma, grid, stream, decode, mode, ev0, ev1);
  return head_dim == 128 ? launch<128, E, KV>(da, ma, grid, stream, decode, mode, ev0, ev1)
                         : launch<64, E, KV>(da, ma, grid, stream, decode, mode, ev0, ev1);
}

// The kernels of one head dimension and element-type pair (both checked by
// the caller).
int launch_any(int head_dim, int dtype, const DecodeArgs& da, const MergeArgs& ma, int grid,
               hipStream_t stream, bool decode, int mode, hipEvent_t ev0 = nullptr,
               hipEvent_t ev1 = nullptr) {
  switch (dtype) {
    case PKV_DTYPE_BF16:
      return launch_d<__bf16, __bf16>(head_dim, da, ma, grid, stream, decode, mode, ev0, ev1);
    case PKV_DTYPE_F16_KV_FP8:
      return launch_d<_Float16, Fp8E4M3>(head_dim, da, ma, grid, stream, decode, mode, ev0, ev1);
    case PKV_DTYPE_BF16_KV_FP8:
      return launch_d<__bf16, Fp8E4M3>(head_dim, da, ma, grid, stream, decode, mode, ev0, ev1);
    default:
      return launch_d<_Float16, _Float16>(head_dim, da, ma, grid, stream, decode, mode, ev0, ev1);
  }
}

}  // namespace pkv

extern "C" {

#ifdef PKV_TIMELINE
// Profiling build only: copy the per-workgroup timeline of the last launch
// (kTimelineWorkgroups x kTimelineSlots uint64, row w for workgroup w) to
// host memory.  Returns PKV_OK or PKV_ERR_HIP.
int pkv_timeline_read(void* host, size_t bytes) {
  const size_t all = sizeof(pkv::timeline);
  if (!host) return PKV_ERR_INVALID_ARG;
  const hipError_t e = hipMemcpyFromSymbol(host, HIP_SYMBOL(pkv::timeline),
                                           bytes < all ? bytes : all, 0,
                                           hipMemcpyDeviceToHost);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
#endif

int pkv_page_load_mode(int32_t head_dim, int32_t dtype, int64_t num_tasks, int32_t num_cus,
                       int32_t* mode) {
  if (!mode || num_cus < 1 || dtype < PKV_DTYPE_F16 || dtype > PKV_DTYPE_BF16_KV_FP8)
    return PKV_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return PKV_ERR_UNSUPPORTED;
  *mode = pkv::load_mode(head_dim, dtype, num_tasks < 0 ? -1 : num_tasks, num_cus);
  return PKV_OK;
}

int pkv_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || workspace_bytes < PKV_WORKSPACE_HEADER_BYTES) return PKV_ERR_INVALID_ARG;
  hipError_t e = hipMemsetAsync(workspace, 0, PKV_WORKSPACE_HEADER_BYTES,
                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    pkv::set_hip_error(static_cast<int>(e));
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
    pkv::set_hip_error(static_cast<int>(e));
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
            int32_t page_size, int32_t dtype, float scale, float k_scale, float v_scale,
            void* out, float* lse, void* workspace, size_t workspace_bytes, bool need_decode,
            pkv::DecodeArgs* da, pkv::MergeArgs* ma) {
  if (B < 0 || Hq < 1 || Hkv < 1 || num_pages < 0 || max_pages_per_row < 0 || num_tasks < 0 ||
      num_tasks > INT32_MAX || num_partial_slots < 0 || !(scale == scale) ||
      !(k_scale > 0.f && k_scale <= FLT_MAX) || !(v_scale > 0.f && v_scale <= FLT_MAX))
    return PKV_ERR_INVALID_ARG;
  if (page_size != pkv::kPage || (head_dim != 64 && head_dim != 128 && head_dim != 256) ||
      Hq % Hkv != 0 || dtype < PKV_DTYPE_F16 || dtype > PKV_DTYPE_BF16_KV_FP8)
    return PKV_ERR_UNSUPPORTED;
  const int G = Hq / Hkv;   // one MFMA column per query head of the group
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return PKV_ERR_UNSUPPORTED;
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
  float* part_o = reinterpret_cast<float*>(ws + PKV_WORKSPACE_HEADER_BYTES);
  float2* part_ml = reinterpret_cast<float2*>(ws + PKV_WORKSPACE_HEADER_BYTES +
                                              static_cast<size_t>(num_partial_slots) * Hq *
                                                  head_dim * sizeof(float));
  uint32_t* ctrl = reinterpret_cast<uint32_t*>(ws);

  da->q = q;
  da->k = k_pool;
  da->v = v_pool;
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
  da->scale_log2 = scale * k_scale * 1.44269504088896340736f;
  da->v_scale = v_scale;
  da->out = out;
  da->lse = lse;
  da->ctrl = ctrl;
  da->arrive = ctrl + 64;
  da->fuse = 0;
  da->part_o = part_o;
  da->part_ml = part_ml;

  ma->split_offsets = split_offsets;
  ma->num_slots = num_partial_slots;
  ma->B = B;
  ma->Hq = Hq;
  ma->Hkv = Hkv;
  ma->G = G;
  ma->part_o = part_o;
  ma->part_ml = part_ml;
  ma->out = out;
  ma->lse = lse;
  ma->ctrl = ctrl;
  return PKV_OK;
}

int run(const void* q, const void* k_pool, const void* v_pool, int64_t num_pages,
        const int32_t* block_table, int32_t max_pages_per_row, const int32_t* seq_lens,
        const int32_t* tasks, int64_t num_tasks, const int32_t* split_offsets,
        int64_t num_partial_slots, int32_t B, int32_t Hq, int32_t Hkv, int32_t head_dim,
        int32_t page_size, int32_t dtype, float scale, float k_scale, float v_scale, void* out,
        float* lse, void* workspace, size_t workspace_bytes, void* stream, bool do_decode,
        bool do_merge, bool fused, void* ev0 = nullptr, void* ev1 = nullptr) {
  pkv::DecodeArgs da{};
  pkv::MergeArgs ma{};
  int st = prepare(q, k_pool, v_pool, num_pages, block_table, max_pages_per_row, seq_lens, tasks,
                   num_tasks, split_offsets, num_partial_slots, B, Hq, Hkv, head_dim, page_size,
                   dtype, scale, k_scale, v_scale, out, lse, workspace, workspace_bytes, do_decode,
                   &da, &ma);
  if (st != PKV_OK || B == 0) return st;
  // Fused single launch when the arrival counters fit and there is work for
  // the decode kernel; otherwise the two-launch form.
  if (fused && do_decode && num_tasks > 0 &&
      static_cast<int64_t>(B) * Hkv <= PKV_MAX_FUSED_GROUPS) {
    da.fuse = 1;
    do_merge = false;
  }
  int grid = 1;
  int load = 0;
  if (do_decode) {
    int cus = 0;
    st = pkv::num_cus_of_current_device(&cus);
    if (st != PKV_OK) return st;
    load = pkv::load_mode(head_dim, dtype, num_tasks, cus);
    // as many workgroups as fit at once (persistent: a workgroup that had to
    // wait for a slot would hold its static tasks until the others finish)
    int64_t g = static_cast<int64_t>(cus) * (head_dim == 256 ? 1 : 2);
    if (g > num_tasks) g = num_tasks;
    grid = static_cast<int>(g < 1 ? 1 : g);
  } else {
    da.num_tasks = 0;
  }
  if (!do_merge) ma.B = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool decode = da.num_tasks > 0;
  da.task_cap = da.num_tasks > 0 ? da.num_tasks : 1;
  return pkv::launch_any(head_dim, dtype, da, ma, grid, s, decode, load,
                         static_cast<hipEvent_t>(ev0), static_cast<hipEvent_t>(ev1));
}

}  // namespace

extern "C++" {   // internal, C++ linkage, inside the extern "C" block
namespace pkv {
int decode_timed(const void* q, const void* k_pool, const void* v_pool, int64_t num_pages,
                 const int32_t* block_table, int32_t max_pages_per_row, const int32_t* seq_lens,
                 const int32_t* tasks, int64_t num_tasks, const int32_t* split_offsets,
                 int64_t num_partial_slots, int32_t B, int32_t Hq, int32_t Hkv, int32_t head_dim,
                 int32_t page_size, int32_t dtype, float scale, float k_scale, float v_scale,
                 void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream,
                 bool fused, void* ev0, void* ev1) {
  return run(q, k_pool, v_pool, num_pages, block_table, max_pages_per_row, seq_lens, tasks,
             num_tasks, split_offsets, num_partial_slots, B, Hq, Hkv, head_dim, page_size, dtype,
             scale, k_scale, v_scale, out, lse, workspace, workspace_bytes, stream, true, true,
             fused, ev0, ev1);
}
}  // namespace pkv
}

int pkv_decode(const void* q, const void* k_pool, const void* v_pool, int64_t num_pages,
               const int32_t* block_table, int32_t max_pages_per_row,
               const int32_t* seq_lens, const int32_t* tasks, int64_t num_tasks,
               const int32_t* split_offsets, int64_t num_partial_slots, int32_t B,
               int32_t Hq, int32_t Hkv, int32_t head_dim, int32_t page_size, int32_t dtype,
               float scale, float k_scale, float v_scale, void* out, float* lse,
               void* workspace, size_t workspace_bytes, void* stream) {
  return run(q, k_pool, v_pool, num_pages, block_table, max_pages_per_row, seq_lens, tasks,
             num_tasks, split_offsets, num_partial_slots, B, Hq, Hkv, head_dim, page_size, dtype,
             scale, k_scale, v_scale, out, lse, workspace, workspace_bytes, stream, true, true,
             true);
}

int pkv_decode_splits(const void* q, const void* k_pool, const void* v_pool, int64_t num_pages,
                      const int32_t* block_table, int32_t max_pages_per_row,
                      const int32_t* seq_lens, const int32_t* tasks, int64_t num_tasks,
                      const int32_t* split_offsets, int64_t num_partial_slots, int32_t B,
                      int32_t Hq, int32_t Hkv, int32_t head_dim, int32_t page_size,
                      int32_t dtype, float scale, float k_scale, float v_scale, void* out,
                      float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return run(q, k_pool, v_pool, num_pages, block_table, max_pages_per_row, seq_lens, tasks,
             num_tasks, split_offsets, num_partial_slots, B, Hq, Hkv, head_dim, page_size, dtype,
             scale, k_scale, v_scale, out, lse, workspace, workspace_bytes, stream, true, false,
             false);
}

int pkv_merge(const int32_t* split_offsets, int64_t num_partial_slots, int32_t B, int32_t Hq,
              int32_t Hkv, int32_t head_dim, int32_t dtype, void* out, float* lse,
              void* workspace, size_t workspace_bytes, void* stream) {
  return run(nullptr, nullptr, nullptr, 0, nullptr, 0, nullptr, nullptr, 0, split_offsets,
             num_partial_slots, B, Hq, Hkv, head_dim, pkv::kPage, dtype, 1.0f, 1.0f, 1.0f, out,
             lse, workspace, workspace_bytes, stream, false, true, false);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// pkv_decode_static: pkv_decode with its workspace in a static device array,
// for callers that cannot allocate (graph capture, serving loops, harnesses
// that forbid it).

namespace pkv {

// The workspace of one step (control block, arrival counters, partial
// states), one copy per GPU, held until the process ends.
constexpr size_t kStaticScratchBytes = PKV_STATIC_SCRATCH_BYTES;
static_assert(4 * (64 + PKV_MAX_FUSED_GROUPS) <= PKV_WORKSPACE_HEADER_BYTES,
              "the zeroed control words lie in the header");
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// Zero n 32-bit words at p: the control block and the arrival counters of
// the static workspace before each step (a kernel rather than a memset, so
// that a captured graph replays it as an ordinary kernel node).
__global__ void __launch_bounds__(256) pkv_zero_kernel(uint32_t* p, int n) {
  for (int i = static_cast<int>(blockIdx.x * 256 + threadIdx.x); i < n;
       i += static_cast<int>(gridDim.x * 256))
    p[i] = 0u;
}

// Device address of `scratch` on the current device.  In host code the
// array's name only stands for the symbol, so it is never passed to a
// kernel: its address is looked up once per device, with that device
// current, and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_hip_error(static_cast<int>(e));
    return PKV_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return PKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      set_hip_error(static_cast<int>(e));
      return PKV_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace pkv

extern "C" {

int pkv_decode_static(const void* q, const void* k_pool, const void* v_pool, int64_t num_pages,
                      const int32_t* block_table, int32_t max_pages_per_row,
                      const int32_t* seq_lens, const int32_t* tasks, int64_t num_tasks,
                      const int32_t* split_offsets, int64_t num_partial_slots, int32_t B,
                      int32_t Hq, int32_t Hkv, int32_t head_dim, int32_t page_size,
                      int32_t dtype, float scale, float k_scale, float v_scale, void* out,
                      float* lse, void* stream) {
  size_t need = 0;
  if (pkv_workspace_size(num_partial_slots, Hq, head_dim, &need) != PKV_OK)
    return PKV_ERR_INVALID_ARG;
  if (need > pkv::kStaticScratchBytes) return PKV_ERR_SCRATCH_TOO_SMALL;
  if (B <= 0 || Hkv < 1) {
    // nothing to launch (B == 0), or invalid; the checks of run() decide
    return run(q, k_pool, v_pool, num_pages, block_table, max_pages_per_row, seq_lens, tasks,
               num_tasks, split_offsets, num_partial_slots, B, Hq, Hkv, head_dim, page_size,
               dtype, scale, k_scale, v_scale, out, lse, nullptr, 0, stream, true, true, true);
  }
  void* ws = nullptr;
  int st = pkv::static_scratch(&ws);
  if (st != PKV_OK) return st;
  // the control block and this step's arrival counters start at zero
  const int64_t groups = static_cast<int64_t>(B) * Hkv;
  const int n = 64 + static_cast<int>(groups < PKV_MAX_FUSED_GROUPS ? groups
                                                                     : PKV_MAX_FUSED_GROUPS);
  const int blocks = (n + 255) / 256 < 64 ? (n + 255) / 256 : 64;
  hipLaunchKernelGGL(pkv::pkv_zero_kernel, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint32_t*>(ws), n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    pkv::set_hip_error(static_cast<int>(e));
    return PKV_ERR_HIP;
  }
  return run(q, k_pool, v_pool, num_pages, block_table, max_pages_per_row, seq_lens, tasks,
             num_tasks, split_offsets, num_partial_slots, B, Hq, Hkv, head_dim, page_size, dtype,
             scale, k_scale, v_scale, out, lse, ws, pkv::kStaticScratchBytes, stream, true, true,
             true);
}

}  // extern "C"

namespace {

// Layout of the device-planned workspace: the ordinary workspace for
// B * max_splits partial slots, then the plan area: the header (64 B), the
// split offsets (B+1, padded to 16 B), the task records.
struct DevicePlanLayout {
  int64_t slot_cap = 0, task_cap = 0;
  size_t plan_off = 0, offs_off = 0, tasks_off = 0, bytes = 0;
};

int device_plan_layout(int32_t B, int32_t Hq, int32_t Hkv, int32_t head_dim, int32_t max_splits,
                       DevicePlanLayout* L) {
  if (B < 0 || Hq < 1 || Hkv < 1 || head_dim < 1 || max_splits < 1) return PKV_ERR_INVALID_ARG;
  L->slot_cap = static_cast<int64_t>(B) * max_splits;
  L->task_cap = L->slot_cap * Hkv;
  if (L->task_cap > INT32_MAX) return PKV_ERR_INVALID_ARG;
  size_t ws = 0;
  const int st = pkv_workspace_size(L->slot_cap, Hq, head_dim, &ws);
  if (st != PKV_OK) return st;
  L->plan_off = ws;
  L->offs_off = ws + pkv::kPlanHdrInts * sizeof(int32_t);
  const size_t offs_bytes = ((static_cast<size_t>(B) + 1) * sizeof(int32_t) + 15) & ~size_t(15);
  L->tasks_off = L->offs_off + offs_bytes;
  const size_t task_bytes = static_cast<size_t>(L->task_cap > 0 ? L->task_cap : 1) * 16;
  L->bytes = (L->tasks_off + task_bytes + 255) & ~size_t(255);
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_workspace_size_device_plan(int32_t B, int32_t Hq, int32_t Hkv, int32_t head_dim,
                                   int32_t max_splits, size_t* bytes) {
  if (!bytes) return PKV_ERR_INVALID_ARG;
  DevicePlanLayout L;
  const int st = device_plan_layout(B, Hq, Hkv, head_dim, max_splits, &L);
  if (st != PKV_OK) return st;
  *bytes = L.bytes;
  return PKV_OK;
}

int pkv_decode_device_plan(const void* q, const void* k_pool, const void* v_pool,
                           int64_t num_pages, const int32_t* block_table,
                           int32_t max_pages_per_row, const int32_t* seq_lens, int32_t B,
                           int32_t Hq, int32_t Hkv, int32_t head_dim, int32_t page_size,
                           int32_t dtype, float scale, float k_scale, float v_scale,
                           int32_t mode, int32_t param, int32_t max_splits,
                           const pkv_policy_params* policy, int32_t num_cus, void* out,
                           float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  pkv_policy_params pol;
  if (policy) {
    pol = *policy;
  } else {
    pkv_policy_defaults(&pol);
  }
  if (mode < -1 || mode > PKV_MODE_WORKQUEUE || max_splits < 1 || max_pages_per_row < 0)
    return PKV_ERR_INVALID_ARG;
  if (pol.split_max < 1 || pol.chunk_min < 1 || pol.chunk_max < pol.chunk_min ||
      pol.fuse_max_splits < 0 || pol.fuse_max_group_splits < 0 || !(pol.cu_gbps > 0.0) ||
      !(pol.hbm_gbps > 0.0))
    return PKV_ERR_INVALID_ARG;
  // Capacity: no row may get more than max_splits splits.  Checked on the
  // host from max_pages_per_row alone, so the device never overruns.
  const int64_t M = max_pages_per_row;
  if (mode == PKV_MODE_SPLIT && (param < 1 || param > max_splits)) return PKV_ERR_INVALID_ARG;
  if (mode == PKV_MODE_WORKQUEUE && (param < 1 || pkv::cdiv(M, param) > max_splits))
    return PKV_ERR_INVALID_ARG;
  if (mode < 0) {
    // the candidate sets, limited to the capacity
    if (pol.split_max > max_splits) pol.split_max = max_splits;
    int64_t c = pol.chunk_min;
    while (c <= pol.chunk_max && pkv::cdiv(M, c) > max_splits) c *= 2;
    if (c > pol.chunk_max) {
      pol.chunk_min = pol.chunk_max + 1;   // no workqueue candidate fits
    } else {
      pol.chunk_min = static_cast<int32_t>(c);
    }
  }
  // Groups within the fused merge's arrival counters: the step is always the
  // fused single launch, so the policy times every candidate in that form.
  const int32_t groups_fit = static_cast<int64_t>(B) * Hkv <= PKV_MAX_FUSED_GROUPS ? 1 : 0;
  if (groups_fit) pol.fuse_max_splits = INT32_MAX;
  DevicePlanLayout L;
  int st = device_plan_layout(B, Hq, Hkv, head_dim, max_splits, &L);
  if (st != PKV_OK || B == 0) return st;
  if (!workspace || !out || !seq_lens) return PKV_ERR_INVALID_ARG;
  if (workspace_bytes < L.bytes) return PKV_ERR_BUFFER_TOO_SMALL;
  char* ws = static_cast<char*>(workspace);
  int32_t* hdr = reinterpret_cast<int32_t*>(ws + L.plan_off);
  int32_t* offs = reinterpret_cast<int32_t*>(ws + L.offs_off);
  int32_t* tasks = reinterpret_cast<int32_t*>(ws + L.tasks_off);

  pkv::DecodeArgs da{};
  pkv::MergeArgs ma{};
  st = prepare(q, k_pool, v_pool, num_pages, block_table, max_pages_per_row, seq_lens, tasks,
               L.task_cap, offs, L.slot_cap, B, Hq, Hkv, head_dim, page_size, dtype, scale,
               k_scale, v_scale, out, lse, workspace, workspace_bytes, true, &da, &ma);
  if (st != PKV_OK || B == 0) return st;
  if (num_cus <= 0) {
    st = pkv::num_cus_of_current_device(&num_cus);
    if (st != PKV_OK) return st;
  }
  pkv::PlanArgs pa{};
  pa.seq_lens = seq_lens;
  pa.B = B;
  pa.Hkv = Hkv;
  // the model's tile bytes assume 2-byte elements: an fp8 pool moves half
  pa.head_dim = pkv::policy_head_dim(head_dim, dtype);
  pa.page_size = page_size;
  pa.num_cus = num_cus;
  pa.max_pages = max_pages_per_row;
  pa.mode = mode;
  pa.param = param;
  pa.groups_fit = groups_fit;
  pa.pol = pol;
  pa.hdr = hdr;
  pa.offs = offs;
  pa.tasks = reinterpret_cast<int4*>(tasks);
  pa.ctrl = da.ctrl;
  da.task_cap = static_cast<int32_t>(L.task_cap > 0 ? L.task_cap : 1);
  da.num_tasks = 0;
  ma.plan_hdr = hdr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B <= pkv::kRowStage) {
    // One launch: every decode workgroup plans from the lengths it stages
    // anyway (the same policy and plan as the planner kernel).
    da.plan_mode = mode;
    da.plan_param = param;
    da.plan_num_cus = num_cus;
    da.plan_head_dim = pa.head_dim;
    da.plan_groups_fit = pa.groups_fit;
    da.plan_pol = pol;
    da.plan_out = hdr;
    da.plan_offs_out = offs;
    da.plan_tasks_out = reinterpret_cast<int4*>(tasks);
  } else {
    da.plan_hdr = hdr;
    hipLaunchKernelGGL(pkv::pkv_plan_kernel, dim3(1), dim3(pkv::kThreads), 0, s, pa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
      pkv::set_hip_error(static_cast<int>(e));
      return PKV_ERR_HIP;
    }
  }
  // The task count is known only on the device: one workgroup per CU (as
  // fast as two per CU on the measured workloads, and with no pair of
  // workgroups sharing a CU while others idle); workgroups past the count
  // exit at once.  A fused step launches no merge kernel.
  const int grid = num_cus;
  if (groups_fit) ma.B = 0;
  return pkv::launch_any(head_dim, dtype, da, ma, grid, s, true,
                         pkv::load_mode(head_dim, dtype, -1, num_cus));
}

int pkv_device_plan_read(const void* workspace, size_t workspace_bytes, int32_t B, int32_t Hq,
                         int32_t Hkv, int32_t head_dim, int32_t max_splits, int32_t* header,
                         int32_t* split_offsets, int32_t* tasks, int64_t task_capacity,
                         void* stream) {
  if (!workspace || !header) return PKV_ERR_INVALID_ARG;
  DevicePlanLayout L;
  int st = device_plan_layout(B, Hq, Hkv, head_dim, max_splits, &L);
  if (st != PKV_OK) return st;
  if (workspace_bytes < L.bytes) return PKV_ERR_BUFFER_TOO_SMALL;
  const char* ws = static_cast<const char*>(workspace);
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess)
    e = hipMemcpy(header, ws + L.plan_off, 8 * sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e == hipSuccess && split_offsets)
    e = hipMemcpy(split_offsets, ws + L.offs_off, (static_cast<size_t>(B) + 1) * sizeof(int32_t),
                  hipMemcpyDeviceToHost);
  if (e == hipSuccess && tasks) {
    if (header[0] < 0 || header[0] > task_capacity) return PKV_ERR_BUFFER_TOO_SMALL;
    if (header[0] > 0)
      e = hipMemcpy(tasks, ws + L.tasks_off, static_cast<size_t>(header[0]) * 16,
                    hipMemcpyDeviceToHost);
  }
  if (e != hipSuccess) {
    pkv::set_hip_error(static_cast<int>(e));
    return PKV_ERR_HIP;
  }
  return PKV_OK;
}

}  // extern "C"
