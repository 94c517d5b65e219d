// Device helpers and internal launcher declarations shared by the libcsa
// sources.  gfx950 (CDNA4) only: wave64, bf16 MFMA, 160 KiB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa.h"

namespace csa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Top-k radix key: an order-preserving map from fp32 to uint32 (larger float
// -> larger key).  -0.0 is folded onto +0.0 so that equal values tie.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Number of top key bits histogrammed by the first (multi-workgroup) pass.
constexpr int kHistBits = 11;
constexpr int kHistBins = 1 << kHistBits;

// Visible-block count of a token; flags inconsistent metadata.  Mirrors the
// causal rule: blocks strictly before the query's own block, capped by the
// blocks stored for the sequence.
__device__ __forceinline__ int64_t visible_count(int64_t pos, int ratio, int32_t n_comp,
                                                 uint32_t* flags) {
  if (pos < 0 || n_comp < 0) {
    *flags |= CSA_DERR_BAD_META;
    return 0;
  }
  int64_t v = pos / ratio;
  return v < (int64_t)n_comp ? v : (int64_t)n_comp;
}

__device__ __forceinline__ void report(uint32_t* err, uint32_t flags) {
  if (err != nullptr && flags != 0u) atomicOr(err, flags);
}

// Agent-scope release / acquire fences for the "last workgroup finishes"
// pattern (the caches of the eight XCDs are not coherent with each other).
__device__ __forceinline__ void fence_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void fence_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Internal launchers (host).  Arguments are validated by the C ABI layer.
// ---------------------------------------------------------------------------
struct IndexScoreLaunch {
  const uint16_t* q_idx; const float* w; const uint16_t* k_idx; int64_t k_rows;
  const int64_t* pos; const int64_t* seq_kv; const int32_t* n_comp;
  int T, n_ih, ihd, ratio;
  float* scores; int64_t ld;
  uint32_t* hist;   // [T, kHistBins] or nullptr: fused top-bits histogram
  uint32_t* err;
};
hipError_t launch_index_score(const IndexScoreLaunch& a, hipStream_t s);

// Top-k workspace, per token: hist[kHistBins] u32, ctr[4] u32, cand[ld] u64.
struct TopkWs {
  uint32_t* hist;    // [T, kHistBins]
  uint32_t* ctr;     // [T, 4]: above count, candidate count, ticket, spare
  uint64_t* cand;    // [T, ld]
};
size_t topk_ws_bytes(int T, int64_t ld);
TopkWs topk_ws_carve(void* ws, int T, int64_t ld);
hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t s);
hipError_t launch_score_hist(const float* scores, int64_t ld, const int64_t* pos,
                             const int32_t* n_comp, int T, int ratio, uint32_t* hist,
                             uint32_t* err, hipStream_t s);
hipError_t launch_topk_select(const float* scores, int64_t ld, const int64_t* pos,
                              const int32_t* n_comp, int T, int ratio, int top_k,
                              int32_t* idx, int32_t* count, const TopkWs& ws,
                              uint32_t* err, hipStream_t s);

struct GatherLaunch {
  const uint16_t* comp_kv; int64_t comp_rows; const int64_t* seq_kv;
  const int32_t* idx; const int32_t* count; int top_k;
  const uint16_t* swa; int64_t swa_rows; const int64_t* swa_row0; const int32_t* swa_len;
  int window, T, head_dim;
  uint16_t* all_kv; int32_t* n_kv; uint32_t* err;
};
hipError_t launch_gather(const GatherLaunch& a, hipStream_t s);

// Segment A of the attention row set is described either explicitly
// (row0/len arrays) or, for the HCA path, derived from the visibility rule
// (row0 = seq_kv[t], len = n_vis[t]); or, for the CSA path, as token t's slice
// of all_kv (row0 = t*a_stride, len = n_kv[t]).
struct AttendLaunch {
  const uint16_t* q; int T, n_heads, head_dim; float scale; const float* sink;
  const uint16_t* kv_a; int64_t a_rows; const int64_t* a_row0; const int32_t* a_len;
  int64_t a_stride;                       // >0: row0 = t*a_stride (a_row0 unused)
  const int64_t* vis_pos; const int32_t* vis_ncomp; int vis_ratio;  // HCA: len = n_vis
  const uint16_t* kv_b; int64_t b_rows; const int64_t* b_row0; const int32_t* b_len;
  int max_rows;
  uint16_t* out; float* lse;
  void* ws; uint32_t* err;
};
size_t attend_ws_bytes(int T, int n_heads, int head_dim, int max_rows);
hipError_t launch_attend(const AttendLaunch& a, hipStream_t s);

}  // namespace csa
