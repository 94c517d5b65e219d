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

// ReLU on the bits: a float with the sign bit set (negative, -0, -inf, a
// NaN with the sign set) becomes +0, any other keeps its value.  One integer
// max, where fmaxf(x, 0) would first canonicalize x (a second instruction).
__device__ __forceinline__ float relu_f32(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// Composite selection key of block s with score f: the score key in the high
// word, the complemented block index in the low word.  Unique per block;
// larger score first, then lower block index.  Zero marks an empty slot.
__device__ __forceinline__ uint64_t block_key(float f, uint32_t s) {
  return ((uint64_t)score_key(f) << 32) | (uint32_t)(~s);
}

// Largest value over the wave: DPP max steps within each row of 16 lanes
// (quad swaps, half-row and row mirrors), then row broadcasts carry the row
// maxima up to lane 63, which holds the total.  Register-to-register only.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // half-row mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
}

// Lane i of each 16-lane row receives lane i-1's value; lane 0 of a row
// receives all ones.
__device__ __forceinline__ uint64_t row_shr1_u64(uint64_t v) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)(uint32_t)(v >> 32), 0x111, 0xF, 0xF, false);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)(uint32_t)v, 0x111, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}

// One round of a wave-level selection: the largest nonzero score key over the
// lanes (sk), its owner (the lowest lane holding it; lane order is block
// order for equal scores), and that lane's low word.  The owner's sk is
// cleared.  Returns the composite key.
__device__ __forceinline__ uint64_t wave_take_max(uint32_t& sk, uint32_t lo) {
  const int lane = threadIdx.x & 63;
  const uint32_t M = wave_max_u32(sk);
  const int owner = __ffsll((unsigned long long)__ballot(sk == M)) - 1;
  const uint32_t olo = (uint32_t)__builtin_amdgcn_readlane((int)lo, owner);
  if (lane == owner) sk = 0u;
  return ((uint64_t)M << 32) | olo;
}

// Smallest value over the wave (DPP, as wave_max_u32).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0xB1, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x4E, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x141, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x140, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x142, 0xA, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Largest and summed float over the wave, in lane 63 (as wave_max_u32: DPP
// quad swaps, half-row and row mirrors, then row broadcasts; each step's
// neutral value fills the rows a broadcast does not write).
__device__ __forceinline__ float dpp_f32(float old, float v, int ctrl, int row_mask) {
  switch (ctrl) {  // the control word must be a constant
    case 0xB1: return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), 0xB1, 0xF, 0xF, false));
    case 0x4E: return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), 0x4E, 0xF, 0xF, false));
    case 0x141: return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), 0x141, 0xF, 0xF, false));
    case 0x140: return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), 0x140, 0xF, 0xF, false));
    case 0x142: return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), 0x142, 0xA, 0xF, false));
    default: return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), 0x143, 0xC, 0xF, false));
  }
}
__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, dpp_f32(-INFINITY, v, 0xB1, 0xF));
  v = fmaxf(v, dpp_f32(-INFINITY, v, 0x4E, 0xF));
  v = fmaxf(v, dpp_f32(-INFINITY, v, 0x141, 0xF));
  v = fmaxf(v, dpp_f32(-INFINITY, v, 0x140, 0xF));
  v = fmaxf(v, dpp_f32(-INFINITY, v, 0x142, 0xA));
  v = fmaxf(v, dpp_f32(-INFINITY, v, 0x143, 0xC));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32(0.f, v, 0xB1, 0xF);
  v += dpp_f32(0.f, v, 0x4E, 0xF);
  v += dpp_f32(0.f, v, 0x141, 0xF);
  v += dpp_f32(0.f, v, 0x140, 0xF);
  v += dpp_f32(0.f, v, 0x142, 0xA);
  v += dpp_f32(0.f, v, 0x143, 0xC);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Inclusive prefix sum over the wave's lanes: shifts by 1, 2, 4 and 8 lanes
// within each 16-lane row (zero filled), then row broadcasts carry the row
// totals across rows (lane 15 into row 1 and 3, lane 31 into rows 2 and 3).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Wave-level top-m of the blocks whose scores the lanes hold: for q < KPL,
// lane L holds score sc[q] of block blk[q] where ok[q].  Block indices must
// ascend in (q, lane) order.  Returns the number of valid blocks; lane r < m
// receives in *val the r-th largest composite key (larger score, then lower
// index), zero beyond the valid blocks.  One key per round: the wave maximum
// of the 32-bit score keys, then the lowest (q, lane) holding it.
template <int KPL>
__device__ __forceinline__ uint32_t wave_top_m(const float (&sc)[KPL], const bool (&ok)[KPL],
                                               const uint32_t (&blk)[KPL], uint32_t m,
                                               uint64_t* val) {
  const int lane = threadIdx.x & 63;
  uint32_t sk[KPL];  // 0 = empty (score keys of non-NaN scores are nonzero)
  uint32_t n_ok = 0;
#pragma unroll
  for (int q = 0; q < KPL; ++q) {
    sk[q] = ok[q] ? score_key(sc[q]) : 0u;
    n_ok += (uint32_t)__popcll(__ballot(ok[q]));
  }
  const uint32_t take = n_ok < m ? n_ok : m;
  uint64_t v = 0ull;
  for (uint32_t r = 0; r < take; ++r) {
    uint32_t lm = 0;
#pragma unroll
    for (int q = 0; q < KPL; ++q) lm = max(lm, sk[q]);
    const uint32_t M = wave_max_u32(lm);
    int oq = -1;
    uint64_t mask = 0;
#pragma unroll
    for (int q = 0; q < KPL; ++q) {
      if (oq < 0) {  // wave-uniform
        const uint64_t b = __ballot(sk[q] == M);
        if (b != 0ull) {
          oq = q;
          mask = b;
        }
      }
    }
    const int owner = __ffsll((unsigned long long)mask) - 1;
    uint32_t ob = 0;
#pragma unroll
    for (int q = 0; q < KPL; ++q)
      if (q == oq) ob = blk[q];
    ob = (uint32_t)__builtin_amdgcn_readlane((int)ob, owner);
    if (lane == owner) {
#pragma unroll
      for (int q = 0; q < KPL; ++q)
        if (q == oq) sk[q] = 0u;
    }
    if (lane == (int)r) v = ((uint64_t)M << 32) | (uint32_t)~ob;
  }
  *val = v;
  return n_ok;
}

// Visible-block count of a token; flags inconsistent metadata.  Mirrors the
// causal rule: blocks strictly before the query's own block, capped by the
// blocks stored for the sequence.
__device__ __forceinline__ int64_t visible_count(int64_t pos, int ratio, int32_t n_comp,
                                                 uint32_t* flags) {
  if (pos < 0 || n_comp < 0) {
    *flags |= CSA_DERR_BAD_META;
    return 0;
  }
  // 32-bit division when the position fits (a 64-bit one is a long scalar
  // sequence)
  int64_t v = pos < (int64_t)0x7FFFFFFF ? (int64_t)((uint32_t)pos / (uint32_t)ratio) : pos / ratio;
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

// Candidate lists of the top-k, written by the indexer epilogue (or by
// score_cands_kernel for caller-given scores) and read by the select.  A
// token's blocks are cut into groups of consecutive blocks: one indexer
// wave's blocks, or with merging one indexer workgroup's.  Group g of token t
// has list_len composite keys at cand[(t*groups_per_token + g)*list_len],
// zero-padded, and a bound gcut[t*groups_per_token + g] that
// is >= the key of every block of the group missing from the list (0: the
// list holds every block of the group).
constexpr int kIndexWaves = 8;      // waves per indexer workgroup
constexpr int kMergeMaxWaveM = 8;   // merged waves' lists fit one wave: kIndexWaves * 8 = 64
constexpr int kMergedLen = 16;      // keys per merged list
constexpr int kMergeScratch = 2 * kMergedLen;  // LDS words per wave the merge needs
struct CandArgs {
  uint64_t* cand; uint64_t* gcut;
  int wave_m;            // keys each wave keeps of its own blocks
  int merge;             // 1: a group is a workgroup; its waves' lists are merged
  int list_len;          // keys per group list
  int groups_per_token;
};

// Publishes a wave's candidate list: lane r < wave_m holds the wave's r-th
// largest composite key (zero past its valid blocks) and n_ok counts the
// wave's valid blocks.  Lists are stored in ascending block order, zero keys
// last, so that the select can list its selection in block order from slot
// positions.  Without merging the list is its group's list and the
// group bound is the list's last key when the wave has more valid blocks.
// With merging every wave of the workgroup calls this (it holds two
// barriers): each wave's list and bound go to LDS (wave w's kMergeMaxWaveM + 1
// words at lds + w*lds_stride, lds_stride >= kMergeScratch); every wave ranks
// its own keys among all kIndexWaves*kMergeMaxWaveM of them, and the keys of
// rank below list_len go to LDS by rank, from where wave 0 stores them.  A block missing from the merged list is either
// below the largest key left out of it, or missing from its wave's list and
// so below that wave's last key; the bound is the larger of those.
__device__ __forceinline__ void cand_publish(uint64_t val, uint32_t n_ok, const CandArgs& ca,
                                             int64_t t, int64_t wave_in_token,
                                             int64_t wg_in_token, uint64_t* lds,
                                             int lds_stride) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = ca.wave_m;
  const uint64_t wlast = readlane_u64(val, m - 1);
  const uint64_t wbound = n_ok > (uint32_t)m ? wlast : 0ull;
  if (!ca.merge) {
    const int64_t g = t * ca.groups_per_token + wave_in_token;
    // block order: the nonzero keys are lanes 0..nnz-1
    const uint32_t blk = ~(uint32_t)val;
    const int nnz = __popcll(__ballot(lane < m && val != 0ull));
    uint32_t pos = 0;
    for (int j = 0; j < nnz; ++j) pos += (uint32_t)__builtin_amdgcn_readlane((int)blk, j) < blk ? 1u : 0u;
    if (lane >= nnz) pos = (uint32_t)lane;
    if (lane < m) ca.cand[g * ca.list_len + pos] = val;
    if (lane == 0) ca.gcut[g] = wbound;
    return;
  }
  static_assert(kIndexWaves == 8 && kMergeMaxWaveM == 8, "one 8-lane group per listed key");
  uint64_t* mine = lds + wave * lds_stride;
  uint64_t* tmp = lds + kMergedLen;                // wave 0's region past its list: kept keys by rank
  uint64_t* cut_slot = lds + kMergeMaxWaveM + 1;   // ... and the largest key left out
  if (lane < kMergeMaxWaveM) mine[lane] = lane < m ? val : 0ull;
  if (lane == 0) mine[kMergeMaxWaveM] = wbound;
  if (wave == 0 && lane == 0) *cut_slot = 0ull;
  __syncthreads();
  // Key e = lane / 8 of this wave's list: lane c = lane % 8 of its 8-lane
  // group counts the larger keys (and the nonzero keys) among wave c's
  // slots; the group's sums are the key's rank (keys are unique where
  // nonzero) and the number of nonzero keys in all the lists.
  const uint64_t key = mine[lane >> 3];
  const uint64_t* other = lds + (lane & 7) * lds_stride;
  uint32_t above = 0, nz = 0;
#pragma unroll
  for (int e = 0; e < kMergeMaxWaveM; ++e) {
    const uint64_t o = other[e];
    above += o > key ? 1u : 0u;
    nz += o != 0ull ? 1u : 0u;
  }
  above += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)above, 0xB1, 0xF, 0xF, false);  // quad [1,0,3,2]
  above += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)above, 0x4E, 0xF, 0xF, false);  // quad [2,3,0,1]
  above += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)above, 0x141, 0xF, 0xF, false); // half-row mirror
  nz += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)nz, 0xB1, 0xF, 0xF, false);
  nz += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)nz, 0x4E, 0xF, 0xF, false);
  nz += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)nz, 0x141, 0xF, 0xF, false);
  if ((lane & 7) == 0 && key != 0ull) {
    if (above < (uint32_t)ca.list_len) tmp[above] = key;
    else if (above == (uint32_t)ca.list_len) *cut_slot = key;
  }
  __syncthreads();
  if (wave != 0) return;
  const int64_t g = t * ca.groups_per_token + wg_in_token;
  // the kept keys in key order are tmp[0 .. nnz_l); each list slot takes its
  // block-order position among them, zero keys last
  const uint32_t nnz_l = min(nz, (uint32_t)ca.list_len);
  if (lane < ca.list_len) {
    const uint64_t kl = (uint32_t)lane < nnz_l ? tmp[lane] : 0ull;
    const uint32_t bl = ~(uint32_t)kl;
    uint32_t pos = (uint32_t)lane;
    if ((uint32_t)lane < nnz_l) {
      pos = 0;
      for (uint32_t j = 0; j < nnz_l; ++j) pos += ~(uint32_t)tmp[j] < bl ? 1u : 0u;
    }
    ca.cand[g * ca.list_len + pos] = kl;
  }
  // the largest key left out of the list, and the waves' own bounds
  uint64_t cut = *cut_slot;
#pragma unroll
  for (int v = 0; v < kIndexWaves; ++v) {
    const uint64_t wc = lds[v * lds_stride + kMergeMaxWaveM];
    cut = wc > cut ? wc : cut;
  }
  if (lane == 0) ca.gcut[g] = cut;
}

// ---------------------------------------------------------------------------
// Internal launchers (host).  Arguments are validated by the C ABI layer.
// ---------------------------------------------------------------------------
// Keys the decode step's select holds: four register slots per thread of a
// 1024-thread workgroup (the fast select's capacity).
constexpr int kStepPool = 4096;
struct IndexScoreLaunch {
  const void* q_idx; const float* w; const void* k_idx; int64_t k_rows;  // bf16, or E4M3 codes
  int e4m3;                                  // 1: q_idx/k_idx are E4M3 codes scaled by
  const float* q_scale; const float* k_scale;  // q_scale [T, n_ih] and k_scale [k_rows]
  const int64_t* pos; const int64_t* seq_kv; const int32_t* n_comp;
  int T, n_ih, ihd, ratio;
  float* scores; int64_t ld;
  CandArgs cand;    // cand.cand == nullptr: no candidate lists
  uint32_t* err;
  int one_seq;      // 1: every token's key rows start at the same seq_kv
};
// Tokens per workgroup of the GEMM form of the indexer (one wave a token);
// the workgroup reads the key rows of its first token for all of them.
constexpr int kGemmTokens = 8;
// Whether launch_index_score takes the GEMM form for these arguments.
bool gemm_indexer(const IndexScoreLaunch& a);
struct IndexPlan {
  int tiles_per_wave, wgs_per_token;
  int waves_per_token() const { return wgs_per_token * kIndexWaves; }
  int blocks_per_wave() const { return 32 * tiles_per_wave; }
};
IndexPlan plan_index(int T, int64_t ld);
hipError_t launch_index_score(const IndexScoreLaunch& a, hipStream_t s);
// bf16 rescoring of candidate blocks (the E4M3 prefilter's): for token t and
// j < count[t] (<= C), key[t*C + j] is the composite key of block
// idx[t*C + j] with its bf16 indexer score; zero for count[t] <= j < C;
// gcut[t] = 0, so that key[t*C ..] reads as one complete candidate list.
struct RescoreLaunch {
  const uint16_t* q_idx; const float* w; const uint16_t* k_idx; const int64_t* seq_kv;
  const int32_t* idx; const int32_t* count;
  int T, n_ih, ihd, C;
  uint64_t* key; uint64_t* gcut;
};
hipError_t launch_rescore(const RescoreLaunch& a, hipStream_t s);
// The prefilter's select (S with top_k = C, whose idx and count it does not
// write) fused with the rescore of its candidates: one launch instead of
// launch_step_select + launch_rescore, for up to 64 indexer heads and ihd 64
// or 128 (prefilter_rescore_fits).
bool prefilter_rescore_fits(const RescoreLaunch& a);
struct SelectLaunch;
hipError_t launch_prefilter_rescore(const SelectLaunch& sl, const RescoreLaunch& a, int T,
                                    hipStream_t s);
// The producer side of one decode step (produce.hip): both compressors'
// projections of the new tokens, the ring of recent projections, the
// sliding-window append and, at block ends, the pooled compressed rows.
struct CompressLaunch {
  const uint16_t* x; int T, H;
  const uint16_t* w_kv; int hd; const uint16_t* w_ik; int ihd;
  const int32_t* seq; const int64_t* pos; int S, ratio, window;
  float* ring; uint16_t* swa; int32_t* swa_head; int32_t* swa_len;
  uint16_t* comp_kv; uint16_t* k_idx; const int64_t* seq_kv; int32_t* n_comp; int64_t comp_rows;
  void* ws; uint32_t* err;
};
size_t compress_ws_bytes(int T, int H, int hd, int ihd);
hipError_t launch_compress_append(const CompressLaunch& c, hipStream_t s);

// Row quantisation to E4M3 with one power-of-two scale per row (quant.hip).
hipError_t launch_quant_e4m3(const uint16_t* src, int64_t rows, int d, uint8_t* codes,
                             float* scale, hipStream_t s);

// Top-k (see topk.hip).
constexpr int kPoolCap = 12288;   // keys the select workgroup holds in registers
constexpr int kMaxGroups = 2048;  // group bounds the select holds (two per thread)
struct TopkPlan {
  int waves_per_token, blocks_per_wave;  // indexer geometry
  int wave_m, merge;                     // see CandArgs
  int list_len;                          // keys per group list (0: no lists)
  int groups_per_token, blocks_per_group;
};
// pool: keys the select holds in registers (kPoolCap for the top-k kernel,
// kStepPool in the decode step)
TopkPlan plan_topk(int T, int64_t ld, int top_k, int pool);
struct TopkWs {
  uint64_t* cand;  // [T, groups_per_token, list_len]
  uint64_t* gcut;  // [T, groups_per_token]
  size_t bytes;
};
TopkWs topk_ws_layout(void* ws, int T, const TopkPlan& p);
CandArgs cand_args(const TopkPlan& p, const TopkWs& w);
int select_slots(const TopkPlan& p);  // register key slots per select thread: 4 or 12
hipError_t launch_score_cands(const float* scores, int64_t ld, const int64_t* pos,
                              const int32_t* n_comp, int T, int ratio, const TopkPlan& p,
                              const TopkWs& ws, uint32_t* err, hipStream_t s);
// seq_kv == nullptr: caller-given scores with no key buffer to check
hipError_t launch_topk_select(const float* scores, int64_t ld, const int64_t* pos,
                              const int32_t* n_comp, const int64_t* seq_kv, int64_t k_rows,
                              int T, int ratio, int top_k,
                              const TopkPlan& p, const TopkWs& ws, int32_t* idx,
                              int32_t* count, uint32_t* err, hipStream_t s);

struct GatherLaunch {
  const uint16_t* comp_kv; int64_t comp_rows; const int64_t* seq_kv;
  const int32_t* idx; const int32_t* count; int top_k;
  const uint16_t* swa; int64_t swa_rows; const int64_t* swa_row0; const int32_t* swa_len;
  int window, T, head_dim;
  uint16_t* all_kv; int32_t* n_kv; uint32_t* err;
};
hipError_t launch_gather(const GatherLaunch& a, hipStream_t s);

// Row set of each token: segment A then segment B.  Segment A is one of
//   * explicit: rows a_row0[t] .. +a_len[t] of kv_a;
//   * visibility (HCA): rows a_row0[t] .. +n_vis[t] (vis_pos != nullptr);
//   * gather (CSA decode step, sel_idx != nullptr): rows a_row0[t] + sel_idx[t, j]
//     for j < sel_cnt[t], also copied to copy_out[t, j] with the SWA rows after
//     them, and n_kv_out[t] = rows used.
struct AttendLaunch {
  const uint16_t* q; int T, n_heads, head_dim; float scale; const float* sink;
  const uint16_t* kv_a; int64_t a_rows; const int64_t* a_row0; const int32_t* a_len;
  int64_t a_stride;                       // a_row0 == nullptr: row0 = t*a_stride
  const int64_t* vis_pos; const int32_t* vis_ncomp; int vis_ratio;
  const int32_t* sel_idx; const int32_t* sel_cnt; int sel_stride;
  const uint16_t* kv_b; int64_t b_rows; const int64_t* b_row0; const int32_t* b_len;
  int b_cap;                              // gather mode: at most this many B rows
  uint16_t* copy_out; int64_t copy_stride; int32_t* n_kv_out;
  int max_rows;
  int split_tiles;                        // 64-row tiles per row split (0: planned for ~256 workgroups)
  uint16_t* out; float* lse;
  void* ws; uint32_t* err;
};
// Rows per split of the decode step's attention: one 64-row tile per
// workgroup, so that each fetches its rows in one round trip; the bf16 split
// partials of all splits are then about as large as the rows themselves.
constexpr int kStepSplitTiles = 1;
size_t attend_ws_bytes(int T, int n_heads, int head_dim, int max_rows, int split_tiles);
hipError_t launch_attend(const AttendLaunch& a, hipStream_t s);

// The decode step's top-k (S2) over the indexer's scores and candidate lists:
// either inside the attention kernel (select_attend_kernel: every workgroup of
// a token selects, then attends over its own share of the selected rows) or,
// for larger batches, in a select kernel of one workgroup per token followed
// by the gather-mode attention kernel.
struct SelectLaunch {
  const float* scores; int64_t ld; const int64_t* pos; const int32_t* n_comp;
  const int64_t* seq_kv; int64_t k_rows;  // the indexer's key range check
  int ratio, top_k;
  const uint64_t* cand; const uint64_t* gcut;
  int list_len, groups_per_token, blocks_per_group;
  int lists_complete;  // 1: the lists are the whole candidate set, for rows of any length
  int32_t* idx; int32_t* count;
  uint32_t* err;
  int row0_group;  // kGemmTokens after the GEMM indexer, else 0: see select_row0
};
// The key offset the select checks for token t.  After the GEMM indexer a
// token whose seq_kv differs from that of the first token of its workgroup
// was scored over no block (and raised BAD_META); -1 makes the select agree.
__device__ __forceinline__ int64_t select_row0(const SelectLaunch& sl, int t) {
  const int64_t r = sl.seq_kv[t];
  if (sl.row0_group > 0 && sl.seq_kv[t - t % sl.row0_group] != r) return -1;
  return r;
}
bool select_attend_fits(int T, int n_heads, int max_rows, int split_tiles);
// 64-row tiles per split of the decode step's attention: kStepSplitTiles when
// the select runs inside the attention kernel (small batches); otherwise as
// many as give about kStepTargetWgs workgroups (fewer, longer splits: less
// partial-output traffic for the combine).
constexpr int kStepTargetWgs = 256;
int step_split_tiles(int T, int n_heads, int max_rows);
hipError_t launch_select_attend(const SelectLaunch& s, const AttendLaunch& a, hipStream_t st);
hipError_t launch_step_select(const SelectLaunch& s, int T, hipStream_t st);

}  // namespace csa
