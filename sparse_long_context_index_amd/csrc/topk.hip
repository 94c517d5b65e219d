// S2 -- causal top-k over the indexer scores (post-probe audit, F3:
// tk = min(top_k, n_comp) and a top-k over the scores; PART A, suspect 3: only
// blocks strictly before the query's own block are candidates).
//
// Exact radix select on an order-preserving uint32 key of each fp32 score,
// extended by the complemented block index so that every element has a unique
// 64-bit key and equal scores resolve to the lower block index:
//
//   pass 1 (multi-workgroup, usually fused into the indexer epilogue):
//       histogram of the top kHistBits key bits per token;
//   pass 2 (multi-workgroup, this file): every workgroup finds the threshold
//       bin b* from the histogram, streams its chunk of scores once, appends
//       blocks above b* straight into idx and blocks inside b* into a small
//       candidate list;
//   pass 3 (the last workgroup of each token, found with an atomic ticket):
//       resolves the remaining key and index bits of the candidates with 8-bit
//       LDS radix passes, then writes the selected blocks in ascending order by
//       scanning an LDS bitmap of the visible range.
//
// The candidate list holds the blocks whose score shares the threshold bin --
// a few hundred to a few thousand for continuous scores; it lives in LDS when
// it fits and is read from the workspace otherwise (e.g. all scores equal).
#include "csa_common.h"

namespace csa {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 8;
constexpr int kChunk = kThreads * kPerThread;  // scores per filter workgroup
constexpr int kCandCap = 4096;                 // candidates staged in LDS
constexpr int kMaxTopk = 2048;
constexpr int kBitmapWords = 8192;             // 262,144 blocks per emission sweep

// Block-wide search in a histogram distributed over the workgroup: thread i
// owns bins [i*BPT, i*BPT+BPT) in `c`.  Finds the bin b with
//   (items in bins > b) < need <= (items in bins >= b)
// and returns b and the count above it.  Requires 1 <= need <= total.
template <int BPT>
__device__ void find_threshold_bin(const uint32_t (&c)[BPT], uint32_t need,
                                   uint32_t* scratch, uint32_t& bin, uint32_t& above) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t tot = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) tot += c[i];
  uint32_t x = tot;  // inclusive suffix sum within the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_down(x, d);
    if (lane + d < 64) x += y;
  }
  if (lane == 0) scratch[wave] = x;
  __syncthreads();
  uint32_t acc = x - tot;
  for (int wv = wave + 1; wv < kThreads / 64; ++wv) acc += scratch[wv];
#pragma unroll
  for (int i = BPT - 1; i >= 0; --i) {
    if (acc < need && acc + c[i] >= need) {
      scratch[4] = (uint32_t)(tid * BPT + i);
      scratch[5] = acc;
    }
    acc += c[i];
  }
  __syncthreads();
  bin = scratch[4];
  above = scratch[5];
  __syncthreads();
}

// Exclusive prefix sum over the workgroup (ascending thread order).
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* scratch, uint32_t& total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  uint32_t base = 0;
  total = 0;
  for (int wv = 0; wv < kThreads / 64; ++wv) {
    if (wv < wave) base += scratch[wv];
    total += scratch[wv];
  }
  __syncthreads();
  return base + x - v;
}

// Wave-aggregated append: one atomic per wave for all lanes with `pred`.
__device__ __forceinline__ uint32_t wave_append(bool pred, uint32_t* counter) {
  const uint64_t mask = __ballot(pred);
  if (mask == 0) return 0u;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((unsigned long long)mask) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(mask));
  base = __shfl(base, leader);
  const uint64_t lower = lane == 0 ? 0ull : (mask & (~0ull >> (64 - lane)));
  return base + (uint32_t)__popcll(lower);
}

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// Stand-alone pass 1 (when the scores come from the caller).
__global__ __launch_bounds__(256) void score_hist_kernel(
    const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ pos,
    const int32_t* __restrict__ n_comp, int ratio, uint32_t* __restrict__ hist,
    uint32_t* __restrict__ err) {
  __shared__ uint32_t lh[kHistBins];
  const int t = blockIdx.y;
  uint32_t flags = 0;
  int64_t n_vis = visible_count(pos[t], ratio, n_comp[t], &flags);
  if (n_vis > ld) {
    flags |= CSA_DERR_VIS_OVER_LD;
    n_vis = ld;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) report(err, flags);
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  if (c0 >= n_vis) return;
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) lh[i] = 0u;
  __syncthreads();
  const float* row = scores + (int64_t)t * ld;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int64_t s = c0 + i * kThreads + threadIdx.x;
    if (s < n_vis) atomicAdd(&lh[score_key(row[s]) >> (32 - kHistBits)], 1u);
  }
  __syncthreads();
  uint32_t* ht = hist + (int64_t)t * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) {
    const uint32_t v = lh[i];
    if (v != 0u) atomicAdd(ht + i, v);
  }
}

struct SelectShared {
  uint32_t scratch[16];
  uint32_t last;
  uint32_t dh[256];
  uint32_t above_list[kMaxTopk];
  uint64_t cand[kCandCap];
  uint32_t bitmap[kBitmapWords];
};

__global__ __launch_bounds__(256) void topk_select_kernel(
    const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ pos,
    const int32_t* __restrict__ n_comp, int ratio, int top_k, int32_t* __restrict__ idx,
    int32_t* __restrict__ count, const uint32_t* __restrict__ hist_all,
    uint32_t* __restrict__ ctr_all, uint64_t* __restrict__ cand_all,
    uint32_t* __restrict__ err) {
  __shared__ SelectShared sh;
  const int tid = threadIdx.x;
  const int t = blockIdx.y;
  uint32_t flags = 0;
  int64_t n_vis = visible_count(pos[t], ratio, n_comp[t], &flags);
  if (n_vis > ld) n_vis = ld;  // reported by the histogram pass
  const uint32_t k_eff = (uint32_t)(n_vis < (int64_t)top_k ? n_vis : (int64_t)top_k);
  const uint32_t* hist = hist_all + (int64_t)t * kHistBins;
  uint32_t* ctr = ctr_all + (int64_t)t * 4;
  uint64_t* cand = cand_all + (int64_t)t * ld;
  int32_t* out = idx + (int64_t)t * top_k;

  // ---- threshold bin from the histogram (every workgroup) ----
  uint32_t bstar = 0, above = 0, total = 0;
  if (k_eff > 0) {
    uint32_t c[kHistBins / kThreads];
    const u32x4* hv = reinterpret_cast<const u32x4*>(hist + tid * (kHistBins / kThreads));
#pragma unroll
    for (int j = 0; j < kHistBins / kThreads / 4; ++j) {
      const u32x4 v = hv[j];
      c[4 * j + 0] = v.x; c[4 * j + 1] = v.y; c[4 * j + 2] = v.z; c[4 * j + 3] = v.w;
    }
    uint32_t tot = 0;
#pragma unroll
    for (int j = 0; j < kHistBins / kThreads; ++j) tot += c[j];
    uint32_t sum_all;
    block_excl_scan(tot, sh.scratch, sum_all);
    if (sum_all >= k_eff) {
      find_threshold_bin<kHistBins / kThreads>(c, k_eff, sh.scratch, bstar, above);
      total = sum_all;
    } else {
      total = 0;  // histogram disagrees with the scores: nothing selected
    }
  }

  // ---- filter this workgroup's chunk ----
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  if (total > 0 && c0 < n_vis) {
    const float* row = scores + (int64_t)t * ld;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int64_t s = c0 + i * kThreads + tid;
      const bool valid = s < n_vis;
      const uint32_t key = valid ? score_key(row[s]) : 0u;
      const uint32_t b = key >> (32 - kHistBits);
      const bool up = valid && b > bstar;
      const bool in = valid && b == bstar;
      const uint32_t sa = wave_append(up, ctr + 0);
      if (up && sa < (uint32_t)top_k) out[sa] = (int32_t)s;
      const uint32_t sc = wave_append(in, ctr + 1);
      if (in && sc < (uint64_t)ld) cand[sc] = ((uint64_t)key << 32) | (uint32_t)(~(uint32_t)s);
    }
  }

  // ---- the last workgroup of this token finishes ----
  fence_release();
  __syncthreads();
  if (tid == 0) sh.last = (atomicAdd(ctr + 2, 1u) == gridDim.x - 1) ? 1u : 0u;
  __syncthreads();
  if (sh.last == 0u) return;
  fence_acquire();

  if (total == 0) {
    if (k_eff > 0) report(err, CSA_DERR_BAD_META);
    for (int i = tid; i < top_k; i += kThreads) out[i] = -1;
    if (tid == 0) count[t] = 0;
    return;
  }

  const uint32_t n_above = min(__hip_atomic_load(ctr + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), (uint32_t)top_k);
  const uint64_t n_cand64 = __hip_atomic_load(ctr + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t n_cand = (uint32_t)(n_cand64 < (uint64_t)ld ? n_cand64 : (uint64_t)ld);
  uint32_t need = k_eff - min(n_above, k_eff);
  if (n_above != above || need > n_cand) {
    report(err, CSA_DERR_BAD_META);
    need = min(need, n_cand);
  }

  for (uint32_t i = tid; i < n_above; i += kThreads) sh.above_list[i] = (uint32_t)out[i];
  const bool in_lds = n_cand <= (uint32_t)kCandCap;
  if (in_lds)
    for (uint32_t i = tid; i < n_cand; i += kThreads) sh.cand[i] = cand[i];
  const uint64_t* cs = in_lds ? sh.cand : cand;
  __syncthreads();

  // ---- resolve the remaining key bits and the index among candidates ----
  // Selected candidates are those with (key64 >> shift) >= prefix.
  bool take_all = need == n_cand;
  uint64_t prefix = bstar;
  int shift = 64 - kHistBits;
  uint32_t need_rem = need;
  for (int pass = 0; !take_all && pass < 8 && need_rem > 0; ++pass) {
    const int nb = shift < 8 ? shift : 8;
    const int nshift = shift - nb;
    const uint32_t mask = (1u << nb) - 1u;
    sh.dh[tid] = 0u;
    __syncthreads();
    for (uint32_t i = tid; i < n_cand; i += kThreads) {
      const uint64_t c = cs[i];
      if ((c >> shift) == prefix) atomicAdd(&sh.dh[(uint32_t)(c >> nshift) & mask], 1u);
    }
    __syncthreads();
    uint32_t cnt[1] = {sh.dh[tid]};
    uint32_t d, above_d;
    find_threshold_bin<1>(cnt, need_rem, sh.scratch, d, above_d);
    const uint32_t in_bin = sh.dh[d];
    need_rem -= above_d;
    prefix = (prefix << nb) | d;
    shift = nshift;
    __syncthreads();
    if (in_bin == need_rem) break;
  }
  const bool none = need == 0;

  // ---- emit selected blocks in ascending order ----
  uint32_t emitted = 0;
  const int64_t span = (int64_t)kBitmapWords * 32;
  for (int64_t base = 0; base < n_vis; base += span) {
    const int64_t len = min(span, n_vis - base);
    const int words = (int)((len + 31) / 32);
    for (int i = tid; i < words; i += kThreads) sh.bitmap[i] = 0u;
    __syncthreads();
    for (uint32_t i = tid; i < n_above; i += kThreads) {
      const int64_t s = (int64_t)sh.above_list[i] - base;
      if (s >= 0 && s < len) atomicOr(&sh.bitmap[s >> 5], 1u << (s & 31));
    }
    if (!none) {
      for (uint32_t i = tid; i < n_cand; i += kThreads) {
        const uint64_t c = cs[i];
        const bool sel = take_all || (shift == 0 ? c >= prefix : (c >> shift) >= prefix);
        if (sel) {
          const int64_t s = (int64_t)(~(uint32_t)c) - base;
          if (s >= 0 && s < len) atomicOr(&sh.bitmap[s >> 5], 1u << (s & 31));
        }
      }
    }
    __syncthreads();
    const int per = (words + kThreads - 1) / kThreads;
    const int w0 = tid * per;
    uint32_t mine = 0;
    for (int k = 0; k < per; ++k)
      if (w0 + k < words) mine += (uint32_t)__popc(sh.bitmap[w0 + k]);
    uint32_t sweep_total;
    uint32_t o = emitted + block_excl_scan(mine, sh.scratch, sweep_total);
    for (int k = 0; k < per; ++k) {
      if (w0 + k >= words) break;
      uint32_t bits = sh.bitmap[w0 + k];
      while (bits) {
        const int b = __ffs(bits) - 1;
        bits &= bits - 1u;
        if (o < (uint32_t)top_k) out[o] = (int32_t)(base + (int64_t)(w0 + k) * 32 + b);
        ++o;
      }
    }
    emitted += sweep_total;
    __syncthreads();
  }
  if (emitted > (uint32_t)top_k) emitted = (uint32_t)top_k;
  for (uint32_t i = emitted + tid; i < (uint32_t)top_k; i += kThreads) out[i] = -1;
  if (tid == 0) count[t] = (int32_t)emitted;
}

}  // namespace

size_t topk_ws_bytes(int T, int64_t ld) {
  size_t b = (size_t)T * kHistBins * 4;
  b = (b + 255) & ~(size_t)255;
  b += (size_t)T * 4 * 4;
  b = (b + 255) & ~(size_t)255;
  b += (size_t)T * (size_t)ld * 8;
  return (b + 255) & ~(size_t)255;
}

TopkWs topk_ws_carve(void* ws, int T, int64_t ld) {
  char* p = static_cast<char*>(ws);
  TopkWs w;
  w.hist = reinterpret_cast<uint32_t*>(p);
  size_t off = ((size_t)T * kHistBins * 4 + 255) & ~(size_t)255;
  w.ctr = reinterpret_cast<uint32_t*>(p + off);
  off += ((size_t)T * 16 + 255) & ~(size_t)255;
  w.cand = reinterpret_cast<uint64_t*>(p + off);
  return w;
}

hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_score_hist(const float* scores, int64_t ld, const int64_t* pos,
                             const int32_t* n_comp, int T, int ratio, uint32_t* hist,
                             uint32_t* err, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)((ld + kChunk - 1) / kChunk), (unsigned)T);
  hipLaunchKernelGGL(score_hist_kernel, grid, dim3(kThreads), 0, s, scores, ld, pos, n_comp,
                     ratio, hist, err);
  return hipGetLastError();
}

hipError_t launch_topk_select(const float* scores, int64_t ld, const int64_t* pos,
                              const int32_t* n_comp, int T, int ratio, int top_k,
                              int32_t* idx, int32_t* count, const TopkWs& ws, uint32_t* err,
                              hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)((ld + kChunk - 1) / kChunk), (unsigned)T);
  hipLaunchKernelGGL(topk_select_kernel, grid, dim3(kThreads), 0, s, scores, ld, pos, n_comp,
                     ratio, top_k, idx, count, ws.hist, ws.ctr, ws.cand, err);
  return hipGetLastError();
}

}  // namespace csa
