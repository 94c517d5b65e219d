// S2 -- causal top-k over the indexer scores (post-probe audit, F3:
// tk = min(top_k, n_comp) and a top-k over the scores; PART A, suspect 3: only
// blocks strictly before the query's own block are candidates).
//
// Every block s gets the composite key (score key << 32 | ~s): unique, larger
// score first, then lower block index, so the selected set is exactly the
// k_eff largest keys and ties at the k-th score go to the lower index.
//
// One 1024-thread workgroup per token selects from a key set held in
// registers (12 keys per thread) plus an LDS overflow area:
//   * n_vis <= kPoolCap: the keys are every visible block (exact, direct);
//   * otherwise the keys are the candidate lists -- the top-m keys of every
//     group of blocks handled by one indexer wave, written by the indexer
//     epilogue (or score_cands_kernel).  Let T1 be the k_eff-th largest
//     listed key.  A group whose list is full (it has more than m blocks) and
//     whose m-th key is >= T1 may hold unlisted blocks above T1; its unlisted
//     blocks are added and the threshold is found again.  Every other
//     unlisted block is below its group's m-th key < T1, below k_eff listed
//     keys, so the result is exact.  At most k_eff/m groups can qualify (each
//     puts m keys >= T1 into the set, and only k_eff keys are >= T1);
//   * if the extra blocks would not fit, the select runs over the token's
//     scores in global memory (slow, exact; only for adversarial layouts).
//
// The k-th key is found in one histogram pass over 2048 bins laid linearly
// over [min, max] of the scores (a monotone map, so bins are ordered), then an
// exact rank among the few keys of the threshold bin.  Linear bins spread the
// keys, which keeps LDS atomics free of same-address conflicts; where the
// threshold bin is crowded (ties, clustered values) an exact 8-bit radix
// select over the composite keys takes over.  The selection is written in
// ascending block order by scanning an LDS bitmap of the visible range.
//
// No global atomics: cross-workgroup communication is plain stores plus the
// kernel boundary.
#include <math.h>

#include "csa_common.h"

namespace csa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int KPT = kPoolCap / kThreads;  // register keys per thread
constexpr int kBins = 2 * kThreads;       // linear bins, two per thread
constexpr int kXCap = 4096;               // keys of re-scanned groups (LDS)
constexpr int kListCap = 1024;            // threshold-bin keys ranked exactly
constexpr int kMaxOv = 512;               // groups re-scanned before falling back
constexpr int kBitmapWords = 8192;        // 262,144 blocks per emission sweep
constexpr int kMaxTopK = 2048;
static_assert(KPT * kThreads == kPoolCap, "pool must split evenly");
static_assert(kBitmapWords % (8 * kThreads) == 0, "8 bitmap words per thread");

struct SelShared {
  uint32_t bitmap[kBitmapWords];
  uint64_t xk[kXCap];
  uint64_t list[kListCap];
  uint32_t hist[kBins];
  uint32_t ov_w[kMaxOv];
  uint32_t ov_nv[kMaxOv];
  uint64_t ov_cut[kMaxOv];
  int32_t outl[kMaxTopK];                 // the selection, ascending, before the output copy
  uint32_t scratch[2 * kWaves + 8];
  uint32_t rc[kWaves];                    // per-wave count / range of kth_key
  float rlo[kWaves], rhi[kWaves];
  uint32_t fb_w[kWaves];                  // per-wave bin totals of kth_key
  uint32_t fb_bin, fb_above;
  uint64_t red64[2 * kWaves];
  uint64_t thr;
  uint32_t n_x, n_ov, n_list;
};

// Score of a composite key (inverse of score_key on the high word).
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t u = (uint32_t)(key >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Linear bin of a key's score: non-decreasing in the key for s > 0 (the
// subtraction, product, clamp and truncation are all monotone).
__device__ __forceinline__ uint32_t key_bin(uint64_t key, float lo, float s) {
  const float x = (key_value(key) - lo) * s;
  return (uint32_t)fminf(fmaxf(x, 0.0f), (float)(kBins - 1));
}

// Appends v (where p) to list[0..cap) at *n; one LDS atomic per wave.
__device__ __forceinline__ void wave_append(bool p, uint64_t v, uint64_t* list, uint32_t* n,
                                            uint32_t cap) {
  const uint64_t mask = __ballot(p);
  if (mask == 0ull) return;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((unsigned long long)mask) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(n, (uint32_t)__popcll(mask));
  base = __shfl(base, leader);
  if (p) {
    const uint32_t o = base + (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
    if (o < cap) list[o] = v;
  }
}

// Block-wide search in a histogram distributed over the workgroup: thread i
// owns bins [i*BPT, i*BPT+BPT) in `c`.  Finds the bin b with
//   (items in bins > b) < need <= (items in bins >= b)
// and returns b and the count above it.  Requires 1 <= need <= total.
template <int BPT>
__device__ __forceinline__ void find_threshold_bin(const uint32_t (&c)[BPT], uint32_t need,
                                                   uint32_t* scratch, uint32_t& bin,
                                                   uint32_t& above) {
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
  for (int wv = wave + 1; wv < kWaves; ++wv) acc += scratch[wv];
#pragma unroll
  for (int i = BPT - 1; i >= 0; --i) {
    if (acc < need && acc + c[i] >= need) {
      scratch[kWaves] = (uint32_t)(tid * BPT + i);
      scratch[kWaves + 1] = acc;
    }
    acc += c[i];
  }
  __syncthreads();
  bin = scratch[kWaves];
  above = scratch[kWaves + 1];
  __syncthreads();
}

// Exclusive prefix sum over the workgroup (ascending thread order).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* scratch,
                                                    uint32_t& total) {
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
  for (int wv = 0; wv < kWaves; ++wv) {
    if (wv < wave) base += scratch[wv];
    total += scratch[wv];
  }
  __syncthreads();
  return base + x - v;
}

__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* scratch) {
  uint32_t total;
  block_excl_scan(v, scratch, total);
  return total;
}

// Block-wide min over nonzero keys and max of 64-bit keys.
__device__ __forceinline__ void block_minmax64(uint64_t lo, uint64_t hi, SelShared& sh,
                                               uint64_t& blo, uint64_t& bhi) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t a = __shfl_xor((unsigned long long)lo, off);
    const uint64_t b = __shfl_xor((unsigned long long)hi, off);
    lo = a < lo ? a : lo;
    hi = b > hi ? b : hi;
  }
  if (lane == 0) {
    sh.red64[wave] = lo;
    sh.red64[kWaves + wave] = hi;
  }
  __syncthreads();
  blo = sh.red64[0];
  bhi = sh.red64[kWaves];
  for (int w = 1; w < kWaves; ++w) {
    blo = sh.red64[w] < blo ? sh.red64[w] : blo;
    bhi = sh.red64[kWaves + w] > bhi ? sh.red64[kWaves + w] : bhi;
  }
  __syncthreads();
}

// Exact k-th largest of the nonzero keys get(0..n) by 8-bit radix passes over
// the 64-bit keys, starting below the leading bits that all of them share and
// stopping once the threshold bin holds exactly the remaining need.  Requires
// at least k nonzero keys.  `get(j)` may return zero for an empty slot.
template <class Get>
__device__ uint64_t radix_kth(Get get, uint32_t n, uint32_t k, SelShared& sh) {
  const int tid = threadIdx.x;
  uint64_t lo = ~0ull, hi = 0ull;
  for (uint32_t j = tid; j < n; j += kThreads) {
    const uint64_t c = get(j);
    if (c != 0ull && c < lo) lo = c;
    if (c > hi) hi = c;
  }
  uint64_t blo, bhi;
  block_minmax64(lo, hi, sh, blo, bhi);
  if (blo >= bhi) return bhi;  // a single nonzero key
  const int top = 63 - __clzll((long long)(blo ^ bhi));  // highest differing bit
  int shift = top + 1;
  uint64_t prefix = shift >= 64 ? 0ull : (bhi >> shift);
  uint32_t need = k;
  for (int pass = 0; pass < 9 && shift > 0; ++pass) {
    const int nb = shift < 8 ? shift : 8;
    const int nshift = shift - nb;
    const uint32_t mask = (1u << nb) - 1u;
    if (tid < 256) sh.hist[tid] = 0u;
    __syncthreads();
#pragma unroll 4
    for (uint32_t j = tid; j < n; j += kThreads) {
      const uint64_t c = get(j);
      if (c != 0ull && (shift >= 64 || (c >> shift) == prefix))
        atomicAdd(&sh.hist[(uint32_t)(c >> nshift) & mask], 1u);
    }
    __syncthreads();
    uint32_t cnt[1] = {tid < 256 ? sh.hist[tid] : 0u};
    uint32_t d, above;
    find_threshold_bin<1>(cnt, need, sh.scratch, d, above);
    const uint32_t in_bin = sh.hist[d];
    need -= above;
    prefix = (shift >= 64 ? 0ull : (prefix << nb)) | d;
    shift = nshift;
    __syncthreads();
    if (in_bin == need) break;
  }
  return prefix << shift;
}

// The k-th largest of the nonzero keys in key[0..KPT) of every thread and in
// sh.xk[0..n_x); 0 when fewer than k keys are nonzero.  1 <= k.  Each phase
// writes its own LDS slots, so six barriers separate the phases (a barrier
// between a phase's reads and the next call's writes always intervenes).
__device__ __forceinline__ uint64_t kth_key(const uint64_t (&key)[KPT], uint32_t n_x, uint32_t k,
                                            SelShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // ---- count and score range of the nonzero keys; clear the histogram ----
  uint32_t nz = 0;
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (key[i] != 0ull) {
      const float v = key_value(key[i]);
      ++nz;
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
    }
  }
  for (uint32_t j = tid; j < n_x; j += kThreads) {
    const float v = key_value(sh.xk[j]);
    ++nz;
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  for (int b = tid; b < kBins; b += kThreads) sh.hist[b] = 0u;
  if (tid == 0) sh.n_list = 0u;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    nz += __shfl_xor(nz, off);
    lo = fminf(lo, __shfl_xor(lo, off));
    hi = fmaxf(hi, __shfl_xor(hi, off));
  }
  if (lane == 0) {
    sh.rc[wave] = nz;
    sh.rlo[wave] = lo;
    sh.rhi[wave] = hi;
  }
  __syncthreads();
  uint32_t n_nz = 0;
  float blo = INFINITY, bhi = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    n_nz += sh.rc[w];
    blo = fminf(blo, sh.rlo[w]);
    bhi = fmaxf(bhi, sh.rhi[w]);
  }
  if (n_nz < k) return 0ull;
  const float s = (float)kBins / (bhi - blo);  // +inf when all scores are equal
  bool crowded = !(s > 0.0f && s < INFINITY);
  if (!crowded) {
    // ---- histogram of the linear bins ----
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (key[i] != 0ull) atomicAdd(&sh.hist[key_bin(key[i], blo, s)], 1u);
    for (uint32_t j = tid; j < n_x; j += kThreads)
      atomicAdd(&sh.hist[key_bin(sh.xk[j], blo, s)], 1u);
    __syncthreads();
    // ---- the bin b with (keys in bins > b) < k <= (keys in bins >= b);
    // thread i owns bins 2i, 2i+1 ----
    const uint32_t c0 = sh.hist[2 * tid], c1 = sh.hist[2 * tid + 1];
    const uint32_t tot = c0 + c1;
    uint32_t x = tot;  // inclusive suffix sum within the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t y = __shfl_down(x, d);
      if (lane + d < 64) x += y;
    }
    if (lane == 0) sh.fb_w[wave] = x;
    __syncthreads();
    uint32_t acc = x - tot;
    for (int wv = wave + 1; wv < kWaves; ++wv) acc += sh.fb_w[wv];
    if (acc < k && acc + c1 >= k) {
      sh.fb_bin = 2u * tid + 1u;
      sh.fb_above = acc;
    } else if (acc + c1 < k && acc + c1 + c0 >= k) {
      sh.fb_bin = 2u * tid;
      sh.fb_above = acc + c1;
    }
    __syncthreads();
    const uint32_t b = sh.fb_bin;
    const uint32_t need = k - sh.fb_above;
    const uint32_t in_bin = sh.hist[b];
    crowded = in_bin > (uint32_t)kListCap;
    if (!crowded) {
      // ---- exact rank among the keys of bin b ----
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        wave_append(key[i] != 0ull && key_bin(key[i], blo, s) == b, key[i], sh.list, &sh.n_list,
                    kListCap);
      for (uint32_t j0 = 0; j0 < n_x; j0 += kThreads) {
        const uint32_t j = j0 + tid;
        const uint64_t v = j < n_x ? sh.xk[j] : 0ull;
        wave_append(j < n_x && key_bin(v, blo, s) == b, v, sh.list, &sh.n_list, kListCap);
      }
      __syncthreads();
      if ((uint32_t)tid < in_bin) {
        const uint64_t v = sh.list[tid];
        uint32_t r = 0;
        for (uint32_t j = 0; j < in_bin; ++j) r += sh.list[j] > v ? 1u : 0u;
        if (r == need - 1u) sh.thr = v;
      }
      __syncthreads();
      return sh.thr;
    }
  }
  // ties or tightly clustered scores: exact radix select over all the keys
  auto get = [&](uint32_t j) -> uint64_t {
    if (j < (uint32_t)kPoolCap) {
      // register slot of j is (thread j % kThreads, index j / kThreads); only
      // the calling thread's own slots are ever asked for
      const int i = (int)(j / kThreads);
      uint64_t v = 0ull;
#pragma unroll
      for (int q = 0; q < KPT; ++q)
        if (q == i) v = key[q];
      return v;
    }
    return sh.xk[j - kPoolCap];
  };
  return radix_kth(get, (uint32_t)kPoolCap + n_x, k, sh);
}

// Marks {block of key : key >= thr, key != 0} of the keys in registers, the
// LDS extras and (if any) the row, in the bitmap (already clear on entry),
// then lists them in ascending block order at sh.outl[0..top_k); returns how
// many were marked.
template <class Mark>
__device__ __forceinline__ uint32_t emit_bitmap(Mark mark, int64_t n_vis, int top_k,
                                                SelShared& sh) {
  const int tid = threadIdx.x;
  uint32_t emitted = 0;
  const int64_t span = (int64_t)kBitmapWords * 32;
  constexpr int WPT = kBitmapWords / kThreads;  // bitmap words per thread
  u32x4* bm4 = reinterpret_cast<u32x4*>(sh.bitmap);
  for (int64_t base = 0; base < n_vis; base += span) {
    const int64_t len = min(span, n_vis - base);
    if (base > 0) {
      for (int i = tid; i < kBitmapWords / 4; i += kThreads) bm4[i] = u32x4{0u, 0u, 0u, 0u};
      __syncthreads();
    }
    mark(base, len);
    __syncthreads();
    uint32_t wv[WPT];
    uint32_t mine = 0;
#pragma unroll
    for (int q = 0; q < WPT / 4; ++q) {
      const u32x4 x = bm4[tid * (WPT / 4) + q];
      wv[4 * q + 0] = x.x;
      wv[4 * q + 1] = x.y;
      wv[4 * q + 2] = x.z;
      wv[4 * q + 3] = x.w;
    }
#pragma unroll
    for (int q = 0; q < WPT; ++q) mine += (uint32_t)__popc(wv[q]);
    uint32_t sweep_total;
    uint32_t o = emitted + block_excl_scan(mine, sh.scratch, sweep_total);
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
      uint32_t bits = wv[q];
      while (bits) {
        const int bb = __ffs(bits) - 1;
        bits &= bits - 1u;
        if (o < (uint32_t)top_k) sh.outl[o] = (int32_t)(base + (int64_t)(tid * WPT + q) * 32 + bb);
        ++o;
      }
    }
    emitted += sweep_total;
    __syncthreads();
  }
  return emitted;
}

__device__ __forceinline__ void mark_block(uint64_t c, int64_t base, int64_t len, SelShared& sh) {
  const int64_t s = (int64_t)(~(uint32_t)c) - base;
  if (s >= 0 && s < len) atomicOr(&sh.bitmap[s >> 5], 1u << (s & 31));
}

__global__ __launch_bounds__(kThreads) void topk_select_kernel(
    const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ pos,
    const int32_t* __restrict__ n_comp, int ratio, int top_k,
    const uint64_t* __restrict__ cand_all, const uint32_t* __restrict__ nvalid_all,
    int waves_per_token, int blocks_per_wave, int cand_m, int32_t* __restrict__ idx,
    int32_t* __restrict__ count, uint32_t* __restrict__ err) {
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  int32_t* out = idx + (int64_t)t * top_k;
  const float* srow = scores + (int64_t)t * ld;

  // Loads that do not depend on the row length go out together: the token's
  // metadata and, when there are candidate lists, every list of the token
  // (the indexer writes all of them, zero keys for waves without blocks) with
  // the size of the group whose m-th key each slot holds.
  const int64_t pos_t = pos[t];
  const int32_t ncomp_t = n_comp[t];
  const uint32_t m = cand_m > 0 ? (uint32_t)cand_m : 1u;
  const uint32_t CT = cand_m > 0 ? min((uint32_t)waves_per_token * m, (uint32_t)kPoolCap) : 0u;
  const uint64_t* cand = cand_all + (int64_t)t * waves_per_token * cand_m;
  const uint32_t* nval = nvalid_all + (int64_t)t * waves_per_token;
  uint64_t key[KPT];
  uint32_t nv[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const uint32_t j = (uint32_t)tid + (uint32_t)i * kThreads;
    key[i] = j < CT ? cand[j] : 0ull;
    nv[i] = (j < CT && j % m == m - 1u) ? nval[j / m] : 0u;
  }
  // the emission bitmap is cleared while those loads are in flight
  {
    u32x4* bm4 = reinterpret_cast<u32x4*>(sh.bitmap);
    for (int i = tid; i < kBitmapWords / 4; i += kThreads) bm4[i] = u32x4{0u, 0u, 0u, 0u};
  }
  if (tid == 0) {
    sh.n_ov = 0u;
    sh.n_x = 0u;
  }
  uint32_t f = 0;
  int64_t n_vis = visible_count(pos_t, ratio, ncomp_t, &f);
  if (n_vis > ld) n_vis = ld;
  const uint32_t k_eff = (uint32_t)(n_vis < (int64_t)top_k ? n_vis : (int64_t)top_k);
  __syncthreads();

  uint32_t emitted = 0;
  bool listed = false;  // the selection is in sh.outl
  if (k_eff == 0) {
    emitted = 0;
  } else if ((int64_t)k_eff == n_vis) {
    emitted = k_eff;  // every visible block
  } else {
    listed = true;
    uint32_t n_x = 0;
    bool global_path = false;
    uint64_t thr = 0ull;
    if (n_vis <= kPoolCap || cand_m == 0) {
      // ---- direct: every visible block is a key ----
      const uint32_t n = (uint32_t)min(n_vis, (int64_t)kPoolCap);
      if (n_vis > kPoolCap && tid == 0) report(err, CSA_DERR_BAD_META);  // long row, no lists
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const uint32_t j = (uint32_t)tid + (uint32_t)i * kThreads;
        key[i] = j < n ? block_key(srow[j], j) : 0ull;
        nv[i] = 0u;
      }
      thr = kth_key(key, 0, k_eff, sh);
    } else {
      // ---- candidate lists of the nw groups that cover the row ----
      const int G = blocks_per_wave;
      const uint32_t nw = (uint32_t)((n_vis + G - 1) / G);
      const uint32_t C = min(nw * m, CT);
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const uint32_t j = (uint32_t)tid + (uint32_t)i * kThreads;
        if (j >= C) {
          key[i] = 0ull;
          nv[i] = 0u;
        }
      }
      const uint64_t t1 = C >= k_eff ? kth_key(key, 0, k_eff, sh) : 0ull;
      // groups that may hold unlisted blocks at or above T1
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        if (nv[i] > m && (t1 == 0ull || key[i] >= t1)) {
          const uint32_t slot = atomicAdd(&sh.n_ov, 1u);
          if (slot < (uint32_t)kMaxOv) {
            sh.ov_w[slot] = ((uint32_t)tid + (uint32_t)i * kThreads) / m;
            sh.ov_nv[slot] = nv[i];
            sh.ov_cut[slot] = key[i];
          }
        }
      }
      __syncthreads();
      const uint32_t n_ov = sh.n_ov;
      global_path = n_ov > (uint32_t)kMaxOv || t1 == 0ull;
      thr = t1;
      if (!global_path && n_ov > 0) {
        const uint32_t unlisted =
            block_sum((uint32_t)tid < n_ov ? sh.ov_nv[tid] - m : 0u, sh.scratch);
        if (unlisted > (uint32_t)kXCap) {
          global_path = true;
        } else {
          // every block of the flagged groups that is below the group's m-th
          // key (i.e. not listed) joins the key set
          constexpr int XB = 4;
          const uint32_t span = n_ov * (uint32_t)G;
          for (uint32_t e0 = 0; e0 < span; e0 += XB * kThreads) {
            uint32_t blk[XB];
            bool ok[XB];
            float fv[XB];
#pragma unroll
            for (int u = 0; u < XB; ++u) {
              const uint32_t e = e0 + (uint32_t)u * kThreads + tid;
              const uint32_t g = e / (uint32_t)G, off = e - g * (uint32_t)G;
              ok[u] = e < span && off < sh.ov_nv[g < n_ov ? g : 0];
              blk[u] = ok[u] ? sh.ov_w[g] * (uint32_t)G + off : 0u;
            }
#pragma unroll
            for (int u = 0; u < XB; ++u) fv[u] = ok[u] ? srow[blk[u]] : 0.0f;
#pragma unroll
            for (int u = 0; u < XB; ++u) {
              const uint32_t e = e0 + (uint32_t)u * kThreads + tid;
              const uint64_t c = ok[u] ? block_key(fv[u], blk[u]) : 0ull;
              const bool add = ok[u] && c < sh.ov_cut[e / (uint32_t)G];
              wave_append(add, c, sh.xk, &sh.n_x, kXCap);
            }
          }
          __syncthreads();
          n_x = min(sh.n_x, (uint32_t)kXCap);
          thr = kth_key(key, n_x, k_eff, sh);
          if (thr == 0ull) global_path = true;
        }
      }
    }
    if (!global_path) {
      auto mark = [&](int64_t base, int64_t len) {
#pragma unroll
        for (int i = 0; i < KPT; ++i)
          if (key[i] != 0ull && key[i] >= thr) mark_block(key[i], base, len, sh);
        for (uint32_t j = tid; j < n_x; j += kThreads)
          if (sh.xk[j] >= thr) mark_block(sh.xk[j], base, len, sh);
      };
      emitted = emit_bitmap(mark, n_vis, top_k, sh);
    } else {
      auto getg = [&](uint32_t j) { return block_key(srow[j], j); };
      const uint64_t tg = radix_kth(getg, (uint32_t)n_vis, k_eff, sh);
      auto mark = [&](int64_t base, int64_t len) {
        for (int64_t j = base + tid; j < base + len; j += kThreads) {
          const uint64_t c = getg((uint32_t)j);
          if (c >= tg) mark_block(c, base, len, sh);
        }
      };
      emitted = emit_bitmap(mark, n_vis, top_k, sh);
    }
  }
  if (emitted > (uint32_t)top_k) emitted = (uint32_t)top_k;
  // one coalesced pass writes the selection and the -1 padding
  for (uint32_t i = tid; i < (uint32_t)top_k; i += kThreads)
    out[i] = i < emitted ? (listed ? sh.outl[i] : (int32_t)i) : -1;
  if (tid == 0) count[t] = (int32_t)emitted;
}

// Candidate lists from caller-given scores (same layout as the indexer's).
constexpr int kCandThreads = 256;
__global__ __launch_bounds__(kCandThreads) void score_cands_kernel(
    const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ pos,
    const int32_t* __restrict__ n_comp, int ratio, int blocks_per_wave, int cand_m,
    uint64_t* __restrict__ cand, uint32_t* __restrict__ nvalid, uint32_t* __restrict__ err) {
  constexpr int KPL = 8;  // up to 8 x 32 = 256 blocks per group
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t flags = 0;
  int64_t n_vis = visible_count(pos[t], ratio, n_comp[t], &flags);
  if (n_vis > ld) {
    flags |= CSA_DERR_VIS_OVER_LD;
    n_vis = ld;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) report(err, flags);
  const int64_t wg = (int64_t)blockIdx.x * (kCandThreads / 64) + wave;
  const int64_t wslot = (int64_t)t * gridDim.x * (kCandThreads / 64) + wg;
  const int64_t b0 = wg * blocks_per_wave;
  const int64_t b1 = min(b0 + (int64_t)blocks_per_wave, n_vis);
  const float* srow = scores + (int64_t)t * ld;
  // half-wave h takes the 32-block pieces 2p + h of the group
  constexpr int KPH = KPL / 2;
  float sc[KPH];
  bool ok[KPH];
  uint32_t blk[KPH];
#pragma unroll
  for (int p = 0; p < KPH; ++p) {
    const int piece = 2 * p + (lane >> 5);
    const int64_t b = b0 + piece * 32 + (lane & 31);
    ok[p] = piece * 32 < blocks_per_wave && b < b1;
    blk[p] = (uint32_t)b;
    sc[p] = ok[p] ? srow[b] : 0.0f;
  }
  const uint32_t n_ok = wave_top_m<KPH>(sc, ok, blk, (uint32_t)cand_m, cand + wslot * cand_m);
  if (lane == 0) nvalid[wslot] = n_ok;
}

}  // namespace

TopkPlan plan_topk(int T, int64_t ld, int top_k) {
  (void)top_k;
  const IndexPlan ip = plan_index(T, ld);
  TopkPlan p;
  p.waves_per_token = ip.waves_per_token();
  p.blocks_per_wave = ip.blocks_per_wave();
  if (ld <= kPoolCap) {
    p.cand_m = 0;
    return p;
  }
  // the lists of one token fill at most the select workgroup's registers
  int m = kPoolCap / p.waves_per_token;
  if (m > 32) m = 32;
  if (m < 1) m = 1;
  p.cand_m = m;
  return p;
}

TopkWs topk_ws_layout(void* ws, int T, const TopkPlan& p) {
  TopkWs w{};
  const size_t n = (size_t)T * p.waves_per_token;
  const size_t cand_b = (n * p.cand_m * 8 + 255) & ~(size_t)255;
  const size_t nv_b = (n * 4 + 255) & ~(size_t)255;
  w.bytes = p.cand_m ? cand_b + nv_b : 0;
  if (ws != nullptr && p.cand_m) {
    w.cand = static_cast<uint64_t*>(ws);
    w.nvalid = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + cand_b);
  }
  return w;
}

hipError_t launch_score_cands(const float* scores, int64_t ld, const int64_t* pos,
                              const int32_t* n_comp, int T, int ratio, const TopkPlan& p,
                              const TopkWs& ws, uint32_t* err, hipStream_t s) {
  if (T == 0 || p.cand_m == 0) return hipSuccess;
  dim3 grid((unsigned)(p.waves_per_token / (kCandThreads / 64)), (unsigned)T);
  hipLaunchKernelGGL(score_cands_kernel, grid, dim3(kCandThreads), 0, s, scores, ld, pos, n_comp,
                     ratio, p.blocks_per_wave, p.cand_m, ws.cand, ws.nvalid, err);
  return hipGetLastError();
}

hipError_t launch_topk_select(const float* scores, int64_t ld, const int64_t* pos,
                              const int32_t* n_comp, int T, int ratio, int top_k,
                              const TopkPlan& p, const TopkWs& ws, int32_t* idx,
                              int32_t* count, uint32_t* err, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)T), dim3(kThreads), 0, s, scores, ld,
                     pos, n_comp, ratio, top_k, ws.cand, ws.nvalid, p.waves_per_token,
                     p.blocks_per_wave, p.cand_m, idx, count, err);
  return hipGetLastError();
}

}  // namespace csa
