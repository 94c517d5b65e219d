// S2 -- causal top-k over the indexer scores (post-probe audit, F3:
// tk = min(top_k, n_comp) and a top-k over the scores; PART A, suspect 3: only
// blocks strictly before the query's own block are candidates).
//
// Every block s gets the composite key (score key << 32 | ~s): unique, larger
// score first, then lower block index, so the selected set is exactly the
// k_eff largest keys and ties at the k-th score go to the lower index.
//
// One workgroup per token selects, in LDS, from a pool of keys:
//   * n_vis <= kPoolCap: the pool is every visible block (exact, direct);
//   * otherwise the pool is the candidate lists -- the top-m keys of every
//     group of blocks handled by one indexer wave, written by the indexer
//     epilogue (or score_cands_kernel).  Let T1 be the k_eff-th largest pool
//     key.  A group whose list is full (it has more than m blocks) and whose
//     m-th key is >= T1 may hold unlisted blocks above T1; all its blocks are
//     added to the pool and the selection is repeated.  Every other unlisted
//     block is below its group's m-th key < T1, below k_eff pool keys, so the
//     result is exact.  At most k_eff/m groups can qualify (each puts m keys
//     >= T1 into the pool, and only k_eff pool keys are >= T1), which bounds
//     the extra work;
//   * if the pool would not fit, the select runs over the token's scores in
//     global memory (slow, exact; only for adversarial score layouts).
// The threshold is found by 8-bit radix passes over the 64-bit keys with a
// block-wide bin search; the selection is written in ascending block order
// by scanning an LDS bitmap of the visible range.
//
// No global atomics: on this chip same-address device-scope atomics serialise
// at ~12 ns each, so cross-workgroup communication is plain stores plus the
// kernel boundary.
#include "csa_common.h"

namespace csa {
namespace {

constexpr int kThreads = 256;
constexpr int kBitmapWords = 8192;  // 262,144 blocks per emission sweep
constexpr int kMaxOv = 512;         // groups re-scanned in full before falling back

// Block-wide search in a histogram distributed over the workgroup: thread i
// owns bins [i*BPT, i*BPT+BPT) in `c`.  Finds the bin b with
//   (items in bins > b) < need <= (items in bins >= b)
// and returns b and the count above it.  Requires 1 <= need <= total.
template <int BPT>
__device__ __forceinline__ void find_threshold_bin(const uint32_t (&c)[BPT], uint32_t need,
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
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* scratch, uint32_t& total) {
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

__device__ __forceinline__ int64_t token_visible(const int64_t* pos, const int32_t* n_comp,
                                                 int t, int ratio, int64_t ld) {
  uint32_t f = 0;
  int64_t n_vis = visible_count(pos[t], ratio, n_comp[t], &f);
  return n_vis > ld ? ld : n_vis;
}

struct SelShared {
  uint64_t pool[kPoolCap];
  uint32_t bitmap[kBitmapWords + kBitmapWords / 32];  // word w at w + w/32 (bank padding)
  uint32_t dh4[kThreads / 64][256];                    // per-wave digit histograms
  uint32_t dh[256];
  uint32_t scratch[16];
  uint32_t ov_w[kMaxOv];
  uint32_t ov_off[kMaxOv + 1];
  uint64_t ov_cut[kMaxOv];
  uint64_t red[8];
  uint32_t n_pool, n_ov;
};

// Block-wide max, and min over nonzero values, of 64-bit keys.
__device__ __forceinline__ void block_minmax(uint64_t lo, uint64_t hi, SelShared& sh, uint64_t& blo, uint64_t& bhi) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t a = __shfl_xor((unsigned long long)lo, off);
    const uint64_t b = __shfl_xor((unsigned long long)hi, off);
    lo = a < lo ? a : lo;
    hi = b > hi ? b : hi;
  }
  if (lane == 0) {
    sh.red[wave] = lo;
    sh.red[4 + wave] = hi;
  }
  __syncthreads();
  blo = sh.red[0];
  bhi = sh.red[4];
  for (int w = 1; w < kThreads / 64; ++w) {
    blo = sh.red[w] < blo ? sh.red[w] : blo;
    bhi = sh.red[4 + w] > bhi ? sh.red[4 + w] : bhi;
  }
  __syncthreads();
}

// Threshold T with exactly k of the n keys get(0..n-1) >= T (keys unique,
// 1 <= k; returns 0 when fewer than k keys are nonzero).  Radix passes of up to 8 bits, starting
// below the leading bits that all nonzero keys share, stopping as soon as the
// threshold bin holds exactly the remaining need.
template <class Get>
__device__ uint64_t kth_threshold(Get get, uint32_t n, uint32_t k, SelShared& sh) {
  const int tid = threadIdx.x;
  uint64_t lo = ~0ull, hi = 0ull;
  uint32_t nz = 0;
#pragma unroll 4
  for (uint32_t j = tid; j < n; j += kThreads) {
    const uint64_t c = get(j);
    if (c != 0ull && c < lo) lo = c;
    if (c > hi) hi = c;
    nz += c != 0ull;
  }
  uint32_t n_nonzero;
  block_excl_scan(nz, sh.scratch, n_nonzero);
  if (n_nonzero < k) return 0ull;  // caller falls back
  uint64_t blo, bhi;
  block_minmax(lo, hi, sh, blo, bhi);
  if (blo >= bhi) return bhi;  // a single nonzero key
  const int top = 63 - __clzll((long long)(blo ^ bhi));  // highest differing bit
  int shift = top + 1;
  uint64_t prefix = shift >= 64 ? 0ull : (bhi >> shift);
  uint32_t need = k;
  for (int pass = 0; pass < 9 && shift > 0; ++pass) {
    const int nb = shift < 8 ? shift : 8;
    const int nshift = shift - nb;
    const uint32_t mask = (1u << nb) - 1u;
    sh.dh[tid] = 0u;
    __syncthreads();
#pragma unroll 4
    for (uint32_t j = tid; j < n; j += kThreads) {
      const uint64_t c = get(j);
      if (shift >= 64 || (c >> shift) == prefix) atomicAdd(&sh.dh[(uint32_t)(c >> nshift) & mask], 1u);
    }
    __syncthreads();
    uint32_t cnt[1] = {sh.dh[tid]};
    uint32_t d, above;
    find_threshold_bin<1>(cnt, need, sh.scratch, d, above);
    const uint32_t in_bin = sh.dh[d];
    need -= above;
    prefix = (shift >= 64 ? 0ull : (prefix << nb)) | d;
    shift = nshift;
    __syncthreads();
    if (in_bin == need) break;
  }
  return prefix << shift;
}

// Write the selected blocks {s : key(s) >= thr, key != 0} in ascending order.
template <class Get>
__device__ uint32_t emit_sorted(Get get, uint32_t n_src, uint64_t thr, int64_t n_vis, int top_k,
                                int32_t* out, SelShared& sh) {
  const int tid = threadIdx.x;
  uint32_t emitted = 0;
  const int64_t span = (int64_t)kBitmapWords * 32;
  for (int64_t base = 0; base < n_vis; base += span) {
    const int64_t len = min(span, n_vis - base);
    const int words = (int)((len + 31) / 32);
    for (int i = tid; i < kBitmapWords + kBitmapWords / 32; i += kThreads) sh.bitmap[i] = 0u;
    __syncthreads();
#pragma unroll 4
    for (uint32_t j = tid; j < n_src; j += kThreads) {
      const uint64_t c = get(j);
      if (c != 0ull && c >= thr) {
        const int64_t s = (int64_t)(~(uint32_t)c) - base;
        if (s >= 0 && s < len) atomicOr(&sh.bitmap[(s >> 5) + (s >> 10)], 1u << (s & 31));
      }
    }
    __syncthreads();
    const int per = (words + kThreads - 1) / kThreads;
    const int w0 = tid * per;
    uint32_t mine = 0;
    for (int k = 0; k < per; ++k)
      if (w0 + k < words) mine += (uint32_t)__popc(sh.bitmap[(w0 + k) + ((w0 + k) >> 5)]);
    uint32_t sweep_total;
    uint32_t o = emitted + block_excl_scan(mine, sh.scratch, sweep_total);
    for (int k = 0; k < per; ++k) {
      if (w0 + k >= words) break;
      uint32_t bits = sh.bitmap[(w0 + k) + ((w0 + k) >> 5)];
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
  return emitted;
}

constexpr int KPT = kPoolCap / kThreads;  // pool keys per thread

__device__ __forceinline__ uint32_t bm_index(uint32_t w) { return w + (w >> 5); }

// Threshold T with exactly k of the keys >= T, for keys held in registers
// (key[i], i < KPT; zero = empty).  Returns 0 when fewer than k keys are
// nonzero.  Digit histograms are kept per wave, so a skewed digit only
// contends within a wave.
__device__ __forceinline__ uint64_t kth_regs(const uint64_t (&key)[KPT], uint32_t k, SelShared& sh) {
  const int tid = threadIdx.x, wave = tid >> 6;
  uint64_t lo = ~0ull, hi = 0ull;
  uint32_t nz = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const uint64_t c = key[i];
    if (c != 0ull && c < lo) lo = c;
    if (c > hi) hi = c;
    nz += c != 0ull;
  }
  uint32_t n_nonzero;
  block_excl_scan(nz, sh.scratch, n_nonzero);
  if (n_nonzero < k) return 0ull;
  uint64_t blo, bhi;
  block_minmax(lo, hi, sh, blo, bhi);
  if (blo >= bhi) return bhi;
  const int top = 63 - __clzll((long long)(blo ^ bhi));
  int shift = top + 1;
  uint64_t prefix = shift >= 64 ? 0ull : (bhi >> shift);
  uint32_t need = k;
  for (int pass = 0; pass < 9 && shift > 0; ++pass) {
    const int nb = shift < 8 ? shift : 8;
    const int nshift = shift - nb;
    const uint32_t mask = (1u << nb) - 1u;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) sh.dh4[w][tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const uint64_t c = key[i];
      if (c != 0ull && (shift >= 64 || (c >> shift) == prefix))
        atomicAdd(&sh.dh4[wave][(uint32_t)(c >> nshift) & mask], 1u);
    }
    __syncthreads();
    uint32_t cnt1[1] = {sh.dh4[0][tid] + sh.dh4[1][tid] + sh.dh4[2][tid] + sh.dh4[3][tid]};
    sh.dh[tid] = cnt1[0];
    uint32_t d, above;
    find_threshold_bin<1>(cnt1, need, sh.scratch, d, above);
    const uint32_t in_bin = sh.dh[d];
    need -= above;
    prefix = (shift >= 64 ? 0ull : (prefix << nb)) | d;
    shift = nshift;
    __syncthreads();
    if (in_bin == need) break;
  }
  return prefix << shift;
}

// Write {block of key : key >= thr, key != 0} (keys in registers) in
// ascending block order: mark a padded LDS bitmap, then every thread scans a
// contiguous run of words and emits its bits at its prefix-sum offset.
__device__ __forceinline__ uint32_t emit_regs(const uint64_t (&key)[KPT], uint64_t thr, int64_t n_vis, int top_k,
                              int32_t* out, SelShared& sh) {
  const int tid = threadIdx.x;
  uint32_t emitted = 0;
  const int64_t span = (int64_t)kBitmapWords * 32;
  for (int64_t base = 0; base < n_vis; base += span) {
    const int64_t len = min(span, n_vis - base);
    const int words = (int)((len + 31) / 32);
    for (int i = tid; i < kBitmapWords + kBitmapWords / 32; i += kThreads) sh.bitmap[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const uint64_t c = key[i];
      if (c != 0ull && c >= thr) {
        const int64_t s = (int64_t)(~(uint32_t)c) - base;
        if (s >= 0 && s < len) atomicOr(&sh.bitmap[bm_index((uint32_t)(s >> 5))], 1u << (s & 31));
      }
    }
    __syncthreads();
    const int per = (words + kThreads - 1) / kThreads;
    const int w0 = tid * per;
    uint32_t wv[32];
    uint32_t mine = 0;
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      wv[q] = (q < per && w0 + q < words) ? sh.bitmap[bm_index((uint32_t)(w0 + q))] : 0u;
      mine += (uint32_t)__popc(wv[q]);
    }
    uint32_t sweep_total;
    uint32_t o = emitted + block_excl_scan(mine, sh.scratch, sweep_total);
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      uint32_t bits = wv[q];
      while (bits) {
        const int b = __ffs(bits) - 1;
        bits &= bits - 1u;
        if (o < (uint32_t)top_k) out[o] = (int32_t)(base + (int64_t)(w0 + q) * 32 + b);
        ++o;
      }
    }
    emitted += sweep_total;
    __syncthreads();
  }
  return emitted;
}

// Keys of the LDS pool entries tid, tid + 256, ... into registers.
__device__ __forceinline__ void pool_to_regs(const SelShared& sh, uint32_t n, uint64_t (&key)[KPT]) {
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const uint32_t j = (uint32_t)threadIdx.x + (uint32_t)i * kThreads;
    key[i] = j < n ? sh.pool[j] : 0ull;
  }
}

__global__ __launch_bounds__(256) void topk_select_kernel(
    const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ pos,
    const int32_t* __restrict__ n_comp, int ratio, int top_k,
    const uint64_t* __restrict__ cand_all, const uint32_t* __restrict__ nvalid_all,
    int waves_per_token, int blocks_per_wave, int cand_m, int32_t* __restrict__ idx,
    int32_t* __restrict__ count, uint32_t* __restrict__ err) {
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  const int64_t n_vis = token_visible(pos, n_comp, t, ratio, ld);
  const uint32_t k_eff = (uint32_t)(n_vis < (int64_t)top_k ? n_vis : (int64_t)top_k);
  int32_t* out = idx + (int64_t)t * top_k;
  const float* srow = scores + (int64_t)t * ld;
  uint32_t emitted = 0;

  if (k_eff == 0) {
    emitted = 0;
  } else if ((int64_t)k_eff == n_vis) {
    for (uint32_t j = tid; j < k_eff; j += kThreads) out[j] = (int32_t)j;
    emitted = k_eff;
  } else if (n_vis <= kPoolCap || cand_m == 0) {
    // ---- direct: every visible block is a key ----
    const uint32_t n = (uint32_t)min(n_vis, (int64_t)kPoolCap);
    if (n_vis > kPoolCap && tid == 0) report(err, CSA_DERR_BAD_META);  // no candidates for a long row
    uint64_t key[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const uint32_t j = (uint32_t)tid + (uint32_t)i * kThreads;
      key[i] = j < n ? block_key(srow[j], j) : 0ull;
    }
    const uint64_t thr = kth_regs(key, k_eff, sh);
    emitted = emit_regs(key, thr, n_vis, top_k, out, sh);
  } else {
    // ---- candidate lists ----
    const int G = blocks_per_wave;
    const int m = cand_m;
    const uint32_t nw = (uint32_t)((n_vis + G - 1) / G);
    const uint64_t* cand = cand_all + (int64_t)t * waves_per_token * m;
    const uint32_t* nval = nvalid_all + (int64_t)t * waves_per_token;
    const uint32_t C = nw * (uint32_t)m;  // <= 2/3 kPoolCap by the plan
    // the lists go straight into registers (and the LDS pool, for the
    // re-scan); the group sizes are loaded in the same batch
    uint64_t key[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const uint32_t j = (uint32_t)tid + (uint32_t)i * kThreads;
      key[i] = j < C ? cand[j] : 0ull;
    }
    constexpr int NB = 8;
    uint32_t nv[NB];  // sizes of groups tid + 256 u
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const uint32_t w = (uint32_t)u * kThreads + tid;
      nv[u] = w < nw ? nval[w] : 0u;
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const uint32_t j = (uint32_t)tid + (uint32_t)i * kThreads;
      if (j < C) sh.pool[j] = key[i];
    }
    if (tid == 0) {
      sh.n_ov = 0u;
      sh.n_pool = C;
    }
    __syncthreads();
    const uint64_t t1 = C >= k_eff ? kth_regs(key, k_eff, sh) : 0ull;
    // groups that may hold unlisted blocks at or above T1
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const uint32_t w = (uint32_t)u * kThreads + tid;
      if (w < nw) {
        const uint64_t cut = sh.pool[w * m + m - 1];
        if (nv[u] > (uint32_t)m && (t1 == 0ull || cut >= t1)) {
          const uint32_t slot = atomicAdd(&sh.n_ov, 1u);
          if (slot < (uint32_t)kMaxOv) {
            sh.ov_w[slot] = w;
            sh.ov_cut[slot] = cut;
          }
        }
      }
    }
    for (uint32_t w = NB * kThreads + tid; w < nw; w += kThreads) {  // very long rows
      const uint64_t cut = sh.pool[w * m + m - 1];
      if (nval[w] > (uint32_t)m && (t1 == 0ull || cut >= t1)) {
        const uint32_t slot = atomicAdd(&sh.n_ov, 1u);
        if (slot < (uint32_t)kMaxOv) {
          sh.ov_w[slot] = w;
          sh.ov_cut[slot] = cut;
        }
      }
    }
    __syncthreads();
    const uint32_t n_ov = sh.n_ov;
    bool global_path = n_ov > (uint32_t)kMaxOv || t1 == 0ull;
    uint64_t thr = t1;
    if (!global_path && n_ov > 0) {
      if (tid == 0) {  // prefix of the groups' block counts (n_ov <= kMaxOv)
        uint32_t acc = 0;
        for (uint32_t i = 0; i < n_ov; ++i) {
          sh.ov_off[i] = acc;
          acc += nval[sh.ov_w[i]];
        }
        sh.ov_off[n_ov] = acc;
      }
      __syncthreads();
      const uint32_t extra = sh.ov_off[n_ov];
      if (C + extra > (uint32_t)kPoolCap) {
        global_path = true;
      } else {
        constexpr int XB = 4;
        for (uint32_t j0 = 0; j0 < extra; j0 += XB * kThreads) {
          uint32_t blk[XB];
          int own[XB];
#pragma unroll
          for (int u = 0; u < XB; ++u) {
            const uint32_t j = j0 + u * kThreads + tid;
            int lo = 0, hi = (int)n_ov - 1;
            while (lo < hi) {
              const int mid = (lo + hi + 1) >> 1;
              if (sh.ov_off[mid] <= j) lo = mid; else hi = mid - 1;
            }
            own[u] = j < extra ? lo : -1;
            blk[u] = j < extra ? sh.ov_w[lo] * (uint32_t)G + (j - sh.ov_off[lo]) : 0u;
          }
          float f[XB];
#pragma unroll
          for (int u = 0; u < XB; ++u) f[u] = own[u] >= 0 ? srow[blk[u]] : 0.0f;
#pragma unroll
          for (int u = 0; u < XB; ++u) {
            if (own[u] >= 0) {
              const uint64_t c = block_key(f[u], blk[u]);
              if (c < sh.ov_cut[own[u]]) sh.pool[atomicAdd(&sh.n_pool, 1u)] = c;  // not yet listed
            }
          }
        }
        __syncthreads();
        pool_to_regs(sh, sh.n_pool, key);
        __syncthreads();
        thr = kth_regs(key, k_eff, sh);
        if (thr == 0ull) global_path = true;
      }
    }
    if (!global_path) {
      emitted = emit_regs(key, thr, n_vis, top_k, out, sh);
    } else {
      auto getg = [&](uint32_t j) { return block_key(srow[j], j); };
      const uint64_t tg = kth_threshold(getg, (uint32_t)n_vis, k_eff, sh);
      emitted = emit_sorted(getg, (uint32_t)n_vis, tg, n_vis, top_k, out, sh);
    }
  }
  if (emitted > (uint32_t)top_k) emitted = (uint32_t)top_k;
  for (uint32_t i = emitted + tid; i < (uint32_t)top_k; i += kThreads) out[i] = -1;
  if (tid == 0) count[t] = (int32_t)emitted;
}

// Candidate lists from caller-given scores (same layout as the indexer's).
__global__ __launch_bounds__(256) void score_cands_kernel(
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
  const int64_t wg = (int64_t)blockIdx.x * (kThreads / 64) + wave;
  const int64_t wslot = (int64_t)t * gridDim.x * (kThreads / 64) + wg;
  const int64_t b0 = wg * blocks_per_wave;
  const int64_t b1 = min(b0 + (int64_t)blocks_per_wave, n_vis);
  uint64_t key[KPL];
  const float* srow = scores + (int64_t)t * ld;
#pragma unroll
  for (int q = 0; q < KPL; ++q) {
    const int64_t blk = b0 + q * 32 + (lane & 31);
    key[q] = (lane < 32 && q * 32 < blocks_per_wave && blk < b1) ? block_key(srow[blk], (uint32_t)blk)
                                                                  : 0ull;
  }
  wave_top_m<KPL>(key, cand_m, cand + wslot * cand_m);
  if (lane == 0) nvalid[wslot] = b1 > b0 ? (uint32_t)(b1 - b0) : 0u;
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
  // keep a third of the pool free for groups re-scanned in full
  int m = (2 * kPoolCap) / (3 * p.waves_per_token);
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
  dim3 grid((unsigned)(p.waves_per_token / (kThreads / 64)), (unsigned)T);
  hipLaunchKernelGGL(score_cands_kernel, grid, dim3(kThreads), 0, s, scores, ld, pos, n_comp,
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
