// Exact causal top-k of one token by one workgroup of NT threads (1024 in the
// top-k kernel, 512 at the tail of the indexer in the decode step).
//
// Every block s gets the composite key (score key << 32 | ~s): unique, larger
// score first, then lower block index, so the selected set is exactly the
// k_eff largest keys and ties at the k-th score go to the lower index
// (post-probe audit, F3: tk = min(top_k, n_comp) and a top-k over the scores;
// PART A, suspect 3: only blocks strictly before the query's own block).
//
// The workgroup selects from a key set held in registers (KP keys per
// thread) plus an LDS overflow area:
//   * n_vis <= KP * NT: the keys are every visible block (exact, direct);
//   * otherwise the keys are the candidate lists of the groups that cover
//     the row (see CandArgs).  Let T1 be the k_eff-th largest listed key.  A
//     group whose bound (>= every key it did not list) is >= T1 may hold
//     unlisted blocks at or above T1: its listed keys leave the set and all
//     its visible blocks join it, and the threshold is found again.  Every
//     other unlisted block is below T1, below k_eff listed keys, so the
//     result is exact;
//   * if the extra blocks would not fit, or a long row has no lists, the
//     select runs over the token's scores in global memory (slow, exact).
//
// The k-th key is found in one histogram pass over 2*NT bins laid linearly
// over [min, max] of the keys' order-preserving uint32 score words (a monotone
// map, so bins are ordered; two integer operations per key), then an exact
// rank among the few keys of the threshold bin.  Within one binade the words
// are linear in the score, so the bins spread the keys, which keeps LDS
// atomics free of same-address conflicts; where the
// threshold bin is crowded (ties, clustered values) an exact 8-bit radix
// select over the composite keys takes over.  The selection is listed in
// ascending block order from the slot order of the keys (lists stored in
// block order) or by scanning an LDS bitmap of the visible range.
#pragma once

#include <math.h>

#include "csa_common.h"

namespace csa {
namespace {
namespace sel {

// The select runs in a workgroup of NT threads (1024 in the top-k kernel, 512
// at the tail of the indexer), with up to KP register keys per thread.
constexpr int kMaxThreads = 1024;
constexpr int kMaxWaves = kMaxThreads / 64;
constexpr int kMaxKP = kPoolCap / kMaxThreads;  // register keys per thread, at most (1024 threads)
constexpr int KPT = kMaxKP;
constexpr int kXCap = 4096;               // keys of re-scanned groups (LDS)
constexpr int kListCap = 1024;            // threshold-bin keys ranked exactly
constexpr int kMaxOv = 512;               // groups re-scanned before falling back
constexpr int kBitmapWords = 8192;        // 262,144 blocks per emission sweep
constexpr int kMaxTopK = 2048;
constexpr int kThreads = kMaxThreads;     // the top-k kernel's workgroup
static_assert(kMaxKP * kMaxThreads == kPoolCap, "pool must split evenly");

template <int NT>
struct Geo {
  static constexpr int kWaves = NT / 64;
  static constexpr int kBins = 2 * NT;    // linear bins, two per thread
  static constexpr int kGPT = kMaxGroups / NT;  // group bounds per thread
  static_assert(NT == 512 || NT == 1024, "select workgroup size");
  static_assert(kBitmapWords % (8 * NT) == 0, "whole u32x4 bitmap reads per thread");
  static_assert(kMaxOv <= NT, "one flagged group per thread");
};

template <int NT>
struct SelShared {
  static constexpr int W = Geo<NT>::kWaves;
  uint32_t bitmap[kBitmapWords];
  uint64_t xk[kXCap];
  uint64_t list[kListCap];
  uint32_t hist[Geo<NT>::kBins];
  uint32_t ov_g[kMaxOv];                  // flagged groups (re-scanned whole)
  uint32_t gflag[kMaxGroups / 32];        // the same groups as a bitmap
  int32_t outl[kMaxTopK];                 // the selection, ascending, before the output copy
  uint32_t scratch[2 * W + 8];
  uint32_t plane[(kMaxKP + 1) / 2 * W];   // per-wave packed slot-plane counts of emit_slots
  uint32_t rc[W];                         // per-wave count / score-word range of kth_key
  uint32_t rlo[W], rhi[W];
  uint32_t fb_w[W];                       // per-wave bin totals of kth_key
  uint32_t fb_bin, fb_above;
  uint64_t red64[2 * W];
  uint64_t thr;
  uint32_t n_x, n_ov, n_list;
};

// Appends v (where p) to list[0..cap) at *n; one LDS atomic per wave.
__device__ __forceinline__ void wave_append(bool p, uint64_t v, uint64_t* list, uint32_t* n,
                                            uint32_t cap) {
  const uint64_t mask = __ballot(p);
  if (mask == 0ull) return;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((unsigned long long)mask) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(n, (uint32_t)__popcll(mask));
  base = (uint32_t)__builtin_amdgcn_readlane((int)base, leader);
  if (p) {
    const uint32_t o = base + (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
    if (o < cap) list[o] = v;
  }
}

// Per-wave values vals[0..kWaves) in LDS (one per wave of the workgroup):
// lane w < kWaves reads value w, so one read and a DPP scan give the sum of
// the values before this wave's, the sum after it, and the total.
template <int NT>
__device__ __forceinline__ void cross_wave_sums(const uint32_t* vals, uint32_t& before,
                                                uint32_t& after, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t v = lane < Geo<NT>::kWaves ? vals[lane] : 0u;
  const uint32_t incl = wave_incl_scan_u32(v);
  total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  const uint32_t upto = (uint32_t)__builtin_amdgcn_readlane((int)incl, wave);
  before = upto - (uint32_t)__builtin_amdgcn_readlane((int)v, wave);
  after = total - upto;
}

// Block-wide search in a histogram distributed over the workgroup: thread i
// owns bins [i*BPT, i*BPT+BPT) in `c`.  Finds the bin b with
//   (items in bins > b) < need <= (items in bins >= b)
// and returns b and the count above it.  Requires 1 <= need <= total.
template <int NT, int BPT>
__device__ __forceinline__ void find_threshold_bin(const uint32_t (&c)[BPT], uint32_t need,
                                                   uint32_t* scratch, uint32_t& bin,
                                                   uint32_t& above) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t tot = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) tot += c[i];
  // inclusive suffix sum within the wave
  const uint32_t pre = wave_incl_scan_u32(tot);
  const uint32_t x = (uint32_t)__builtin_amdgcn_readlane((int)pre, 63) - pre + tot;
  if (lane == 0) scratch[wave] = x;
  __syncthreads();
  uint32_t before_w, after_w, total_w;
  cross_wave_sums<NT>(scratch, before_w, after_w, total_w);
  uint32_t acc = x - tot + after_w;
#pragma unroll
  for (int i = BPT - 1; i >= 0; --i) {
    if (acc < need && acc + c[i] >= need) {
      scratch[Geo<NT>::kWaves] = (uint32_t)(tid * BPT + i);
      scratch[Geo<NT>::kWaves + 1] = acc;
    }
    acc += c[i];
  }
  __syncthreads();
  bin = scratch[Geo<NT>::kWaves];
  above = scratch[Geo<NT>::kWaves + 1];
  __syncthreads();
}

// Exclusive prefix sum over the workgroup (ascending thread order).
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* scratch,
                                                    uint32_t& total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t x = wave_incl_scan_u32(v);
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  uint32_t base, after;
  cross_wave_sums<NT>(scratch, base, after, total);
  __syncthreads();
  return base + x - v;
}

template <int NT>
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* scratch) {
  uint32_t total;
  block_excl_scan<NT>(v, scratch, total);
  return total;
}

// Block-wide min over nonzero keys and max of 64-bit keys.
template <int NT>
__device__ __forceinline__ void block_minmax64(uint64_t lo, uint64_t hi, SelShared<NT>& sh,
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
    sh.red64[Geo<NT>::kWaves + wave] = hi;
  }
  __syncthreads();
  blo = sh.red64[0];
  bhi = sh.red64[Geo<NT>::kWaves];
  for (int w = 1; w < Geo<NT>::kWaves; ++w) {
    blo = sh.red64[w] < blo ? sh.red64[w] : blo;
    bhi = sh.red64[Geo<NT>::kWaves + w] > bhi ? sh.red64[Geo<NT>::kWaves + w] : bhi;
  }
  __syncthreads();
}

// Exact k-th largest of the nonzero keys get(0..n) by 8-bit radix passes over
// the 64-bit keys, starting below the leading bits that all of them share and
// stopping once the threshold bin holds exactly the remaining need.  Requires
// at least k nonzero keys.  `get(j)` may return zero for an empty slot.
template <int NT, class Get>
__device__ __forceinline__ uint64_t radix_kth(Get get, uint32_t n, uint32_t k, SelShared<NT>& sh) {
  const int tid = threadIdx.x;
  uint64_t lo = ~0ull, hi = 0ull;
  for (uint32_t j = tid; j < n; j += NT) {
    const uint64_t c = get(j);
    if (c != 0ull && c < lo) lo = c;
    if (c > hi) hi = c;
  }
  uint64_t blo, bhi;
  block_minmax64<NT>(lo, hi, sh, blo, bhi);
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
    for (uint32_t j = tid; j < n; j += NT) {
      const uint64_t c = get(j);
      if (c != 0ull && (shift >= 64 || (c >> shift) == prefix))
        atomicAdd(&sh.hist[(uint32_t)(c >> nshift) & mask], 1u);
    }
    __syncthreads();
    uint32_t cnt[1] = {tid < 256 ? sh.hist[tid] : 0u};
    uint32_t d, above;
    find_threshold_bin<NT, 1>(cnt, need, sh.scratch, d, above);
    const uint32_t in_bin = sh.hist[d];
    need -= above;
    prefix = (shift >= 64 ? 0ull : (prefix << nb)) | d;
    shift = nshift;
    __syncthreads();
    if (in_bin == need) break;
  }
  return prefix << shift;
}

// Bin of a score word h >= ulo among kBins bins laid linearly over the
// ordered-uint32 score words [ulo, ulo + range]: the word difference itself
// when the range has fewer values than bins, else its product with mul
// (about kBins * 2^32 / (range + 1)), high half, capped at kBins - 1.
// Non-decreasing in h for any mul, so the bins are ordered.
template <int NT>
__device__ __forceinline__ uint32_t word_bin(uint32_t h, uint32_t ulo, bool small, uint32_t mul) {
  const uint32_t d = h - ulo;
  return small ? d : min(__umulhi(d, mul), (uint32_t)Geo<NT>::kBins - 1u);
}

// The k-th largest of the nonzero keys in key[0..KP) of every thread (slots
// i with i*NT >= nk are zero and skipped) and in sh.xk[0..n_x); 0 when
// fewer than k keys are nonzero.  1 <= k.  Each phase
// writes its own LDS slots, so six barriers separate the phases (a barrier
// between a phase's reads and the next call's writes always intervenes).
template <int NT, int KP>
__device__ __forceinline__ uint64_t kth_key(const uint64_t (&key)[KP], uint32_t nk, uint32_t n_x,
                                            uint32_t k, SelShared<NT>& sh) {
  constexpr int W = Geo<NT>::kWaves;
  constexpr int kBins = Geo<NT>::kBins;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // ---- count and score-word range of the nonzero keys; clear the histogram ----
  uint32_t nz = 0, ulo = 0xFFFFFFFFu, uhi = 0u;
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    if ((uint32_t)i * NT < nk) {
      const bool p = key[i] != 0ull;
      const uint32_t h = (uint32_t)(key[i] >> 32);
      nz += p ? 1u : 0u;
      ulo = min(ulo, p ? h : 0xFFFFFFFFu);
      uhi = max(uhi, h);
    }
  }
  for (uint32_t j = tid; j < n_x; j += NT) {
    const uint32_t h = (uint32_t)(sh.xk[j] >> 32);
    ++nz;
    ulo = min(ulo, h);
    uhi = max(uhi, h);
  }
  static_assert(kBins == 2 * NT, "two bins per thread");
  sh.hist[tid] = 0u;
  sh.hist[tid + NT] = 0u;
  if (tid == 0) sh.n_list = 0u;
  nz = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan_u32(nz), 63);
  ulo = wave_min_u32(ulo);
  uhi = wave_max_u32(uhi);
  if (lane == 0) {
    sh.rc[wave] = nz;
    sh.rlo[wave] = ulo;
    sh.rhi[wave] = uhi;
  }
  __syncthreads();
  uint32_t n_nz, blo, bhi;
  {
    uint32_t before_w, after_w;
    cross_wave_sums<NT>(sh.rc, before_w, after_w, n_nz);
    blo = wave_min_u32(lane < W ? sh.rlo[lane] : 0xFFFFFFFFu);
    bhi = wave_max_u32(lane < W ? sh.rhi[lane] : 0u);
  }
  if (n_nz < k) return 0ull;
  const uint32_t range = bhi - blo;
  const bool small = range < (uint32_t)kBins;
  // single-precision reciprocal (a 64-bit division is a long scalar sequence
  // that every wave would repeat); range >= kBins here, so mul < 2^32
  const uint32_t mul =
      small ? 0u : (uint32_t)((float)kBins * 4294967296.0f / ((float)range + 1.0f) * 0.99999f);
  bool crowded = range == 0u;  // one score value: the radix select orders by index
  if (!crowded) {
    // ---- histogram of the linear bins ----
#pragma unroll
    for (int i = 0; i < KP; ++i)
      if ((uint32_t)i * NT < nk && key[i] != 0ull)
        atomicAdd(&sh.hist[word_bin<NT>((uint32_t)(key[i] >> 32), blo, small, mul)], 1u);
    for (uint32_t j = tid; j < n_x; j += NT)
      atomicAdd(&sh.hist[word_bin<NT>((uint32_t)(sh.xk[j] >> 32), blo, small, mul)], 1u);
    __syncthreads();
    // ---- the bin b with (keys in bins > b) < k <= (keys in bins >= b);
    // thread i owns bins 2i, 2i+1 ----
    const uint32_t c0 = sh.hist[2 * tid], c1 = sh.hist[2 * tid + 1];
    const uint32_t tot = c0 + c1;
    // inclusive suffix sum within the wave
    const uint32_t pre = wave_incl_scan_u32(tot);
    const uint32_t x = (uint32_t)__builtin_amdgcn_readlane((int)pre, 63) - pre + tot;
    if (lane == 0) sh.fb_w[wave] = x;
    __syncthreads();
    uint32_t before_w, after_w, total_w;
    cross_wave_sums<NT>(sh.fb_w, before_w, after_w, total_w);
    uint32_t acc = x - tot + after_w;
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
      for (int i = 0; i < KP; ++i)
        if ((uint32_t)i * NT < nk)
          wave_append(key[i] != 0ull && word_bin<NT>((uint32_t)(key[i] >> 32), blo, small, mul) == b,
                    key[i], sh.list, &sh.n_list, kListCap);
      for (uint32_t j0 = 0; j0 < n_x; j0 += NT) {
        const uint32_t j = j0 + tid;
        const uint64_t v = j < n_x ? sh.xk[j] : 0ull;
        wave_append(j < n_x && word_bin<NT>((uint32_t)(v >> 32), blo, small, mul) == b, v, sh.list,
                    &sh.n_list, kListCap);
      }
      __syncthreads();
      for (uint32_t i = (uint32_t)tid; i < in_bin; i += NT) {
        const uint64_t v = sh.list[i];
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
    if (j < (uint32_t)(KP * NT)) {
      // register slot of j is (thread j % NT, index j / NT); only the
      // calling thread's own slots are ever asked for
      const int i = (int)(j / NT);
      uint64_t v = 0ull;
#pragma unroll
      for (int q = 0; q < KP; ++q)
        if (q == i) v = key[q];
      return v;
    }
    return sh.xk[j - KP * NT];
  };
  return radix_kth<NT>(get, (uint32_t)(KP * NT) + n_x, k, sh);
}

// Marks {block of key : key >= thr, key != 0} of the keys in registers, the
// LDS extras and (if any) the row, in the bitmap,
// then lists those at positions [e_lo, e_hi) of the ascending block order at
// dst[0..e_hi-e_lo) (positions below top_k only); returns how
// many were marked.
template <int NT, class Mark>
__device__ __forceinline__ uint32_t emit_bitmap(Mark mark, int64_t n_vis, int top_k,
                                                SelShared<NT>& sh, int32_t* dst, uint32_t e_lo,
                                                uint32_t e_hi) {
  if (e_hi > (uint32_t)top_k) e_hi = (uint32_t)top_k;
  const int tid = threadIdx.x;
  uint32_t emitted = 0;
  const int64_t span = (int64_t)kBitmapWords * 32;
  constexpr int WPT = kBitmapWords / NT;  // bitmap words per thread
  u32x4* bm4 = reinterpret_cast<u32x4*>(sh.bitmap);
  for (int64_t base = 0; base < n_vis; base += span) {
    const int64_t len = min(span, n_vis - base);
    for (int i = tid; i < kBitmapWords / 4; i += NT) bm4[i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
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
    uint32_t o = emitted + block_excl_scan<NT>(mine, sh.scratch, sweep_total);
    if (o < e_hi && o + mine > e_lo) {  // this thread's bits reach the window
#pragma unroll
      for (int q = 0; q < WPT; ++q) {
        uint32_t bits = wv[q];
        const uint32_t c = (uint32_t)__popc(bits);
        if (o < e_hi && o + c > e_lo) {
          while (bits) {
            const int bb = __ffs(bits) - 1;
            bits &= bits - 1u;
            if (o >= e_lo && o < e_hi)
              dst[o - e_lo] = (int32_t)(base + (int64_t)(tid * WPT + q) * 32 + bb);
            ++o;
          }
        } else {
          o += c;
        }
      }
    }
    emitted += sweep_total;
    __syncthreads();
  }
  return emitted;
}

// Emission when the register slots hold keys in ascending block order (slot
// j = tid + i*NT; every visible block in its own slot, or candidate
// lists stored in block order, group after group) and there are no LDS
// extras: a selected key's position is the number of selected keys in lower
// slots.  Each thread packs its slot planes' selected flags two to a word in
// 16-bit fields (a plane counts at most NT), and one workgroup scan of
// the packed words gives every position.  Writes positions [e_lo, e_hi)
// below top_k to dst like emit_bitmap; returns the number selected.
template <int NT, int KP>
__device__ __forceinline__ uint32_t emit_slots(const uint64_t (&key)[KP], uint32_t nk,
                                               uint64_t thr, int top_k, SelShared<NT>& sh,
                                               int32_t* dst, uint32_t e_lo, uint32_t e_hi) {
  constexpr int NP = (KP + 1) / 2;
  constexpr int W = Geo<NT>::kWaves;
  static_assert(NP <= (kMaxKP + 1) / 2, "slot planes");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (e_hi > (uint32_t)top_k) e_hi = (uint32_t)top_k;
  bool sel[KP];
  uint32_t pk[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) pk[p] = 0u;
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    sel[i] = (uint32_t)i * NT < nk && key[i] != 0ull && key[i] >= thr;
    pk[i / 2] |= (sel[i] ? 1u : 0u) << (16 * (i & 1));
  }
  uint32_t incl[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    incl[p] = wave_incl_scan_u32(pk[p]);
    if (lane == 63) sh.plane[p * W + wave] = incl[p];
  }
  __syncthreads();
  uint32_t base = 0;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    uint32_t before, after, total;
    cross_wave_sums<NT>(&sh.plane[p * W], before, after, total);
    const uint32_t excl = before + incl[p] - pk[p];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = 2 * p + h;
      if (i < KP) {
        const uint32_t o = base + ((excl >> (16 * h)) & 0xFFFFu);
        if (sel[i] && o >= e_lo && o < e_hi) dst[o - e_lo] = (int32_t)~(uint32_t)key[i];
        base += (total >> (16 * h)) & 0xFFFFu;
      }
    }
  }
  __syncthreads();
  return base;
}

template <int NT>
__device__ __forceinline__ void mark_block(uint64_t c, int64_t base, int64_t len, SelShared<NT>& sh) {
  const int64_t s = (int64_t)(~(uint32_t)c) - base;
  if (s >= 0 && s < len) atomicOr(&sh.bitmap[s >> 5], 1u << (s & 31));
}

struct SelResult {
  uint32_t emitted;  // selected blocks (<= top_k)
  bool listed;       // the selection's window is in dst; otherwise the blocks are 0..emitted-1
  uint32_t flags;    // CSA_DERR_* found in the token's metadata
};

// Top-k of one token over its scores row `srow` (ld entries, n_vis of them
// visible), holding up to KP keys per thread in registers: every thread of the 1024-thread workgroup calls this with the same
// arguments.  A token whose keys would run past the key buffer (key_row0 < 0
// or key_row0 + n_vis > key_rows) was scored as 0 blocks by the indexer and
// selects nothing here.  `cand`/`gcut` are the token's candidate lists and group bounds
// (list_len keys per group of blocks_per_group blocks, groups_per_token
// groups; list_len == 0 means none).  On return (after a barrier) the
// selection is described by the result and, when listed, by dst: the blocks
// at positions [e_lo, e_hi) of the ascending selection, dst[i] holding
// position e_lo + i (positions at or past the count are not written).
template <int NT, int KP>
__device__ __forceinline__ SelResult select_token(const float* __restrict__ srow, int64_t ld,
                                                  int64_t pos_t, int32_t ncomp_t, int ratio,
                                                  int64_t key_row0, int64_t key_rows,
                                                  int top_k, const uint64_t* __restrict__ cand,
                                                  const uint64_t* __restrict__ gcut, int list_len,
                                                  int groups_per_token, int blocks_per_group,
                                                  SelShared<NT>& sh, int32_t* dst, uint32_t e_lo,
                                                  uint32_t e_hi) {
  const int tid = threadIdx.x;
  // The candidate lists do not depend on the row length, so they are loaded
  // before it is known: every list of the token (empty groups have zero keys)
  // and the bounds of up to two groups per thread.  Every load is
  // unconditional (indices clamped into the arrays) and masked afterwards,
  // so that all of them are in flight together.
  const uint32_t L = list_len > 0 ? (uint32_t)list_len : 1u;
  const uint32_t NG = list_len > 0 ? (uint32_t)groups_per_token : 0u;
  const uint32_t CT = NG * L <= (uint32_t)(KP * NT) ? NG * L : 0u;  // NG <= kMaxGroups (plan_topk)
  uint64_t key[KP];
  constexpr int GPT = Geo<NT>::kGPT;
  uint64_t gc[GPT];
  if (CT > 0u) {
#pragma unroll
    for (int i = 0; i < KP; ++i)
      key[i] = (uint32_t)i * NT < CT ? cand[min((uint32_t)tid + (uint32_t)i * NT, CT - 1u)]
                                           : 0ull;
#pragma unroll
    for (int i = 0; i < GPT; ++i) gc[i] = gcut[min((uint32_t)tid + (uint32_t)i * NT, NG - 1u)];
#pragma unroll
    for (int i = 0; i < KP; ++i)
      if ((uint32_t)tid + (uint32_t)i * NT >= CT) key[i] = 0ull;
#pragma unroll
    for (int i = 0; i < GPT; ++i)
      if ((uint32_t)tid + (uint32_t)i * NT >= NG) gc[i] = 0ull;
  } else {
#pragma unroll
    for (int i = 0; i < KP; ++i) key[i] = 0ull;
#pragma unroll
    for (int i = 0; i < GPT; ++i) gc[i] = 0ull;
  }
  if (tid == 0) {
    sh.n_ov = 0u;
    sh.n_x = 0u;
  }
  if (tid < kMaxGroups / 32) sh.gflag[tid] = 0u;
  uint32_t f = 0;
  int64_t n_vis = visible_count(pos_t, ratio, ncomp_t, &f);
  if (key_row0 < 0 || key_row0 + n_vis > key_rows) n_vis = 0;  // flagged by the indexer
  if (n_vis > ld) {
    f |= CSA_DERR_VIS_OVER_LD;
    n_vis = ld;
  }
  const uint32_t k_eff = (uint32_t)(n_vis < (int64_t)top_k ? n_vis : (int64_t)top_k);
  __syncthreads();

  SelResult res{0u, false, f};
  if (k_eff == 0) {
    res.emitted = 0;
  } else if ((int64_t)k_eff == n_vis) {
    res.emitted = k_eff;  // every visible block
  } else {
    res.listed = true;
    uint32_t n_x = 0;
    uint32_t nk = 0;  // register key slots in use (i*NT < nk)
    // a long row without candidate lists selects over its scores in memory
    bool global_path = n_vis > KP * NT && CT == 0u;
    uint64_t thr = 0ull;
    if (n_vis <= KP * NT) {
      // ---- direct: every visible block is a key ----
      const uint32_t n = (uint32_t)n_vis;  // >= 1 here
      float sv[KP];
#pragma unroll
      for (int i = 0; i < KP; ++i) sv[i] = srow[min((uint32_t)tid + (uint32_t)i * NT, n - 1u)];
#pragma unroll
      for (int i = 0; i < KP; ++i) {
        const uint32_t j = (uint32_t)tid + (uint32_t)i * NT;
        key[i] = j < n ? block_key(sv[i], j) : 0ull;
      }
      nk = n;
      thr = kth_key<NT, KP>(key, nk, 0, k_eff, sh);
    } else if (!global_path) {
      // ---- candidate lists of the ng groups that cover the row ----
      const uint32_t G = (uint32_t)blocks_per_group;
      const uint32_t ng = ((uint32_t)n_vis + G - 1u) / G;  // n_vis < 2^31
      const uint32_t C = min(ng * L, CT);
      nk = C;
#pragma unroll
      for (int i = 0; i < KP; ++i)
        if ((uint32_t)tid + (uint32_t)i * NT >= C) key[i] = 0ull;
      const uint64_t t1 = C >= k_eff ? kth_key<NT, KP>(key, nk, 0, k_eff, sh) : 0ull;
      // groups that may hold unlisted blocks at or above T1
#pragma unroll
      for (int i = 0; i < GPT; ++i) {
        const uint32_t g = (uint32_t)tid + (uint32_t)i * NT;
        if (g < ng && gc[i] != 0ull && (t1 == 0ull || gc[i] >= t1)) {
          const uint32_t slot = atomicAdd(&sh.n_ov, 1u);
          if (slot < (uint32_t)kMaxOv) sh.ov_g[slot] = g;
          atomicOr(&sh.gflag[g >> 5], 1u << (g & 31));
        }
      }
      __syncthreads();
      const uint32_t n_ov = sh.n_ov;
      global_path = n_ov > (uint32_t)kMaxOv || t1 == 0ull;
      thr = t1;
      if (!global_path && n_ov > 0) {
        uint32_t span_g = 0;  // visible blocks of flagged group tid
        if ((uint32_t)tid < n_ov) {
          const int64_t b0 = (int64_t)sh.ov_g[tid] * G;
          span_g = (uint32_t)min((int64_t)G, n_vis - b0);
        }
        const uint32_t extra = block_sum<NT>(span_g, sh.scratch);
        if (extra > (uint32_t)kXCap) {
          global_path = true;
        } else {
          // a flagged group's listed keys leave the register set ...
          const uint32_t dq = (uint32_t)NT / L, dr = (uint32_t)NT - dq * L;
          uint32_t q = (uint32_t)tid / L, r = (uint32_t)tid - q * L;
#pragma unroll
          for (int i = 0; i < KP; ++i) {
            if ((uint32_t)i * NT < nk && q < ng && ((sh.gflag[q >> 5] >> (q & 31)) & 1u))
              key[i] = 0ull;
            q += dq;
            r += dr;
            if (r >= L) {
              r -= L;
              ++q;
            }
          }
          // ... and every visible block of the group joins the LDS extras
          constexpr int XB = 4;
          const uint32_t span = n_ov * G;
          for (uint32_t e0 = 0; e0 < span; e0 += XB * NT) {
            uint32_t blk[XB];
            bool ok[XB];
            float fv[XB];
#pragma unroll
            for (int u = 0; u < XB; ++u) {
              const uint32_t e = e0 + (uint32_t)u * NT + tid;
              const uint32_t g = e / G;
              const int64_t b = (int64_t)sh.ov_g[g < n_ov ? g : 0] * G + (e - g * G);
              ok[u] = e < span && b < n_vis;
              blk[u] = ok[u] ? (uint32_t)b : 0u;
            }
#pragma unroll
            for (int u = 0; u < XB; ++u) fv[u] = ok[u] ? srow[blk[u]] : 0.0f;
#pragma unroll
            for (int u = 0; u < XB; ++u)
              wave_append(ok[u], ok[u] ? block_key(fv[u], blk[u]) : 0ull, sh.xk, &sh.n_x, kXCap);
          }
          __syncthreads();
          n_x = min(sh.n_x, (uint32_t)kXCap);
          thr = kth_key<NT, KP>(key, nk, n_x, k_eff, sh);
          if (thr == 0ull) global_path = true;
        }
      }
    }
    if (!global_path && n_x == 0u) {
      res.emitted = emit_slots<NT, KP>(key, nk, thr, top_k, sh, dst, e_lo, e_hi);
    } else if (!global_path) {
      auto mark = [&](int64_t base, int64_t len) {
#pragma unroll
        for (int i = 0; i < KP; ++i)
          if ((uint32_t)i * NT < nk && key[i] != 0ull && key[i] >= thr)
            mark_block<NT>(key[i], base, len, sh);
        for (uint32_t j = tid; j < n_x; j += NT)
          if (sh.xk[j] >= thr) mark_block<NT>(sh.xk[j], base, len, sh);
      };
      res.emitted = emit_bitmap<NT>(mark, n_vis, top_k, sh, dst, e_lo, e_hi);
    } else {
      auto getg = [&](uint32_t j) { return block_key(srow[j], j); };
      const uint64_t tg = radix_kth<NT>(getg, (uint32_t)n_vis, k_eff, sh);
      auto mark = [&](int64_t base, int64_t len) {
        for (int64_t j = base + tid; j < base + len; j += NT) {
          const uint64_t c = getg((uint32_t)j);
          if (c >= tg) mark_block<NT>(c, base, len, sh);
        }
      };
      res.emitted = emit_bitmap<NT>(mark, n_vis, top_k, sh, dst, e_lo, e_hi);
    }
  }
  if (res.emitted > (uint32_t)top_k) res.emitted = (uint32_t)top_k;
  return res;
}

// ---------------------------------------------------------------------------
// Fast exact select for the common case.  The keys are in registers, KP
// consecutive slots per thread (slot j = tid*KP + i), slot order being block
// order: every visible block in its own slot, or candidate lists stored in
// block order, group after group.  Per-key work is spread over every thread;
// the work that is the same for the whole workgroup (scanning the histogram,
// ranking the threshold bin) runs in wave 0 alone and reaches the other
// waves through LDS and a barrier: with 16 waves, four share each SIMD, so
// work repeated in every wave costs four times its length.
//   1. range [min, max] of the keys' score words (DPP reductions, one LDS
//      exchange) and a cleared histogram;
//   2. a histogram of kFastBins bins laid linearly over that range (LDS
//      atomics);
//   3. wave 0 reads the histogram (lane l takes the 16-byte groups q*64 + l,
//      conflict-free) and finds the threshold bin with four DPP scans;
//   4. the keys of that bin go to one LDS array (one LDS atomic per wave
//      places each wave's run), and each 16-lane row ranks one of them: its
//      lanes count the larger keys among four slots apiece, the row sums the
//      counts, and the key of rank need - 1 is the threshold;
//   5. each thread checks its group bounds against it and counts its
//      selected keys, and one exchange gives each thread its first output
//      position.
// It gives up (returns false, uniformly, after a barrier) when a group bound
// reaches the threshold (the group may hide unlisted keys at or above it),
// when all keys share one score value, or when the threshold bin is crowded;
// the caller then runs select_token, which handles every case.  Lane reads
// (readlane, ballot) are all made where every lane of the wave is active.
// Sum over each 16-lane row, in every lane of the row: DPP quad swaps, then
// the half-row and row mirrors.
__device__ __forceinline__ uint32_t row_sum16_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);   // quad [1,0,3,2]
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);   // quad [2,3,0,1]
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);  // half-row mirror
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false);  // row mirror
  return v;
}

constexpr int kFastBins = 1024;
constexpr int kFastQ = kFastBins / 256;  // 16-byte histogram groups per lane
constexpr int kFastBinCap = 64;
template <int NT>
struct FastShared {
  static constexpr int W = NT / 64;
  uint32_t hist[kFastBins];
  uint64_t bk[kFastBinCap];  // the keys of the threshold bin, in no order
  uint32_t nb;               // keys placed in bk so far
  uint32_t wmin[W], wmax[W], wsel[W], wflag[W];
  uint32_t bin, need, in_bin, total;  // wave 0's verdict on the histogram
  uint64_t thr;                       // wave 0's k-th key
};

// On success the selected blocks at positions [e_lo, e_hi) of the ascending
// selection are at dst[0 .. e_hi - e_lo) (positions past the count are not
// written), *emitted is k, and a barrier has passed.
template <int NT, int KP, int GB>
__device__ __forceinline__ bool fast_select(const uint64_t (&key)[KP], const uint64_t (&gb)[GB],
                                            uint32_t k, FastShared<NT>& sh, int32_t* dst,
                                            uint32_t e_lo, uint32_t e_hi, uint32_t* emitted) {
  constexpr int W = NT / 64;
  static_assert(W * 4 == kFastBinCap, "step 4 ranks four keys per wave");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // ---- 1. range; clear the histogram ----
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const uint32_t h = (uint32_t)(key[i] >> 32);
    lo = min(lo, key[i] != 0ull ? h : 0xFFFFFFFFu);
    hi = max(hi, h);
  }
  for (int b = tid; b < kFastBins; b += NT) sh.hist[b] = 0u;
  if (tid == 0) sh.nb = 0u;
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane == 0) {
    sh.wmin[wave] = lo;
    sh.wmax[wave] = hi;
  }
  __syncthreads();
  // The keys still in play have score words in [blo, bhi]; kk of them are
  // at or above the threshold.  A pass bins them linearly over that range;
  // when the threshold bin is crowded (a few far outliers stretch the range)
  // the next pass re-bins that bin's keys alone, over their own range.
  uint32_t blo = wave_min_u32(lane < W ? sh.wmin[lane] : 0xFFFFFFFFu);
  uint32_t bhi = wave_max_u32(lane < W ? sh.wmax[lane] : 0u);
  if (bhi == 0u || bhi == blo) {  // no keys, or a single score value
    __syncthreads();
    return false;
  }
  uint32_t kk = k;
  bool small = false;
  uint32_t mul = 0u;
  auto in_play = [&](uint64_t c) {
    const uint32_t h = (uint32_t)(c >> 32);
    return c != 0ull && h >= blo && h <= bhi;
  };
  auto bin_of = [&](uint64_t c) {
    const uint32_t d = (uint32_t)(c >> 32) - blo;
    return small ? d : min(__umulhi(d, mul), (uint32_t)kFastBins - 1u);
  };
  uint32_t b = 0, need = 0, in_bin = 0;
  for (int pass = 0;; ++pass) {
    const uint32_t range = bhi - blo;
    small = range < (uint32_t)kFastBins;
    mul = small ? 0u
                : (uint32_t)((float)kFastBins * 4294967296.0f / ((float)range + 1.0f) * 0.99999f);
    // ---- 2. histogram ----
#pragma unroll
    for (int i = 0; i < KP; ++i)
      if (in_play(key[i])) atomicAdd(&sh.hist[bin_of(key[i])], 1u);
    __syncthreads();
    // ---- 3. wave 0: the threshold bin.  Lane l holds bins 256*q + 4*l + e;
    // bins descend with q, then lane, then e ----
    if (wave == 0) {
      uint32_t c[kFastQ][4], tq[kFastQ], incl[kFastQ], qtot[kFastQ];
#pragma unroll
      for (int q = 0; q < kFastQ; ++q) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(&sh.hist[(q * 64 + lane) * 4]);
        c[q][0] = x.x;
        c[q][1] = x.y;
        c[q][2] = x.z;
        c[q][3] = x.w;
        tq[q] = x.x + x.y + x.z + x.w;
      }
#pragma unroll
      for (int q = 0; q < kFastQ; ++q) {
        incl[q] = wave_incl_scan_u32(tq[q]);
        qtot[q] = (uint32_t)__builtin_amdgcn_readlane((int)incl[q], 63);
      }
      uint32_t total = 0;
#pragma unroll
      for (int q = 0; q < kFastQ; ++q) total += qtot[q];
      // the (q, lane) holding the threshold bin, and the keys above that lane
      uint32_t fq = 0, above_fq = 0, base = 0;
      uint64_t own = 0ull;
#pragma unroll
      for (int q = kFastQ - 1; q >= 0; --q) {
        const uint32_t above_l = base + qtot[q] - incl[q];  // bins of higher q or higher lanes
        const uint64_t m = __ballot(above_l < kk && above_l + tq[q] >= kk);
        if (own == 0ull && m != 0ull) {  // wave-uniform
          own = m;
          fq = (uint32_t)q;
          above_fq = above_l;
        }
        base += qtot[q];
      }
      const int L = own != 0ull ? __ffsll((unsigned long long)own) - 1 : 0;
      uint32_t cf[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cf[e] = c[0][e];
#pragma unroll
        for (int q = 1; q < kFastQ; ++q)
          if (fq == (uint32_t)q) cf[e] = c[q][e];
      }
      uint32_t bsel = 0, babove = 0, bcnt = 0, acc = above_fq;
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        if (acc < kk && acc + cf[e] >= kk) {
          bsel = 256u * fq + 4u * (uint32_t)lane + (uint32_t)e;
          babove = acc;
          bcnt = cf[e];
        }
        acc += cf[e];
      }
      const uint32_t vb = (uint32_t)__builtin_amdgcn_readlane((int)bsel, L);
      const uint32_t va = (uint32_t)__builtin_amdgcn_readlane((int)babove, L);
      const uint32_t vc = (uint32_t)__builtin_amdgcn_readlane((int)bcnt, L);
      if (lane == 0) {
        sh.bin = vb;
        sh.need = kk - va;
        sh.in_bin = vc;
        sh.total = total;
      }
    }
    __syncthreads();
    b = sh.bin;
    need = sh.need;
    in_bin = sh.in_bin;
    if (sh.total < kk) {
      __syncthreads();
      return false;
    }
    if (in_bin <= (uint32_t)kFastBinCap) break;
    if (small || pass == 2) {  // one score value per bin already, or still crowded
      __syncthreads();
      return false;
    }
    // ---- narrow to the threshold bin: its keys' range, a cleared histogram ----
    uint32_t nlo = 0xFFFFFFFFu, nhi = 0u;
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      if (in_play(key[i]) && bin_of(key[i]) == b) {
        const uint32_t h = (uint32_t)(key[i] >> 32);
        nlo = min(nlo, h);
        nhi = max(nhi, h);
      }
    }
    nlo = wave_min_u32(nlo);
    nhi = wave_max_u32(nhi);
    // (wave 0 read the histogram before the last barrier, and every wave
    // read wmin / wmax before the one ahead of the histogram)
    for (int e = tid; e < kFastBins; e += NT) sh.hist[e] = 0u;
    if (lane == 0) {
      sh.wmin[wave] = nlo;
      sh.wmax[wave] = nhi;
    }
    __syncthreads();
    blo = wave_min_u32(lane < W ? sh.wmin[lane] : 0xFFFFFFFFu);
    bhi = wave_max_u32(lane < W ? sh.wmax[lane] : 0u);
    kk = need;
    if (bhi == blo) {  // the bin is one score value: ties the bins cannot split
      __syncthreads();
      return false;
    }
  }
  // ---- 4. the bin's keys (in_bin <= kFastBinCap of them) into bk, then
  // row r of wave w ranks key 4w + r: lane c of the row counts the larger
  // keys among slots 4c .. 4c+3 (keys are unique), and the row's sum is the
  // key's rank ----
  uint64_t bm[KP];
  uint32_t wcnt = 0;
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    bm[i] = __ballot(in_play(key[i]) && bin_of(key[i]) == b);
    wcnt += (uint32_t)__popcll(bm[i]);
  }
  if (wcnt != 0u) {  // wave-uniform
    uint32_t o = 0;
    if (lane == 0) o = atomicAdd(&sh.nb, wcnt);
    o = (uint32_t)__builtin_amdgcn_readfirstlane((int)o);
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      if ((bm[i] >> lane) & 1ull) sh.bk[o + (uint32_t)__popcll(bm[i] & ((1ull << lane) - 1ull))] = key[i];
      o += (uint32_t)__popcll(bm[i]);
    }
  }
  __syncthreads();
  {
    const uint32_t j = 4u * (uint32_t)wave + (uint32_t)(lane >> 4);
    const uint32_t m0 = 4u * (uint32_t)(lane & 15);
    const uint64_t kj = j < in_bin ? sh.bk[j] : 0ull;
    uint32_t gt = 0;
#pragma unroll
    for (uint32_t e = 0; e < 4u; ++e) {
      const uint64_t km = m0 + e < in_bin ? sh.bk[m0 + e] : 0ull;
      gt += km > kj ? 1u : 0u;
    }
    gt = row_sum16_u32(gt);
    if ((lane & 15) == 0 && j < in_bin && gt == need - 1u) sh.thr = kj;
  }
  __syncthreads();
  // ---- 5. group bounds and output positions ----
  const uint64_t thr = sh.thr;
  bool flagged = false;
#pragma unroll
  for (int g = 0; g < GB; ++g) flagged |= gb[g] != 0ull && gb[g] >= thr;
  uint32_t selc = 0;
#pragma unroll
  for (int i = 0; i < KP; ++i) selc += (key[i] != 0ull && key[i] >= thr) ? 1u : 0u;
  const uint32_t sincl = wave_incl_scan_u32(selc);
  const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)sincl, 63);
  const uint64_t fl = __ballot(flagged);
  if (lane == 0) {
    sh.wsel[wave] = wtot;
    sh.wflag[wave] = fl != 0ull ? 1u : 0u;
  }
  __syncthreads();
  const uint32_t ws = lane < W ? sh.wsel[lane] : 0u;
  const uint32_t any_flag = __ballot(lane < W && sh.wflag[lane] != 0u) != 0ull ? 1u : 0u;
  if (any_flag != 0u) {
    __syncthreads();
    return false;
  }
  const uint32_t wsi = wave_incl_scan_u32(ws);
  const uint32_t before = (uint32_t)__builtin_amdgcn_readlane((int)(wsi - ws), wave);
  uint32_t o = before + sincl - selc;
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    if (key[i] != 0ull && key[i] >= thr) {
      if (o >= e_lo && o < e_hi) dst[o - e_lo] = (int32_t)~(uint32_t)key[i];
      ++o;
    }
  }
  *emitted = k;
  __syncthreads();
  return true;
}

// The decode step's select of one token: the fast select over KP register
// keys per thread (the token's candidate lists, or every visible block of a
// row of at most KP*NT blocks), and select_token when the fast select gives
// up or the keys do not fit.  lists_complete: the lists are the whole
// candidate set (the E4M3 prefilter's rescored keys), to be used whatever
// the row's length.  fsh and ssh may overlay each other.  Same contract as
// select_token.
template <int NT, int KP = 4>
__device__ __forceinline__ SelResult step_select(
    const float* __restrict__ srow, int64_t ld, int64_t pos_t, int32_t ncomp_t, int ratio,
    int64_t key_row0, int64_t key_rows, int top_k, const uint64_t* __restrict__ cand,
    const uint64_t* __restrict__ gcut, int list_len, int groups_per_token, int blocks_per_group,
    bool lists_complete, FastShared<NT>& fsh, SelShared<NT>& ssh, int32_t* dst, uint32_t e_lo,
    uint32_t e_hi) {
  constexpr int GB = kMaxGroups / NT;
  const uint32_t tid = threadIdx.x;
  const uint32_t L = list_len > 0 ? (uint32_t)list_len : 1u;
  const uint32_t NG = list_len > 0 ? (uint32_t)groups_per_token : 0u;
  const uint32_t CT = NG * L;
  const bool lists = CT > 0u && CT <= (uint32_t)(KP * NT);
  // every load is unconditional (indices clamped) and masked afterwards, so
  // that all are in flight together with the caller's own loads
  uint64_t key[KP];
  uint64_t gb[GB];
  float sv[KP];
  const uint32_t nl = (uint32_t)min(ld, (int64_t)(KP * NT));
  if (lists) {
#pragma unroll
    for (int i = 0; i < KP; ++i) key[i] = cand[min(tid * KP + (uint32_t)i, CT - 1u)];
#pragma unroll
    for (int g = 0; g < GB; ++g) gb[g] = gcut[min(tid + (uint32_t)(g * NT), NG - 1u)];
  } else {
#pragma unroll
    for (int i = 0; i < KP; ++i) sv[i] = srow[min(tid * KP + (uint32_t)i, nl - 1u)];
  }
  uint32_t f = 0;
  int64_t n_vis = visible_count(pos_t, ratio, ncomp_t, &f);
  if (key_row0 < 0 || key_row0 + n_vis > key_rows) n_vis = 0;  // flagged by the indexer
  if (n_vis > ld) {
    f |= CSA_DERR_VIS_OVER_LD;
    n_vis = ld;
  }
  const uint32_t k_eff = (uint32_t)(n_vis < (int64_t)top_k ? n_vis : (int64_t)top_k);
  SelResult res{0u, false, f};
  if (k_eff == 0u) return res;
  if ((int64_t)k_eff == n_vis) {
    res.emitted = k_eff;  // every visible block
    return res;
  }
  bool ok = false;
  if (lists && !lists_complete && n_vis <= (int64_t)(KP * NT)) {
    // a row short enough to hold every block beats its lists (which may hold
    // fewer than top_k keys): its scores, in one more round trip
#pragma unroll
    for (int i = 0; i < KP; ++i) sv[i] = srow[min(tid * KP + (uint32_t)i, (uint32_t)n_vis - 1u)];
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const uint32_t j = tid * KP + (uint32_t)i;
      key[i] = j < (uint32_t)n_vis ? block_key(sv[i], j) : 0ull;
    }
#pragma unroll
    for (int g = 0; g < GB; ++g) gb[g] = 0ull;
    ok = fast_select<NT, KP, GB>(key, gb, k_eff, fsh, dst, e_lo, e_hi, &res.emitted);
  } else if (lists) {
    // the candidate lists of the groups that cover the row
    const uint32_t G = (uint32_t)blocks_per_group;
    const uint32_t ng = ((uint32_t)n_vis + G - 1u) / G;
    const uint32_t C = min(ng * L, CT);
#pragma unroll
    for (int i = 0; i < KP; ++i)
      if (tid * KP + (uint32_t)i >= C) key[i] = 0ull;
#pragma unroll
    for (int g = 0; g < GB; ++g)
      if (tid + (uint32_t)(g * NT) >= ng) gb[g] = 0ull;
    ok = fast_select<NT, KP, GB>(key, gb, k_eff, fsh, dst, e_lo, e_hi, &res.emitted);
  } else if (n_vis <= (int64_t)(KP * NT)) {
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const uint32_t j = tid * KP + (uint32_t)i;
      key[i] = j < (uint32_t)n_vis ? block_key(sv[i], j) : 0ull;
    }
#pragma unroll
    for (int g = 0; g < GB; ++g) gb[g] = 0ull;
    ok = fast_select<NT, KP, GB>(key, gb, k_eff, fsh, dst, e_lo, e_hi, &res.emitted);
  }
  if (ok) {
    res.listed = true;
    return res;
  }
  return select_token<NT, KP>(srow, ld, pos_t, ncomp_t, ratio, key_row0, key_rows, top_k, cand,
                              gcut, list_len, groups_per_token, blocks_per_group, ssh, dst, e_lo,
                              e_hi);
}

}  // namespace sel
}  // namespace
}  // namespace csa
