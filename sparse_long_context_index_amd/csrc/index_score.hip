// S1 -- lightning-indexer scoring on gfx950 bf16 MFMA.
//
// Computes, per query token t and visible block s (post-probe audit, F1/F3;
// eq. 16 of DeepSeek-V4 sec. 2.3.1 as restated there):
//     I[t,s] = sum_h w[t,h] * ReLU(q_idx[t,h,:] . K[s,:])
// with one key row per block shared by every indexer head.
//
// Mapping: indexer heads are the MFMA M dimension (32-row tiles, padded with
// zero queries and zero weights), compressed blocks are N (32 blocks per
// v_mfma_f32_32x32x16_bf16 tile), ihd is K.  The (heads x blocks) logits never
// leave the accumulators: ReLU, the per-head weight and the head sum are
// applied in registers, the two half-waves are added with one cross-lane
// exchange, and one fp32 score per block is produced.
//
// Decode is HBM-bound (64 flop per key byte at n_ih = 64, far below the MFMA
// ridge), so the kernel is built around streaming the keys:
//   * a workgroup is eight waves, one workgroup per CU on a 1M-block row;
//     every wave walks a contiguous run of 32-block tiles; each tile is
//     fetched with global_load_lds_dwordx4, 1 KiB (whole key rows) per
//     instruction, straight into a per-wave LDS buffer -- no VGPRs, fully
//     coalesced, two tiles in flight (double buffer);
//   * the 16-byte chunk slots of each row are XOR-swizzled by the row index,
//     chosen through the per-lane global address, so that the MFMA operand
//     reads (lane = block column or head, 16 bytes of that row) are
//     bank-conflict free;
//   * the token's query block (the same for every wave) is brought into LDS
//     once per workgroup by the same DMA, together with the token metadata
//     and head weights (one round trip), instead of every wave reading it
//     from L2; the first key tiles are issued before the one workgroup
//     barrier, after which each wave copies its query operands to VGPRs.
//     The only memory operations pending in the loop are then tile DMAs,
//     waited for with explicit vmcnt counts; the tile loop is unrolled so the
//     per-tile scores stay in VGPRs until the wave's tiles are done.
//
// Optionally the epilogue also emits the candidate lists of the top-k: each
// wave's top-m composite selection keys (score, then lower block index),
// merged per workgroup when the plan asks for it.
#include <type_traits>

#include "csa_common.h"

namespace csa {
namespace {

constexpr int kTileN = 32;
constexpr int kWaves = kIndexWaves;
constexpr int kMaxTpw = 8;  // tiles per wave (scores held in VGPRs)
// Lists of up to this many keys are rebuilt by rounds of wave maxima; longer
// ones by a rank merge (whose cost does not grow with the list).
constexpr int kMergeRoundsMax = 8;

__device__ __forceinline__ void lds_dma16(const void* gsrc, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(gsrc, lds_dst, 16, 0, 0);
}

// The same DMA, issued so that the compiler does not track it.  For a ring
// of LDS tiles indexed at run time the compiler cannot tell which slot a
// read touches and would wait for every DMA in flight before each read; the
// ring's users order their reads with explicit vmcnt waits and barriers
// instead.  (No VGPR is written: the data goes to LDS at M0 + 16 * lane.)
__device__ __forceinline__ void lds_dma16_untracked(const void* gsrc, void* lds_dst) {
  // M0 is kept as it was: the DMA reads it when it issues.
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds_dst));
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(keep)
      : "v"(gsrc), "s"(m0)
      : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// The group of tiles of workgroup L among G.  The dispatcher deals
// workgroups to the eight XCDs in turn (L % 8), so with groups in workgroup
// order XCD x would read only groups x, x + 8, ...: one fixed eighth of every
// eight consecutive groups (at 1M, of every 2 MiB of keys), at a rate that was
// measured to differ from XCD to XCD by up to a fifth.  The diagonal order
// gives XCD x the groups 8k + (x + k) % 8 instead, every position equally
// often.
__device__ __forceinline__ int index_group(int L, int G) {
  return (G & 7) == 0 ? (L & ~7) | (((L & 7) + (L >> 3)) & 7) : L;
}

// Merges one scored tile into a wave's running candidate list while the next
// tile's DMA is in flight: lanes r < m hold the r-th largest composite key of
// the wave's blocks so far (sorted, descending; zero beyond its valid blocks)
// and n_ok counts them.  Lanes 32..63 hold the tile's scores (part) for blocks
// tile_blk0 + lane % 32 (the same scores as lanes 0..31); blocks at or past
// n_vis are not keys.
__device__ __forceinline__ void list_merge_tile(uint64_t& rl, uint32_t& n_ok, float part,
                                                int64_t tile_blk0, int64_t n_vis, int m) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  const int64_t b = tile_blk0 + col;
  const bool tv = half == 1 && b < n_vis;
  const uint32_t tsk = tv ? score_key(part) : 0u;
  const uint64_t tkey = tsk != 0u ? ((uint64_t)tsk << 32) | (uint32_t)~(uint32_t)b : 0ull;
  n_ok += (uint32_t)__popcll(__ballot(tv));
  const uint64_t cut = readlane_u64(rl, m - 1);  // 0 until the list is full
  uint64_t cmask = __ballot(tkey > cut);
  const int nc = __popcll(cmask);
  if (nc > 0 && nc <= 8) {
    // few keys beat the list: insert each (lane i takes its own entry,
    // the key, or the entry above it; m <= 32, so only lane 16 needs
    // its upper neighbour from another row)
    while (cmask != 0ull) {
      const int l = __ffsll((unsigned long long)cmask) - 1;
      cmask &= cmask - 1ull;
      const uint64_t k = readlane_u64(tkey, l);
      uint64_t prev = row_shr1_u64(rl);  // lane 0 of a row: all ones
      const uint64_t r15 = readlane_u64(rl, 15);
      if (lane == 16) prev = r15;
      if (lane < m) rl = rl > k ? rl : (prev > k ? k : prev);
    }
  } else if (nc > 0 && m > kMergeRoundsMax) {
    // Rank merge of the list (lanes 0..31, sorted, descending) with the
    // tile (lanes 32..63): a key's rank is the number of larger keys
    // among the 64 (keys are unique where nonzero).  A list key's rank
    // is its lane plus the tile keys above it; a tile key's, the list
    // keys and the tile keys above it.  Each key then moves to the
    // lane of its rank (ds_permute), which keeps the list sorted.
    const uint64_t mine = half == 1 ? tkey : rl;
    uint32_t rank = half == 1 ? 0u : (uint32_t)lane;
#pragma unroll 8
    for (int j = 0; j < 32; ++j) {
      const uint64_t tj = readlane_u64(tkey, 32 + j);
      const uint64_t lj = readlane_u64(rl, j);
      rank += tj > mine ? 1u : 0u;
      if (half == 1) rank += lj > mine ? 1u : 0u;
    }
    const uint32_t nnz = (uint32_t)__popcll(__ballot(mine != 0ull));
    const int addr = (int)(min(rank, 63u) * 4u);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_permute(addr, (int)(uint32_t)(mine >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_permute(addr, (int)(uint32_t)mine);
    const uint64_t got = ((uint64_t)hi << 32) | lo;
    if (lane < m) rl = (uint32_t)lane < nnz ? got : 0ull;
  } else if (nc > 0) {
    // wave_m rounds over the list (lanes 0..31) and the tile (lanes
    // 32..63): lane order is block order for equal scores
    uint32_t sk = half == 1 ? tsk : (uint32_t)(rl >> 32);
    const uint32_t lo = half == 1 ? (uint32_t)tkey : (uint32_t)rl;
    const uint32_t avail = (uint32_t)__popcll(__ballot(sk != 0u));
    const uint32_t take = avail < (uint32_t)m ? avail : (uint32_t)m;
    uint64_t nrl = 0ull;
    for (uint32_t r = 0; r < take; ++r) {
      const uint64_t kr = wave_take_max(sk, lo);
      if (lane == (int)r) nrl = kr;
    }
    rl = nrl;
  }
}

// Exclusive prefix over the lanes of a per-lane count c < 8: three ballots
// of its bits, each counted below the lane.
__device__ __forceinline__ uint32_t lane_prefix8(uint32_t c, uint32_t* total) {
  const uint64_t b0 = __ballot(c & 1u), b1 = __ballot(c & 2u), b2 = __ballot(c & 4u);
  auto below = [](uint64_t b) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
  };
  *total = (uint32_t)(__popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2));
  return below(b0) + 2u * below(b1) + 4u * below(b2);
}

// The candidate lists of NG consecutive groups of one token from their
// scores, all at once.  Each group gets the list the tile-by-tile merge above
// ends with (the m <= 32 largest composite keys of its valid blocks), stored
// in block order with zeros after the keys, and its bound (the m-th key when
// more than m blocks are valid, else zero).  Group g's n_blk blocks (a
// multiple of 32, at most 256) start at block blk0 + g * n_blk, their scores
// at sc + g * n_blk, and lane l takes blocks 4l + j, j < 4; groups g >= n_live
// hold no tiles (empty lists), groups g >= n_store are not stored, and blocks
// at or past n_vis are not keys.  A group's m-th largest score key is found
// bit by bit from the top (the largest x with at least m keys >= x), the
// groups' searches in lockstep so that their ballot and count chains overlap;
// a group stops as soon as exactly m keys lie at or above its prefix.
template <int NG>
__device__ __forceinline__ void groups_lists_from_scores(const float* sc, int n_blk, int64_t blk0,
                                                         int64_t n_vis, int m, int n_live,
                                                         int n_store, uint64_t* cand, int list_len,
                                                         uint64_t* gcut) {
  const int lane = threadIdx.x & 63;
  const bool in = 4 * lane < n_blk;
  uint32_t sk[NG][4];
  uint32_t n_ok[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (in && g < n_live) v = *reinterpret_cast<const float4*>(sc + g * n_blk + 4 * lane);
    const float vs[4] = {v.x, v.y, v.z, v.w};
    n_ok[g] = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = in && g < n_live && blk0 + (int64_t)g * n_blk + 4 * lane + j < n_vis;
      sk[g][j] = ok ? score_key(vs[j]) : 0u;
      n_ok[g] += (uint32_t)__popcll(__ballot(ok));
    }
  }
  // thr[g]: the largest value found so far with at least m keys >= it, and
  // cnt[g] how many keys are >= it.  A group is done once exactly m keys are
  // >= thr (then they are its list, whatever the lower bits of the m-th); the
  // search stops when every group is done or the last bit is decided.
  // A group of fewer than m nonzero keys is done at once (thr = 0).
  uint32_t thr[NG], cnt[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    uint32_t nz = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) nz += (uint32_t)__popcll(__ballot(sk[g][j] != 0u));
    thr[g] = 0u;
    cnt[g] = nz < (uint32_t)m ? (uint32_t)m : 256u;  // every slot is >= 0
  }
  for (int bit = 31; bit >= 0; --bit) {
    bool all_done = true;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (cnt[g] == (uint32_t)m) continue;
      all_done = false;
      const uint32_t c = thr[g] | (1u << bit);
      uint32_t n = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) n += (uint32_t)__popcll(__ballot(sk[g][j] >= c));
      if (n >= (uint32_t)m) {
        thr[g] = c;
        cnt[g] = n;
      }
    }
    if (all_done) break;
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (g >= n_store) break;
    uint64_t* list = cand + (int64_t)g * list_len;
    const int64_t gb0 = blk0 + (int64_t)g * n_blk;
    // thr == 0: fewer than m nonzero keys, all listed.  cnt == m: the m keys
    // >= thr (thr > 0).  Otherwise thr is the m-th largest score key itself, shared by
    // several blocks: the keys above it, and of those equal to it the lowest
    // blocks, as many as fill the list.
    uint32_t need = 0;
    if (thr[g] != 0u && cnt[g] != (uint32_t)m) {
      uint32_t n_gt = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) n_gt += (uint32_t)__popcll(__ballot(sk[g][j] > thr[g]));
      need = (uint32_t)m - n_gt;
    }
    bool sel[4];
    uint32_t ce = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) ce += (need != 0u && sk[g][j] == thr[g]) ? 1u : 0u;
    uint32_t n_eq;
    uint32_t r = lane_prefix8(ce, &n_eq);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool eq = need != 0u && sk[g][j] == thr[g];
      sel[j] = thr[g] == 0u ? sk[g][j] != 0u
                            : (need == 0u ? sk[g][j] >= thr[g] : (sk[g][j] > thr[g] || (eq && r < need)));
      r += eq ? 1u : 0u;
    }
    uint32_t cs = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) cs += sel[j] ? 1u : 0u;
    uint32_t n_sel;
    uint32_t p = lane_prefix8(cs, &n_sel);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (sel[j]) list[p++] = ((uint64_t)sk[g][j] << 32) | (uint32_t)~(uint32_t)(gb0 + 4 * lane + j);
    }
    if (lane < m && (uint32_t)lane >= n_sel) list[lane] = 0ull;
    // the bound: the smallest listed composite key (the smallest listed
    // score key, at the highest block that holds it), when blocks were left out
    uint64_t bound = 0ull;
    if (n_ok[g] > (uint32_t)m && thr[g] != 0u) {
      uint32_t lo = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) lo = max(lo, sel[j] ? ~sk[g][j] : 0u);
      const uint32_t smin = ~wave_max_u32(lo);
      uint32_t hb = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        hb = max(hb, sel[j] && sk[g][j] == smin ? (uint32_t)(gb0 + 4 * lane + j) + 1u : 0u);
      const uint32_t b = wave_max_u32(hb) - 1u;
      bound = ((uint64_t)smin << 32) | (uint32_t)~b;
    }
    if (lane == 0) gcut[g] = bound;
  }
}

// Up to 64 indexer heads the register budget is held to two waves per SIMD;
// more heads need more registers and run one wave per SIMD.
//
// F8: queries and keys are OCP FP8 E4M3 codes with one power-of-two scale per
// query head (q_scale [T, n_ih]) and per key block (k_scale [rows]); the
// products run on v_mfma_f32_32x32x16_fp8_fp8 (8 bytes of a row per lane and
// k-step).  A positive per-block scale leaves every head's ReLU in place, so
// I[s] = k_scale[s] * sum_h (w[h] q_scale[h]) ReLU(q8[h] . k8[s]): the query
// scale folds into the head weight and the key scale multiplies the score.
template <int IHD, int MT, bool F8>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(MT <= 2 ? 2 : 1, 2))) void index_score_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k_idx,
    const float* __restrict__ k_scale, int64_t k_rows,
    const int64_t* __restrict__ pos, const int64_t* __restrict__ seq_kv,
    const int32_t* __restrict__ n_comp, int n_ih, int ratio,
    float* __restrict__ scores, int64_t ld, CandArgs ca, uint32_t* __restrict__ err,
    int tiles_per_wave) {
  constexpr int KS = IHD / 16;          // MFMA k-steps of 16 elements
  constexpr int RB = F8 ? IHD : 2 * IHD;  // bytes per key or query row
  constexpr int CPR = RB / 16;          // 16-byte chunks per key or query row
  constexpr int TILE_CHUNKS = kTileN * CPR;
  constexpr int LPT = TILE_CHUNKS / 64; // DMA instructions per tile (1 KiB each)
  constexpr int QCHUNKS = MT * 32 * CPR;
  // Up to 64 heads each wave keeps its query operands in VGPRs; with more,
  // they are read from LDS at every k-step (two waves per SIMD leave no room).
  constexpr bool kQRegs = MT <= 2;
  static_assert(kWaves * 2 * TILE_CHUNKS * 16 + QCHUNKS * 16 <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) u32x4 ktile[kWaves][2][TILE_CHUNKS];
  __shared__ __attribute__((aligned(16))) u32x4 qlds[QCHUNKS];

  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 31;
  const int half = lane >> 5;
  const uint8_t* qt = q_idx + (int64_t)t * n_ih * RB;

  // ---- one round trip: query block (to LDS), head weights, metadata ----
  // Query chunk e = row*CPR + p of the padded head block goes to LDS slot e,
  // holding global chunk p ^ (row % CPR); padded heads re-read the last real
  // head (their weight is zero, so they add nothing).
#pragma unroll
  for (int e0 = 0; e0 < QCHUNKS; e0 += kWaves * 64) {
    const int e = e0 + wave * 64 + lane;
    if (e0 + wave * 64 < QCHUNKS) {  // wave-uniform
      const int r = e / CPR, pp = e % CPR;
      const int hq = r < n_ih ? r : n_ih - 1;
      lds_dma16(qt + (int64_t)hq * RB + (pp ^ (r & (CPR - 1))) * 16, &qlds[e0 + wave * 64]);
    }
  }
  // A operand of k-step s for lane (col, half): q[head = mt*32+col][16*s +
  // 8*half .. +8] (bf16: 16 bytes, chunk 2s + half; E4M3: 8 bytes, half
  // `half` of chunk s); accumulator element r of lane (col, half) is head
  // 8*(r/4) + 4*half + (r%4) of its 32-head tile.
  using Op = typename std::conditional<F8, uint2, u32x4>::type;  // one lane's MFMA operand
  auto q_operand = [&](int mt, int s) -> Op {
    const int r = mt * 32 + col;
    if constexpr (F8) {
      return reinterpret_cast<const uint2*>(qlds)[(r * CPR + (s ^ (r & (CPR - 1)))) * 2 + half];
    } else {
      const int c = 2 * s + half;
      return qlds[r * CPR + (c ^ (r & (CPR - 1)))];
    }
  };
  float wv[MT][16];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int hw = mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      const int64_t hi = (int64_t)t * n_ih + (hw < n_ih ? hw : n_ih - 1);
      wv[mt][r] = F8 ? w[hi] * q_scale[hi] : w[hi];
    }
  }
  // The token metadata and the scalar arguments are read in the same batch
  // (the empty asm takes them as operands), rather than one dependent load
  // after another as the branches below would otherwise order them.
  const int64_t pos_t = pos[t];
  const int32_t ncomp_t = n_comp[t];
  const int64_t row0 = seq_kv[t];
  asm volatile("" ::"s"(pos_t), "s"(ncomp_t), "s"(row0), "s"(k_rows), "s"(ld), "s"(ratio),
               "s"(tiles_per_wave), "s"(n_ih));
  // The first key tiles need only this metadata: they are issued before the
  // query block and head weights are waited for (below).

  uint32_t flags = 0;
  int64_t n_vis = visible_count(pos_t, ratio, ncomp_t, &flags);
  if (row0 < 0) {
    flags |= CSA_DERR_BAD_META;
    n_vis = 0;
  } else if (row0 + n_vis > k_rows) {
    flags |= CSA_DERR_KEY_RANGE;
    n_vis = 0;
  }
  if (n_vis > ld) {
    flags |= CSA_DERR_VIS_OVER_LD;
    n_vis = ld;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) report(err, flags);

  const int64_t n_tiles = (n_vis + kTileN - 1) / kTileN;
  const int grp = index_group((int)blockIdx.x, (int)gridDim.x);
  const int64_t tile_begin = ((int64_t)grp * kWaves + wave) * tiles_per_wave;
  const int64_t tile_end = min(tile_begin + (int64_t)tiles_per_wave, n_tiles);
  const int64_t wave_in_token = (int64_t)grp * kWaves + wave;
  const bool active = tile_begin < tile_end;  // wave-uniform
  const char* kbase = reinterpret_cast<const char*>(k_idx + row0 * RB);

  // DMA of one tile into buffer b: instruction i, lane l -> tile row
  // r = (i*64 + l) / CPR, LDS slot p = l % CPR, holding global chunk p ^ (r % CPR).
  auto issue_tile = [&](int64_t tile, int b) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int e = i * 64 + lane;
      const int r = e / CPR;
      const int p = e % CPR;
      const int c = p ^ (r & (CPR - 1));
      int64_t blk = tile * kTileN + r;
      if (blk > n_vis - 1) blk = n_vis - 1;  // ragged tail: re-read a valid row
      lds_dma16(kbase + blk * RB + c * 16, &ktile[wave][b][i * 64]);
    }
  };
  // E4M3: the key scales of the wave's blocks (lane col's block of each
  // tile), loaded before the first tile DMA so that waiting for a tile also
  // waits for them
  float ksc[kMaxTpw];
  if constexpr (F8) {
#pragma unroll
    for (int j = 0; j < kMaxTpw; ++j) {
      ksc[j] = 1.0f;
      if (j < tiles_per_wave && active) {  // wave-uniform
        int64_t blk = (tile_begin + j) * kTileN + col;
        blk = blk < n_vis ? blk : (n_vis > 0 ? n_vis - 1 : 0);
        ksc[j] = k_scale[row0 + blk];
      }
    }
  }
  const int n_first = active ? (tile_begin + 1 < tile_end ? 2 : 1) : 0;  // wave-uniform
  if (n_first > 0) issue_tile(tile_begin, 0);
  if (n_first > 1) issue_tile(tile_begin + 1, 1);
  // the query DMA and the weight loads, issued before the tiles, have landed
  if (n_first == 2) wait_vmcnt<2 * LPT>();
  else if (n_first == 1) wait_vmcnt<LPT>();
  else wait_vmcnt<0>();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int hw = mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (hw >= n_ih) wv[mt][r] = 0.0f;
    }
  }
  __syncthreads();  // the query block is in LDS for every wave
  // After its last tile each wave's own tile buffers hold its candidate list
  // for the workgroup merge (no DMA into them is pending by then).
  uint64_t* cand_lds = reinterpret_cast<uint64_t*>(&ktile[0][0][0]);
  constexpr int kCandStride = 2 * TILE_CHUNKS * 2;  // u64 words per wave's buffers
  static_assert(kCandStride >= kMergeScratch, "merge scratch fits a wave's buffers");
  if (!active) {
    if (ca.cand != nullptr)  // empty list and bound (and the merge barrier)
      cand_publish(0ull, 0u, ca, t, wave_in_token, grp, cand_lds, kCandStride);
    return;
  }
  Op qv[kQRegs ? MT : 1][KS];
  if constexpr (kQRegs) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < KS; ++s) qv[mt][s] = q_operand(mt, s);
  }

  float sc[kMaxTpw];
  // Running candidate list: lane r < wave_m holds the r-th largest composite
  // key of the wave's blocks so far (zero beyond them); n_ok counts them.
  uint64_t rl = 0ull;
  uint32_t n_ok = 0;
#pragma unroll
  for (int j = 0; j < kMaxTpw; ++j) {
    sc[j] = 0.0f;
    const int64_t tile = tile_begin + j;
    if (tile < tile_end) {  // wave-uniform
      const int b = j & 1;
      // all but the next tile's DMA (if issued) have landed
      if (tile + 1 < tile_end) wait_vmcnt<LPT>(); else wait_vmcnt<0>();
      Op kb[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if constexpr (F8) {
          kb[s] = reinterpret_cast<const uint2*>(&ktile[wave][b][0])[(col * CPR + (s ^ (col & (CPR - 1)))) * 2 + half];
        } else {
          const int c = 2 * s + half;
          kb[s] = ktile[wave][b][col * CPR + (c ^ (col & (CPR - 1)))];
        }
      }
      wait_lgkmcnt0();  // buffer b is free again
      if (tile + 2 < tile_end) issue_tile(tile + 2, b);

      f32x16 acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const Op qa = kQRegs ? qv[kQRegs ? mt : 0][s] : q_operand(mt, s);
          if constexpr (F8)
            acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(
                __builtin_bit_cast(long, qa), __builtin_bit_cast(long, kb[s]), acc[mt], 0, 0, 0);
          else
            acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, qa), __builtin_bit_cast(bf16x8, kb[s]), acc[mt], 0, 0, 0);
        }
      }
      float part = 0.0f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) part += wv[mt][r] * relu_f32(acc[mt][r]);
      }
      part += __shfl_xor(part, 32);
      if constexpr (F8) part *= ksc[j];
      sc[j] = part;
      if (ca.cand != nullptr) list_merge_tile(rl, n_ok, part, tile * kTileN, n_vis, ca.wave_m);
    }
  }

  // coalesced score stores: lanes 0..31 hold consecutive blocks of each tile
  const int nt = (int)(tile_end - tile_begin);
  float* srow = scores + (int64_t)t * ld;
#pragma unroll
  for (int q = 0; q < kMaxTpw; ++q) {
    const int64_t blk = (tile_begin + q) * kTileN + col;
    if (q < nt && half == 0 && blk < n_vis) srow[blk] = sc[q];
  }

  if (ca.cand != nullptr)
    cand_publish(rl, n_ok, ca, t, wave_in_token, grp, cand_lds, kCandStride);
}

// Batches of 2..kBatchMaxT rows: a persistent grid of one workgroup per CU
// over the non-empty 256-block items (token, chunk) of all rows, each
// workgroup taking a contiguous, equal share of them.  A grid of
// (row, chunk) workgroups planned for the longest row leaves the shorter
// rows' workgroups idle and ends in a partly filled round; here every CU
// streams about the same number of tiles.  Wave w takes tile 8*chunk + w of
// each item, with two tiles in flight across item boundaries; the query
// block and head weights are reloaded (pipeline drained) when the token
// changes.  Scores, candidate lists and their layout are those of
// index_score_kernel with one tile per wave.
constexpr int kBatchMaxT = 512;
constexpr int kBatchGrid = 256;

template <int IHD, int MT>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void index_batch_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint16_t* __restrict__ k_idx, int64_t k_rows, const int64_t* __restrict__ pos,
    const int64_t* __restrict__ seq_kv, const int32_t* __restrict__ n_comp, int T, int n_ih,
    int ratio, float* __restrict__ scores, int64_t ld, CandArgs ca, uint32_t* __restrict__ err) {
  constexpr int KS = IHD / 16;
  constexpr int RB = 2 * IHD;
  constexpr int CPR = RB / 16;
  constexpr int TILE_CHUNKS = kTileN * CPR;
  constexpr int LPT = TILE_CHUNKS / 64;
  constexpr int QCHUNKS = MT * 32 * CPR;
  static_assert(kWaves * 2 * TILE_CHUNKS * 16 + QCHUNKS * 16 + (kBatchMaxT + 1) * 4 +
                    kBatchMaxT * 12 <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) u32x4 ktile[kWaves][2][TILE_CHUNKS];
  __shared__ __attribute__((aligned(16))) u32x4 qlds[QCHUNKS];
  __shared__ uint32_t s_pref[kBatchMaxT + 1];  // items before token t
  __shared__ int64_t s_row0[kBatchMaxT];
  __shared__ int32_t s_nvis[kBatchMaxT];
  __shared__ uint32_t s_wsum[kWaves];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;

  // ---- every row's visible blocks and item count; a block-wide scan ----
  uint32_t items = 0;
  if (threadIdx.x < T) {
    const int t = threadIdx.x;
    uint32_t flags = 0;
    int64_t n_vis = visible_count(pos[t], ratio, n_comp[t], &flags);
    const int64_t row0 = seq_kv[t];
    if (row0 < 0) {
      flags |= CSA_DERR_BAD_META;
      n_vis = 0;
    } else if (row0 + n_vis > k_rows) {
      flags |= CSA_DERR_KEY_RANGE;
      n_vis = 0;
    }
    if (n_vis > ld) {
      flags |= CSA_DERR_VIS_OVER_LD;
      n_vis = ld;
    }
    if (blockIdx.x == 0) report(err, flags);
    s_row0[t] = row0 < 0 ? 0 : row0;
    s_nvis[t] = (int32_t)n_vis;
    items = (uint32_t)((n_vis + kTileN * kWaves - 1) / (kTileN * kWaves));
  }
  const uint32_t incl = wave_incl_scan_u32(items);
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) before += v < wave ? s_wsum[v] : 0u;
  if (threadIdx.x < T) s_pref[threadIdx.x + 1] = before + incl;
  if (threadIdx.x == 0) s_pref[0] = 0;
  __syncthreads();
  const uint32_t N = s_pref[T];
  const uint32_t I0 = (uint32_t)(((uint64_t)N * blockIdx.x) / gridDim.x);
  const uint32_t I1 = (uint32_t)(((uint64_t)N * (blockIdx.x + 1)) / gridDim.x);
  if (I0 >= I1) return;  // workgroup-uniform

  // the token of item k (items in order: the token only moves forward)
  int tk = 0;
  auto token_of = [&](uint32_t k, int from) {
    int t = from;
    while (s_pref[t + 1] <= k) ++t;
    return t;
  };
  auto issue_tile = [&](uint32_t k, int b) {
    const int t = token_of(k, tk);
    const int64_t n_vis = s_nvis[t];
    const int64_t tile = (int64_t)(k - s_pref[t]) * kWaves + wave;
    const char* kbase = reinterpret_cast<const char*>(k_idx + s_row0[t] * IHD);
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int e = i * 64 + lane;
      const int r = e / CPR;
      const int p = e % CPR;
      const int c = p ^ (r & (CPR - 1));
      int64_t blk = tile * kTileN + r;
      if (blk > n_vis - 1) blk = n_vis - 1;  // past the row's end: re-read a valid row
      lds_dma16(kbase + blk * RB + c * 16, &ktile[wave][b][i * 64]);
    }
  };
  // both first tiles before the first query load
  issue_tile(I0, 0);
  if (I0 + 1 < I1) issue_tile(I0 + 1, 1);

  float wv[MT][16];
  int cur_t = -1;
  // An item's results are stored one iteration later, after the wait for
  // the next tile, so that the wait never covers stores just issued.
  struct Pending {
    bool ok = false, store = false;
    int t = 0;
    int64_t tile = 0, blk = 0;
    float part = 0.f;
    uint64_t val = 0ull;
    uint32_t n_ok = 0;
  } pd;
  auto flush = [&]() {
    if (!pd.ok) return;  // wave-uniform
    if (pd.store) scores[(int64_t)pd.t * ld + pd.blk] = pd.part;
    if (ca.cand != nullptr) cand_publish(pd.val, pd.n_ok, ca, pd.t, pd.tile, 0, nullptr, 0);
    pd.ok = false;
  };
  tk = token_of(I0, 0);
  for (uint32_t k = I0; k < I1; ++k) {
    const int t = token_of(k, tk);
    tk = t;
    const int b = (int)((k - I0) & 1u);
    if (t != cur_t) {  // workgroup-uniform: drain, then this token's queries and weights
      wait_vmcnt<0>();
      __syncthreads();  // every wave is done with the previous query block
      const uint16_t* qt = q_idx + (int64_t)t * n_ih * IHD;
#pragma unroll
      for (int e0 = 0; e0 < QCHUNKS; e0 += kWaves * 64) {
        const int e = e0 + wave * 64 + lane;
        if (e0 + wave * 64 < QCHUNKS) {  // wave-uniform
          const int r = e / CPR, pp = e % CPR;
          const int hq = r < n_ih ? r : n_ih - 1;
          lds_dma16(reinterpret_cast<const char*>(qt) + (int64_t)hq * RB + (pp ^ (r & (CPR - 1))) * 16,
                    &qlds[e0 + wave * 64]);
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int hw = mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          const float x = w[(int64_t)t * n_ih + (hw < n_ih ? hw : n_ih - 1)];
          wv[mt][r] = hw < n_ih ? x : 0.0f;
        }
      }
      wait_vmcnt<0>();
      __syncthreads();  // the query block is in LDS for every wave
      cur_t = t;
    }
    // all but the next item's tile DMA (if issued) have landed: vector
    // memory operations complete in order, and the stores issued since that
    // DMA are the previous item's, issued an iteration ago
    if (k + 1 < I1) wait_vmcnt<LPT>(); else wait_vmcnt<0>();
    u32x4 kb[KS];
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      const int c = 2 * s2 + half;
      kb[s2] = ktile[wave][b][col * CPR + (c ^ (col & (CPR - 1)))];
    }
    wait_lgkmcnt0();  // buffer b is free again
    flush();          // the previous item's scores and list
    if (k + 2 < I1) issue_tile(k + 2, b);

    f32x16 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};
    // query operands from LDS at each k-step (the registers go to the
    // pipeline and the deferred results)
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = mt * 32 + col;
        const int c = 2 * s2 + half;
        const u32x4 qa = qlds[r * CPR + (c ^ (r & (CPR - 1)))];
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qa),
                                                          __builtin_bit_cast(bf16x8, kb[s2]),
                                                          acc[mt], 0, 0, 0);
      }
    }
    float part = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) part += wv[mt][r] * relu_f32(acc[mt][r]);
    }
    part += __shfl_xor(part, 32);

    const int64_t n_vis = s_nvis[t];
    const int64_t tile = (int64_t)(k - s_pref[t]) * kWaves + wave;
    const int64_t blk = tile * kTileN + col;
    pd.ok = tile * kTileN < n_vis;  // wave-uniform
    pd.t = t;
    pd.tile = tile;
    pd.part = part;
    pd.store = half == 0 && blk < n_vis;
    pd.blk = blk;
    if (ca.cand != nullptr && pd.ok) {
      // the tile's top-m keys in lanes 0..m-1, descending (its group's list)
      const bool tv = half == 1 && blk < n_vis;
      const uint32_t tsk = tv ? score_key(part) : 0u;
      const uint64_t tkey = tsk != 0u ? ((uint64_t)tsk << 32) | (uint32_t)~(uint32_t)blk : 0ull;
      uint32_t rank = 0;
#pragma unroll 8
      for (int j = 0; j < 32; ++j) rank += readlane_u64(tkey, 32 + j) > tkey ? 1u : 0u;
      const uint32_t nnz = (uint32_t)__popcll(__ballot(tkey != 0ull));
      const int addr = (int)(min(rank, 63u) * 4u);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_permute(addr, (int)(uint32_t)(tkey >> 32));
      const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_permute(addr, (int)(uint32_t)tkey);
      const uint64_t got = ((uint64_t)hi << 32) | lo;
      pd.val = lane < ca.wave_m && (uint32_t)lane < nnz ? got : 0ull;
      pd.n_ok = (uint32_t)__popcll(__ballot(tv));
    }
  }
  flush();
}

template <int IHD, int MT>
hipError_t launch_t(const IndexScoreLaunch& a, const IndexPlan& p, hipStream_t s) {
  dim3 grid(p.wgs_per_token, a.T);
  const uint8_t* q = static_cast<const uint8_t*>(a.q_idx);
  const uint8_t* k = static_cast<const uint8_t*>(a.k_idx);
  if (a.e4m3)
    hipLaunchKernelGGL((index_score_kernel<IHD, MT, true>), grid, dim3(kWaves * 64), 0, s, q,
                       a.q_scale, a.w, k, a.k_scale, a.k_rows, a.pos, a.seq_kv, a.n_comp, a.n_ih,
                       a.ratio, a.scores, a.ld, a.cand, a.err, p.tiles_per_wave);
  else
    hipLaunchKernelGGL((index_score_kernel<IHD, MT, false>), grid, dim3(kWaves * 64), 0, s, q,
                       nullptr, a.w, k, nullptr, a.k_rows, a.pos, a.seq_kv, a.n_comp, a.n_ih,
                       a.ratio, a.scores, a.ld, a.cand, a.err, p.tiles_per_wave);
  return hipGetLastError();
}

template <int IHD>
hipError_t launch_ihd(const IndexScoreLaunch& a, const IndexPlan& p, hipStream_t s) {
  switch ((a.n_ih + 31) / 32) {
    case 1: return launch_t<IHD, 1>(a, p, s);
    case 2: return launch_t<IHD, 2>(a, p, s);
    case 3: return launch_t<IHD, 3>(a, p, s);
    case 4: return launch_t<IHD, 4>(a, p, s);
    default: return hipErrorInvalidValue;
  }
}

// Rescoring of the E4M3 prefilter's candidates with the bf16 queries and
// keys.  A wave takes 32 candidates as one MFMA tile: lane (col, half) reads
// its candidate's key row straight into the B operand registers (16 bytes a
// k-step) and its query rows from L2, and the score is formed by the same
// sequence of operations as in the bf16 indexer kernel, so that a candidate's
// score is the bf16 indexer's score of its block.
template <int IHD, int MT>
__global__ __launch_bounds__(256) void rescore_kernel(RescoreLaunch a) {
  constexpr int KS = IHD / 16;
  constexpr int RB = 2 * IHD;
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  if (blockIdx.x == 0 && threadIdx.x == 0) a.gcut[t] = 0ull;
  const int64_t j0 = ((int64_t)blockIdx.x * 4 + wave) * 32;
  if (j0 >= a.C) return;  // wave-uniform
  const int64_t j = j0 + col;
  uint64_t* out = a.key + (int64_t)t * a.C;
  // one round trip: the count, this lane's candidate slot (clamped into the
  // C slots), the token's first key row, then (below) its queries and weights
  const int32_t cnt = a.count[t];
  const int32_t bj = a.idx[(int64_t)t * a.C + (j < a.C ? j : a.C - 1)];
  const int64_t row0 = a.seq_kv[t];
  if (j0 >= cnt) {  // wave-uniform: no candidate in this tile
    if (half == 0 && j < a.C) out[j] = 0ull;
    return;
  }
  // lanes past the count take lane 0's candidate (j0 < cnt: a valid row)
  const bool valid = j < cnt;
  const int32_t b = valid ? bj : __shfl(bj, 0);
  const char* krow = reinterpret_cast<const char*>(a.k_idx) + (row0 + b) * RB;
  u32x4 kb[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) kb[s] = *reinterpret_cast<const u32x4*>(krow + (2 * s + half) * 16);
  u32x4 qa[MT][KS];
  float wv[MT][16];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int hq = mt * 32 + col < a.n_ih ? mt * 32 + col : a.n_ih - 1;
    const char* qrow = reinterpret_cast<const char*>(a.q_idx) + ((int64_t)t * a.n_ih + hq) * RB;
#pragma unroll
    for (int s = 0; s < KS; ++s) qa[mt][s] = *reinterpret_cast<const u32x4*>(qrow + (2 * s + half) * 16);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int hw = mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      wv[mt][r] = hw < a.n_ih ? a.w[(int64_t)t * a.n_ih + hw] : 0.0f;
    }
  }
  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qa[mt][s]),
                                                        __builtin_bit_cast(bf16x8, kb[s]), acc[mt],
                                                        0, 0, 0);
  }
  float part = 0.0f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) part += wv[mt][r] * relu_f32(acc[mt][r]);
  }
  part += __shfl_xor(part, 32);
  const uint32_t sk = score_key(part);
  if (half == 0 && j < a.C)
    out[j] = valid && sk != 0u ? ((uint64_t)sk << 32) | (uint32_t)~(uint32_t)b : 0ull;
}

template <int IHD>
hipError_t launch_rescore_ihd(const RescoreLaunch& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.C + 127) / 128), (unsigned)a.T);
  switch ((a.n_ih + 31) / 32) {
    case 1: hipLaunchKernelGGL((rescore_kernel<IHD, 1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((rescore_kernel<IHD, 2>), grid, dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL((rescore_kernel<IHD, 3>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((rescore_kernel<IHD, 4>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int IHD>
hipError_t launch_batch_ihd(const IndexScoreLaunch& a, hipStream_t s) {
  const uint16_t* q = static_cast<const uint16_t*>(a.q_idx);
  const uint16_t* k = static_cast<const uint16_t*>(a.k_idx);
  if (a.n_ih <= 32)
    hipLaunchKernelGGL((index_batch_kernel<IHD, 1>), dim3(kBatchGrid), dim3(kWaves * 64), 0, s, q,
                       a.w, k, a.k_rows, a.pos, a.seq_kv, a.n_comp, a.T, a.n_ih, a.ratio, a.scores,
                       a.ld, a.cand, a.err);
  else
    hipLaunchKernelGGL((index_batch_kernel<IHD, 2>), dim3(kBatchGrid), dim3(kWaves * 64), 0, s, q,
                       a.w, k, a.k_rows, a.pos, a.seq_kv, a.n_comp, a.T, a.n_ih, a.ratio, a.scores,
                       a.ld, a.cand, a.err);
  return hipGetLastError();
}

bool batch_indexer(int T, int n_ih, int ihd, int e4m3) {
  return T > 1 && T <= kBatchMaxT && n_ih <= 64 && !e4m3 && (ihd == 64 || ihd == 128);
}

// ---------------------------------------------------------------------------
// Many query tokens of one sequence (a prefill chunk, one_seq): the scores of
// T tokens are one GEMM of (tokens x heads) by blocks, and a key tile staged
// once in LDS serves eight tokens.  A workgroup is eight waves, wave w scoring
// token 8*blockIdx.y + w over kGemmGroups consecutive groups of the decode
// plan (tiles_per_wave 32-block tiles each, so that the scores and candidate
// lists come out exactly as the decode kernel's).  The eight waves share a
// ring of kGemmSlots key tiles: wave p DMAs the p-th 1 KiB of every tile,
// kGemmDepth tiles ahead, and one barrier per tile publishes a tile to all.
// Queries and head weights stay in VGPRs.  Each wave keeps its token's
// scores in LDS and stores them after the tile loop (a store among the
// counted DMA waits would make the counts ambiguous: loads and stores share
// the counter and need not complete in order); the candidate list of each
// group is then built from the group's scores at once, not merged tile by
// tile as in the decode kernel, which left the tile loop bound by that
// merge's VALU work.
constexpr int kGemmGroups = 4;
constexpr int kGemmSlots = 12;
constexpr int kGemmDepth = 8;
constexpr int kGemmMinT = 64;
static_assert(kGemmDepth < kGemmSlots, "a slot is refilled after every wave has used it");
static_assert(kWaves == kGemmTokens, "one wave a token");

template <int IHD, int MT>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void index_gemm_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint16_t* __restrict__ k_idx, int64_t k_rows, const int64_t* __restrict__ pos,
    const int64_t* __restrict__ seq_kv, const int32_t* __restrict__ n_comp, int T, int n_ih,
    int ratio, float* __restrict__ scores, int64_t ld, CandArgs ca, uint32_t* __restrict__ err,
    int tpw, int n_groups) {
  constexpr int KS = IHD / 16;
  constexpr int RB = 2 * IHD;             // bytes per key or query row
  constexpr int CPR = RB / 16;            // 16-byte chunks per row
  constexpr int TILE_CHUNKS = kTileN * CPR;
  constexpr int LPT = TILE_CHUNKS / 64;   // DMA instructions (1 KiB) per tile: one per wave p < LPT
  static_assert(LPT <= kWaves, "one DMA instruction per wave and tile");
  constexpr int kMaxTiles = kGemmGroups * kMaxTpw;
  // the key ring, then each wave's scores; before the first key DMA the same
  // bytes stage the eight tokens' query rows (QB bytes a wave)
  constexpr int RING_B = kGemmSlots * TILE_CHUNKS * 16;
  constexpr int SC_B = kWaves * kMaxTiles * kTileN * 4;
  constexpr int QB = MT * 32 * RB;
  static_assert(kWaves * QB <= RING_B + SC_B, "query staging fits the ring and score space");
  __shared__ __attribute__((aligned(16))) char lds_main[RING_B + SC_B];
  __shared__ int64_t s_nvis[kWaves];
  u32x4 (*ring)[TILE_CHUNKS] = reinterpret_cast<u32x4 (*)[TILE_CHUNKS]>(lds_main);
  float (*s_sc)[kMaxTiles * kTileN] = reinterpret_cast<float (*)[kMaxTiles * kTileN]>(lds_main + RING_B);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int tw = blockIdx.y * kWaves + wave;   // this wave's token
  const int t = tw < T ? tw : T - 1;
  const int t0 = blockIdx.y * kWaves;          // its key rows serve the workgroup

  // The token's query rows go to LDS by DMA, 1 KiB per instruction (chunk p
  // of row r at position p ^ (r % CPR), as in the key tiles), and are read
  // from there in the MFMA A layout (lane (col, half) holds head mt*32 + col,
  // elements 16s + 8*half .. +8): loaded in that layout straight from memory,
  // each instruction would touch 32 rows 32 B apiece, and those loads held
  // the workgroup's start for several thousand cycles.  One load a lane
  // brings the head weights.  Both are in flight with the metadata.
  char* qst = lds_main + wave * QB;
  {
    const char* qsrc = reinterpret_cast<const char*>(q_idx + (int64_t)t * n_ih * IHD);
    const int q_chunks = n_ih * CPR;
    for (int e0 = 0; e0 < q_chunks; e0 += 64) {
      const int c = min(e0 + lane, q_chunks - 1);  // the LDS chunk e0 + lane (past the rows: a copy)
      const int r = c / CPR, p = (c % CPR) ^ (r & (CPR - 1));
      lds_dma16_untracked(qsrc + (r * CPR + p) * 16, qst + e0 * 16);
    }
  }
  const float wl = w[(int64_t)t * n_ih + min(lane, n_ih - 1)];
  const int64_t pos_t = pos[t];
  const int32_t ncomp_t = n_comp[t];
  const int64_t row0_t = seq_kv[t];
  const int64_t row0 = seq_kv[t0];
  // all the metadata and scalar arguments the first key DMAs need, in one
  // round trip (the empty asm takes them as operands; otherwise the compiler
  // sinks some of these loads to their first use, a round trip later)
  asm volatile("" ::"s"(pos_t), "s"(ncomp_t), "s"(row0_t), "s"(row0), "s"(k_rows), "s"(ld),
               "s"(ratio), "s"(tpw), "s"(n_groups), "s"(T));
  wait_vmcnt<0>();  // the query DMAs (not counted by the compiler) and the weights
  u32x4 qa[MT][KS];
  float wv[MT][16];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int hq = mt * 32 + col < n_ih ? mt * 32 + col : n_ih - 1;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qa[mt][s] = *reinterpret_cast<const u32x4*>(qst + (hq * CPR + ((2 * s + half) ^ (hq & (CPR - 1)))) * 16);
    // heads past n_ih (their query rows repeat the last head's) weigh zero
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int hw = mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      const float v = __shfl(wl, hw < n_ih ? hw : 0);
      wv[mt][r] = hw < n_ih ? v : 0.0f;
    }
  }
  uint32_t flags = 0;
  int64_t n_vis = visible_count(pos_t, ratio, ncomp_t, &flags);
  if (row0_t < 0) {
    flags |= CSA_DERR_BAD_META;
    n_vis = 0;
  } else if (row0_t + n_vis > k_rows) {
    flags |= CSA_DERR_KEY_RANGE;
    n_vis = 0;
  }
  if (n_vis > ld) {
    flags |= CSA_DERR_VIS_OVER_LD;
    n_vis = ld;
  }
  if (row0_t != row0 && n_vis > 0) {  // the promise of one sequence is broken
    flags |= CSA_DERR_BAD_META;
    n_vis = 0;
  }
  if (tw >= T) {
    flags = 0;
    n_vis = 0;
  }
  if (blockIdx.x == 0 && lane == 0) report(err, flags);
  if (lane == 0) s_nvis[wave] = n_vis;
  __syncthreads();
  int64_t max_nvis = 0;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) max_nvis = max(max_nvis, s_nvis[v]);

  // the workgroup's tiles: groups [gbeg, gend) of the row, up to the last
  // tile that holds a visible block of one of its tokens
  const int gbeg = blockIdx.x * kGemmGroups;
  const int gend = min(gbeg + kGemmGroups, n_groups);
  const int64_t tile0 = (int64_t)gbeg * tpw;
  int nt = (gend - gbeg) * tpw;
  const int64_t vis_tiles = (max_nvis + kTileN - 1) / kTileN - tile0;
  if (vis_tiles < nt) nt = vis_tiles > 0 ? (int)vis_tiles : 0;
  // every row read lies below max_nvis, the visible count of a token whose
  // rows start at row0 and were checked against k_rows
  const char* kbase = reinterpret_cast<const char*>(k_idx) + row0 * RB;
  // tile i goes to ring slot i % kGemmSlots
  auto issue = [&](int i) {
    if (wave < LPT) {  // instruction `wave` of tile i: rows (64*wave + lane) / CPR
      const int e = wave * 64 + lane;
      const int r = e / CPR, p = e % CPR;
      const int c = p ^ (r & (CPR - 1));
      int64_t blk = (tile0 + i) * kTileN + r;
      if (blk > max_nvis - 1) blk = max_nvis - 1;
      lds_dma16_untracked(kbase + blk * RB + c * 16, &ring[i % kGemmSlots][wave * 64]);
    }
  };
  for (int i = 0; i < kGemmDepth && i < nt; ++i) issue(i);

  // two tiles a step: one barrier per pair, and two independent MFMA chains
  // per wave (the epilogue of one overlaps the products of the other)
  for (int i = 0; i < nt; i += 2) {
    const bool two = i + 1 < nt;
    // this wave's parts of tiles i and i + 1 have landed (one DMA per tile
    // and wave, no other memory operation in flight), then every wave's have
    if (i + kGemmDepth <= nt) wait_vmcnt<kGemmDepth - 2>(); else wait_vmcnt<0>();
    __syncthreads();  // tiles i, i + 1 complete; every wave is done with i - 2, i - 1
    // the next DMAs go into the slots that tiles i + depth - slots, + 1 left
    if (i + kGemmDepth < nt) issue(i + kGemmDepth);
    if (i + kGemmDepth + 1 < nt) issue(i + kGemmDepth + 1);
    const int64_t tt = tile0 + i;
    if (tt * kTileN < n_vis) {  // wave-uniform: the token sees a block of tile i
      // a lone last tile is computed twice and kept once
      const u32x4* kt0 = ring[i % kGemmSlots];
      const u32x4* kt1 = ring[(two ? i + 1 : i) % kGemmSlots];
      u32x4 kb0[KS], kb1[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int c = col * CPR + ((2 * s + half) ^ (col & (CPR - 1)));
        kb0[s] = kt0[c];
        kb1[s] = kt1[c];
      }
      f32x16 acc0[MT], acc1[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc0[mt] = f32x16{};
        acc1[mt] = f32x16{};
      }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc0[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qa[mt][s]),
                                                             __builtin_bit_cast(bf16x8, kb0[s]), acc0[mt],
                                                             0, 0, 0);
          acc1[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qa[mt][s]),
                                                             __builtin_bit_cast(bf16x8, kb1[s]), acc1[mt],
                                                             0, 0, 0);
        }
      }
      float part0 = 0.0f, part1 = 0.0f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          part0 += wv[mt][r] * relu_f32(acc0[mt][r]);
          part1 += wv[mt][r] * relu_f32(acc1[mt][r]);
        }
      }
      part0 += __shfl_xor(part0, 32);
      part1 += __shfl_xor(part1, 32);
      if (half == 0) {
        s_sc[wave][i * kTileN + col] = part0;
        if (two) s_sc[wave][(i + 1) * kTileN + col] = part1;
      }
    }
  }

  // after the loop (its last wait drained every DMA): this wave's scores,
  // two tiles per store, and one list per group (empty past the tiles)
  if (tw >= T) return;
  float* srow = scores + (int64_t)tw * ld;
  for (int i = half; i < nt; i += 2) {
    const int64_t blk = (tile0 + i) * kTileN + col;
    if (blk < n_vis) srow[blk] = s_sc[wave][i * kTileN + col];
  }
  if (ca.cand != nullptr) {
    // one list per group (empty past the tiles), in block order
    const int64_t g0 = (int64_t)tw * ca.groups_per_token + gbeg;
    groups_lists_from_scores<kGemmGroups>(s_sc[wave], tpw * kTileN, tile0 * kTileN, n_vis,
                                          ca.wave_m, (nt + tpw - 1) / tpw, gend - gbeg,
                                          ca.cand + g0 * ca.list_len, ca.list_len, ca.gcut + g0);
  }
}

template <int IHD>
hipError_t launch_gemm_ihd(const IndexScoreLaunch& a, const IndexPlan& p, hipStream_t s) {
  const int n_groups = p.waves_per_token();
  const dim3 grid((unsigned)((n_groups + kGemmGroups - 1) / kGemmGroups),
                  (unsigned)((a.T + kWaves - 1) / kWaves));
  const auto* q = static_cast<const uint16_t*>(a.q_idx);
  const auto* k = static_cast<const uint16_t*>(a.k_idx);
  if (a.n_ih <= 32)
    hipLaunchKernelGGL((index_gemm_kernel<IHD, 1>), grid, dim3(kWaves * 64), 0, s, q, a.w, k,
                       a.k_rows, a.pos, a.seq_kv, a.n_comp, a.T, a.n_ih, a.ratio, a.scores, a.ld,
                       a.cand, a.err, p.tiles_per_wave, n_groups);
  else
    hipLaunchKernelGGL((index_gemm_kernel<IHD, 2>), grid, dim3(kWaves * 64), 0, s, q, a.w, k,
                       a.k_rows, a.pos, a.seq_kv, a.n_comp, a.T, a.n_ih, a.ratio, a.scores, a.ld,
                       a.cand, a.err, p.tiles_per_wave, n_groups);
  return hipGetLastError();
}

}  // namespace

// The batch kernel takes batches of short rows (one tile a wave), also of
// one sequence; the GEMM form the rest of one_seq's launches it can run.
static bool uses_batch_indexer(const IndexScoreLaunch& a, const IndexPlan& p) {
  return batch_indexer(a.T, a.n_ih, a.ihd, a.e4m3) && p.tiles_per_wave == 1 &&
         (a.cand.cand == nullptr || !a.cand.merge);
}

bool gemm_indexer(const IndexScoreLaunch& a) {
  return a.one_seq && !a.e4m3 && a.T >= kGemmMinT && a.n_ih <= 64 && (a.ihd == 64 || a.ihd == 128) &&
         (a.cand.cand == nullptr || !a.cand.merge) && !uses_batch_indexer(a, plan_index(a.T, a.ld));
}

IndexPlan plan_index(int T, int64_t ld) {
  // Every wave owns `tpw` consecutive 32-block tiles; about one resident
  // workgroup per CU (256 CUs x kWaves waves) over the whole batch, at most
  // kMaxTpw tiles per wave.
  IndexPlan p;
  const int64_t tiles = (ld + kTileN - 1) / kTileN;
  const int64_t total = tiles * (T > 0 ? T : 1);
  int64_t tpw = (total + kWaves * 256 - 1) / (kWaves * 256);
  if (tpw < 1) tpw = 1;
  // A batch of rows of different lengths is planned for its longest.  Up to
  // 2048 tiles a row (the select holds that many group bounds), a batch has
  // one tile per wave: the geometry of index_batch_kernel's items.  Longer
  // rows in a batch take half the tiles per wave, so that the workgroups of
  // the longer rows do not run alone at the end (large prefill chunks keep
  // the full length).
  if (T > 1 && T <= kBatchMaxT) tpw = tiles <= kMaxGroups ? 1 : (tpw < kMaxTpw / 2 ? tpw : kMaxTpw / 2);
  if (tpw > kMaxTpw) tpw = kMaxTpw;
  p.tiles_per_wave = (int)tpw;
  p.wgs_per_token = (int)((tiles + kWaves * tpw - 1) / (kWaves * tpw));
  return p;
}

hipError_t launch_index_score(const IndexScoreLaunch& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const IndexPlan bp = plan_index(a.T, a.ld);
  if (uses_batch_indexer(a, bp)) return a.ihd == 64 ? launch_batch_ihd<64>(a, s) : launch_batch_ihd<128>(a, s);
  const IndexPlan& p = bp;
  if (gemm_indexer(a)) return a.ihd == 64 ? launch_gemm_ihd<64>(a, p, s) : launch_gemm_ihd<128>(a, p, s);
  switch (a.ihd) {
    case 32: return launch_ihd<32>(a, p, s);
    case 64: return launch_ihd<64>(a, p, s);
    case 128: return launch_ihd<128>(a, p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_rescore(const RescoreLaunch& a, hipStream_t s) {
  if (a.T == 0 || a.C == 0) return hipSuccess;
  switch (a.ihd) {
    case 32: return launch_rescore_ihd<32>(a, s);
    case 64: return launch_rescore_ihd<64>(a, s);
    case 128: return launch_rescore_ihd<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace csa
