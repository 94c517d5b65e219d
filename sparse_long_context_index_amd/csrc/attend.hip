// S4 -- shared-KV MQA softmax attention (post-probe audit, F3 "shared key-value
// MQA": every row is both key and value, shared by all query heads; 1M-context
// audit, D4: the dense HCA row set is the whole visible compressed history
// followed by the SWA rows; D6: the sink is a per-head logit added to the
// softmax denominator).
//
// Split-K flash decoding on gfx950 bf16 MFMA (v_mfma_f32_16x16x32_bf16), with
// the products transposed so that each lane owns one query head:
//   * a workgroup = 4 waves serving 16 query heads (one per lane column) on a
//     run of 64-row tiles; the grid is (row splits, 16-head groups, tokens),
//     so a decode token's rows spread over many CUs while each workgroup
//     fetches only its heads' queries and writes only their partials;
//   * rows stream through LDS in 64-row tiles; each tile is staged twice from
//     one set of 16-byte global loads: row-major (A operand of S^T = K Q^T) and
//     8-row interleaved (A operand of O^T += V^T P^T), the latter transposed in
//     registers with v_perm so that both products read 16 bytes per lane;
//   * wave w computes S^T for tile rows 16w..16w+15; the fp32 online softmax
//     (exp2 domain) combines the waves' row maxima and sums through LDS, and
//     P is exchanged there in the row order of the interleaved V^T groups
//     (attention does not depend on the order of its rows);
//   * wave w then accumulates O^T for its quarter of head_dim; each lane holds
//     four consecutive d of its head, stored 16 bytes at a time: unnormalised
//     partial outputs plus (max, sum) per split, merged by a small combine
//     kernel (which also applies the sink).  With one split the workgroup
//     writes the final output directly.
// The row set of token t is segment A followed by segment B, read in place, so
// the HCA path needs no concatenation.  In the decode step the CSA rows are
// gathered here (selected compressed rows through their block indices, then
// the SWA rows) and copied into all_kv while they are staged, which fuses the
// gather stage into the attention.
#include <type_traits>

#include "select_core.h"

namespace csa {
namespace {

constexpr int kRT = 64;          // rows per tile
constexpr int kHeadsPerWg = 16;  // query heads per workgroup (one per lane column)
constexpr int kMaxSplits = 256;
constexpr int64_t kSegB = 1ll << 62;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
struct Layout {
  static constexpr int RM = D + 8;                   // row-major row stride (bf16)
  static constexpr int ILG = D * 8 + (D / 8) * 8;    // interleaved 8-row group stride
  static constexpr int RM_ELEMS = kRT * RM;
  static constexpr int IL_ELEMS = (kRT / 8) * ILG;
};

// Row-set mode of segment A (a template parameter of the split kernel, so
// that the token metadata loads are unconditional and go out together).
enum : int { kModeExplicit = 0, kModeVisible = 1, kModeGather = 2 };

struct SegDesc {
  int64_t a0, b0;
  int alen, blen;
};

// Per-token row metadata of the mode, read in one batch.
struct TokMeta {
  int64_t a_row0, vis_pos, b_row0;
  int32_t a_cnt, vis_ncomp, b_len;
};
template <int MODE, bool HAS_B>
__device__ __forceinline__ TokMeta load_meta(const AttendLaunch& p, int t) {
  TokMeta m{};
  m.a_row0 = p.a_row0 != nullptr ? p.a_row0[t] : (int64_t)t * p.a_stride;
  if constexpr (MODE == kModeGather) m.a_cnt = p.sel_cnt[t];
  if constexpr (MODE == kModeExplicit) m.a_cnt = p.a_len[t];
  if constexpr (MODE == kModeVisible) {
    m.vis_pos = p.vis_pos[t];
    m.vis_ncomp = p.vis_ncomp[t];
  }
  if constexpr (HAS_B) {
    m.b_row0 = p.b_row0[t];
    m.b_len = p.b_len[t];
  }
  return m;
}

// Row set of token t.  Gather mode: segment A is the selected compressed rows
// comp_kv[seq_kv[t] + sel_idx[t, j]], j < sel_cnt[t], segment B the SWA rows;
// the rows are also copied into all_kv while staged.
template <int MODE, bool HAS_B>
__device__ __forceinline__ SegDesc token_rows(const AttendLaunch& p, const TokMeta& m, uint32_t& flags) {
  SegDesc s;
  int64_t alen;
  s.a0 = m.a_row0;
  if constexpr (MODE == kModeGather) {
    alen = m.a_cnt;
    if (alen < 0 || alen > p.sel_stride) {
      flags |= CSA_DERR_COUNT_RANGE;
      alen = alen < 0 ? 0 : p.sel_stride;
    }
  } else {
    if constexpr (MODE == kModeVisible) {
      alen = visible_count(m.vis_pos, p.vis_ratio, m.vis_ncomp, &flags);
    } else {
      alen = m.a_cnt;
    }
    if (s.a0 < 0 || alen < 0 || s.a0 + alen > p.a_rows) {
      flags |= CSA_DERR_ROW_RANGE;
      alen = 0;
    }
  }
  int64_t blen = 0;
  s.b0 = 0;
  if constexpr (HAS_B) {
    s.b0 = m.b_row0;
    blen = m.b_len;
    if (MODE == kModeGather && blen > p.b_cap) {
      flags |= CSA_DERR_COUNT_RANGE;
      blen = p.b_cap;
    }
    if (s.b0 < 0 || blen < 0 || s.b0 + blen > p.b_rows) {
      flags |= CSA_DERR_ROW_RANGE;
      blen = 0;
    }
  }
  if (alen + blen > p.max_rows) {
    flags |= CSA_DERR_ROWS_OVER_MAX;
    if (alen > p.max_rows) alen = p.max_rows;
    blen = p.max_rows - alen;
  }
  s.alen = (int)alen;
  s.blen = (int)blen;
  return s;
}

__device__ __forceinline__ uint32_t perm(uint32_t hi_src, uint32_t lo_src, uint32_t sel) {
  return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}

// Work item of workgroup L of a 1-D grid of N = n_splits * n_hg * T.  The
// dispatcher deals workgroups to the eight XCDs in turn (L % 8), and each XCD
// has its own L2; workgroups are numbered so that each XCD takes a run of
// consecutive items, in which the head groups of one row split (the same
// rows) are neighbours and share that XCD's L2.
struct WorkItem {
  int split, hg, t;
};
__device__ __forceinline__ WorkItem work_item(int n_splits, int n_hg) {
  const int N = (int)gridDim.x, L = (int)blockIdx.x;
  const int x = L & 7, slot = L >> 3;
  const int i = x * (N >> 3) + min(x, N & 7) + slot;
  WorkItem w;
  w.hg = i % n_hg;
  w.split = (i / n_hg) % n_splits;
  w.t = i / (n_hg * n_splits);
  return w;
}

// Split partials in the workspace: (max, sum) fp32 pairs per (token, split,
// head), then the bf16 outputs, 256-byte aligned.
__host__ __device__ inline size_t part_ml_floats(int T, int n_splits, int n_heads) {
  const size_t n = (size_t)T * n_splits * n_heads * 2;
  return (n + 63) & ~(size_t)63;
}

// LDS of the tile loop.
template <int D>
struct alignas(16) AttSmem {
  using L = Layout<D>;
  uint16_t rm[L::RM_ELEMS];              // tile, row-major
  uint16_t il[L::IL_ELEMS];              // tile, 8-row groups transposed
  uint16_t pl[kHeadsPerWg * kRT];        // P[head][tile row], bf16
  float red_m[4][kHeadsPerWg], red_l[4][kHeadsPerWg];
  int64_t rsrc[kRT];  // element offset of each tile row (kSegB: segment B), -1: none
};

// The tile loop and epilogue of one workgroup: rows [row_begin, row_end) of
// token t for the 16 heads of group hg.  NT threads stage the tiles; waves
// 0-3 run the products and the softmax (the others only join the barriers).
// Q comes from registers (qa) or from LDS (qlds, 16 rows of D+8); in gather
// mode the block index of row rr comes from a prefetch of sel_idx (pidx holds
// the first tile's) or, when SEL_LDS, from selrow[rr - row_begin] (rr itself
// when sel_listed is false: every visible block is selected).  With SEL_LDS
// the first tile's loads are issued before the tile loop's first barrier, so
// that they are in flight across it.
template <int D, int MODE, bool HAS_B, int NT, bool Q_LDS, bool SEL_LDS>
__device__ __forceinline__ void attend_tiles(const AttendLaunch& p, AttSmem<D>& sm, int t,
                                             int hg, int split, int n_splits, int row_begin,
                                             int row_end,
                                             const SegDesc& sd, int32_t pidx,
                                             const int32_t* selrow, bool sel_listed,
                                             const bf16x8 (&qa)[D / 32], const uint16_t* qlds,
                                             bool copy_rows) {
  constexpr bool kGather = MODE == kModeGather;
  using L = Layout<D>;
  constexpr int KSQ = D / 32;  // k-steps of S^T = K Q^T
  constexpr int NTW = D / 64;  // 16-wide d tiles of O^T per wave (a quarter of D)
  constexpr int DP = D / 8;    // 16-byte pieces per row
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, quad = lane >> 4;
  const bool mma = NT == 256 || wave < 4;       // waves of the products
  const int h = hg * kHeadsPerWg + li;  // this lane's query head
  uint32_t flags = 0;
  const float sl2 = p.scale * kLog2e;

  // o[nn][r] = O^T[d = (wave*NTW + nn)*16 + 4*quad + r][head h] (unnormalised)
  f32x4 o[NTW];
#pragma unroll
  for (int n = 0; n < NTW; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const uint16_t* kv_a = p.kv_a;
  const uint16_t* kv_b = p.kv_b;
  // One tile; the first tile of a SEL_LDS call is staged directly (see above).
  auto tile = [&](auto direct_tag, const int r0) {
    constexpr bool direct = decltype(direct_tag)::value;
      if constexpr (!direct) {
        __syncthreads();  // the previous tile has been consumed
        // ---- row sources of this tile: one thread per row resolves the block
        // index (gather mode) or segment B, into an LDS table ----
        if (tid < kRT) {
          const int rr = r0 + tid;
          int64_t src = -1;
          if (rr < row_end) {
            if (rr < sd.alen) {
              int64_t ar = sd.a0 + rr;
              if constexpr (kGather) {
                ar = sd.a0 + (SEL_LDS ? (sel_listed ? selrow[rr - row_begin] : rr) : pidx);
                if (ar < 0 || ar >= p.a_rows) {
                  flags |= CSA_DERR_ROW_RANGE;
                  ar = -1;
                }
              }
              src = ar < 0 ? -1 : ar * D;
            } else {
              src = ((sd.b0 + (rr - sd.alen)) * D) | kSegB;
            }
          }
          sm.rsrc[tid] = src;
          // prefetch the next tile's block indices
          if (kGather && !SEL_LDS && r0 + kRT < row_end)
            pidx = p.sel_idx[(int64_t)t * p.sel_stride + min(r0 + kRT + tid, p.sel_stride - 1)];
        }
        __syncthreads();
      }
      // ---- stage the tile.  The P V product takes its 32 rows per k-step in
      // the order the S^T accumulators hold them, so 8-row group g = 4*kp + qg
      // is rows 32*kp + 16*(j/4) + 4*qg + j%4, j < 8.  Each thread loads one
      // 8x8 (rows x d) block of a group, writes it row-major (A operand of S^T)
      // and transposed (A operand of O^T), and (head group 0) copies it to
      // all_kv. ----
      constexpr int NB = (kRT / 8) * DP;     // 8x8 blocks per tile
      constexpr int BPTH = (NB + NT - 1) / NT;  // blocks per thread
      // Every load is issued unconditionally (a load under a branch per row
      // keeps the loads from overlapping: measured 2.6x slower for a 64-row
      // tile): a missing row reads this token's own query row instead, an
      // address always in bounds, and is zeroed once it has arrived.
      const uint16_t* safe = p.q + (int64_t)t * p.n_heads * D;
      u32x4 rows[BPTH][8];
      bool have[BPTH][8];
  #pragma unroll
      for (int q = 0; q < BPTH; ++q) {
        const int b = tid + q * NT;
        const int g = b / DP, dp = b - g * DP;
  #pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int row = 32 * (g >> 2) + 16 * (k >> 2) + 4 * (g & 3) + (k & 3);
          int64_t src = -1;
          if constexpr (direct) {
            const int rr = r0 + row;  // the first tile of the split: r0 == row_begin
            const int32_t sidx = selrow[row];
            const int64_t ar = sd.a0 + (sel_listed ? sidx : rr);
            const bool in_a = rr < sd.alen;
            const bool ok_a = ar >= 0 && ar < p.a_rows;
            if (b < NB && rr < row_end && in_a && !ok_a) flags |= CSA_DERR_ROW_RANGE;
            src = (b < NB && rr < row_end)
                      ? (in_a ? (ok_a ? ar * D : -1) : (((sd.b0 + (rr - sd.alen)) * D) | kSegB))
                      : -1;
          } else {
            src = b < NB ? sm.rsrc[row] : -1;
          }
          have[q][k] = src >= 0;
          const uint16_t* base = (src & kSegB) ? kv_b : kv_a;
          const uint16_t* a = src >= 0 ? base + (src & ~kSegB) + dp * 8 : safe + (dp & (DP - 1)) * 8;
          rows[q][k] = *reinterpret_cast<const u32x4*>(a);
        }
      }
  #pragma unroll
      for (int q = 0; q < BPTH; ++q)
  #pragma unroll
        for (int k = 0; k < 8; ++k)
          if (!have[q][k]) rows[q][k] = u32x4{0u, 0u, 0u, 0u};
      if constexpr (direct) __syncthreads();  // the select's LDS (aliased by sm) is free from here
  #pragma unroll
      for (int q = 0; q < BPTH; ++q) {
        const int b = tid + q * NT;
        if (b >= NB) break;
        const int g = b / DP, dp = b - g * DP;
  #pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int row = 32 * (g >> 2) + 16 * (k >> 2) + 4 * (g & 3) + (k & 3);
          *reinterpret_cast<u32x4*>(&sm.rm[row * L::RM + dp * 8]) = rows[q][k];
          if (copy_rows && r0 + row < row_end)
            *reinterpret_cast<u32x4*>(p.copy_out + ((int64_t)t * p.copy_stride + r0 + row) * D +
                                      dp * 8) = rows[q][k];
        }
        uint16_t* ilg = &sm.il[g * L::ILG + dp * 8 * 8 + dp * 8];
  #pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          const int wi = e >> 1;
          u32x4 c;
          c.x = perm(rows[q][1][wi], rows[q][0][wi], sel);
          c.y = perm(rows[q][3][wi], rows[q][2][wi], sel);
          c.z = perm(rows[q][5][wi], rows[q][4][wi], sel);
          c.w = perm(rows[q][7][wi], rows[q][6][wi], sel);
          *reinterpret_cast<u32x4*>(ilg + e * 8) = c;
        }
      }
      __syncthreads();

      float x[4];
      if (mma) {
        // ---- S^T = K Q^T for this wave's 16 tile rows x the 16 heads.  The
        // fragments of k-step ks+1 are read from LDS while the MFMA of ks runs.
        f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint16_t* krow = &sm.rm[(wave * 16 + li) * L::RM + quad * 8];
        const uint16_t* qrow = qlds + li * (D + 8) + quad * 8;
        bf16x8 kb[2], qb[2];
        kb[0] = *reinterpret_cast<const bf16x8*>(krow);
        if constexpr (Q_LDS) qb[0] = *reinterpret_cast<const bf16x8*>(qrow);
  #pragma unroll
        for (int ks = 0; ks < KSQ; ++ks) {
          if (ks + 1 < KSQ) {
            kb[(ks + 1) & 1] = *reinterpret_cast<const bf16x8*>(krow + (ks + 1) * 32);
            if constexpr (Q_LDS) qb[(ks + 1) & 1] = *reinterpret_cast<const bf16x8*>(qrow + (ks + 1) * 32);
          }
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[ks & 1], Q_LDS ? qb[ks & 1] : qa[ks], s, 0,
                                                      0, 0);
        }
        // s[r] = S[head h][tile row wave*16 + 4*quad + r]
        // ---- online softmax (exp2 domain): per-wave maxima over 16 rows, then
        // the tile maximum of each head through LDS ----
        float mloc = -INFINITY;
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool valid = r0 + wave * 16 + 4 * quad + r < row_end;
          x[r] = valid ? s[r] * sl2 : -INFINITY;
          mloc = fmaxf(mloc, x[r]);
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        if (quad == 0) sm.red_m[wave][li] = mloc;
      }
      __syncthreads();
      float alpha = 1.f;
      if (mma) {
        const float mtile = fmaxf(fmaxf(sm.red_m[0][li], sm.red_m[1][li]),
                                  fmaxf(sm.red_m[2][li], sm.red_m[3][li]));
        const float mnew = fmaxf(m_run, mtile);
        alpha = (mnew == -INFINITY) ? 1.f : exp2f(m_run - mnew);
        float lsum = 0.f;
        float pv[4];
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          pv[r] = (x[r] == -INFINITY) ? 0.f : exp2f(x[r] - mnew);
          lsum += pv[r];
        }
        lsum += __shfl_xor(lsum, 16);
        lsum += __shfl_xor(lsum, 32);
        // P[head li][tile rows wave*16 + 4*quad .. +4] as bf16
        *reinterpret_cast<uint2*>(&sm.pl[li * kRT + wave * 16 + 4 * quad]) =
            make_uint2((uint32_t)f32_to_bf16(pv[0]) | ((uint32_t)f32_to_bf16(pv[1]) << 16),
                       (uint32_t)f32_to_bf16(pv[2]) | ((uint32_t)f32_to_bf16(pv[3]) << 16));
        if (quad == 0) sm.red_l[wave][li] = lsum;
        m_run = mnew;
      }
      __syncthreads();
      if (mma) {
        l_run = l_run * alpha +
                (sm.red_l[0][li] + sm.red_l[1][li] + sm.red_l[2][li] + sm.red_l[3][li]);
  #pragma unroll
        for (int n = 0; n < NTW; ++n) o[n] *= alpha;
        // P^T (B operand of O^T) for k-step kp: rows 32kp + 4*quad + 0..3 and
        // 32kp + 16 + 4*quad + 0..3 of head li
        bf16x8 pb[2];
  #pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          const uint2 lo = *reinterpret_cast<const uint2*>(&sm.pl[li * kRT + 32 * kp + 4 * quad]);
          const uint2 hi =
              *reinterpret_cast<const uint2*>(&sm.pl[li * kRT + 32 * kp + 16 + 4 * quad]);
          pb[kp] = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
        }
        // ---- O^T += V^T P^T for this wave's quarter of D ----
  #pragma unroll
        for (int kp = 0; kp < kRT / 32; ++kp) {
          const uint16_t* ilg = &sm.il[(kp * 4 + quad) * L::ILG];
          bf16x8 vb[NTW];
  #pragma unroll
          for (int nn = 0; nn < NTW; ++nn) {
            const int d = (wave * NTW + nn) * 16 + li;
            vb[nn] = *reinterpret_cast<const bf16x8*>(ilg + d * 8 + (d >> 3) * 8);
          }
  #pragma unroll
          for (int nn = 0; nn < NTW; ++nn)
            o[nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb[nn], pb[kp], o[nn], 0, 0, 0);
        }
      }
  };
  int r0 = row_begin;
  if constexpr (SEL_LDS) {
    if (r0 < row_end) {
      tile(std::true_type{}, r0);
      r0 += kRT;
    }
  }
  for (; r0 < row_end; r0 += kRT) tile(std::false_type{}, r0);

  report(p.err, flags);
  // ---- epilogue: lane (li, quad) of wave w holds d = (w*NTW + nn)*16 +
  // 4*quad + r of head h ----
  if (!mma || h >= p.n_heads) return;
  if (n_splits == 1) {
    float M = m_run;
    float Lsum = l_run;
    float f = 1.f;
    if (p.sink != nullptr) {
      const float s2 = p.sink[h] * kLog2e;
      const float Mn = fmaxf(M, s2);
      f = (M == -INFINITY) ? 0.f : exp2f(M - Mn);
      Lsum = Lsum * f + exp2f(s2 - Mn);
      M = Mn;
    }
    const float inv = Lsum > 0.f ? f / Lsum : 0.f;
    uint16_t* oh = p.out + ((int64_t)t * p.n_heads + h) * D + 4 * quad;
#pragma unroll
    for (int nn = 0; nn < NTW; ++nn) {
      const uint32_t lo = (uint32_t)f32_to_bf16(o[nn][0] * inv) | ((uint32_t)f32_to_bf16(o[nn][1] * inv) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16(o[nn][2] * inv) | ((uint32_t)f32_to_bf16(o[nn][3] * inv) << 16);
      *reinterpret_cast<uint2*>(oh + (wave * NTW + nn) * 16) = make_uint2(lo, hi);
    }
    if (p.lse != nullptr && wave == 0 && quad == 0)
      p.lse[(int64_t)t * p.n_heads + h] = Lsum > 0.f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
  } else {
    // split partial: the split's own softmax output (normalised by its sum)
    // in bf16, and its (max, sum) in fp32
    float* part_ml = static_cast<float*>(p.ws);
    uint16_t* part_o = reinterpret_cast<uint16_t*>(part_ml + part_ml_floats(p.T, n_splits, p.n_heads));
    const size_t slot = ((size_t)t * n_splits + split) * p.n_heads + h;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    uint16_t* po = part_o + slot * D + 4 * quad;
#pragma unroll
    for (int nn = 0; nn < NTW; ++nn) {
      const uint32_t lo = (uint32_t)f32_to_bf16(o[nn][0] * inv) | ((uint32_t)f32_to_bf16(o[nn][1] * inv) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16(o[nn][2] * inv) | ((uint32_t)f32_to_bf16(o[nn][3] * inv) << 16);
      *reinterpret_cast<uint2*>(po + (wave * NTW + nn) * 16) = make_uint2(lo, hi);
    }
    if (wave == 0 && quad == 0) {
      part_ml[slot * 2 + 0] = m_run;
      part_ml[slot * 2 + 1] = l_run;
    }
  }
}

template <int D, int MODE, bool HAS_B>
__global__ __launch_bounds__(256) void attend_split_kernel(AttendLaunch p, int tiles_per_split,
                                                           int n_splits) {
  constexpr bool kGather = MODE == kModeGather;
  constexpr int KSQ = D / 32;
  __shared__ AttSmem<D> sm;
  const WorkItem wi = work_item(n_splits, (p.n_heads + kHeadsPerWg - 1) / kHeadsPerWg);
  const int t = wi.t, split = wi.split, hg = wi.hg;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int li = lane & 15, quad = lane >> 4;
  const int h = hg * kHeadsPerWg + li;

  // Everything the first tile waits on is loaded up front: its selected block
  // indices (idx rows always hold sel_stride entries), Q, the row metadata.
  int32_t pidx = 0;
  const int row_begin = split * tiles_per_split * kRT;
  if (kGather && tid < kRT)
    pidx = p.sel_idx[(int64_t)t * p.sel_stride + min(row_begin + tid, p.sel_stride - 1)];
  // Q as the B operand of S^T = K Q^T: lane holds Q[h][ks*32 + quad*8 .. +8].
  // A lane beyond n_heads computes with the last real head's query; its own
  // results are never stored, and the softmax statistics are per head.
  bf16x8 qa[KSQ];
  {
    const int hq = h < p.n_heads ? h : p.n_heads - 1;
    const uint16_t* qh = p.q + ((int64_t)t * p.n_heads + hq) * D + quad * 8;
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks)
      qa[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qh + ks * 32));
  }
  const TokMeta meta = load_meta<MODE, HAS_B>(p, t);
  uint32_t flags = 0;
  const SegDesc sd = token_rows<MODE, HAS_B>(p, meta, flags);
  if (split == 0 && hg == 0 && tid == 0) {
    report(p.err, flags);
    if (p.n_kv_out != nullptr) p.n_kv_out[t] = sd.alen + sd.blen;
  }
  const int n_rows = sd.alen + sd.blen;
  const int row_end = min(row_begin + tiles_per_split * kRT, n_rows);
  const bool copy_rows = kGather && p.copy_out != nullptr && hg == 0;
  attend_tiles<D, MODE, HAS_B, 256, false, false>(p, sm, t, hg, split, n_splits, row_begin, row_end,
                                                  sd, pidx, nullptr, false, qa, nullptr,
                                                  copy_rows);
}

// Gather-mode attention of the decode step (CSA rows: the selected
// compressed rows through their block indices, then the SWA rows in place).
// A 1024-thread workgroup per (row split, 16-head group, token): the split's
// block indices, the queries (to LDS) and the row metadata are loaded
// together, then 512 threads fetch each 64-row tile with eight 16-byte loads
// apiece, all in flight at once.
template <int D, bool HAS_B>
__global__ __launch_bounds__(1024) void gather_attend_kernel(AttendLaunch p, int tiles_per_split,
                                                             int n_splits) {
  constexpr int KSQ = D / 32;
  constexpr int QPR = D / 8;  // 16-byte pieces per query row
  __shared__ AttSmem<D> sm;
  __shared__ __attribute__((aligned(16))) uint16_t qlds[kHeadsPerWg * (D + 8)];
  const WorkItem wi = work_item(n_splits, (p.n_heads + kHeadsPerWg - 1) / kHeadsPerWg);
  const int t = wi.t, split = wi.split, hg = wi.hg;
  const int tid = threadIdx.x;
  const int row_begin = split * tiles_per_split * kRT;
  int32_t pidx = 0;
  if (tid < kRT)
    pidx = p.sel_idx[(int64_t)t * p.sel_stride + min(row_begin + tid, p.sel_stride - 1)];
  u32x4 qv = u32x4{0u, 0u, 0u, 0u};
  const int hl = tid / QPR;
  if (tid < kHeadsPerWg * QPR) {
    const int hq = min(hg * kHeadsPerWg + hl, p.n_heads - 1);
    qv = *reinterpret_cast<const u32x4*>(p.q + ((int64_t)t * p.n_heads + hq) * D +
                                         (tid - hl * QPR) * 8);
  }
  const TokMeta meta = load_meta<kModeGather, HAS_B>(p, t);
  uint32_t flags = 0;
  const SegDesc sd = token_rows<kModeGather, HAS_B>(p, meta, flags);
  if (tid < kHeadsPerWg * QPR)
    *reinterpret_cast<u32x4*>(&qlds[hl * (D + 8) + (tid - hl * QPR) * 8]) = qv;
  if (split == 0 && hg == 0 && tid == 0) {
    report(p.err, flags);
    if (p.n_kv_out != nullptr) p.n_kv_out[t] = sd.alen + sd.blen;
  }
  const int n_rows = sd.alen + sd.blen;
  const int row_end = min(row_begin + tiles_per_split * kRT, n_rows);
  const bool copy_rows = p.copy_out != nullptr && hg == 0;
  const bf16x8 qa_unused[KSQ] = {};
  // the tile loop's first barrier also orders the query stores above
  attend_tiles<D, kModeGather, HAS_B, 1024, true, false>(p, sm, t, hg, split, n_splits, row_begin,
                                                         row_end, sd, pidx, nullptr, false,
                                                         qa_unused, qlds, copy_rows);
}

// Select and attend in one kernel (decode step, CSA, small batches).  Every
// workgroup of token t -- one per (row split, 16-head group) -- runs the
// token's exact top-k (step_select: the fast select over the indexer's
// candidate lists, select_token when it gives up), which lists the selected
// block indices of its own split's rows in LDS; the queries, the row
// metadata and the candidate lists are all in flight together before it.
// The first tile's rows are then fetched straight from that list, with no
// global handoff or kernel boundary between the two stages.  The select's
// LDS is reused for the tiles.  Head-group-0 workgroups write the idx
// entries of their rows; split 0 writes the count.
constexpr int kFuseThreads = sel::kThreads;
constexpr int kFuseMaxTiles = 4;  // tiles per split the fused kernel takes

template <int D>
union FusedSmem {
  sel::SelShared<kFuseThreads> s;
  sel::FastShared<kFuseThreads> f;
  AttSmem<D> a;
};

template <int D, bool HAS_B>
__global__ __launch_bounds__(kFuseThreads) void select_attend_kernel(SelectLaunch sl,
                                                                     AttendLaunch p,
                                                                     int tiles_per_split,
                                                                     int n_splits) {
  constexpr int KSQ = D / 32;
  constexpr int QPR = D / 8;  // 16-byte pieces per query row
  __shared__ FusedSmem<D> u;
  __shared__ __attribute__((aligned(16))) uint16_t qlds[kHeadsPerWg * (D + 8)];
  __shared__ int32_t selrow[kFuseMaxTiles * kRT];
  const WorkItem wi = work_item(n_splits, (p.n_heads + kHeadsPerWg - 1) / kHeadsPerWg);
  const int t = wi.t, split = wi.split, hg = wi.hg;
  const int tid = threadIdx.x;
  const int row_begin = split * tiles_per_split * kRT;

  u32x4 qv = u32x4{0u, 0u, 0u, 0u};
  const int hl = tid / QPR;
  if (tid < kHeadsPerWg * QPR) {
    const int hq = min(hg * kHeadsPerWg + hl, p.n_heads - 1);
    qv = *reinterpret_cast<const u32x4*>(p.q + ((int64_t)t * p.n_heads + hq) * D +
                                         (tid - hl * QPR) * 8);
  }
  TokMeta meta{};
  meta.a_row0 = p.a_row0 != nullptr ? p.a_row0[t] : (int64_t)t * p.a_stride;
  if constexpr (HAS_B) {
    meta.b_row0 = p.b_row0[t];
    meta.b_len = p.b_len[t];
  }

  const uint32_t win = (uint32_t)(tiles_per_split * kRT);  // this split's rows
  const sel::SelResult r = sel::step_select<kFuseThreads>(
      sl.scores + (int64_t)t * sl.ld, sl.ld, sl.pos[t], sl.n_comp[t], sl.ratio, select_row0(sl, t),
      sl.k_rows, sl.top_k, sl.cand + (int64_t)t * sl.groups_per_token * sl.list_len,
      sl.gcut + (int64_t)t * sl.groups_per_token, sl.list_len, sl.groups_per_token,
      sl.blocks_per_group, sl.lists_complete != 0, u.f, u.s, selrow, (uint32_t)row_begin,
      (uint32_t)row_begin + win);

  if (tid < kHeadsPerWg * QPR)
    *reinterpret_cast<u32x4*>(&qlds[hl * (D + 8) + (tid - hl * QPR) * 8]) = qv;
  meta.a_cnt = (int32_t)r.emitted;
  uint32_t flags = 0;
  const SegDesc sd = token_rows<kModeGather, HAS_B>(p, meta, flags);
  if (hg == 0) {
    // idx entries [row_begin, row_begin + win) below top_k: the selection,
    // then -1
    int32_t* out = sl.idx + (int64_t)t * sl.top_k;
    const uint32_t i = (uint32_t)row_begin + (uint32_t)tid;
    if ((uint32_t)tid < win && i < (uint32_t)sl.top_k)
      out[i] = i < r.emitted ? (r.listed ? selrow[tid] : (int32_t)i) : -1;
  }
  if (split == 0 && hg == 0 && tid == 0) {
    sl.count[t] = (int32_t)r.emitted;
    report(p.err, flags | r.flags);
    if (p.n_kv_out != nullptr) p.n_kv_out[t] = sd.alen + sd.blen;
  }
  const int n_rows = sd.alen + sd.blen;
  const int row_end = min(row_begin + tiles_per_split * kRT, n_rows);
  const bool copy_rows = p.copy_out != nullptr && hg == 0;
  const bf16x8 qa_unused[KSQ] = {};
  attend_tiles<D, kModeGather, HAS_B, kFuseThreads, true, true>(
      p, u.a, t, hg, split, n_splits, row_begin, row_end, sd, 0, selrow, r.listed, qa_unused, qlds,
      copy_rows);
}

// Merge of the split partials of one (token, head): out = sum_s w_s o_s with
// w_s = l_s e^{m_s - M} / (sum_s' l_s' e^{m_s' - M} [+ e^{sink - M}]), where
// o_s is split s's normalised bf16 output.  A workgroup is one wave per 256
// output elements of the head (two waves at head_dim 512), and the waves
// share nothing: each reads every split's (max, sum) -- lane l takes splits
// l, l + 64, ... -- and reduces them with DPP, then its part of every split's
// output in rounds of kCombCh splits, all of a round's loads in flight
// together.  No LDS, no barrier.
constexpr int kCombCh = 32;
template <int D>
constexpr int comb_waves() { return D >= 512 ? D / 256 : 1; }
template <int EPL> struct CombRaw;
template <> struct CombRaw<4> { using T = uint2; };
template <> struct CombRaw<2> { using T = uint32_t; };
template <> struct CombRaw<1> { using T = uint16_t; };
template <int EPL>
__device__ __forceinline__ float comb_elem(const typename CombRaw<EPL>::T& r, int j) {
  if constexpr (EPL == 4) {
    const uint32_t w = j < 2 ? r.x : r.y;
    return __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
  } else if constexpr (EPL == 2) {
    return __uint_as_float((j & 1) ? (r & 0xFFFF0000u) : (r << 16));
  } else {
    return __uint_as_float((uint32_t)r << 16);
  }
}

template <int D>
__global__ __launch_bounds__(64 * comb_waves<D>()) void attend_combine_kernel(AttendLaunch p, int n_splits) {
  constexpr int NW = comb_waves<D>();
  constexpr int EPL = D / (64 * NW);  // output elements per lane
  constexpr int MLR = kMaxSplits / 64;
  using Raw = typename CombRaw<EPL>::T;
  const int h = blockIdx.x, t = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* part_ml = static_cast<const float*>(p.ws);
  const uint16_t* part_o =
      reinterpret_cast<const uint16_t*>(part_ml + part_ml_floats(p.T, n_splits, p.n_heads));
  const size_t slot0 = (size_t)t * n_splits * p.n_heads + h;
  const size_t sstride = (size_t)p.n_heads * D;
  const int e0 = wave * (D / NW) + lane * EPL;  // this lane's first output element
  const uint16_t* pbase = part_o + slot0 * D + e0;

  // Every load is unconditional (split index clamped, value masked after): a
  // load under a per-lane branch waits for its data before the branch closes.
  float m_s[MLR], l_s[MLR];
#pragma unroll
  for (int r = 0; r < MLR; ++r) {
    const int s = lane + 64 * r;
    const float2 ml = *reinterpret_cast<const float2*>(
        part_ml + (slot0 + (size_t)min(s, n_splits - 1) * p.n_heads) * 2);
    m_s[r] = s < n_splits ? ml.x : -INFINITY;
    l_s[r] = s < n_splits ? ml.y : 0.f;
  }
  Raw raw[kCombCh];
  auto load_round = [&](int c0) {
#pragma unroll
    for (int c = 0; c < kCombCh; ++c)
      raw[c] = *reinterpret_cast<const Raw*>(pbase + (size_t)min(c0 + c, n_splits - 1) * sstride);
  };
  load_round(0);

  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < MLR; ++r) mx = fmaxf(mx, l_s[r] > 0.f ? m_s[r] : -INFINITY);
  float M = wave_max_f32(mx);
  float s2 = -INFINITY;
  if (p.sink != nullptr) {
    s2 = p.sink[h] * kLog2e;
    M = fmaxf(M, s2);
  }
  float f[MLR];
  float fs = 0.f;
#pragma unroll
  for (int r = 0; r < MLR; ++r) {
    f[r] = l_s[r] > 0.f ? l_s[r] * exp2f(m_s[r] - M) : 0.f;
    fs += f[r];
  }
  float Lsum = wave_sum_f32(fs);
  if (p.sink != nullptr) Lsum += exp2f(s2 - M);

  float acc[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) acc[j] = 0.f;
  for (int c0 = 0; c0 < n_splits; c0 += kCombCh) {
    if (c0 > 0) load_round(c0);
#pragma unroll
    for (int c = 0; c < kCombCh; ++c) {
      const int s = c0 + c;
      if (s < n_splits) {  // wave-uniform
        // split s's weight sits in lane s % 64 of f[s / 64]
        const int r = s >> 6;
        float fr = f[0];
#pragma unroll
        for (int rr = 1; rr < MLR; ++rr) fr = r == rr ? f[rr] : fr;
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fr), s & 63));
#pragma unroll
        for (int j = 0; j < EPL; ++j) acc[j] += w * comb_elem<EPL>(raw[c], j);
      }
    }
  }
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  uint16_t* oh = p.out + ((size_t)t * p.n_heads + h) * D + e0;
#pragma unroll
  for (int j = 0; j < EPL; ++j) oh[j] = f32_to_bf16(acc[j] * inv);
  if (p.lse != nullptr && threadIdx.x == 0)
    p.lse[(size_t)t * p.n_heads + h] = Lsum > 0.f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
}

struct SplitPlan {
  int tiles_per_split, n_splits;
};

// Row splits of a launch: split_tiles tiles per split when the caller fixes it
// (the decode step), else enough splits for about 256 workgroups.
SplitPlan plan_splits(int T, int n_heads, int max_rows, int split_tiles) {
  SplitPlan sp;
  const int n_tiles = max_rows > 0 ? (max_rows + kRT - 1) / kRT : 1;
  if (split_tiles > 0) {
    sp.tiles_per_split = split_tiles < n_tiles ? split_tiles : n_tiles;
    sp.n_splits = (n_tiles + sp.tiles_per_split - 1) / sp.tiles_per_split;
    if (sp.n_splits <= kMaxSplits) return sp;
  }
  const int n_hg = (n_heads + kHeadsPerWg - 1) / kHeadsPerWg;
  int want = (256 + T * n_hg - 1) / (T * n_hg);
  if (want < 1) want = 1;
  if (want > n_tiles) want = n_tiles;
  if (want > kMaxSplits) want = kMaxSplits;
  sp.tiles_per_split = (n_tiles + want - 1) / want;
  sp.n_splits = (n_tiles + sp.tiles_per_split - 1) / sp.tiles_per_split;
  return sp;
}

template <int D>
hipError_t launch_d(const AttendLaunch& a, hipStream_t s) {
  const SplitPlan sp = plan_splits(a.T, a.n_heads, a.max_rows, a.split_tiles);
  const int n_hg = (a.n_heads + kHeadsPerWg - 1) / kHeadsPerWg;
  dim3 grid((unsigned)(sp.n_splits * n_hg * a.T));
  const int mode = a.sel_idx != nullptr ? kModeGather
                   : a.vis_pos != nullptr ? kModeVisible
                                          : kModeExplicit;
#define CSA_SPLIT(MODE, HB)                                                                  \
  hipLaunchKernelGGL((attend_split_kernel<D, MODE, HB>), grid, dim3(256), 0, s, a,          \
                     sp.tiles_per_split, sp.n_splits)
  if (mode == kModeGather) {
    if (a.kv_b != nullptr)
      hipLaunchKernelGGL((gather_attend_kernel<D, true>), grid, dim3(1024), 0, s, a,
                         sp.tiles_per_split, sp.n_splits);
    else
      hipLaunchKernelGGL((gather_attend_kernel<D, false>), grid, dim3(1024), 0, s, a,
                         sp.tiles_per_split, sp.n_splits);
  } else if (mode == kModeVisible) {
    if (a.kv_b != nullptr) CSA_SPLIT(kModeVisible, true); else CSA_SPLIT(kModeVisible, false);
  } else {
    if (a.kv_b != nullptr) CSA_SPLIT(kModeExplicit, true); else CSA_SPLIT(kModeExplicit, false);
  }
#undef CSA_SPLIT
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sp.n_splits == 1) return e;
  hipLaunchKernelGGL((attend_combine_kernel<D>), dim3((unsigned)a.n_heads, (unsigned)a.T),
                     dim3(64 * comb_waves<D>()), 0, s, a, sp.n_splits);
  return hipGetLastError();
}

// The fused kernel takes a launch whose grid fills the chip at most once
// (one 1024-thread workgroup per CU by its LDS), so that the repeated selects
// run side by side, and whose splits fit its LDS list of selected rows.
bool fused_fits(const SplitPlan& sp, int T, int n_heads) {
  const int n_hg = (n_heads + kHeadsPerWg - 1) / kHeadsPerWg;
  return sp.tiles_per_split <= kFuseMaxTiles && (int64_t)sp.n_splits * n_hg * T <= 256;
}

template <int D>
hipError_t launch_fused_d(const SelectLaunch& sl, const AttendLaunch& a, hipStream_t s) {
  const SplitPlan sp = plan_splits(a.T, a.n_heads, a.max_rows, a.split_tiles);
  const int n_hg = (a.n_heads + kHeadsPerWg - 1) / kHeadsPerWg;
  dim3 grid((unsigned)(sp.n_splits * n_hg * a.T));
  if (a.kv_b != nullptr)
    hipLaunchKernelGGL((select_attend_kernel<D, true>), grid, dim3(kFuseThreads), 0, s, sl, a,
                       sp.tiles_per_split, sp.n_splits);
  else
    hipLaunchKernelGGL((select_attend_kernel<D, false>), grid, dim3(kFuseThreads), 0, s, sl, a,
                       sp.tiles_per_split, sp.n_splits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sp.n_splits == 1) return e;
  hipLaunchKernelGGL((attend_combine_kernel<D>), dim3((unsigned)a.n_heads, (unsigned)a.T),
                     dim3(64 * comb_waves<D>()), 0, s, a, sp.n_splits);
  return hipGetLastError();
}

}  // namespace

bool select_attend_fits(int T, int n_heads, int max_rows, int split_tiles) {
  return T > 0 && fused_fits(plan_splits(T, n_heads, max_rows, split_tiles), T, n_heads);
}

int step_split_tiles(int T, int n_heads, int max_rows) {
  if (select_attend_fits(T, n_heads, max_rows, kStepSplitTiles)) return kStepSplitTiles;
  const int n_tiles = max_rows > 0 ? (max_rows + kRT - 1) / kRT : 1;
  const int n_hg = (n_heads + kHeadsPerWg - 1) / kHeadsPerWg;
  int64_t want = (kStepTargetWgs + (int64_t)T * n_hg - 1) / ((int64_t)T * n_hg);
  if (want < 1) want = 1;
  if (want > n_tiles) want = n_tiles;
  return (int)((n_tiles + want - 1) / want);
}

hipError_t launch_select_attend(const SelectLaunch& sl, const AttendLaunch& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (!select_attend_fits(a.T, a.n_heads, a.max_rows, a.split_tiles) || a.sel_stride != sl.top_k)
    return hipErrorInvalidValue;
  switch (a.head_dim) {
    case 64: return launch_fused_d<64>(sl, a, s);
    case 128: return launch_fused_d<128>(sl, a, s);
    case 256: return launch_fused_d<256>(sl, a, s);
    case 512: return launch_fused_d<512>(sl, a, s);
    default: return hipErrorInvalidValue;
  }
}

size_t attend_ws_bytes(int T, int n_heads, int head_dim, int max_rows, int split_tiles) {
  const SplitPlan sp = plan_splits(T, n_heads, max_rows, split_tiles);
  if (sp.n_splits == 1) return 256;
  const size_t n = (size_t)T * sp.n_splits * n_heads;
  size_t b = part_ml_floats(T, sp.n_splits, n_heads) * 4 + n * head_dim * 2;
  return (b + 255) & ~(size_t)255;
}

hipError_t launch_attend(const AttendLaunch& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  switch (a.head_dim) {
    case 64: return launch_d<64>(a, s);
    case 128: return launch_d<128>(a, s);
    case 256: return launch_d<256>(a, s);
    case 512: return launch_d<512>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace csa
