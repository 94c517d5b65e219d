// S4 -- shared-KV MQA softmax attention (post-probe audit, F3 "shared key-value
// MQA": every row is both key and value, shared by all query heads; 1M-context
// audit, D4: the dense HCA row set is the whole visible compressed history
// followed by the SWA rows; D6: the sink is a per-head logit added to the
// softmax denominator).
//
// Split-K flash decoding on gfx950 bf16 MFMA (v_mfma_f32_16x16x32_bf16):
//   * a workgroup = 4 waves = up to 64 query heads (16 per wave, the MFMA M);
//     the grid is (row splits, 64-head groups, tokens);
//   * rows stream through LDS in 64-row tiles; each tile is staged twice from
//     one set of 16-byte global loads: row-major (B operand of S = Q K^T, K = D)
//     and 8-row interleaved (B operand of O += P V, K = rows), the latter
//     transposed in registers with v_perm so that both products read 16 bytes
//     per lane from LDS;
//   * fp32 online softmax in the exp2 domain, P rounded to bf16 and passed
//     through a per-wave LDS buffer into the A-operand layout;
//   * each split writes unnormalised partial outputs plus (max, sum); a small
//     combine kernel merges them (and applies the sink).  With one split the
//     workgroup writes the final output directly.
// The row set of token t is segment A followed by segment B, read in place, so
// the HCA path needs no concatenation.  In the decode step the CSA rows are
// gathered here (selected compressed rows through their block indices, then
// the SWA rows) and copied into all_kv while they are staged, which fuses the
// gather stage into the attention.
#include "csa_common.h"

namespace csa {
namespace {

constexpr int kRT = 64;          // rows per tile
constexpr int kHeadsPerWg = 64;  // 4 waves x 16 heads
constexpr int kMaxSplits = 256;
constexpr int64_t kSegB = 1ll << 62;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
struct Layout {
  static constexpr int RM = D + 8;                   // row-major row stride (bf16)
  static constexpr int ILG = D * 8 + (D / 8) * 8;    // interleaved 8-row group stride
  static constexpr int PS = kRT + 8;                 // P row stride
  static constexpr int RM_ELEMS = kRT * RM;
  static constexpr int IL_ELEMS = (kRT / 8) * ILG;
  static constexpr int P_ELEMS = 4 * 16 * PS;
};

struct SegDesc {
  int64_t a0, b0;
  int alen, blen;
};

// Row set of token t.  Gather mode (p.sel_idx != nullptr): segment A is the
// selected compressed rows comp_kv[seq_kv[t] + sel_idx[t, j]], j < sel_cnt[t],
// segment B the SWA rows; the rows are also copied into all_kv while staged.
__device__ SegDesc token_rows(const AttendLaunch& p, int t, uint32_t& flags) {
  SegDesc s;
  int64_t alen;
  if (p.sel_idx != nullptr) {
    s.a0 = p.a_row0[t];  // seq_kv
    alen = p.sel_cnt[t];
    if (alen < 0 || alen > p.sel_stride) {
      flags |= CSA_DERR_COUNT_RANGE;
      alen = alen < 0 ? 0 : p.sel_stride;
    }
  } else {
    s.a0 = p.a_row0 != nullptr ? p.a_row0[t] : (int64_t)t * p.a_stride;
    if (p.vis_pos != nullptr) {
      alen = visible_count(p.vis_pos[t], p.vis_ratio, p.vis_ncomp[t], &flags);
    } else {
      alen = p.a_len[t];
    }
    if (s.a0 < 0 || alen < 0 || s.a0 + alen > p.a_rows) {
      flags |= CSA_DERR_ROW_RANGE;
      alen = 0;
    }
  }
  int64_t blen = 0;
  s.b0 = 0;
  if (p.kv_b != nullptr) {
    s.b0 = p.b_row0[t];
    blen = p.b_len[t];
    if (p.sel_idx != nullptr && blen > p.b_cap) {
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

template <int D>
__global__ __launch_bounds__(256) void attend_split_kernel(AttendLaunch p, int tiles_per_split,
                                                           int n_splits) {
  using L = Layout<D>;
  constexpr int KSQ = D / 32;   // k-steps of S = Q K^T
  constexpr int NTO = D / 16;   // 16-wide output tiles
  constexpr int DP = D / 8;     // 16-byte pieces per row
  __shared__ __attribute__((aligned(16))) uint16_t rm[L::RM_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t il[L::IL_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t pb[L::P_ELEMS];
  __shared__ int64_t rsrc[kRT];  // element offset of each tile row (kSegB: segment B), -1: none

  const int t = blockIdx.z;
  const int split = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, quad = lane >> 4;
  const int h0 = blockIdx.y * kHeadsPerWg + wave * 16;

  // selected block indices of the first tile, loaded before anything they
  // would wait on (idx rows always hold sel_stride entries)
  int32_t pidx = 0;
  const int row_begin = split * tiles_per_split * kRT;
  if (p.sel_idx != nullptr && tid < kRT)
    pidx = p.sel_idx[(int64_t)t * p.sel_stride + min(row_begin + tid, p.sel_stride - 1)];
  uint32_t flags = 0;
  const SegDesc sd = token_rows(p, t, flags);
  if (split == 0 && blockIdx.y == 0 && tid == 0) {
    report(p.err, flags);
    if (p.n_kv_out != nullptr) p.n_kv_out[t] = sd.alen + sd.blen;
  }
  flags = 0;
  const int n_rows = sd.alen + sd.blen;
  const int row_end = min(row_begin + tiles_per_split * kRT, n_rows);

  // Q (A operand): lane holds head h0+li, d = ks*32 + quad*8 .. +8.
  bf16x8 qa[KSQ];
  {
    const int h = h0 + li;
    const uint16_t* qh = p.q + ((int64_t)t * p.n_heads + h) * D + quad * 8;
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) {
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (h < p.n_heads) v = *reinterpret_cast<const u32x4*>(qh + ks * 32);
      qa[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  const float sl2 = p.scale * kLog2e;

  f32x4 o[NTO];
#pragma unroll
  for (int n = 0; n < NTO; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
  }

  const uint16_t* kv_a = p.kv_a;
  const uint16_t* kv_b = p.kv_b;
  for (int r0 = row_begin; r0 < row_end; r0 += kRT) {
    __syncthreads();  // the previous tile has been consumed
    // ---- row sources of this tile: one thread per row resolves the block
    // index (gather mode) or segment B, into an LDS table ----
    if (tid < kRT) {
      const int rr = r0 + tid;
      int64_t o = -1;
      if (rr < row_end) {
        if (rr < sd.alen) {
          int64_t ar = sd.a0 + rr;
          if (p.sel_idx != nullptr) {
            ar = sd.a0 + pidx;
            if (ar < 0 || ar >= p.a_rows) {
              flags |= CSA_DERR_ROW_RANGE;
              ar = -1;
            }
          }
          o = ar < 0 ? -1 : ar * D;
        } else {
          o = ((sd.b0 + (rr - sd.alen)) * D) | kSegB;
        }
      }
      rsrc[tid] = o;
      // prefetch the next tile's block indices
      if (p.sel_idx != nullptr && r0 + kRT < row_end)
        pidx = p.sel_idx[(int64_t)t * p.sel_stride + min(r0 + kRT + tid, p.sel_stride - 1)];
    }
    __syncthreads();
    // ---- stage the tile: 8x8 (rows x d) blocks; all loads issued first ----
    constexpr int NB = (kRT / 8) * DP;             // 8x8 blocks per tile
    constexpr int BPTH = (NB + 255) / 256;         // blocks per thread
    u32x4 rows[BPTH][8];
#pragma unroll
    for (int q = 0; q < BPTH; ++q) {
      const int b = tid + q * 256;
      const int g = b / DP, dp = b - g * DP;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int64_t o = b < NB ? rsrc[g * 8 + k] : -1;
        rows[q][k] = u32x4{0u, 0u, 0u, 0u};
        if (o >= 0) {
          const uint16_t* base = (o & kSegB) ? kv_b : kv_a;
          rows[q][k] = *reinterpret_cast<const u32x4*>(base + (o & ~kSegB) + dp * 8);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < BPTH; ++q) {
      const int b = tid + q * 256;
      if (b >= NB) break;
      const int g = b / DP, dp = b - g * DP;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        *reinterpret_cast<u32x4*>(&rm[(g * 8 + k) * L::RM + dp * 8]) = rows[q][k];
      uint16_t* ilg = &il[g * L::ILG + dp * 8 * 8 + dp * 8];
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

    // ---- S = Q K^T for 16 heads x 64 rows ----
    f32x4 s[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) s[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const bf16x8 kb = *reinterpret_cast<const bf16x8*>(&rm[(nt * 16 + li) * L::RM + ks * 32 + quad * 8]);
        s[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kb, s[nt], 0, 0, 0);
      }
    }
    // s[nt][r] = S[head 4*quad + r][row r0 + nt*16 + li]

    // ---- online softmax (exp2 domain) ----
    float x[4][4];
    float mloc[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const bool valid = r0 + nt * 16 + li < row_end;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[nt][r] = valid ? s[nt][r] * sl2 : -INFINITY;
        mloc[r] = fmaxf(mloc[r], x[nt][r]);
      }
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) mloc[r] = fmaxf(mloc[r], __shfl_xor(mloc[r], off));
    }
    float alpha[4], mnew[4], lsum[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      mnew[r] = fmaxf(m_run[r], mloc[r]);
      alpha[r] = (mnew[r] == -INFINITY) ? 1.f : exp2f(m_run[r] - mnew[r]);
      lsum[r] = 0.f;
    }
    uint16_t* pw = &pb[wave * 16 * L::PS];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pv = (x[nt][r] == -INFINITY) ? 0.f : exp2f(x[nt][r] - mnew[r]);
        lsum[r] += pv;
        pw[(4 * quad + r) * L::PS + nt * 16 + li] = f32_to_bf16(pv);
      }
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) lsum[r] += __shfl_xor(lsum[r], off);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      l_run[r] = l_run[r] * alpha[r] + lsum[r];
      m_run[r] = mnew[r];
    }
#pragma unroll
    for (int n = 0; n < NTO; ++n) {
#pragma unroll
      for (int r = 0; r < 4; ++r) o[n][r] *= alpha[r];
    }
    __syncthreads();  // P visible in the A-operand layout

    // ---- O += P V ----
#pragma unroll
    for (int kp = 0; kp < kRT / 32; ++kp) {
      const bf16x8 pa = *reinterpret_cast<const bf16x8*>(&pw[li * L::PS + kp * 32 + quad * 8]);
      const uint16_t* ilg = &il[(kp * 4 + quad) * L::ILG];
#pragma unroll
      for (int n = 0; n < NTO; ++n) {
        const int d = n * 16 + li;
        const bf16x8 vb = *reinterpret_cast<const bf16x8*>(ilg + d * 8 + (d >> 3) * 8);
        o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, o[n], 0, 0, 0);
      }
    }
    // gather mode: copy the staged rows to all_kv (off the staging critical path)
    if (p.copy_out != nullptr) {
      for (int c = tid; c < kRT * DP; c += 256) {
        const int r = c / DP, dp = c - r * DP;
        const int rr = r0 + r;
        if (rr < row_end)
          *reinterpret_cast<u32x4*>(p.copy_out + ((int64_t)t * p.copy_stride + rr) * D + dp * 8) =
              *reinterpret_cast<const u32x4*>(&rm[r * L::RM + dp * 8]);
      }
    }
  }

  report(p.err, flags);
  // ---- epilogue: o[n][r] = O[head 4*quad + r][d = n*16 + li] ----
  if (n_splits == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = h0 + 4 * quad + r;
      if (h >= p.n_heads) continue;
      float M = m_run[r];
      float Lsum = l_run[r];
      float f = 1.f;
      if (p.sink != nullptr) {
        const float s2 = p.sink[h] * kLog2e;
        const float Mn = fmaxf(M, s2);
        f = (M == -INFINITY) ? 0.f : exp2f(M - Mn);
        Lsum = Lsum * f + exp2f(s2 - Mn);
        M = Mn;
      }
      const float inv = Lsum > 0.f ? f / Lsum : 0.f;
      uint16_t* oh = p.out + ((int64_t)t * p.n_heads + h) * D;
#pragma unroll
      for (int n = 0; n < NTO; ++n) oh[n * 16 + li] = f32_to_bf16(o[n][r] * inv);
      if (p.lse != nullptr && li == 0)
        p.lse[(int64_t)t * p.n_heads + h] = Lsum > 0.f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
    }
  } else {
    float* part_o = static_cast<float*>(p.ws);
    float* part_ml = part_o + (size_t)p.T * n_splits * p.n_heads * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = h0 + 4 * quad + r;
      if (h >= p.n_heads) continue;
      const size_t slot = ((size_t)t * n_splits + split) * p.n_heads + h;
      float* po = part_o + slot * D;
#pragma unroll
      for (int n = 0; n < NTO; ++n) po[n * 16 + li] = o[n][r];
      if (li == 0) {
        part_ml[slot * 2 + 0] = m_run[r];
        part_ml[slot * 2 + 1] = l_run[r];
      }
    }
  }
}

// Merge of the split partials of one (token, head): all split weights are
// formed at once (one split per lane), then the partial rows are accumulated
// with their loads batched four splits at a time.
template <int D>
__global__ __launch_bounds__(64) void attend_combine_kernel(AttendLaunch p, int n_splits) {
  constexpr int EPL = D / 64;
  __shared__ float fw[kMaxSplits];
  const int h = blockIdx.x, t = blockIdx.y, lane = threadIdx.x;
  const float* part_o = static_cast<const float*>(p.ws);
  const float* part_ml = part_o + (size_t)p.T * n_splits * p.n_heads * D;
  const size_t slot0 = (size_t)t * n_splits * p.n_heads + h;
  constexpr int SPL = kMaxSplits / 64;
  float m[SPL], l[SPL];
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    const int s = lane + 64 * i;
    m[i] = -INFINITY;
    l[i] = 0.f;
    if (s < n_splits) {
      const size_t slot = slot0 + (size_t)s * p.n_heads;
      m[i] = part_ml[slot * 2];
      l[i] = part_ml[slot * 2 + 1];
      if (l[i] > 0.f) M = fmaxf(M, m[i]);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float s2 = -INFINITY;
  if (p.sink != nullptr) {
    s2 = p.sink[h] * kLog2e;
    M = fmaxf(M, s2);
  }
  float Lsum = 0.f;
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    const int s = lane + 64 * i;
    const float f = (l[i] > 0.f) ? exp2f(m[i] - M) : 0.f;
    Lsum += l[i] * f;
    if (s < n_splits) fw[s] = f;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) Lsum += __shfl_xor(Lsum, off);
  if (p.sink != nullptr) Lsum += exp2f(s2 - M);
  __syncthreads();
  float acc[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) acc[j] = 0.f;
  const float* pb = part_o + slot0 * D + lane * EPL;
  const size_t sstride = (size_t)p.n_heads * D;
  for (int s0 = 0; s0 < n_splits; s0 += 4) {
    float v[4][EPL];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int s = s0 + u;
#pragma unroll
      for (int j = 0; j < EPL; ++j) v[u][j] = 0.f;
      if (s < n_splits && fw[s] != 0.f) {
#pragma unroll
        for (int j = 0; j < EPL; ++j) v[u][j] = pb[(size_t)s * sstride + j];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int s = s0 + u;
      const float f = s < n_splits ? fw[s] : 0.f;
#pragma unroll
      for (int j = 0; j < EPL; ++j) acc[j] += f * v[u][j];
    }
  }
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  uint16_t* oh = p.out + ((size_t)t * p.n_heads + h) * D + lane * EPL;
#pragma unroll
  for (int j = 0; j < EPL; ++j) oh[j] = f32_to_bf16(acc[j] * inv);
  if (p.lse != nullptr && lane == 0)
    p.lse[(size_t)t * p.n_heads + h] = Lsum > 0.f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
}

struct SplitPlan {
  int tiles_per_split, n_splits;
};

SplitPlan plan_splits(int T, int n_heads, int max_rows) {
  SplitPlan sp;
  const int n_tiles = max_rows > 0 ? (max_rows + kRT - 1) / kRT : 1;
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
  const SplitPlan sp = plan_splits(a.T, a.n_heads, a.max_rows);
  const int n_hg = (a.n_heads + kHeadsPerWg - 1) / kHeadsPerWg;
  dim3 grid((unsigned)sp.n_splits, (unsigned)n_hg, (unsigned)a.T);
  hipLaunchKernelGGL((attend_split_kernel<D>), grid, dim3(256), 0, s, a, sp.tiles_per_split,
                     sp.n_splits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sp.n_splits == 1) return e;
  hipLaunchKernelGGL((attend_combine_kernel<D>), dim3((unsigned)a.n_heads, (unsigned)a.T),
                     dim3(64), 0, s, a, sp.n_splits);
  return hipGetLastError();
}

}  // namespace

size_t attend_ws_bytes(int T, int n_heads, int head_dim, int max_rows) {
  const SplitPlan sp = plan_splits(T, n_heads, max_rows);
  if (sp.n_splits == 1) return 256;
  const size_t n = (size_t)T * sp.n_splits * n_heads;
  size_t b = n * head_dim * 4 + n * 2 * 4;
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
