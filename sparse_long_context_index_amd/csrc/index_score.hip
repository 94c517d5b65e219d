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
// exchange, and one fp32 score per block is stored.
//
// Decode is HBM-bound (64 flop per key byte at n_ih = 64, far below the MFMA
// ridge), so the kernel is organised around streaming the key rows: each
// lane reads one contiguous half-row (IHD/2 bf16, 128 B at ihd = 128) of its
// block, which is exactly the B operand it feeds to the MFMA across the IHD/16
// k-steps -- the reduction index d is permuted identically in A (queries), so
// no LDS staging or shuffles are needed.  Each wave keeps the token's queries
// resident in VGPRs and walks a contiguous run of 32-block tiles with the next
// tile's loads in flight.
//
// Optionally the epilogue also builds the histogram of the top kHistBits bits
// of the order-preserving score key (an LDS histogram per workgroup, flushed
// with one global atomic per non-empty bin), which is the first pass of the
// top-k radix select.
#include "csa_common.h"

namespace csa {
namespace {

constexpr int kTileN = 32;
constexpr int kWaves = 4;

template <int IHD, int MT>
__global__ __launch_bounds__(256) void index_score_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint16_t* __restrict__ k_idx, int64_t k_rows,
    const int64_t* __restrict__ pos, const int64_t* __restrict__ seq_kv,
    const int32_t* __restrict__ n_comp, int n_ih, int ratio,
    float* __restrict__ scores, int64_t ld, uint32_t* __restrict__ hist,
    uint32_t* __restrict__ err, int tiles_per_wave) {
  constexpr int KS = IHD / 16;   // MFMA k-steps
  constexpr int HALF = IHD / 2;  // key elements per lane
  __shared__ uint32_t lhist[kHistBins];

  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 31;
  const int half = lane >> 5;

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
  if (blockIdx.x == 0 && threadIdx.x == 0) report(err, flags);

  const int64_t n_tiles = (n_vis + kTileN - 1) / kTileN;
  const int64_t wg_tile0 = (int64_t)blockIdx.x * kWaves * tiles_per_wave;
  if (wg_tile0 >= n_tiles) return;  // uniform across the workgroup

  const bool do_hist = hist != nullptr;
  if (do_hist) {
    for (int i = threadIdx.x; i < kHistBins; i += 256) lhist[i] = 0u;
    __syncthreads();
  }

  // A operand: lane (col, half) holds q[head = mt*32+col][half*HALF + s*8 + 0..7]
  // for k-step s; padded heads are zero.
  bf16x8 qa[MT][KS];
  const uint16_t* qt = q_idx + (int64_t)t * n_ih * IHD;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int head = mt * 32 + col;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (head < n_ih) {
        u32x4 v = *reinterpret_cast<const u32x4*>(qt + (int64_t)head * IHD + half * HALF + s * 8);
        qa[mt][s] = __builtin_bit_cast(bf16x8, v);
      } else {
        qa[mt][s] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      }
    }
  }
  // Accumulator element r of lane (col, half) holds head row
  // 8*(r/4) + 4*half + (r%4) of its 32-head tile, block column col.
  float wv[MT][16];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int head = mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      wv[mt][r] = head < n_ih ? w[(int64_t)t * n_ih + head] : 0.0f;
    }
  }

  const int64_t tile_begin = wg_tile0 + (int64_t)wave * tiles_per_wave;
  const int64_t tile_end = min(tile_begin + (int64_t)tiles_per_wave, n_tiles);
  const uint16_t* kbase = k_idx + row0 * IHD + half * HALF;
  float* srow = scores + (int64_t)t * ld;

  u32x4 kc[KS], kn[KS];
  auto load_tile = [&](int64_t tile, u32x4* dst) {
    int64_t blk = tile * kTileN + col;
    if (blk > n_vis - 1) blk = n_vis - 1;  // ragged tail: re-read a valid row
    const u32x4* src = reinterpret_cast<const u32x4*>(kbase + blk * IHD);
#pragma unroll
    for (int s = 0; s < KS; ++s) dst[s] = __builtin_nontemporal_load(src + s);
  };

  if (tile_begin < tile_end) load_tile(tile_begin, kc);
  for (int64_t tile = tile_begin; tile < tile_end; ++tile) {
    if (tile + 1 < tile_end) load_tile(tile + 1, kn);
    f32x16 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 kb = __builtin_bit_cast(bf16x8, kc[s]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mt][s], kb, acc[mt], 0, 0, 0);
    }
    float part = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) part += wv[mt][r] * fmaxf(acc[mt][r], 0.0f);
    }
    part += __shfl_xor(part, 32);
    const int64_t blk = tile * kTileN + col;
    if (half == 0 && blk < n_vis) {
      srow[blk] = part;
      if (do_hist) atomicAdd(&lhist[score_key(part) >> (32 - kHistBits)], 1u);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) kc[s] = kn[s];
  }

  if (do_hist) {
    __syncthreads();
    uint32_t* ht = hist + (int64_t)t * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += 256) {
      const uint32_t v = lhist[i];
      if (v != 0u) atomicAdd(ht + i, v);
    }
  }
}

template <int IHD, int MT>
hipError_t launch_t(const IndexScoreLaunch& a, int tiles_per_wave, int wgs, hipStream_t s) {
  dim3 grid(wgs, a.T);
  hipLaunchKernelGGL((index_score_kernel<IHD, MT>), grid, dim3(256), 0, s, a.q_idx, a.w,
                     a.k_idx, a.k_rows, a.pos, a.seq_kv, a.n_comp, a.n_ih, a.ratio, a.scores,
                     a.ld, a.hist, a.err, tiles_per_wave);
  return hipGetLastError();
}

template <int IHD>
hipError_t launch_ihd(const IndexScoreLaunch& a, int tpw, int wgs, hipStream_t s) {
  const int mt = (a.n_ih + 31) / 32;
  switch (mt) {
    case 1: return launch_t<IHD, 1>(a, tpw, wgs, s);
    case 2: return launch_t<IHD, 2>(a, tpw, wgs, s);
    case 3: return launch_t<IHD, 3>(a, tpw, wgs, s);
    case 4: return launch_t<IHD, 4>(a, tpw, wgs, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_index_score(const IndexScoreLaunch& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  // Work split: every wave owns `tpw` consecutive 32-block tiles.  Aim for
  // about two resident workgroups per CU over the whole batch (256 CUs).
  const int64_t tiles = (a.ld + kTileN - 1) / kTileN;
  const int64_t total = tiles * a.T;
  int64_t tpw = (total + kWaves * 512 - 1) / (kWaves * 512);
  if (tpw < 1) tpw = 1;
  if (tpw > 32) tpw = 32;
  const int64_t wgs = (tiles + kWaves * tpw - 1) / (kWaves * tpw);
  switch (a.ihd) {
    case 32: return launch_ihd<32>(a, (int)tpw, (int)wgs, s);
    case 64: return launch_ihd<64>(a, (int)tpw, (int)wgs, s);
    case 128: return launch_ihd<128>(a, (int)tpw, (int)wgs, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace csa
