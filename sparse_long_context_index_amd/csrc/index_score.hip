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
//   * every wave walks a contiguous run of 32-block tiles; each tile is
//     fetched with global_load_lds_dwordx4, 1 KiB (whole key rows) per
//     instruction, straight into a per-wave LDS buffer -- no VGPRs, fully
//     coalesced, two tiles in flight (double buffer);
//   * the 16-byte chunk slots of each row are XOR-swizzled by the row index,
//     chosen through the per-lane global address, so that the MFMA B-operand
//     reads (lane = block column, 16 bytes of that row) are bank-conflict free;
//   * the token's queries and head weights are loaded into VGPRs and settled
//     before the loop, so the only memory operations in flight inside it are
//     the tile DMAs, waited for with explicit vmcnt counts; scores stay in
//     VGPRs until the wave's tiles are done.
//
// Optionally the epilogue also emits each wave's top-m composite selection
// keys (score, then lower block index) -- the candidate lists of the top-k.
#include "csa_common.h"

namespace csa {
namespace {

constexpr int kTileN = 32;
constexpr int kWaves = kIndexWaves;
constexpr int kMaxTpw = 8;  // tiles per wave (scores held in VGPRs)

__device__ __forceinline__ void lds_dma16(const void* gsrc, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(gsrc, lds_dst, 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int IHD, int MT>
__global__ __launch_bounds__(256) void index_score_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint16_t* __restrict__ k_idx, int64_t k_rows,
    const int64_t* __restrict__ pos, const int64_t* __restrict__ seq_kv,
    const int32_t* __restrict__ n_comp, int n_ih, int ratio,
    float* __restrict__ scores, int64_t ld, uint64_t* __restrict__ cand,
    uint32_t* __restrict__ nvalid, int cand_m, uint32_t* __restrict__ err,
    int tiles_per_wave) {
  constexpr int KS = IHD / 16;          // MFMA k-steps (one 16-byte chunk per lane each)
  constexpr int CPR = IHD / 8;          // 16-byte chunks per key row
  constexpr int TILE_CHUNKS = kTileN * CPR;
  constexpr int LPT = TILE_CHUNKS / 64; // DMA instructions per tile (1 KiB each)
  __shared__ __attribute__((aligned(16))) u32x4 ktile[kWaves][2][TILE_CHUNKS];

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
  const int64_t tile_begin = ((int64_t)blockIdx.x * kWaves + wave) * tiles_per_wave;
  const int64_t tile_end = min(tile_begin + (int64_t)tiles_per_wave, n_tiles);
  const int64_t wslot = (int64_t)t * gridDim.x * kWaves + (int64_t)blockIdx.x * kWaves + wave;
  if (tile_begin >= tile_end) {  // wave-uniform; no workgroup barrier follows
    if (cand != nullptr && lane == 0) {
      nvalid[wslot] = 0u;
      for (int i = 0; i < cand_m; ++i) cand[wslot * cand_m + i] = 0ull;
    }
    return;
  }
  const char* kbase = reinterpret_cast<const char*>(k_idx + row0 * IHD);

  // A operand: lane (col, half) holds q[head = mt*32+col][16*s + 8*half .. +8]
  // for k-step s; padded heads are zero.  Accumulator element r of lane
  // (col, half) is head 8*(r/4) + 4*half + (r%4) of its 32-head tile.
  u32x4 qv[MT][KS];
  float wv[MT][16];
  const uint16_t* qt = q_idx + (int64_t)t * n_ih * IHD;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int head = mt * 32 + col;
    const int hq = head < n_ih ? head : n_ih - 1;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qt + (int64_t)hq * IHD + 16 * s + 8 * half);
      qv[mt][s] = head < n_ih ? v : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int hw = mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      const float x = w[(int64_t)t * n_ih + (hw < n_ih ? hw : n_ih - 1)];
      wv[mt][r] = hw < n_ih ? x : 0.0f;
    }
  }
  // Settle those loads here: the loop then carries no pending register loads
  // and its waits count tile DMAs only.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" : "+v"(qv[mt][s]));
#pragma unroll
    for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(wv[mt][r]));
  }

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
      lds_dma16(kbase + blk * (IHD * 2) + c * 16, &ktile[wave][b][i * 64]);
    }
  };
  issue_tile(tile_begin, 0);
  if (tile_begin + 1 < tile_end) issue_tile(tile_begin + 1, 1);

  float sc[kMaxTpw];
#pragma unroll
  for (int j = 0; j < kMaxTpw; ++j) sc[j] = 0.0f;

  int j = 0;
  for (int64_t tile = tile_begin; tile < tile_end; ++tile, ++j) {
    const int b = j & 1;
    // all but the next tile's DMA (if issued) have landed
    if (tile + 1 < tile_end) wait_vmcnt<LPT>(); else wait_vmcnt<0>();
    u32x4 kb[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int c = 2 * s + half;
      kb[s] = ktile[wave][b][col * CPR + (c ^ (col & (CPR - 1)))];
    }
    wait_lgkmcnt0();  // buffer b is free again
    if (tile + 2 < tile_end) issue_tile(tile + 2, b);

    f32x16 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 kv = __builtin_bit_cast(bf16x8, kb[s]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qv[mt][s]),
                                                          kv, acc[mt], 0, 0, 0);
    }
    float part = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) part += wv[mt][r] * fmaxf(acc[mt][r], 0.0f);
    }
    part += __shfl_xor(part, 32);
#pragma unroll
    for (int q = 0; q < kMaxTpw; ++q)
      if (q == j) sc[q] = part;
  }

  // coalesced score stores: lanes 0..31 hold consecutive blocks of each tile
  const int nt = (int)(tile_end - tile_begin);
  float* srow = scores + (int64_t)t * ld;
#pragma unroll
  for (int q = 0; q < kMaxTpw; ++q) {
    const int64_t blk = (tile_begin + q) * kTileN + col;
    if (q < nt && half == 0 && blk < n_vis) srow[blk] = sc[q];
  }

  if (cand != nullptr) {
    uint64_t key[kMaxTpw];
#pragma unroll
    for (int q = 0; q < kMaxTpw; ++q) {
      const int64_t blk = (tile_begin + q) * kTileN + col;
      key[q] = (q < nt && half == 0 && blk < n_vis) ? block_key(sc[q], (uint32_t)blk) : 0ull;
    }
    wave_top_m<kMaxTpw>(key, cand_m, cand + wslot * cand_m);
    if (lane == 0) nvalid[wslot] = (uint32_t)(min(n_vis, tile_end * kTileN) - tile_begin * kTileN);
  }
}

template <int IHD, int MT>
hipError_t launch_t(const IndexScoreLaunch& a, const IndexPlan& p, hipStream_t s) {
  dim3 grid(p.wgs_per_token, a.T);
  hipLaunchKernelGGL((index_score_kernel<IHD, MT>), grid, dim3(256), 0, s, a.q_idx, a.w,
                     a.k_idx, a.k_rows, a.pos, a.seq_kv, a.n_comp, a.n_ih, a.ratio, a.scores,
                     a.ld, a.cand, a.nvalid, a.cand_m, a.err, p.tiles_per_wave);
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

}  // namespace

IndexPlan plan_index(int T, int64_t ld) {
  // Every wave owns `tpw` consecutive 32-block tiles; about two resident
  // workgroups per CU over the whole batch (256 CUs), at most kMaxTpw tiles
  // per wave.
  IndexPlan p;
  const int64_t tiles = (ld + kTileN - 1) / kTileN;
  const int64_t total = tiles * (T > 0 ? T : 1);
  int64_t tpw = (total + kWaves * 512 - 1) / (kWaves * 512);
  if (tpw < 1) tpw = 1;
  if (tpw > kMaxTpw) tpw = kMaxTpw;
  p.tiles_per_wave = (int)tpw;
  p.wgs_per_token = (int)((tiles + kWaves * tpw - 1) / (kWaves * tpw));
  return p;
}

hipError_t launch_index_score(const IndexScoreLaunch& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const IndexPlan p = plan_index(a.T, a.ld);
  switch (a.ihd) {
    case 32: return launch_ihd<32>(a, p, s);
    case 64: return launch_ihd<64>(a, p, s);
    case 128: return launch_ihd<128>(a, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace csa
