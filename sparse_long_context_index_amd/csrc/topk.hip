// S2 -- causal top-k over the indexer scores (post-probe audit, F3:
// tk = min(top_k, n_comp) and a top-k over the scores; PART A, suspect 3: only
// blocks strictly before the query's own block are candidates).
//
// One 1024-thread workgroup per token runs the exact select of
// select_core.h and writes the selection in ascending block order, padded
// with -1 to top_k entries.  The candidate lists it starts from are written
// by the indexer epilogue, or by score_cands_kernel for caller-given scores.
#include "select_core.h"

namespace csa {
namespace {

template <int KP>
__global__ __launch_bounds__(sel::kThreads) void topk_select_kernel(
    const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ pos,
    const int32_t* __restrict__ n_comp, const int64_t* __restrict__ seq_kv, int64_t k_rows,
    int ratio, int top_k, const uint64_t* __restrict__ cand_all, const uint64_t* __restrict__ gcut_all, int list_len,
    int groups_per_token, int blocks_per_group, int32_t* __restrict__ idx,
    int32_t* __restrict__ count, uint32_t* __restrict__ err) {
  __shared__ sel::SelShared<sel::kThreads> sh;
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  const sel::SelResult r = sel::select_token<sel::kThreads, KP>(
      scores + (int64_t)t * ld, ld, pos[t], n_comp[t], ratio,
      seq_kv != nullptr ? seq_kv[t] : 0, seq_kv != nullptr ? k_rows : INT64_MAX, top_k, cand_all + (int64_t)t * groups_per_token * list_len, gcut_all + (int64_t)t * groups_per_token,
      list_len, groups_per_token, blocks_per_group, sh, sh.outl, 0u, (uint32_t)top_k);
  // one coalesced pass writes the selection and the -1 padding
  int32_t* out = idx + (int64_t)t * top_k;
  for (uint32_t i = tid; i < (uint32_t)top_k; i += sel::kThreads)
    out[i] = i < r.emitted ? (r.listed ? sh.outl[i] : (int32_t)i) : -1;
  if (tid == 0) {
    count[t] = (int32_t)r.emitted;
    report(err, r.flags);
  }
}

// The decode step's top-k for larger batches: one workgroup per token, the
// fast select (select_token when it gives up), the selection written straight
// to idx in ascending block order and padded with -1.  KP key slots per
// thread: with twelve, rows of up to 12,288 blocks select over all their
// blocks (the shorter rows of a ragged batch, whose lists would hold too few
// keys); four do a third of the per-slot work on a long row's lists.
template <int KP>
__global__ __launch_bounds__(sel::kThreads) void step_select_kernel(SelectLaunch sl) {
  __shared__ union {
    sel::SelShared<sel::kThreads> s;
    sel::FastShared<sel::kThreads> f;
  } u;
  const int t = blockIdx.x;
  int32_t* out = sl.idx + (int64_t)t * sl.top_k;
  const sel::SelResult r = sel::step_select<sel::kThreads, KP>(
      sl.scores + (int64_t)t * sl.ld, sl.ld, sl.pos[t], sl.n_comp[t], sl.ratio, select_row0(sl, t),
      sl.k_rows, sl.top_k, sl.cand + (int64_t)t * sl.groups_per_token * sl.list_len,
      sl.gcut + (int64_t)t * sl.groups_per_token, sl.list_len, sl.groups_per_token,
      sl.blocks_per_group, sl.lists_complete != 0, u.f, u.s, out, 0u, (uint32_t)sl.top_k);
  for (uint32_t i = threadIdx.x; i < (uint32_t)sl.top_k; i += sel::kThreads) {
    if (i >= r.emitted) out[i] = -1;
    else if (!r.listed) out[i] = (int32_t)i;
  }
  if (threadIdx.x == 0) {
    sl.count[t] = (int32_t)r.emitted;
    report(sl.err, r.flags);
  }
}

// Candidate lists from caller-given scores, in the indexer's layout: a
// workgroup of kIndexWaves waves per indexer workgroup, wave w scoring the
// same blocks as the indexer wave it stands for.
constexpr int kCandThreads = kIndexWaves * 64;
__global__ __launch_bounds__(kCandThreads) void score_cands_kernel(
    const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ pos,
    const int32_t* __restrict__ n_comp, int ratio, int blocks_per_wave, CandArgs ca,
    uint32_t* __restrict__ err) {
  constexpr int KPL = 8;  // up to 8 x 32 = 256 blocks per wave
  constexpr int KPH = KPL / 2;
  constexpr int kStride = kMergeScratch;
  __shared__ uint64_t lds[kIndexWaves * kStride];
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t flags = 0;
  int64_t n_vis = visible_count(pos[t], ratio, n_comp[t], &flags);
  if (n_vis > ld) {
    flags |= CSA_DERR_VIS_OVER_LD;
    n_vis = ld;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) report(err, flags);
  const int64_t wave_in_token = (int64_t)blockIdx.x * kIndexWaves + wave;
  const int64_t b0 = wave_in_token * blocks_per_wave;
  const int64_t b1 = min(b0 + (int64_t)blocks_per_wave, n_vis);
  const float* srow = scores + (int64_t)t * ld;
  // half-wave h takes the 32-block pieces 2p + h of the wave's blocks
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
  uint64_t val;
  const uint32_t n_ok = wave_top_m<KPH>(sc, ok, blk, (uint32_t)ca.wave_m, &val);
  cand_publish(val, n_ok, ca, t, wave_in_token, blockIdx.x, lds, kStride);
}

// The E4M3 prefilter and its bf16 rescore in one launch.  Workgroup x of
// token t runs the exact select of the C best blocks by E4M3 score (every
// workgroup of the token reaches the same selection) but keeps only its
// positions [128x, 128x + 128) of the ascending block order; four of its
// waves then rescore those, 32 a wave, as rescore_kernel does (lane (col,
// half) reads its candidate's bf16 key row into the B operand registers;
// the same operations in the same order as the bf16 indexer, so a score is
// that indexer's score of the block), with the query block and weights in
// LDS.  Against a select kernel of one workgroup a token and the rescore
// launch after it: one kernel boundary and one round trip fewer.
constexpr int kRescorePerWg = 128;
template <int IHD, int MT, int KP>
__global__ __launch_bounds__(sel::kThreads) void prefilter_rescore_kernel(SelectLaunch sl,
                                                                        RescoreLaunch a) {
  constexpr int KS = IHD / 16;
  constexpr int RB = 2 * IHD;
  constexpr int CPR = RB / 16;
  constexpr int QCH = MT * 32 * CPR;
  __shared__ union {
    sel::SelShared<sel::kThreads> s;
    sel::FastShared<sel::kThreads> f;
  } u;
  __shared__ int32_t cand[kRescorePerWg];
  __shared__ __attribute__((aligned(16))) u32x4 qlds[QCH];
  __shared__ float wl[MT * 32];
  const int t = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  // the query rows (chunk p of row r at slot r*CPR + (p ^ (r % CPR)); rows
  // past n_ih repeat the last head, whose weight here is zero) and weights
  const char* qt = reinterpret_cast<const char*>(a.q_idx) + (int64_t)t * a.n_ih * RB;
  for (int e = tid; e < QCH; e += sel::kThreads) {
    const int r = e / CPR, pp = e % CPR;
    const int hq = r < a.n_ih ? r : a.n_ih - 1;
    qlds[r * CPR + (pp ^ (r & (CPR - 1)))] = *reinterpret_cast<const u32x4*>(qt + (int64_t)hq * RB + pp * 16);
  }
  if (tid < MT * 32) wl[tid] = tid < a.n_ih ? a.w[(int64_t)t * a.n_ih + tid] : 0.0f;
  const uint32_t e_lo = blockIdx.x * kRescorePerWg;
  const sel::SelResult r = sel::step_select<sel::kThreads, KP>(
      sl.scores + (int64_t)t * sl.ld, sl.ld, sl.pos[t], sl.n_comp[t], sl.ratio, select_row0(sl, t),
      sl.k_rows, sl.top_k, sl.cand + (int64_t)t * sl.groups_per_token * sl.list_len,
      sl.gcut + (int64_t)t * sl.groups_per_token, sl.list_len, sl.groups_per_token,
      sl.blocks_per_group, sl.lists_complete != 0, u.f, u.s, cand, e_lo, e_lo + kRescorePerWg);
  __syncthreads();  // this workgroup's candidates, the queries and weights are in LDS
  if (blockIdx.x == 0 && tid == 0) {
    a.gcut[t] = 0ull;
    report(sl.err, r.flags);
  }
  if (wave >= kRescorePerWg / 32) return;
  const int64_t j0 = (int64_t)e_lo + wave * 32;
  if (j0 >= a.C) return;  // wave-uniform
  const int64_t j = j0 + col;
  uint64_t* out = a.key + (int64_t)t * a.C;
  const int64_t cnt = r.emitted;
  if (j0 >= cnt) {  // wave-uniform: no candidate in this tile
    if (half == 0 && j < a.C) out[j] = 0ull;
    return;
  }
  // lanes past the count take the tile's first candidate (j0 < cnt)
  const bool valid = j < cnt;
  const int64_t pj = valid ? j : j0;
  const int32_t b = r.listed ? cand[pj - e_lo] : (int32_t)pj;
  const char* krow = reinterpret_cast<const char*>(a.k_idx) + (a.seq_kv[t] + b) * RB;
  u32x4 kb[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) kb[s] = *reinterpret_cast<const u32x4*>(krow + (2 * s + half) * 16);
  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int qr = mt * 32 + col;
      const u32x4 qa = qlds[qr * CPR + ((2 * s + half) ^ (qr & (CPR - 1)))];
      acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qa),
                                                        __builtin_bit_cast(bf16x8, kb[s]), acc[mt],
                                                        0, 0, 0);
    }
  }
  float part = 0.0f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
      part += wl[mt * 32 + 8 * (rr >> 2) + 4 * half + (rr & 3)] * relu_f32(acc[mt][rr]);
  }
  part += __shfl_xor(part, 32);
  const uint32_t sk = score_key(part);
  if (half == 0 && j < a.C)
    out[j] = valid && sk != 0u ? ((uint64_t)sk << 32) | (uint32_t)~(uint32_t)b : 0ull;
}

template <int IHD, int MT>
void launch_prefilter_rescore_t(const SelectLaunch& sl, const RescoreLaunch& a, int T, hipStream_t s) {
  const dim3 grid((unsigned)((a.C + kRescorePerWg - 1) / kRescorePerWg), (unsigned)T);
  // a batch may mix row lengths; a single row is the long row its lists serve
  if (T > 1)
    hipLaunchKernelGGL((prefilter_rescore_kernel<IHD, MT, 12>), grid, dim3(sel::kThreads), 0, s, sl, a);
  else
    hipLaunchKernelGGL((prefilter_rescore_kernel<IHD, MT, 4>), grid, dim3(sel::kThreads), 0, s, sl, a);
}

}  // namespace

TopkPlan plan_topk(int T, int64_t ld, int top_k, int pool) {
  const IndexPlan ip = plan_index(T, ld);
  TopkPlan p{};
  p.waves_per_token = ip.waves_per_token();
  p.blocks_per_wave = ip.blocks_per_wave();
  // Short rows select over all their blocks.  Rows with more groups than the
  // select holds bounds for take its global path.
  if (ld <= pool || p.waves_per_token > kMaxGroups) return p;
  // A workgroup merges its waves' lists into one of 16 keys when the token's
  // merged lists fit the pool and still hold at least three times top_k
  // keys: a group's expected share of a full row's top-k is then at most
  // 16/3 keys, well inside its list.  Each wave keeps its top 8 for the
  // merge, which bounds the group's unlisted blocks tightly.
  const int64_t merged = (int64_t)ip.wgs_per_token * kMergedLen;
  if (merged <= pool && merged >= 3 * (int64_t)top_k) {
    p.wave_m = kMergeMaxWaveM;
    p.merge = 1;
    p.list_len = kMergedLen;
    p.groups_per_token = ip.wgs_per_token;
    p.blocks_per_group = kIndexWaves * p.blocks_per_wave;
    return p;
  }
  // otherwise every wave keeps its share of the select's key set
  int m = pool / p.waves_per_token;
  if (m > 32) m = 32;
  if (m < 1) m = 1;
  p.wave_m = m;
  p.list_len = m;
  p.groups_per_token = p.waves_per_token;
  p.blocks_per_group = p.blocks_per_wave;
  return p;
}

int select_slots(const TopkPlan& p) {
  // with candidate lists of at most 4096 keys, four register slots per
  // thread hold them (and rows of up to 4096 blocks directly); the select's
  // per-slot work is then a third of the twelve-slot variant's
  return p.list_len > 0 && (int64_t)p.groups_per_token * p.list_len <= 4096 ? 4 : 12;
}

CandArgs cand_args(const TopkPlan& p, const TopkWs& w) {
  CandArgs c{};
  c.cand = w.cand;
  c.gcut = w.gcut;
  c.wave_m = p.wave_m;
  c.merge = p.merge;
  c.list_len = p.list_len;
  c.groups_per_token = p.groups_per_token;
  return c;
}

TopkWs topk_ws_layout(void* ws, int T, const TopkPlan& p) {
  TopkWs w{};
  const size_t n = (size_t)T * p.groups_per_token;
  const size_t cand_b = (n * p.list_len * 8 + 255) & ~(size_t)255;
  const size_t cut_b = (n * 8 + 255) & ~(size_t)255;
  w.bytes = p.list_len ? cand_b + cut_b : 0;
  if (ws != nullptr && p.list_len) {
    w.cand = static_cast<uint64_t*>(ws);
    w.gcut = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + cand_b);
  }
  return w;
}

hipError_t launch_score_cands(const float* scores, int64_t ld, const int64_t* pos,
                              const int32_t* n_comp, int T, int ratio, const TopkPlan& p,
                              const TopkWs& ws, uint32_t* err, hipStream_t s) {
  if (T == 0 || p.list_len == 0) return hipSuccess;
  dim3 grid((unsigned)(p.waves_per_token / kIndexWaves), (unsigned)T);
  hipLaunchKernelGGL(score_cands_kernel, grid, dim3(kCandThreads), 0, s, scores, ld, pos, n_comp,
                     ratio, p.blocks_per_wave, cand_args(p, ws), err);
  return hipGetLastError();
}

hipError_t launch_step_select(const SelectLaunch& sl, int T, hipStream_t s) {
  if (T == 0) return hipSuccess;
  // a batch may mix row lengths; a single row is the long row its lists serve
  if (T > 1)
    hipLaunchKernelGGL(step_select_kernel<12>, dim3((unsigned)T), dim3(sel::kThreads), 0, s, sl);
  else
    hipLaunchKernelGGL(step_select_kernel<4>, dim3((unsigned)T), dim3(sel::kThreads), 0, s, sl);
  return hipGetLastError();
}

hipError_t launch_topk_select(const float* scores, int64_t ld, const int64_t* pos,
                              const int32_t* n_comp, const int64_t* seq_kv, int64_t k_rows,
                              int T, int ratio, int top_k,
                              const TopkPlan& p, const TopkWs& ws, int32_t* idx,
                              int32_t* count, uint32_t* err, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (select_slots(p) == 4)
    hipLaunchKernelGGL((topk_select_kernel<4>), dim3((unsigned)T), dim3(sel::kThreads), 0, s, scores,
                       ld, pos, n_comp, seq_kv, k_rows, ratio, top_k, ws.cand, ws.gcut, p.list_len,
                       p.groups_per_token, p.blocks_per_group, idx, count, err);
  else
    hipLaunchKernelGGL((topk_select_kernel<sel::KPT>), dim3((unsigned)T), dim3(sel::kThreads), 0, s,
                       scores, ld, pos, n_comp, seq_kv, k_rows, ratio, top_k, ws.cand, ws.gcut, p.list_len,
                       p.groups_per_token, p.blocks_per_group, idx, count, err);
  return hipGetLastError();
}

bool prefilter_rescore_fits(const RescoreLaunch& a) {
  return a.C > 0 && a.n_ih <= 64 && (a.ihd == 64 || a.ihd == 128);
}

hipError_t launch_prefilter_rescore(const SelectLaunch& sl, const RescoreLaunch& a, int T,
                                    hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (!prefilter_rescore_fits(a)) return hipErrorInvalidValue;
  const bool one = a.n_ih <= 32;
  if (a.ihd == 64) {
    if (one) launch_prefilter_rescore_t<64, 1>(sl, a, T, s); else launch_prefilter_rescore_t<64, 2>(sl, a, T, s);
  } else {
    if (one) launch_prefilter_rescore_t<128, 1>(sl, a, T, s); else launch_prefilter_rescore_t<128, 2>(sl, a, T, s);
  }
  return hipGetLastError();
}

}  // namespace csa
