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

__global__ __launch_bounds__(sel::kThreads) void topk_select_kernel(
    const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ pos,
    const int32_t* __restrict__ n_comp, int ratio, int top_k,
    const uint64_t* __restrict__ cand_all, const uint32_t* __restrict__ nvalid_all,
    int waves_per_token, int blocks_per_wave, int cand_m, int32_t* __restrict__ idx,
    int32_t* __restrict__ count, uint32_t* __restrict__ err) {
  __shared__ sel::SelShared sh;
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  const sel::SelResult r = sel::select_token(
      scores + (int64_t)t * ld, ld, pos[t], n_comp[t], ratio, top_k,
      cand_all + (int64_t)t * waves_per_token * cand_m, nvalid_all + (int64_t)t * waves_per_token,
      waves_per_token, blocks_per_wave, cand_m, sh);
  // one coalesced pass writes the selection and the -1 padding
  int32_t* out = idx + (int64_t)t * top_k;
  for (uint32_t i = tid; i < (uint32_t)top_k; i += sel::kThreads)
    out[i] = i < r.emitted ? (r.listed ? sh.outl[i] : (int32_t)i) : -1;
  if (tid == 0) {
    count[t] = (int32_t)r.emitted;
    report(err, r.flags);
  }
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
  // short rows select over all their blocks; rows whose lists would not fit
  // the select's key set (over kPoolCap groups) take its global path
  if (ld <= kPoolCap || p.waves_per_token > kPoolCap) {
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
  hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)T), dim3(sel::kThreads), 0, s, scores, ld,
                     pos, n_comp, ratio, top_k, ws.cand, ws.nvalid, p.waves_per_token,
                     p.blocks_per_wave, p.cand_m, idx, count, err);
  return hipGetLastError();
}

}  // namespace csa
