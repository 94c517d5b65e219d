// S3 -- gather of the selected compressed rows followed by the sliding-window
// rows into one preallocated buffer (post-probe audit, B1/B2 and C2; 1M-context
// audit, D3/D5): all_kv[t] = cat(comp_kv[seq_kv[t] + idx[t, :count[t]]],
// swa[swa_row0[t] : swa_row0[t] + swa_len[t]]).  A bit-exact row copy with
// 16-byte accesses; consecutive lanes move consecutive 16-byte pieces of a row,
// so every 1 KiB row (head_dim 512) is one fully coalesced wave access.
#include "csa_common.h"

namespace csa {
namespace {

constexpr int kRowsPerWg = 16;

template <int D>
__global__ __launch_bounds__(256) void gather_kernel(
    const uint16_t* __restrict__ comp_kv, int64_t comp_rows, const int64_t* __restrict__ seq_kv,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ count, int top_k,
    const uint16_t* __restrict__ swa, int64_t swa_rows, const int64_t* __restrict__ swa_row0,
    const int32_t* __restrict__ swa_len, int window, uint16_t* __restrict__ all_kv,
    int32_t* __restrict__ n_kv, uint32_t* __restrict__ err) {
  constexpr int CPR = D / 8;  // 16-byte pieces per row
  const int t = blockIdx.y;
  uint32_t flags = 0;
  int32_t cnt = count[t];
  int32_t sl = swa_len[t];
  if (cnt < 0 || cnt > top_k) {
    flags |= CSA_DERR_COUNT_RANGE;
    cnt = cnt < 0 ? 0 : top_k;
  }
  if (sl < 0 || sl > window) {
    flags |= CSA_DERR_COUNT_RANGE;
    sl = sl < 0 ? 0 : window;
  }
  const int n = cnt + sl;
  if (blockIdx.x == 0 && threadIdx.x == 0) n_kv[t] = n;
  const int64_t row0 = seq_kv[t];
  const int64_t srow0 = swa_row0[t];
  const int r_begin = blockIdx.x * kRowsPerWg;
  uint16_t* dst_t = all_kv + (int64_t)t * (top_k + window) * D;
  for (int c = threadIdx.x; c < kRowsPerWg * CPR; c += 256) {
    const int r = r_begin + c / CPR;
    const int part = c % CPR;
    if (r >= n) break;  // rows are visited in increasing order per thread
    int64_t src_row;
    const uint16_t* base;
    int64_t limit;
    if (r < cnt) {
      src_row = row0 + idx[(int64_t)t * top_k + r];
      base = comp_kv;
      limit = comp_rows;
    } else {
      src_row = srow0 + (r - cnt);
      base = swa;
      limit = swa_rows;
    }
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (src_row >= 0 && src_row < limit) {
      v = *reinterpret_cast<const u32x4*>(base + src_row * D + part * 8);
    } else {
      flags |= CSA_DERR_ROW_RANGE;
    }
    *reinterpret_cast<u32x4*>(dst_t + (int64_t)r * D + part * 8) = v;
  }
  report(err, flags);
}

template <int D>
hipError_t launch_d(const GatherLaunch& a, hipStream_t s) {
  const int rows = a.top_k + a.window;
  dim3 grid((unsigned)((rows + kRowsPerWg - 1) / kRowsPerWg), (unsigned)a.T);
  if (rows == 0) grid.x = 1;  // still write n_kv
  hipLaunchKernelGGL((gather_kernel<D>), grid, dim3(256), 0, s, a.comp_kv, a.comp_rows, a.seq_kv,
                     a.idx, a.count, a.top_k, a.swa, a.swa_rows, a.swa_row0, a.swa_len, a.window,
                     a.all_kv, a.n_kv, a.err);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gather(const GatherLaunch& a, hipStream_t s) {
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
