// Producer side of the CSA caches for one decode step (1M-context audit,
// D1/D2: a main compressor and an indexer-key compressor, each
// Compressor(ratio, width, H) projecting the hidden state to 2 x width per
// token; its closing assessment: overlapped 2m-token windows with softmax
// weights; D5: the sliding window ring).  Per token t of sequence s at
// position p:
//   y = [W_kv; W_ik] x_t                  (value and score halves of both)
//   ring[s, p mod 2m] = y                 (the last 2m tokens' projections)
//   swa[s, head] = bf16(c_kv); head = (head + 1) mod window; len = min(len+1, window)
//   if p + 1 = (i + 1) m:                 (block i complete)
//     row_i = sum_j softmax_j(z_j) c_j    per channel over tokens [(i-1)m, (i+1)m)
//     comp_kv[seq_kv[s] + i], k_idx[seq_kv[s] + i] = bf16(rows); n_comp[s] = i + 1
//
// Two kernels.  project_kernel is the projection as a split-K bf16 MFMA
// product over all the tokens of the call (decode: a weight-streaming
// GEMV/GEMM, 2 x (hd + ihd) x H x 2 bytes of weights read once per call);
// append_kernel, one workgroup per token, sums the split-K partials and does
// the rest.
#include "csa_common.h"

namespace csa {
namespace {

constexpr int kPjKChunk = 1024;  // hidden elements per workgroup (four waves of 256)
constexpr int kPjWaveK = 256;    // per wave: 16 k-steps of 16

// partial[kc][t][n] = sum over k in chunk kc of x[t, k] w[n, k].  Workgroup
// (n-tile of 32 output channels, k-chunk, 32-token tile); each wave one 256-wide
// slice of the chunk: W rows are the MFMA A operand (channel = row), the
// tokens' x rows the B operand (token = column); the four waves' 32 x 32
// accumulators are added through LDS.
__global__ __launch_bounds__(256) void project_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                      const uint16_t* __restrict__ w_kv, int n_kv,
                                                      const uint16_t* __restrict__ w_ik,
                                                      float* __restrict__ part, int N) {
  __shared__ float red[4][32][33];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int n0 = blockIdx.x * 32;
  const int kc = blockIdx.y;
  const int t0 = blockIdx.z * 32;
  const int kbeg = kc * kPjKChunk + wave * kPjWaveK;
  const bool kact = kbeg < H;  // wave-uniform: H is a multiple of 256
  f32x16 acc = f32x16{};
  if (kact) {
    // A: output channel n0 + col; B: token t0 + col (the last token for padding)
    const int n = n0 + col;
    const uint16_t* wrow = n < n_kv ? w_kv + (size_t)n * H : w_ik + (size_t)(n - n_kv) * H;
    const int t = min(t0 + col, T - 1);
    const uint16_t* xrow = x + (size_t)t * H;
    // The sum runs over the wave's 256 k in any order: k-step s of half h
    // takes k = kbeg + 128h + 8s .. +8 in both operands, so that each lane
    // reads 256 contiguous bytes of its row.
    constexpr int KS = kPjWaveK / 16;
    u32x4 a[KS], b[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int k = kbeg + (kPjWaveK / 2) * half + 8 * s;
      a[s] = *reinterpret_cast<const u32x4*>(wrow + k);
      b[s] = *reinterpret_cast<const u32x4*>(xrow + k);
    }
    // keep every load ahead of the products: all 32 in flight at once (the
    // scheduler would otherwise interleave them with the MFMAs, a few at a
    // time, one round trip after another)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[s]),
                                                    __builtin_bit_cast(bf16x8, b[s]), acc, 0, 0, 0);
  }
  // accumulator element r of lane (col, half): channel 8(r/4) + 4 half + r%4, token col
#pragma unroll
  for (int r = 0; r < 16; ++r) red[wave][8 * (r >> 2) + 4 * half + (r & 3)][col] = acc[r];
  __syncthreads();
  for (int e = threadIdx.x; e < 32 * 32; e += 256) {
    const int ch = e & 31, tk = e >> 5;  // consecutive threads: consecutive channels
    const int t = t0 + tk;
    if (t < T) {
      const float v = red[0][ch][tk] + red[1][ch][tk] + red[2][ch][tk] + red[3][ch][tk];
      part[((size_t)kc * T + t) * N + n0 + ch] = v;
    }
  }
}

struct AppendArgs {
  const float* part; int n_kc;
  const int32_t* seq; const int64_t* pos; int T, S, hd, ihd, ratio, window;
  float* ring; uint16_t* swa; int32_t* swa_head; int32_t* swa_len;
  uint16_t* comp_kv; uint16_t* k_idx; const int64_t* seq_kv; int32_t* n_comp; int64_t comp_rows;
  uint32_t* err;
};

// Per channel of one compressor: softmax over the window's ring rows of the
// score column weighting the value column.  The window's cnt <= R tokens sit
// in ring slots (j0 + k) mod R; every load is issued before the first use.
template <int R>
__device__ __forceinline__ float pool_channel(const float* ring_s, int N, int j0, int cnt,
                                              int c_col, int z_col) {
  float c[R], z[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int slot = (j0 + (k < cnt ? k : cnt - 1)) % R;
    c[k] = ring_s[(size_t)slot * N + c_col];
    z[k] = ring_s[(size_t)slot * N + z_col];
  }
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < R; ++k)
    if (k < cnt) m = fmaxf(m, z[k]);
  float num = 0.f, den = 0.f;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    if (k < cnt) {
      const float e = __expf(z[k] - m);
      num += e * c[k];
      den += e;
    }
  }
  return num / den;
}

template <int R>  // 2 * ratio
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  __shared__ int s_head;
  __shared__ int s_ok;
  const int t = blockIdx.x;
  const int hd = a.hd, ihd = a.ihd;
  const int N = 2 * hd + 2 * ihd;
  const int s = a.seq[t];
  const int64_t p = a.pos[t];
  if (threadIdx.x == 0) {
    int ok = s >= 0 && s < a.S && p >= 0;
    if (!ok) report(a.err, CSA_DERR_BAD_META);
    s_ok = ok;
    s_head = ok ? a.swa_head[s] : 0;
  }
  __syncthreads();
  if (!s_ok) return;  // workgroup-uniform
  const bool head_ok = s_head >= 0 && s_head < a.window;
  const int head = head_ok ? s_head : 0;
  float* ring_s = a.ring + (size_t)s * R * N;
  float* slot = ring_s + (size_t)(p % R) * N;
  uint16_t* swa_row = a.swa + ((size_t)s * a.window + head) * hd;
  for (int n = threadIdx.x; n < N; n += 256) {
    // the split-K partials, eight at a time in flight
    float y = 0.f;
    for (int kc0 = 0; kc0 < a.n_kc; kc0 += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = a.part[((size_t)min(kc0 + u, a.n_kc - 1) * a.T + t) * N + n];
#pragma unroll
      for (int u = 0; u < 8; ++u) y += kc0 + u < a.n_kc ? v[u] : 0.f;
    }
    slot[n] = y;
    if (n < hd) swa_row[n] = f32_to_bf16(y);
  }
  const bool complete = (p + 1) % a.ratio == 0;
  __syncthreads();  // the token's ring row is written before it is pooled; head is read
  if (threadIdx.x == 0) {
    if (!head_ok) report(a.err, CSA_DERR_BAD_META);
    a.swa_head[s] = (head + 1) % a.window;
    a.swa_len[s] = min(a.swa_len[s] + 1, a.window);
  }
  if (!complete) return;
  const int64_t i = (p + 1) / a.ratio - 1;
  const int64_t row = a.seq_kv[s] + i;
  if (row < 0 || row >= a.comp_rows) {
    if (threadIdx.x == 0) report(a.err, CSA_DERR_KEY_RANGE);
    return;
  }
  // the window's tokens base .. (i+1)m - 1 sit in ring slots j mod 2m
  const int64_t base = i >= 1 ? (i - 1) * a.ratio : 0;
  const int j0 = (int)(base % R), cnt = (int)((i + 1) * a.ratio - base);
  for (int ch = threadIdx.x; ch < hd + ihd; ch += 256) {
    if (ch < hd) {
      const float v = pool_channel<R>(ring_s, N, j0, cnt, ch, hd + ch);
      a.comp_kv[(size_t)row * hd + ch] = f32_to_bf16(v);
    } else {
      const int c = ch - hd;
      const float v = pool_channel<R>(ring_s, N, j0, cnt, 2 * hd + c, 2 * hd + ihd + c);
      a.k_idx[(size_t)row * ihd + c] = f32_to_bf16(v);
    }
  }
  if (threadIdx.x == 0) {
    if (a.n_comp[s] != (int32_t)i) report(a.err, CSA_DERR_BAD_META);
    a.n_comp[s] = (int32_t)(i + 1);
  }
}

}  // namespace

size_t compress_ws_bytes(int T, int H, int hd, int ihd) {
  const size_t n_kc = (size_t)((H + kPjKChunk - 1) / kPjKChunk);
  return n_kc * (size_t)T * (size_t)(2 * hd + 2 * ihd) * 4;
}

hipError_t launch_compress_append(const CompressLaunch& c, hipStream_t s) {
  if (c.T == 0) return hipSuccess;
  const int N = 2 * c.hd + 2 * c.ihd;
  const int n_kc = (c.H + kPjKChunk - 1) / kPjKChunk;
  float* part = static_cast<float*>(c.ws);
  const dim3 grid((unsigned)(N / 32), (unsigned)n_kc, (unsigned)((c.T + 31) / 32));
  hipLaunchKernelGGL(project_kernel, grid, dim3(256), 0, s, c.x, c.T, c.H, c.w_kv, 2 * c.hd,
                     c.w_ik, part, N);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  AppendArgs a{};
  a.part = part; a.n_kc = n_kc;
  a.seq = c.seq; a.pos = c.pos; a.T = c.T; a.S = c.S; a.hd = c.hd; a.ihd = c.ihd;
  a.ratio = c.ratio; a.window = c.window;
  a.ring = c.ring; a.swa = c.swa; a.swa_head = c.swa_head; a.swa_len = c.swa_len;
  a.comp_kv = c.comp_kv; a.k_idx = c.k_idx; a.seq_kv = c.seq_kv; a.n_comp = c.n_comp;
  a.comp_rows = c.comp_rows; a.err = c.err;
  switch (c.ratio) {
#define CSA_APPEND(M) \
  case M: hipLaunchKernelGGL(append_kernel<2 * M>, dim3((unsigned)c.T), dim3(256), 0, s, a); break;
    CSA_APPEND(1) CSA_APPEND(2) CSA_APPEND(4) CSA_APPEND(8) CSA_APPEND(16)
#undef CSA_APPEND
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace csa
