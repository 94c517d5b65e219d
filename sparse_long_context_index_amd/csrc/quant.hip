// Row quantisation of bf16 rows to OCP FP8 E4M3 with one power-of-two scale
// per row -- the narrow indexer keys and queries of the post-probe audit's C4
// (and the 1M-context audit's M1/A2), stored and scored in eight bits.
//
// For a row x with amax = max|x|: the scale is 2**e for the smallest e with
// amax * 2**-e <= 448 (E4M3's largest finite value; e = 0 for a zero row);
// each code is x * 2**-e rounded to the nearest E4M3 value, ties to even,
// subnormals included (spacing 2**-9).  A power-of-two scale is exact, so the
// codes depend on the inputs alone.  One wave per row, eight elements a lane.
#include "csa_common.h"

namespace csa {
namespace {

// E4M3 code of a finite fp32 value with |y| <= 448 (ties to even).
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t code;
  if (a >= 0.015625f) {  // 2**-6, the smallest normal
    const uint32_t au = __float_as_uint(a);
    int E = (int)((au >> 23) & 0xFFu) - 127;
    const uint32_t f = au & 0x7FFFFFu;
    uint32_t n = f >> 20;  // three mantissa bits
    const uint32_t rem = f & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (n & 1u))) ++n;
    if (n == 8u) {
      n = 0u;
      ++E;
    }
    code = ((uint32_t)(E + 7) << 3) | n;
  } else {
    code = (uint32_t)rintf(a * 512.0f);  // exact product; rint rounds half to even
  }
  return sign | code;
}

// The row's scale exponent from the bits of amax (a non-negative fp32):
// amax = f * 2**E with 1 <= f < 2; e = E - 8 when f <= 1.75, else E - 7.
__device__ __forceinline__ int e4m3_row_exponent(uint32_t amax_bits) {
  if (amax_bits == 0u) return 0;
  int E;
  uint32_t frac;
  const uint32_t ex = amax_bits >> 23;
  if (ex != 0u) {
    E = (int)ex - 127;
    frac = amax_bits & 0x7FFFFFu;
  } else {  // subnormal fp32: amax = amax_bits * 2**-149
    const int p = 31 - __clz((int)amax_bits);  // leading bit, p <= 22
    E = p - 149;
    frac = (amax_bits << (23 - p)) & 0x7FFFFFu;
  }
  return frac <= 0x600000u ? E - 8 : E - 7;
}

template <int EPL>  // elements per lane (d = 64 * EPL)
__global__ __launch_bounds__(256) void quant_e4m3_kernel(const uint16_t* __restrict__ src,
                                                          int64_t rows, int d,
                                                          uint8_t* __restrict__ codes,
                                                          float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // wave-uniform
  const uint16_t* s = src + row * d;
  float x[EPL];
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int j = lane * EPL + i;
    x[i] = j < d ? bf16_to_f32(s[j]) : 0.0f;
    amax = max(amax, __float_as_uint(x[i]) & 0x7FFFFFFFu);  // |x| orders as its bits
  }
  amax = wave_max_u32(amax);
  const int e = e4m3_row_exponent(amax);
  uint8_t* c = codes + row * d;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int j = lane * EPL + i;
    if (j < d) c[j] = (uint8_t)e4m3_rne(ldexpf(x[i], -e));
  }
  if (lane == 0) scale[row] = ldexpf(1.0f, e);
}

}  // namespace

hipError_t launch_quant_e4m3(const uint16_t* src, int64_t rows, int d, uint8_t* codes,
                             float* scale, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 3) / 4));
  switch ((d + 63) / 64) {
    case 1: hipLaunchKernelGGL(quant_e4m3_kernel<1>, grid, dim3(256), 0, s, src, rows, d, codes, scale); break;
    case 2: hipLaunchKernelGGL(quant_e4m3_kernel<2>, grid, dim3(256), 0, s, src, rows, d, codes, scale); break;
    case 3: case 4: hipLaunchKernelGGL(quant_e4m3_kernel<4>, grid, dim3(256), 0, s, src, rows, d, codes, scale); break;
    case 5: case 6: case 7: case 8: hipLaunchKernelGGL(quant_e4m3_kernel<8>, grid, dim3(256), 0, s, src, rows, d, codes, scale); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace csa
