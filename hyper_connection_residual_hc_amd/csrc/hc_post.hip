// Stage 5, hc post: Rout[m, j, :] = post[m, j] * x[m, :] + sum_i comb[m, i, j] * R[m, i, :],
// fp32 arithmetic, one round-to-nearest-even to bf16 (deepseek_v4.py,
// DeepseekV4DecoderLayer.hc_post, hc_post_torch_impl).
//
// Pure streaming: per row 10 KB of x and 40 KB of R in, 40 KB of Rout out. One wavefront
// owns one row and 512 consecutive columns; each lane moves 8 columns of x and of all four
// streams with 16-byte accesses, so every wave-wide access is a contiguous 1 KB. The row's
// 20 coefficients are wave-uniform and come in through scalar loads. x and R are read once
// (non-temporal loads); Rout is stored through the caches, since the next hc pre reads it
// right away and it fits the Infinity Cache at prefill sizes.
#include "hc_launch.h"

namespace hc {

__global__ __launch_bounds__(256) void post_kernel(const uint16_t* __restrict__ x, int64_t ldX,
                                                   const uint16_t* __restrict__ R, int64_t ldR,
                                                   const float* __restrict__ post,
                                                   const float* __restrict__ comb, int M, int H,
                                                   int waves_per_row,
                                                   uint16_t* __restrict__ out, int64_t ldOut) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)blockIdx.x * 4 + (int)(threadIdx.x >> 6));
  const int m = wave / waves_per_row;
  if (m >= M) return;
  const int h = (wave - m * waves_per_row) * 512 + lane * 8;

  const uint16_t* xr = x + (int64_t)m * ldX + h;
  const uint16_t* Rr = R + (int64_t)m * ldR + h;
  const u32x4 xv = ld16_stream(xr);
  u32x4 rv[kHC];
#pragma unroll
  for (int i = 0; i < kHC; ++i) rv[i] = ld16_stream(Rr + (int64_t)i * H);

  const float* pm = post + (int64_t)m * kHC;
  const float* cm = comb + (int64_t)m * kHC * kHC;
  float pj[kHC], cij[kHC][kHC];
#pragma unroll
  for (int j = 0; j < kHC; ++j) pj[j] = pm[j];
#pragma unroll
  for (int i = 0; i < kHC; ++i)
#pragma unroll
    for (int j = 0; j < kHC; ++j) cij[i][j] = cm[i * kHC + j];

  float xf[8], rf[kHC][8];
  unpack8(xv, xf);
#pragma unroll
  for (int i = 0; i < kHC; ++i) unpack8(rv[i], rf[i]);

  uint16_t* orow = out + (int64_t)m * ldOut + h;
#pragma unroll
  for (int j = 0; j < kHC; ++j) {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = pj[j] * xf[e];
#pragma unroll
      for (int i = 0; i < kHC; ++i) a = __fmaf_rn(cij[i][j], rf[i][e], a);
      o[e] = a;
    }
    st16(orow + (int64_t)j * H, pack8(o));
  }
}

hipError_t launch_post(const uint16_t* x, int64_t ldX, const uint16_t* R, int64_t ldR,
                       const float* post, const float* comb, int M, int H, uint16_t* out,
                       int64_t ldOut, hipStream_t s) {
  const int wpr = H / 512;
  const int64_t waves = (int64_t)M * wpr;
  const unsigned blocks = (unsigned)((waves + 3) / 4);
  hipLaunchKernelGGL(post_kernel, dim3(blocks), dim3(256), 0, s, x, ldX, R, ldR, post, comb, M,
                     H, wpr, out, ldOut);
  return hipGetLastError();
}

}  // namespace hc
