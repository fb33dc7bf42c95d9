// Row-local MXFP8 quantizer (prefill_sp.py, module docstring stage 2, _mxfp8_quantize and
// mxfp8_gather: e4m3 elements with one ue8m0 scale per row per 32 columns, linear scales).
//
// Per 32-column block: amax is the largest |y| (for finite bf16, magnitude order is the
// integer order of the low 15 bits). The block exponent is the smallest e with
// amax * 2^-e <= 448 = 1.75 * 2^8: with amax = (1 + f/128) * 2^(E-127), e = E - 135 + [f > 96]
// (1 + f/128 > 1.75 exactly when f > 96), clamped to [-127, 127]; zero and bf16-subnormal
// maxima give -127. The scale byte is e + 127. Elements are y * 2^-e (exact in fp32) rounded
// to nearest even into e4m3fn (bias 7, 3 mantissa bits, subnormal step 2^-9), saturating at
// +-448, with the sign of zero kept.
//
// One thread per block: 64 bytes in (4 x 16-byte loads), 32 code bytes out (2 x 16-byte
// stores) and one scale byte; consecutive lanes take consecutive blocks of a row.
#include "hc_launch.h"

namespace hc {

__device__ __forceinline__ uint32_t e4m3_code(float s) {
  const uint32_t u = __float_as_uint(s);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a >= 0x3C800000u) {  // |s| >= 2^-6: normal e4m3 after rounding
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);  // round to 3 mantissa bits, ties even
    const int ex = (int)(r >> 23) - 127 + 7;
    const uint32_t man = (r >> 20) & 7u;
    code = (ex > 15 || (ex == 15 && man == 7u)) ? 0x7Eu : (((uint32_t)ex << 3) | man);
  } else {  // subnormal range: multiples of 2^-9, rounded to nearest even
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  }
  return code | sign;
}

__global__ __launch_bounds__(256) void mxfp8_kernel(const uint16_t* __restrict__ y, int64_t ldY,
                                                    int M, int G, uint8_t* __restrict__ q,
                                                    int64_t ldQ, uint8_t* __restrict__ sc,
                                                    int64_t ldS) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int m = (int)(gid / G);
  if (m >= M) return;
  const int g = (int)(gid - (int64_t)m * G);
  const uint16_t* src = y + (int64_t)m * ldY + g * 32;
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = ld16_stream(src + 8 * i);

  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = max(amax, v[i][j] & 0x7fffu);
      amax = max(amax, (v[i][j] >> 16) & 0x7fffu);
    }
  const int E = (int)(amax >> 7);
  const int f = (int)(amax & 0x7f);
  int e = (E == 0) ? -127 : E - 135 + (f > 96 ? 1 : 0);
  e = min(max(e, -127), 127);
  sc[(int64_t)m * ldS + g] = (uint8_t)(e + 127);
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, e in [-127, 126]

  u32x4 out[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t word[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t w0 = v[i][2 * h], w1 = v[i][2 * h + 1];
      const uint32_t c0 = e4m3_code(bf_lo(w0) * inv);
      const uint32_t c1 = e4m3_code(bf_hi(w0) * inv);
      const uint32_t c2 = e4m3_code(bf_lo(w1) * inv);
      const uint32_t c3 = e4m3_code(bf_hi(w1) * inv);
      word[h] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
    out[i >> 1][(i & 1) * 2] = word[0];
    out[i >> 1][(i & 1) * 2 + 1] = word[1];
  }
  uint8_t* dst = q + (int64_t)m * ldQ + g * 32;
  st16_stream(dst, out[0]);
  st16_stream(dst + 16, out[1]);
}

hipError_t launch_mxfp8(const uint16_t* y, int64_t ldY, int M, int K, uint8_t* q, int64_t ldQ,
                        uint8_t* scales, int64_t ldS, hipStream_t s) {
  const int G = K / 32;
  const int64_t threads = (int64_t)M * G;
  hipLaunchKernelGGL(mxfp8_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, y,
                     ldY, M, G, q, ldQ, scales, ldS);
  return hipGetLastError();
}

}  // namespace hc
