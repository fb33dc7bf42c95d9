// Row-local MXFP8 quantizer (prefill_sp.py, module docstring stage 2, _mxfp8_quantize and
// mxfp8_gather: e4m3 elements with one ue8m0 scale per row per 32 columns, linear scales).
//
// Per 32-column block: the block exponent e from the largest |y| (mx_block_exponent: the
// smallest e with amax * 2^-e <= 448), scale byte e + 127; elements y * 2^-e (exact in fp32)
// rounded to nearest even into e4m3fn, saturating at +-448, with the sign of zero kept.
//
// One thread per block: 64 bytes in (4 x 16-byte loads), 32 code bytes out (2 x 16-byte
// stores) and one scale byte; consecutive lanes take consecutive blocks of a row.
#include "hc_launch.h"

namespace hc {

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
  for (int i = 0; i < 4; ++i) amax = max(amax, amax_bits8(v[i]));
  const int e = mx_block_exponent(amax);
  sc[(int64_t)m * ldS + g] = (uint8_t)(e + 127);
  const float inv = mx_inv_scale(e);

  u32x4 out[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[i >> 1][(i & 1) * 2] = e4m3_word(v[i][0], v[i][1], inv);
    out[i >> 1][(i & 1) * 2 + 1] = e4m3_word(v[i][2], v[i][3], inv);
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

// ---- 128x4 scale layout ------------------------------------------------------------------
// prefill_sp.py, swizzle_128x4: linear scales [M, G] -> rows zero-padded to a multiple of 128,
// tiles (m / 128, g / 4) in row-tile-major order, 512 bytes each; inside a tile, byte
// (m % 32) * 16 + ((m % 128) / 32) * 4 + g % 4. One thread per output word: the 4 scales of
// one row and one g-quad.
__global__ __launch_bounds__(256) void mx_swizzle_kernel(const uint8_t* __restrict__ sc,
                                                         int64_t ldS, int M, int G,
                                                         uint32_t* __restrict__ out,
                                                         int64_t words) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= words) return;
  const int64_t tile = gid >> 7;  // 128 words per tile
  const int r = (int)(gid & 127);  // (m % 32) * 4 + (m % 128) / 32
  const int tiles_g = G / 4;
  const int64_t tm = tile / tiles_g;
  const int tg = (int)(tile - tm * tiles_g);
  const int64_t m = tm * 128 + (r & 3) * 32 + (r >> 2);
  uint32_t word = 0;
  if (m < M) {
    const uint8_t* src = sc + m * ldS + 4 * tg;
    word = (uint32_t)src[0] | ((uint32_t)src[1] << 8) | ((uint32_t)src[2] << 16) |
           ((uint32_t)src[3] << 24);
  }
  out[gid] = word;
}

hipError_t launch_mx_swizzle(const uint8_t* sc, int64_t ldS, int M, int G, uint8_t* out,
                             hipStream_t s) {
  const int64_t words = (int64_t)((M + 127) / 128) * 128 * G / 4;
  hipLaunchKernelGGL(mx_swizzle_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s,
                     sc, ldS, M, G, reinterpret_cast<uint32_t*>(out), words);
  return hipGetLastError();
}

}  // namespace hc
