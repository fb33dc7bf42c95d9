// Row-local MXFP8 quantizer (prefill_sp.py, module docstring stage 2, _mxfp8_quantize and
// mxfp8_gather: e4m3 elements with one ue8m0 scale per row per 32 columns, linear scales).
//
// Per 32-column block: the block exponent e from the largest |y| (mx_block_exponent: the
// smallest e with amax * 2^-e <= 448), scale byte e + 127; elements y * 2^-e (an exact
// power-of-two scaling) rounded to nearest even into e4m3fn, with the sign of zero kept; the
// rule keeps every scaled value within +-448.
//
// One lane per 8 consecutive values (a 16-byte load, an 8-byte store of codes), T such units
// in flight per lane: a lane quad holds a 32-value block, whose maximum comes from a quad DPP
// max; the quad's first lane writes the scale byte. T is 5 when a row's units come in
// multiples of 320 (K = 5120: two full waves per row), else 8.
#include "hc_launch.h"

namespace hc {

template <int T>
__global__ __launch_bounds__(256) void mxfp8_kernel(const uint16_t* __restrict__ y, int64_t ldY,
                                                    int M, int U, int chunks,
                                                    uint8_t* __restrict__ q, int64_t ldQ,
                                                    uint8_t* __restrict__ sc, int64_t ldS) {
  // A unit is 8 consecutive values of a row; U = K / 8 units per row, a multiple of 4. A wave
  // takes 64 T units of one row (chunk j): lane l holds units 64 (T j + t) + l, t < T, so each
  // load instruction reads 1 KB contiguous and the lane quads hold whole 32-value blocks.
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int m = (int)(wid / chunks);
  if (m >= M) return;  // wave-uniform
  const int j = (int)(wid - (int64_t)m * chunks);
  const uint16_t* yr = y + (int64_t)m * ldY;
  u32x4 v[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int u = 64 * (T * j + t) + lane;
    v[t] = ld16_stream(yr + 8 * (int64_t)min(u, U - 1));  // past the row's end: a valid unit
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int u = 64 * (T * j + t) + lane;  // quads past the end are whole quads (U % 4 == 0)
    const int e = mx_block_exponent(quad_max_u32(amax_bits8(v[t])));
    if (u < U) {
      const float scl = mx_scale(e);
      u32x2 codes;
      codes[0] = e4m3_word(v[t][0], v[t][1], scl);
      codes[1] = e4m3_word(v[t][2], v[t][3], scl);
      __builtin_nontemporal_store(codes, reinterpret_cast<u32x2*>(q + (int64_t)m * ldQ + 8 * (int64_t)u));
      if ((u & 3) == 0) sc[(int64_t)m * ldS + (u >> 2)] = (uint8_t)(e + 127);
    }
  }
}

hipError_t launch_mxfp8(const uint16_t* y, int64_t ldY, int M, int K, uint8_t* q, int64_t ldQ,
                        uint8_t* scales, int64_t ldS, hipStream_t s) {
  const int U = K / 8;
  const int T = U % 320 == 0 ? 5 : 8;
  const int chunks = (U + 64 * T - 1) / (64 * T);
  const int64_t waves = (int64_t)M * chunks;
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  if (T == 5)
    hipLaunchKernelGGL(mxfp8_kernel<5>, grid, block, 0, s, y, ldY, M, U, chunks, q, ldQ, scales,
                       ldS);
  else
    hipLaunchKernelGGL(mxfp8_kernel<8>, grid, block, 0, s, y, ldY, M, U, chunks, q, ldQ, scales,
                       ldS);
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
