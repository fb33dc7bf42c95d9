// Stage 1, mix stats: per row x = R[m] flattened (4H bf16 values),
//   d[f] = sum_k fn[f, k] * x_k (24 dots), sumsq = sum_k x_k^2,
//   mixes[f] = d[f] * rsqrt(sumsq / 4H + eps)
// (deepseek_v4.py, DeepseekV4DecoderLayer.hc_pre: hc_pre_torch_impl and the prenorm-GEMM
// path that returns d and sumsq from one pass over x).
//
// The 24 x 4H projection runs on the matrix cores (v_mfma_f32_16x16x32_bf16). x is exactly
// bf16; fn is fp32, so it is split once per weight into three bf16 parts hi + mid + lo (each
// the round-to-nearest-even of what the earlier parts leave). bf16 x bf16 products are exact
// in fp32 and the three parts carry fn to ~24 significant bits, so the contraction is as
// accurate as an fp32 dot product. The three parts of the 24 rows make 72 B-operand columns,
// padded to 80 = 5 tiles of 16. sumsq comes from the same instruction with x as both operands
// (the diagonal of the 16x16 Gram tile).
//
// Split-K: 8 column slices of H/8 columns of every stream; block b takes slice b % 8, so with
// round-robin dispatch every XCD keeps one slice of packed fn (1/8 of 3.3 MB) in its L2.
// A block owns 64 rows of one slice; wave w of the block owns stream w. Partials go to a
// workspace [8][M][32] and are summed in slice order 0..7 by the consumer. Nothing depends on
// M or on a row's position in its tile, so any row slice of a call gives identical bits.
#include "hc_launch.h"

namespace hc {

// ---- weight packing ------------------------------------------------------------------------
// Packed index (in 8-element units): (((s*4 + w)*NC + c)*5 + t)*64 + lane, NC = H/256.
// Lane (n = lane%16, g = lane/16) of tile t holds packed column 16t+n = part (col/24) of fn row
// (col%24) at flattened columns k = w*H + s*(H/8) + 32c + 8g + [0..7]; columns >= 72 are zero.
__device__ __forceinline__ float bf16_round(float v) { return (float)(__bf16)v; }

__global__ __launch_bounds__(256) void fn_pack_kernel(const float* __restrict__ fn, int H,
                                                      uint16_t* __restrict__ out) {
  const int NC = H >> 8;
  const int HS = H >> 3;
  const int64_t total = (int64_t)kSlices * kHC * NC * kPackTiles * 64;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= total) return;
  const int lane = (int)(gid & 63);
  int64_t r = gid >> 6;
  const int t = (int)(r % kPackTiles);
  r /= kPackTiles;
  const int c = (int)(r % NC);
  r /= NC;
  const int w = (int)(r % kHC);
  const int s = (int)(r / kHC);
  const int col = 16 * t + (lane & 15);
  const int part = col / kMix;
  const int f = col % kMix;
  const int64_t k = (int64_t)w * H + (int64_t)s * HS + 32 * c + 8 * (lane >> 4);
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float val = 0.0f;
    if (col < 3 * kMix) {
      const float a = fn[(int64_t)f * 4 * H + k + e];
      const float hi = bf16_round(a);
      const float r1 = a - hi;  // exact
      const float mid = bf16_round(r1);
      const float r2 = r1 - mid;  // exact
      const float lo = bf16_round(r2);
      val = part == 0 ? hi : (part == 1 ? mid : lo);
    }
    v[e] = val;
  }
  st16(out + gid * 8, pack8(v));  // the parts are exact bf16 values: packing does not round
}

hipError_t launch_fn_pack(const float* fn, int H, uint16_t* fn_packed, hipStream_t s) {
  const int64_t total = (int64_t)kSlices * kHC * (H / 256) * kPackTiles * 64;
  hipLaunchKernelGGL(fn_pack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, fn,
                     H, fn_packed);
  return hipGetLastError();
}

// ---- split-K stats -------------------------------------------------------------------------
constexpr int kSub = kStatsRows / 16;  // 16-row MFMA subtiles per block
constexpr int kLdsCols = kPackTiles * 16 + 1;

__global__ __launch_bounds__(256) void stats_kernel(const uint16_t* __restrict__ R, int64_t ldR,
                                                    const uint16_t* __restrict__ fnp, int M,
                                                    int H, float* __restrict__ part) {
  __shared__ float lds_acc[kHC][kStatsRows][kLdsCols];
  __shared__ float lds_sq[kHC][kStatsRows];

  const int s = blockIdx.x & (kSlices - 1);
  const int row0 = (blockIdx.x >> 3) * kStatsRows;
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int NC = H >> 8;
  const int HS = H >> 3;

  const uint16_t* ap[kSub];
  bool av[kSub];
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub) {
    const int row = row0 + sub * 16 + r16;
    av[sub] = row < M;
    ap[sub] = R + (int64_t)(av[sub] ? row : 0) * ldR + (int64_t)w * H + (int64_t)s * HS + 8 * g;
  }
  const u32x4* bp = reinterpret_cast<const u32x4*>(fnp) +
                    ((int64_t)(s * kHC + w) * NC) * kPackTiles * 64 + lane;

  f32x4 acc[kSub][kPackTiles];
  f32x4 sq[kSub];
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub) {
    sq[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < kPackTiles; ++t) acc[sub][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const u32x4 zero = {0u, 0u, 0u, 0u};

  // software pipeline: chunk c+1's operands are in flight while chunk c's MFMAs run
  u32x4 a_cur[kSub], b_cur[kPackTiles];
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub) a_cur[sub] = av[sub] ? ld16_stream(ap[sub]) : zero;
#pragma unroll
  for (int t = 0; t < kPackTiles; ++t) b_cur[t] = bp[t * 64];

  for (int c = 0; c < NC; ++c) {
    u32x4 a_nxt[kSub], b_nxt[kPackTiles];
    const bool more = c + 1 < NC;
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub)
      a_nxt[sub] = (more && av[sub]) ? ld16_stream(ap[sub] + 32 * (c + 1)) : zero;
#pragma unroll
    for (int t = 0; t < kPackTiles; ++t)
      b_nxt[t] = more ? bp[((int64_t)(c + 1) * kPackTiles + t) * 64] : zero;

#pragma unroll
    for (int sub = 0; sub < kSub; ++sub) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, a_cur[sub]);
#pragma unroll
      for (int t = 0; t < kPackTiles; ++t)
        acc[sub][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            a, __builtin_bit_cast(bf16x8, b_cur[t]), acc[sub][t], 0, 0, 0);
      sq[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, sq[sub], 0, 0, 0);
    }
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub) a_cur[sub] = a_nxt[sub];
#pragma unroll
    for (int t = 0; t < kPackTiles; ++t) b_cur[t] = b_nxt[t];
  }

  // 16x16 accumulator layout: lane holds rows 4*(lane/16) + i, column lane % 16
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = sub * 16 + 4 * g + i;
#pragma unroll
      for (int t = 0; t < kPackTiles; ++t) lds_acc[w][row][16 * t + r16] = acc[sub][t][i];
      if (r16 == 4 * g + i) lds_sq[w][sub * 16 + r16] = sq[sub][i];
    }
  }
  __syncthreads();

  // partial[s][row][f] = sum over streams w (in order) of (hi + mid) + lo; [24] = sumsq
  for (int idx = threadIdx.x; idx < kStatsRows * (kMix + 1); idx += 256) {
    const int row = idx / (kMix + 1);
    const int f = idx - row * (kMix + 1);
    const int grow = row0 + row;
    if (grow >= M) continue;
    float v = 0.0f;
    if (f < kMix) {
#pragma unroll
      for (int ww = 0; ww < kHC; ++ww)
        v += (lds_acc[ww][row][f] + lds_acc[ww][row][kMix + f]) + lds_acc[ww][row][2 * kMix + f];
    } else {
#pragma unroll
      for (int ww = 0; ww < kHC; ++ww) v += lds_sq[ww][row];
    }
    part[((int64_t)s * M + grow) * kPartStride + f] = v;
  }
}

hipError_t launch_stats(const uint16_t* R, int64_t ldR, const uint16_t* fn_packed, int M, int H,
                        float* part, hipStream_t s) {
  const unsigned tiles = (unsigned)((M + kStatsRows - 1) / kStatsRows);
  hipLaunchKernelGGL(stats_kernel, dim3(tiles * kSlices), dim3(256), 0, s, R, ldR, fn_packed, M,
                     H, part);
  return hipGetLastError();
}

// ---- reduction of the slices into mixes ----------------------------------------------------
__global__ __launch_bounds__(256) void stats_reduce_kernel(const float* __restrict__ part, int M,
                                                           float kf, float eps,
                                                           float* __restrict__ mixes,
                                                           float* __restrict__ sumsq) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int m = (int)(gid >> 5);
  const int f = (int)(gid & 31);
  if (m >= M || f > kMix) return;
  const float ss = slice_sum(part, M, m, kMix);
  if (f == kMix) {
    if (sumsq) sumsq[m] = ss;
    return;
  }
  mixes[(int64_t)m * kMix + f] = slice_sum(part, M, m, f) * mix_rscale(ss, kf, eps);
}

hipError_t launch_stats_reduce(const float* part, int M, int H, float rms_eps, float* mixes,
                               float* sumsq, hipStream_t s) {
  const int64_t threads = (int64_t)M * 32;
  hipLaunchKernelGGL(stats_reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     s, part, M, (float)(4 * H), rms_eps, mixes, sumsq);
  return hipGetLastError();
}

}  // namespace hc
