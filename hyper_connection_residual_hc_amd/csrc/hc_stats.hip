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
// packed into 5 tiles of 16 that feed two accumulators (the parts of a row share one).
// sumsq comes from the same instruction with x as both operands (the diagonal of the 16x16
// Gram tile).
//
// Memory: the MFMA operand layout wants 16 rows x 64 bytes per wave instruction, which streams
// HBM poorly; so each block stages 64 rows x 512 B of its column slice through LDS. A wave
// loads 16 of the rows with wave-wide loads of 2 rows x 512 B, writes them to a padded LDS tile
// (row stride 528 B: conflict-free 16-byte reads), and after a barrier reads 64-byte operand
// tiles back. The next stage's loads are in flight while the current stage is multiplied.
//
// Split-K: 8 contiguous column slices of 4H/8 flattened columns; block b takes slice b % 8, so
// with round-robin dispatch each XCD keeps one slice of packed fn (1/8 of 3.3 MB) in its L2.
// A block owns 64 rows; wave q multiplies chunks 2q, 2q+1 of every 8-chunk stage for all 64
// rows (the fn operand of a chunk serves 64 rows). Partials go to a workspace [8][M][32] and
// are summed in slice order 0..7 by the consumer. Nothing depends on M or on a row's position
// in its tile, so any row slice of a call gives identical bits.
#include "hc_launch.h"

namespace hc {

// ---- weight packing ------------------------------------------------------------------------
// Packed index (in 8-element units): ((s*NCS + c)*5 + t)*64 + lane with NCS = H/64 chunks of
// 32 columns per slice. Lane (n = lane%16, g = lane/16) of tile t holds 8 values of fn at
// flattened columns k = s*(H/2) + 32c + 8g + [0..7], for the (part, fn row) the tile assigns
// to n:
//   t0: hi  of row n        t1: mid of row n        t2: lo of row n          (rows 0..15)
//   t3: n < 8: hi of row 16+n;  n >= 8: mid of row 8+n                        (rows 16..23)
//   t4: n < 8: lo of row 16+n;  n >= 8: zero
// Tiles t0..t2 accumulate into one 16-column accumulator (column f = row f), tiles t3..t4 into
// a second one whose column 16+n holds hi + lo of row 16+n and column 24+n its mid part.
__device__ __forceinline__ float bf16_round(float v) { return (float)(__bf16)v; }

__device__ __forceinline__ void pack_slot(int t, int n, int* row, int* part) {
  if (t < 3) {
    *row = n;
    *part = t;
  } else if (t == 3) {
    *row = n < 8 ? 16 + n : 8 + n;
    *part = n < 8 ? 0 : 1;
  } else {
    *row = n < 8 ? 16 + n : -1;
    *part = 2;
  }
}

__global__ __launch_bounds__(256) void fn_pack_kernel(const float* __restrict__ fn, int H,
                                                      uint16_t* __restrict__ out) {
  const int NCS = H >> 6;
  const int64_t total = (int64_t)kSlices * NCS * kPackTiles * 64;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= total) return;
  const int lane = (int)(gid & 63);
  int64_t r = gid >> 6;
  const int t = (int)(r % kPackTiles);
  r /= kPackTiles;
  const int c = (int)(r % NCS);
  const int s = (int)(r / NCS);
  int f, part;
  pack_slot(t, lane & 15, &f, &part);
  const int64_t k = (int64_t)s * (H / 2) + 32 * c + 8 * (lane >> 4);
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float val = 0.0f;
    if (f >= 0) {
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
  const int64_t total = (int64_t)kSlices * (H / 64) * kPackTiles * 64;
  hipLaunchKernelGGL(fn_pack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, fn,
                     H, fn_packed);
  return hipGetLastError();
}

// ---- split-K stats -------------------------------------------------------------------------
constexpr int kSub = kStatsRows / 16;       // 16-row MFMA subtiles per block
constexpr int kStageElems = 256;            // columns of a row per stage (512 B)
constexpr int kStageChunks = kStageElems / 32;
constexpr int kWaveChunks = kStageChunks / 4;  // chunks each wave multiplies per stage
constexpr int kLdsRow = kStageElems + 8;    // padded LDS row stride in elements (528 B)
constexpr int kLdsCols = 33;                // epilogue: 32 accumulator columns + sumsq

struct StatsAcc {
  f32x4 d0[kSub], d1[kSub], sq[kSub];
};

// One 32-column chunk: 5 MFMAs for the projection + 1 for the Gram diagonal, per subtile.
__device__ __forceinline__ void stats_chunk(StatsAcc& acc, const u32x4 (&a)[kSub],
                                            const u32x4* b) {
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub) {
    const bf16x8 x = __builtin_bit_cast(bf16x8, a[sub]);
    acc.d0[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, __builtin_bit_cast(bf16x8, b[0]), acc.d0[sub], 0, 0, 0);
    acc.d1[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, __builtin_bit_cast(bf16x8, b[3]), acc.d1[sub], 0, 0, 0);
    acc.sq[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, x, acc.sq[sub], 0, 0, 0);
    acc.d0[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, __builtin_bit_cast(bf16x8, b[1]), acc.d0[sub], 0, 0, 0);
    acc.d1[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, __builtin_bit_cast(bf16x8, b[4]), acc.d1[sub], 0, 0, 0);
    acc.d0[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, __builtin_bit_cast(bf16x8, b[2]), acc.d0[sub], 0, 0, 0);
  }
}

__global__ __launch_bounds__(256) void stats_kernel(const uint16_t* __restrict__ R, int64_t ldR,
                                                    const uint16_t* __restrict__ fnp, int M,
                                                    int H, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[kStatsRows * kLdsRow];

  const int s = blockIdx.x & (kSlices - 1);
  const int row0 = (blockIdx.x >> 3) * kStatsRows;
  const int q = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int NCS = H >> 6;            // chunks per slice
  const int nstage = H >> 9;         // 512-byte stages per slice row
  // a wave instruction loads 512 B of two rows: lanes 0..31 the first, 32..63 the second
  const int half = lane >> 5;
  const int col = (lane & 31) * 8;
  const uint16_t* rbase = R + (int64_t)s * (H / 2) + col;
  const u32x4* bbase = reinterpret_cast<const u32x4*>(fnp) + (int64_t)s * NCS * kPackTiles * 64 + lane;

  // stage loads: wave q brings rows 16q .. 16q+15 (rows past the end re-read row M-1)
  u32x4 L[8];
  auto issue = [&](int p) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = min(row0 + 16 * q + 2 * i + half, M - 1);
      L[i] = ld16_stream(rbase + (int64_t)row * ldR + p * kStageElems);
    }
  };

  StatsAcc acc;
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub) {
    acc.d0[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc.d1[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc.sq[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // one stage: stash the landed loads into LDS, then multiply this wave's four chunks while
  // (when `next`) the following stage's loads are in flight
  auto stage = [&](int p, bool next) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<u32x4*>(&lds[(16 * q + 2 * i + half) * kLdsRow + col]) = L[i];
    __syncthreads();
    // the fn operands of this stage go out before the next stage's residual loads: loads
    // return in order, so waiting for them does not wait for HBM
    u32x4 b[kWaveChunks][kPackTiles];
#pragma unroll
    for (int jj = 0; jj < kWaveChunks; ++jj)
#pragma unroll
      for (int t = 0; t < kPackTiles; ++t)
        b[jj][t] = bbase[((int64_t)(p * kStageChunks + kWaveChunks * q + jj) * kPackTiles + t) * 64];
    __builtin_amdgcn_sched_barrier(0);
    if (next) issue(p + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int jj = 0; jj < kWaveChunks; ++jj) {
      const int j = kWaveChunks * q + jj;
      u32x4 a[kSub];
#pragma unroll
      for (int sub = 0; sub < kSub; ++sub)
        a[sub] = *reinterpret_cast<const u32x4*>(&lds[(16 * sub + r16) * kLdsRow + 32 * j + 8 * g]);
      stats_chunk(acc, a, b[jj]);
    }
    __syncthreads();
  };

  // the steady-state loop has a single path (the waitcnt pass then keeps the next stage's
  // loads in flight); the last stage issues nothing
  issue(0);
  for (int p = 0; p + 1 < nstage; ++p) stage(p, true);
  stage(nstage - 1, false);

  // epilogue in the (now idle) LDS tile: 16x16 accumulator layout, lane holds rows
  // 4*(lane/16) + i of column lane % 16
  float(*red)[kStatsRows][kLdsCols] = reinterpret_cast<float(*)[kStatsRows][kLdsCols]>(lds);
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = sub * 16 + 4 * g + i;
      red[q][row][r16] = acc.d0[sub][i];
      red[q][row][16 + r16] = acc.d1[sub][i];
      if (r16 == 4 * g + i) red[q][sub * 16 + r16][32] = acc.sq[sub][i];
    }
  }
  __syncthreads();

  // partial[s][row][f]: sum over the four waves' chunk sets in order; rows 16..23 add their
  // mid column
  for (int idx = threadIdx.x; idx < kStatsRows * (kMix + 1); idx += 256) {
    const int row = idx / (kMix + 1);
    const int f = idx - row * (kMix + 1);
    const int grow = row0 + row;
    if (grow >= M) continue;
    float v = 0.0f;
    if (f < 16) {
#pragma unroll
      for (int w = 0; w < 4; ++w) v += red[w][row][f];
    } else if (f < kMix) {
#pragma unroll
      for (int w = 0; w < 4; ++w) v += red[w][row][f] + red[w][row][f + 8];
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) v += red[w][row][32];
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
