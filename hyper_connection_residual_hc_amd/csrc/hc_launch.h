// Host-side launchers of the gfx950 kernels. Each returns the hipError_t of the launch; the
// C-ABI layer (hc_api.cpp) validates every argument before calling them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hc_device.h"

namespace hc {

// Stats split-K geometry: 8 column slices (slice s = columns [s*H/8, (s+1)*H/8) of every
// stream; block b takes slice b % 8, so each XCD keeps one slice's fn in its L2);
// 32-column chunks inside a slice; 5 B-operand tiles of 16 packed columns (hi | mid | lo
// parts of the 24 fn rows, padded to 80).
constexpr int kSlices = 8;
constexpr int kPackTiles = 5;
constexpr int kStatsRows = 64;        // rows per stats tile
constexpr int kPartStride = 32;       // floats per (slice, row) partial record: 24 dots + sumsq
__host__ __device__ inline int64_t chunks_per_slice(int H) { return (int64_t)4 * (H / kSlices) / 32; }
inline int64_t packed_fn_elems(int H) { return (int64_t)kSlices * chunks_per_slice(H) * kPackTiles * 64 * 8; }
inline size_t stats_workspace_bytes(int64_t M) { return (size_t)kSlices * (size_t)M * kPartStride * 4; }

// Sum of one field of a row's slice partials, in slice order. Used by every consumer
// of the partials, so the standalone and the fused pre give identical bits.
__device__ __forceinline__ float slice_sum(const float (&v)[kSlices]) {
  float t = 0.0f;
#pragma unroll
  for (int s = 0; s < kSlices; ++s) t += v[s];
  return t;
}
__device__ __forceinline__ void slice_load(const float* __restrict__ part, int M, int m, int f,
                                           float (&v)[kSlices]) {
#pragma unroll
  for (int s = 0; s < kSlices; ++s) v[s] = part[((int64_t)s * M + m) * kPartStride + f];
}
__device__ __forceinline__ float slice_sum(const float* __restrict__ part, int M, int m, int f) {
  float v[kSlices];
  slice_load(part, M, m, f, v);
  return slice_sum(v);
}

// fn [rows, 4H] (rows <= 24) into the packed stats operands; missing rows are zero
hipError_t launch_fn_pack(const float* fn, int H, int rows, uint16_t* fn_packed, hipStream_t s);
hipError_t launch_stats(const uint16_t* R, int64_t ldR, const uint16_t* fn_packed, int M, int H,
                        float* part, hipStream_t s);
hipError_t launch_stats_reduce(const float* part, int M, int H, float rms_eps, float* mixes,
                               float* sumsq, hipStream_t s);
// hc post fused with the mix stats of its output R' (partials as launch_stats writes them)
hipError_t launch_post_stats(const uint16_t* x, int64_t ldX, const uint16_t* R, int64_t ldR,
                             const float* post, const float* comb, const uint16_t* fn_packed,
                             int M, int H, uint16_t* out, int64_t ldOut, float* part,
                             hipStream_t s);

hipError_t launch_sinkhorn(const float* mixes, int M, const float* scale, const float* base,
                           int iters, float pre_eps, float sk_eps, float post_mult, float* pre,
                           float* post, float* comb, hipStream_t s);
hipError_t launch_combine_norm(const uint16_t* R, int64_t ldR, const float* pre, int64_t ldPre,
                               const uint16_t* w, int M, int H, float eps, uint16_t* y,
                               int64_t ldY, hipStream_t s);
// q == NULL: bf16 y only; otherwise also (or, with y == NULL, only) the MXFP8 form of y
hipError_t launch_pre_finish(const float* part, const uint16_t* R, int64_t ldR,
                             const float* scale, const float* base, const uint16_t* w, int M,
                             int H, float rms_eps, float pre_eps, float sk_eps, int iters,
                             float post_mult, float norm_eps, uint16_t* y, int64_t ldY,
                             uint8_t* q, int64_t ldQ, uint8_t* sc, int64_t ldS, float* pre,
                             float* post, float* comb, hipStream_t s);
// hc_head from the stats partials: pre = sigmoid(mixes[0..3] * scale[0] + base) + hc_eps,
// y = bf16(sum_i pre_i R_i)
hipError_t launch_head_finish(const float* part, const uint16_t* R, int64_t ldR,
                              const float* scale, const float* base, int M, int H,
                              float norm_eps, float hc_eps, uint16_t* y, int64_t ldY,
                              hipStream_t s);
hipError_t launch_mx_swizzle(const uint8_t* sc, int64_t ldS, int M, int G, uint8_t* out,
                             hipStream_t s);

hipError_t launch_post(const uint16_t* x, int64_t ldX, const uint16_t* R, int64_t ldR,
                       const float* post, const float* comb, int M, int H, uint16_t* out,
                       int64_t ldOut, hipStream_t s);

hipError_t launch_mxfp8(const uint16_t* y, int64_t ldY, int M, int K, uint8_t* q, int64_t ldQ,
                        uint8_t* scales, int64_t ldS, hipStream_t s);

// H values with a compiled combine/norm kernel (H = 512 * groups per lane).
bool combine_h_supported(int H);

}  // namespace hc
