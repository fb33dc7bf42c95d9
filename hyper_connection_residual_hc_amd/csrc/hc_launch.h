// Host-side launchers of the gfx950 kernels. Each returns the hipError_t of the launch; the
// C-ABI layer (hc_api.hip) validates every argument before calling them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hc_device.h"

namespace hc {

// Stats split-K geometry. The 4H columns of a flattened row split into S column slices: slice s
// covers columns [s W, (s + 1) W) of every stream, W = H / S = 32 NC (NC MFMA chunks of 32
// columns per stream). NC is the largest even value up to 10 with S = H / (32 NC) a multiple of
// 4 from 8 to kMaxSlices: a stats block keeps its slice's whole packed fn (NC chunks x 5
// B-operand tiles per stream, 20 NC registers per lane) in the registers of four MFMA waves, so
// the slice must stay narrow. The stats kernels take every multiple of 512 up to 8192 that has
// such an NC, which is all of them but 5632 and 6656:
//   H:   512 1024 1536 2048 2560 3072 3584 4096 4608 5120 6144 7168 7680 8192
//   NC:    2    4    6    8   10    8    4    8    6   10    8    8   10    8
//   S:     8    8    8    8    8   12   28   16   24   16   24   28   24   32
// Each (slice, row) gets a partial record of kPartStride floats: the 24 partial dots of that
// slice's columns and their partial sum of squares.
constexpr int kPackTiles = 5;         // B-operand tiles of 16 packed (part, fn row) columns
constexpr int kGroupRows = 16;        // rows of one MFMA row tile (a stats row group)
constexpr int kPartStride = 25;       // floats per (slice, row) partial record: 24 dots + sumsq
constexpr int kMaxStatsH = 8192;
constexpr int kMaxSlices = 32;  // the slice sums below hold up to this many records per row

struct StatsGeom {
  int S;   // column slices
  int NC;  // 32-column MFMA chunks of each stream in a slice
  int W;   // slice width (columns of each stream)
};
__host__ __device__ constexpr StatsGeom stats_geom(int H) {
  StatsGeom g{0, 0, 0};
  if (H <= 0 || H % 512 || H > kMaxStatsH) return g;
  for (int nc = 10; nc >= 2; nc -= 2) {
    if (H % (32 * nc)) continue;
    const int S = H / (32 * nc);
    if (S % 4 || S < 8 || S > kMaxSlices) continue;
    g.S = S;
    g.NC = nc;
    g.W = 32 * nc;
    return g;
  }
  return g;
}
// Rounds of 4 slice records a row's partial sums take at width H (S / 4). Kernels compiled per
// width size their sums with it; widths without mix stats get 1 so that they still compile.
__host__ __device__ constexpr int slice_rounds(int H) {
  return stats_geom(H).S > 0 ? stats_geom(H).S / 4 : 1;
}
inline int64_t packed_fn_elems(int H) { return (int64_t)4 * H * kPackTiles * 16; }
inline size_t stats_workspace_bytes(int64_t M, int H) {
  return (size_t)stats_geom(H).S * (size_t)M * kPartStride * 4;
}

// Sum over the S slices of one field of a row's partial records, in the one order every
// consumer of the partials uses: four interleaved running sums t_g = p[g] + p[g + 4] + ...
// (g = 0..3, slices in increasing order), then (t_0 + t_1) + (t_2 + t_3). S is a multiple of 4,
// at most kMaxSlices. Every value is loaded before the first add (addresses clamped to the last
// slice, extra values unused), so the loads overlap.
constexpr int kMaxSliceRounds = kMaxSlices / 4;
__device__ __forceinline__ const float* part_at(const float* part, int M, int s, int m, int f) {
  return part + ((int64_t)s * M + m) * kPartStride + f;
}
// t_g of slice group g (the running sum over slices g, g + 4, ... < S)
// (NR rounds: slice_rounds(H) in kernels compiled per width, kMaxSliceRounds otherwise)
template <int NR>
__device__ __forceinline__ void slice_group_load(const float* __restrict__ part, int S, int M,
                                                 int m, int f, int g, float (&v)[NR]) {
#pragma unroll
  for (int j = 0; j < NR; ++j) v[j] = *part_at(part, M, min(4 * j + g, S - 1), m, f);
}
template <int NR>
__device__ __forceinline__ float slice_group_sum(const float (&v)[NR], int S, int g) {
  float t = v[0];
#pragma unroll
  for (int j = 1; j < NR; ++j)
    if (4 * j + g < S) t += v[j];
  return t;
}
__device__ __forceinline__ float slice_sum(const float* __restrict__ part, int S, int M, int m,
                                           int f) {
  float v[4][kMaxSliceRounds];
#pragma unroll
  for (int g = 0; g < 4; ++g) slice_group_load(part, S, M, m, f, g, v[g]);
  float t[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) t[g] = slice_group_sum(v[g], S, g);
  return (t[0] + t[1]) + (t[2] + t[3]);
}
// The same sum spread over a wavefront: the lanes of 16-lane group g = lane / 16 hold t_g; two
// butterfly exchanges across the groups give every lane (t_0 + t_1) + (t_2 + t_3) (each add sees
// the same two operands in every lane, in one order or the other, so all lanes agree bit for bit).
__device__ __forceinline__ float slice_group_combine(float t) {
  t = t + __shfl_xor(t, 16, 64);
  return t + __shfl_xor(t, 32, 64);
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
