// Stages 2-4 of hc pre (deepseek_v4.py, DeepseekV4DecoderLayer.hc_pre):
//   split + Sinkhorn of the 24 mixes into pre(4), post(4), comb(4x4), then
//   y = bf16( c * rsqrt(mean(c^2) + eps) * w ),  c = sum_i pre_i * R_i   (one rounding).
//
// Work layout: one wavefront per row. The row's split + Sinkhorn runs on a 16-lane group
// (one lane per comb entry, row sums over the lane quad, column sums over lanes e^4, e^8);
// the wave's four 16-lane groups compute the same row, so every lane ends up holding the row's
// values without LDS or a barrier. The combine then streams the row: each lane owns 8 columns
// of every 512-column block of all four streams (16-byte accesses, wave-wide 1 KB), keeps c in
// registers, reduces sum(c^2) across the wave in a fixed butterfly order and writes y.
#include "hc_launch.h"

namespace hc {

// ---- split + Sinkhorn, standalone -----------------------------------------------------------
__global__ __launch_bounds__(256) void sinkhorn_kernel(const float* __restrict__ mixes, int M,
                                                       const float* __restrict__ scale,
                                                       const float* __restrict__ base, int iters,
                                                       float pre_eps, float sk_eps,
                                                       float post_mult, float* __restrict__ pre,
                                                       float* __restrict__ post,
                                                       float* __restrict__ comb) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int m = (int)(gid >> 4);
  const int e = (int)(gid & 15);
  // every lane of a 16-lane group takes part in the cross-lane sums: rows past the end
  // recompute the last row and store nothing
  const bool valid = m < M;
  const int mm = valid ? m : M - 1;
  const SplitParams sp{scale[0], scale[1], scale[2], iters, pre_eps, sk_eps, post_mult};
  const float* mx = mixes + (int64_t)mm * kMix;
  const float mix_a = e < 8 ? mx[e] : 0.0f;
  const float base_a = e < 8 ? base[e] : 0.0f;
  float pp;
  const float c = split_sinkhorn_lane(e, mix_a, mx[8 + e], base_a, base[8 + e], sp, &pp);
  if (!valid) return;
  comb[(int64_t)mm * 16 + e] = c;
  if (e < 4) {
    pre[(int64_t)mm * kHC + e] = pp;
  } else if (e < 8) {
    post[(int64_t)mm * kHC + (e - 4)] = pp;
  }
}

hipError_t launch_sinkhorn(const float* mixes, int M, const float* scale, const float* base,
                           int iters, float pre_eps, float sk_eps, float post_mult, float* pre,
                           float* post, float* comb, hipStream_t s) {
  const int64_t threads = (int64_t)M * 16;
  hipLaunchKernelGGL(sinkhorn_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     mixes, M, scale, base, iters, pre_eps, sk_eps, post_mult, pre, post, comb);
  return hipGetLastError();
}

// ---- combine + RMSNorm of one row by one wavefront ------------------------------------------
// NG = H / 512 column blocks; lane covers columns [512 g + 8 lane, +8) of each block g.
// Up to H = 5120 the lane also holds its weight columns from the start (with the row and
// the combine's values that still fits two waves per SIMD); wider rows load them at the end.
template <int NG>
constexpr bool kPreloadWeight = NG <= 10;

template <int NG>
struct RowTile {
  u32x4 r[NG][kHC];
  u32x4 w[kPreloadWeight<NG> ? NG : 1];  // the norm weight's columns of this lane
};

// The row (streamed once, non-temporal), then the weight (shared by every row: cached). All
// loads go out together so their latencies overlap.
template <int NG, bool kWeight = true>
__device__ __forceinline__ void load_row(const uint16_t* __restrict__ Rr,
                                         const uint16_t* __restrict__ w, int lane,
                                         RowTile<NG>& t) {
  constexpr int H = NG * 512;
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int i = 0; i < kHC; ++i) t.r[g][i] = ld16_stream(Rr + i * H + g * 512 + lane * 8);
  if constexpr (kWeight && kPreloadWeight<NG>) {
#pragma unroll
    for (int g = 0; g < NG; ++g) t.w[g] = ld16(w + g * 512 + lane * 8);
  }
}

// y's row: written as bf16 when yr is given, and with kMx also as MXFP8 (qr: e4m3 codes,
// sr: one scale byte per 32 columns) quantised from the same bf16 values, with the rule of
// mxfp8_quant_rows. A 32-column block is the 8 columns of each lane of a lane quad. The row
// is stored non-temporally: its consumer is another kernel, and dirty lines left in the L2
// would only lengthen this kernel's end-of-kernel write-back.
template <int NG, bool kMx>
__device__ __forceinline__ void combine_norm_row(const RowTile<NG>& t, const float (&p)[kHC],
                                                 const uint16_t* __restrict__ w, float eps,
                                                 uint16_t* __restrict__ yr, uint8_t* __restrict__ qr,
                                                 uint8_t* __restrict__ sr, int lane) {
  constexpr int H = NG * 512;
  float c[NG][8];
  float ss = 0.0f;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float r[kHC][8];
#pragma unroll
    for (int i = 0; i < kHC; ++i) unpack8(t.r[g][i], r[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = p[0] * r[0][e];
#pragma unroll
      for (int i = 1; i < kHC; ++i) a = __fmaf_rn(p[i], r[i][e], a);
      c[g][e] = a;
      ss = __fmaf_rn(a, a, ss);
    }
  }
  ss = wave_sum(ss);
  const float rn = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float wf[8], o[8];
    if constexpr (kPreloadWeight<NG>)
      unpack8(t.w[g], wf);
    else
      unpack8(ld16(w + g * 512 + lane * 8), wf);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (c[g][e] * rn) * wf[e];
    const u32x4 yb = pack8(o);
    if (!kMx || yr) st16_stream(yr + g * 512 + lane * 8, yb);
    if constexpr (kMx) {
      const int ex = mx_block_exponent(quad_max_u32(amax_bits8(yb)));
      const float scl = mx_scale(ex);
      u32x2 codes;
      codes[0] = e4m3_word(yb[0], yb[1], scl);
      codes[1] = e4m3_word(yb[2], yb[3], scl);
      __builtin_nontemporal_store(codes, reinterpret_cast<u32x2*>(qr + g * 512 + lane * 8));
      if ((lane & 3) == 0) sr[g * 16 + (lane >> 2)] = (uint8_t)(ex + 127);
    }
  }
}

template <int NG>
__global__ __launch_bounds__(256) void combine_norm_kernel(const uint16_t* __restrict__ R,
                                                           int64_t ldR,
                                                           const float* __restrict__ pre,
                                                           int64_t ldPre,
                                                           const uint16_t* __restrict__ w, int M,
                                                           float eps, uint16_t* __restrict__ y,
                                                           int64_t ldY) {
  const int lane = threadIdx.x & 63;
  const int m = __builtin_amdgcn_readfirstlane((int)blockIdx.x * 4 + (int)(threadIdx.x >> 6));
  if (m >= M) return;
  RowTile<NG> t;
  load_row<NG>(R + (int64_t)m * ldR, w, lane, t);
  __builtin_amdgcn_sched_barrier(0);
  float p[kHC];
#pragma unroll
  for (int i = 0; i < kHC; ++i) p[i] = pre[(int64_t)m * ldPre + i];
  combine_norm_row<NG, false>(t, p, w, eps, y + (int64_t)m * ldY, nullptr, nullptr, lane);
}

// ---- fused: slice reduce + split + Sinkhorn + combine + RMSNorm ----------------------------
template <int NG, bool kMx>
__global__ __launch_bounds__(256) void pre_finish_kernel(
    const float* __restrict__ part, const uint16_t* __restrict__ R, int64_t ldR,
    const float* __restrict__ scale, const float* __restrict__ base,
    const uint16_t* __restrict__ w, int M, int S, float kf, float rms_eps, float pre_eps, float sk_eps,
    int iters, float post_mult, float norm_eps, uint16_t* __restrict__ y, int64_t ldY,
    uint8_t* __restrict__ q, int64_t ldQ, uint8_t* __restrict__ sc, int64_t ldS,
    float* __restrict__ pre, float* __restrict__ post, float* __restrict__ comb) {
  const int lane = threadIdx.x & 63;
  const int m = __builtin_amdgcn_readfirstlane((int)blockIdx.x * 4 + (int)(threadIdx.x >> 6));
  if (m >= M) return;  // wave-uniform: the whole wave leaves together
  const int e = lane & 15, sg = lane >> 4;
  // Loads in issue order: this lane's slice partials (its 16-lane group's quarter of the
  // slices), then the row. Vector loads complete in order, so the split + Sinkhorn waits only
  // for the partials and runs while the row is in flight.
  constexpr int NR = slice_rounds(NG * 512);  // S / 4 at this width
  float pa[NR], pc[NR], pq[NR];
  slice_group_load(part, S, M, m, e & 7, sg, pa);
  slice_group_load(part, S, M, m, 8 + e, sg, pc);
  slice_group_load(part, S, M, m, kMix, sg, pq);
  const float base_a = base[e & 7];
  const float base_c = base[8 + e];
  __builtin_amdgcn_sched_barrier(0);
  RowTile<NG> t;
  load_row<NG>(R + (int64_t)m * ldR, w, lane, t);
  __builtin_amdgcn_sched_barrier(0);

  // mixes for this lane's entries, reduced over the slices exactly as stats_reduce does
  const float rs = mix_rscale(slice_group_combine(slice_group_sum(pq, S, sg)), kf, rms_eps);
  // lanes e >= 8 carry a copy of lane e - 8's pre/post input; their pre/post value is unused
  // (no branch here, so the loads above stay ahead of the row's)
  const float mix_a = slice_group_combine(slice_group_sum(pa, S, sg)) * rs;
  const float mix_c = slice_group_combine(slice_group_sum(pc, S, sg)) * rs;
  const SplitParams sp{scale[0], scale[1], scale[2], iters, pre_eps, sk_eps, post_mult};
  float pp;
  const float cv = split_sinkhorn_lane(e, mix_a, mix_c, base_a, base_c, sp, &pp);
  if (lane < 16) {
    comb[(int64_t)m * 16 + e] = cv;
    if (e < 4) {
      if (pre) pre[(int64_t)m * kHC + e] = pp;
    } else if (e < 8) {
      post[(int64_t)m * kHC + (e - 4)] = pp;
    }
  }
  float p[kHC];
#pragma unroll
  for (int i = 0; i < kHC; ++i) p[i] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pp), i));
  combine_norm_row<NG, kMx>(t, p, w, norm_eps, y ? y + (int64_t)m * ldY : nullptr,
                            kMx ? q + (int64_t)m * ldQ : nullptr,
                            kMx ? sc + (int64_t)m * ldS : nullptr, lane);
}

// ---- hc_head: the model's last mix (deepseek_v4.py, hc_head_torch / fused_hc_head) -----------
// From the slice partials of a 4-row fn (packed as rows 0..3 of the 24-row layout):
//   mixes[i] = d[i] * rsqrt(sum x^2 / 4H + norm_eps),  pre_i = sigmoid(mixes[i] * scale + base_i)
//   + hc_eps,  y = bf16(sum_i pre_i R_i) (fp32, one rounding; no norm: the model's final
// RMSNorm follows separately). One wave per row; every lane forms the four pre values.
template <int NG>
__global__ __launch_bounds__(256) void head_finish_kernel(
    const float* __restrict__ part, const uint16_t* __restrict__ R, int64_t ldR,
    const float* __restrict__ scale, const float* __restrict__ base, int M, int S, float kf,
    float norm_eps, float hc_eps, uint16_t* __restrict__ y, int64_t ldY) {
  constexpr int H = NG * 512;
  const int lane = threadIdx.x & 63;
  const int m = __builtin_amdgcn_readfirstlane((int)blockIdx.x * 4 + (int)(threadIdx.x >> 6));
  if (m >= M) return;
  const int sg = lane >> 4;
  constexpr int NR = slice_rounds(NG * 512);  // S / 4 at this width
  float pd[kHC][NR], pq[NR];
#pragma unroll
  for (int i = 0; i < kHC; ++i) slice_group_load(part, S, M, m, i, sg, pd[i]);
  slice_group_load(part, S, M, m, kMix, sg, pq);
  __builtin_amdgcn_sched_barrier(0);
  RowTile<NG> t;
  load_row<NG, false>(R + (int64_t)m * ldR, nullptr, lane, t);
  __builtin_amdgcn_sched_barrier(0);
  const float rs = mix_rscale(slice_group_combine(slice_group_sum(pq, S, sg)), kf, norm_eps);
  const float s0 = scale[0];
  float p[kHC];
#pragma unroll
  for (int i = 0; i < kHC; ++i)
    p[i] = sigmoidf_(__fmaf_rn(slice_group_combine(slice_group_sum(pd[i], S, sg)) * rs, s0, base[i])) + hc_eps;
  uint16_t* yr = y + (int64_t)m * ldY;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float r[kHC][8], o[8];
#pragma unroll
    for (int i = 0; i < kHC; ++i) unpack8(t.r[g][i], r[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = p[0] * r[0][e];
#pragma unroll
      for (int i = 1; i < kHC; ++i) a = __fmaf_rn(p[i], r[i][e], a);
      o[e] = a;
    }
    st16_stream(yr + g * 512 + lane * 8, pack8(o));
  }
  (void)H;
}

// ---- dispatch over the compiled H values ----------------------------------------------------
// One kernel per row width H = 512 n, n = 1 .. 16 (every multiple of 512 up to 8192). The row
// lives in registers, so the count of column blocks is a compile-time constant: a runtime count
// with a compiled maximum was measured at compile time to cost the 5120-wide finish 32 more
// registers (address registers of the blocks a shorter row skips).
#define HC_FOR_EACH_NG(X) \
  X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16)

bool combine_h_supported(int H) {
  if (H % 512) return false;
  switch (H / 512) {
#define HC_CASE(n) case n: return true;
    HC_FOR_EACH_NG(HC_CASE)
#undef HC_CASE
    default: return false;
  }
}

hipError_t launch_combine_norm(const uint16_t* R, int64_t ldR, const float* pre, int64_t ldPre,
                               const uint16_t* w, int M, int H, float eps, uint16_t* y,
                               int64_t ldY, hipStream_t s) {
  const dim3 grid((unsigned)((M + 3) / 4)), block(256);
  switch (H / 512) {
#define HC_CASE(n)                                                                              \
  case n:                                                                                       \
    hipLaunchKernelGGL(combine_norm_kernel<n>, grid, block, 0, s, R, ldR, pre, ldPre, w, M,     \
                       eps, y, ldY);                                                            \
    break;
    HC_FOR_EACH_NG(HC_CASE)
#undef HC_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_pre_finish(const float* part, const uint16_t* R, int64_t ldR,
                             const float* scale, const float* base, const uint16_t* w, int M,
                             int H, float rms_eps, float pre_eps, float sk_eps, int iters,
                             float post_mult, float norm_eps, uint16_t* y, int64_t ldY,
                             uint8_t* q, int64_t ldQ, uint8_t* sc, int64_t ldS, float* pre,
                             float* post, float* comb, hipStream_t s) {
  const dim3 grid((unsigned)((M + 3) / 4)), block(256);
  const float kf = (float)(4 * H);
  const int S = stats_geom(H).S;
  if (S == 0) return hipErrorInvalidValue;
  switch (H / 512) {
#define HC_CASE(n)                                                                              \
  case n:                                                                                       \
    if (q)                                                                                      \
      hipLaunchKernelGGL((pre_finish_kernel<n, true>), grid, block, 0, s, part, R, ldR, scale,  \
                         base, w, M, S, kf, rms_eps, pre_eps, sk_eps, iters, post_mult,         \
                         norm_eps, y, ldY, q, ldQ, sc, ldS, pre, post, comb);                   \
    else                                                                                        \
      hipLaunchKernelGGL((pre_finish_kernel<n, false>), grid, block, 0, s, part, R, ldR, scale, \
                         base, w, M, S, kf, rms_eps, pre_eps, sk_eps, iters, post_mult,         \
                         norm_eps, y, ldY, q, ldQ, sc, ldS, pre, post, comb);                   \
    break;
    HC_FOR_EACH_NG(HC_CASE)
#undef HC_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_head_finish(const float* part, const uint16_t* R, int64_t ldR,
                              const float* scale, const float* base, int M, int H,
                              float norm_eps, float hc_eps, uint16_t* y, int64_t ldY,
                              hipStream_t s) {
  const dim3 grid((unsigned)((M + 3) / 4)), block(256);
  const float kf = (float)(4 * H);
  const int S = stats_geom(H).S;
  if (S == 0) return hipErrorInvalidValue;
  switch (H / 512) {
#define HC_CASE(n)                                                                              \
  case n:                                                                                       \
    hipLaunchKernelGGL(head_finish_kernel<n>, grid, block, 0, s, part, R, ldR, scale, base, M,  \
                       S, kf, norm_eps, hc_eps, y, ldY);                                        \
    break;
    HC_FOR_EACH_NG(HC_CASE)
#undef HC_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hc
