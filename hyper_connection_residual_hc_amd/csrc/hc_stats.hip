// Reduction of the mix-stats partials (S column slices, written by the stats kernel in
// hc_pipe.hip) into mixes[m, f] = d[f] * rsqrt(sumsq / 4H + eps) and sumsq
// (deepseek_v4.py, DeepseekV4DecoderLayer.hc_pre: hc_pre_torch_impl and the prenorm-GEMM path).
#include "hc_launch.h"

namespace hc {

// ---- reduction of the slices into mixes ----------------------------------------------------
__global__ __launch_bounds__(256) void stats_reduce_kernel(const float* __restrict__ part, int M,
                                                           int S, float kf, float eps,
                                                           float* __restrict__ mixes,
                                                           float* __restrict__ sumsq) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int m = (int)(gid >> 5);
  const int f = (int)(gid & 31);
  if (m >= M || f > kMix) return;
  const float ss = slice_sum(part, S, M, m, kMix);
  if (f == kMix) {
    if (sumsq) sumsq[m] = ss;
    return;
  }
  mixes[(int64_t)m * kMix + f] = slice_sum(part, S, M, m, f) * mix_rscale(ss, kf, eps);
}

hipError_t launch_stats_reduce(const float* part, int M, int H, float rms_eps, float* mixes,
                               float* sumsq, hipStream_t s) {
  const int64_t threads = (int64_t)M * 32;
  hipLaunchKernelGGL(stats_reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     s, part, M, stats_geom(H).S, (float)(4 * H), rms_eps, mixes, sumsq);
  return hipGetLastError();
}

}  // namespace hc
