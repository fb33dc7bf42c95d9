// Mix stats of a residual, alone or fused behind hc post (deepseek_v4.py,
// DeepseekV4DecoderLayer.hc_pre's mix stats; DeepseekV4DecoderLayer.forward's fused
// mhc_fused_post_pre, which takes the previous sublayer's hc post together with the next
// hc pre). Per row x (flattened stream-major, 4H values) the kernel produces, for each of S
// column slices, the partial dots d[f] = sum_k fn[f, k] x_k (24 of them) and sum_k x_k^2.
// In the fused form the row is R' = post * x + comb^T R (x the sublayer output, one bf16
// rounding), which the kernel also stores.
//
// Arithmetic: the 24 x 4H projection runs on the matrix cores (v_mfma_f32_16x16x32_bf16).
// x is exactly bf16; fn is fp32, split once per weight into three bf16 parts hi + mid + lo
// (each the round-to-nearest-even of what the earlier parts leave). bf16 products are exact
// in fp32 and the three parts carry fn to ~24 significant bits. The 72 (part, row) columns are
// packed into 5 B-operand tiles of 16 feeding two accumulators; sum x^2 is the diagonal of the
// 16x16 Gram tile of x with itself.
//
// Geometry (hc_launch.h, stats_geom): slice s covers columns [s W, (s + 1) W) of all four
// streams (W = 32 NC; 320 at H = 5120, 16 slices). A block owns one slice for the whole call:
// its four MFMA waves load the slice's packed fn once (stream q's NC chunks x 5 tiles, 20 NC
// registers per lane) and keep it, so no operand traffic competes with the residual's stream.
// Block b takes slice b % S; row groups of 16 rows go round robin over the slice's blocks
// (stage k of block kb is row group k * BPS + kb), so at any time the grid sweeps a band of
// BPS x 16 rows of every slice.
//
// One block of 8 waves per CU:
//  * waves 0-3 stream the residual (and in the fused form the sublayer output): a stage is a
//    16-row group across the whole slice width (row runs of W bf16 = 640 bytes per stream at
//    H = 5120); each wave loads 16 NC (row, 8-column) items with buffer loads, 2.5 wave-wide
//    loads per array at NC = 10 (the half one reads out of range in lanes 32-63: no traffic,
//    no branch, so the compiler's in-order load counts stay exact); in the fused form it
//    computes R' in the same operation order as the hc post kernel (identical bits) and stores
//    it; it writes the stage's bf16 rows into one slot of a two-slot LDS ring. Each item's loads
//    for the next stage go out as soon as the item is done: a steady stream of about one stage
//    (51 KB per CU in the fused form) in flight. Whole stages issued two ahead keep twice that
//    in flight in bursts and measured slower;
//  * waves 4-7 multiply the previous stage: wave q owns stream q, NC chunks x 6 MFMAs into one
//    16-row accumulator set, then writes it to a double-buffered LDS epilogue; a stage later
//    the four waves sum the streams' accumulators (stream order) and store the slice's partial
//    records of the group;
//  * one block barrier per stage.
// The LDS row stores 16-byte unit u (stream-major across the slice) at u ^ (row & 15): the MFMA
// waves' reads of one unit of 16 rows hit 16 distinct bank groups.
//
// Partials go to a workspace [S][M][25] (24 dots, sum of squares). Nothing depends on M or on
// where a row sits in its group (rows past the end recompute row M-1 and store identical bits;
// their partials are not written), so any row slice of a call gives the same bits as the full
// call, and one kernel serves every M.
#include "hc_launch.h"

namespace hc {

constexpr int kEpiCols = 33;   // 32 accumulator columns + sum of squares
constexpr int kCoefs = kHC + kHC * kHC;  // post(4) + comb(16) per row
constexpr uint32_t kOutOfRange = 0x80000000u;  // buffer offset past every descriptor's range

// ---- fn packing -------------------------------------------------------------------------------
// Packed index (8-element units): ((((s * 4 + q) * NC + c) * 5 + t) * 64 + lane. Chunk c of
// stream q in slice s covers flattened columns k = q H + s W + 32 c + [0, 32). Lane (n =
// lane % 16, g = lane / 16) of tile t holds the 8 columns k0 + 8g + [0..7] of the (part, fn row)
// the tile assigns to n:
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

// fn has `rows` rows (24 for the mixes, 4 for the head); rows past it pack as zeros.
__global__ __launch_bounds__(256) void fn_pack_kernel(const float* __restrict__ fn, int H,
                                                      int rows, uint16_t* __restrict__ out) {
  const StatsGeom geo = stats_geom(H);
  const int64_t total = (int64_t)4 * H / 32 * kPackTiles * 64;  // 8-element units
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= total) return;
  const int lane = (int)(gid & 63);
  int64_t r = gid >> 6;
  const int t = (int)(r % kPackTiles);
  r /= kPackTiles;
  const int c = (int)(r % geo.NC);
  r /= geo.NC;
  const int q = (int)(r % kHC);
  const int s = (int)(r / kHC);
  int f, part;
  pack_slot(t, lane & 15, &f, &part);
  const int64_t k = (int64_t)q * H + (int64_t)s * geo.W + 32 * c + 8 * (lane >> 4);
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float val = 0.0f;
    if (f >= 0 && f < rows) {
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

hipError_t launch_fn_pack(const float* fn, int H, int rows, uint16_t* fn_packed,
                          hipStream_t s) {
  const int64_t total = (int64_t)4 * H / 32 * kPackTiles * 64;
  hipLaunchKernelGGL(fn_pack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, fn,
                     H, rows, fn_packed);
  return hipGetLastError();
}

// ---- the stats kernel -------------------------------------------------------------------------
struct PipeArgs {
  const uint16_t* x;  // fused form: the sublayer output [M, H]
  int64_t ldX;
  const uint16_t* R;  // residual [M, 4, H]
  int64_t ldR;
  const float* post;  // fused form: [M, 4]
  const float* comb;  // fused form: [M, 4, 4]
  const uint16_t* fnp;
  uint16_t* out;      // fused form: R' [M, 4, H]
  int64_t ldOut;
  float* part;        // [S][M][25]
  int M, H, S;
  int groups;         // ceil(M / 16)
  int blocks_per_slice;
};

__device__ __forceinline__ u32x4 buf_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  // non-temporal (streamed once)
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2));
}
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                          const u32x4& v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, 0);
}
// A buffer descriptor for the 16 rows of a group starting at `base` with row stride `ld`
// elements: byte offsets at or past 16 * ld * 2 (kOutOfRange among them) read zero and drop
// stores. The host checks ld < 2^26, so the range stays below 2^31.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t group_rsrc(const uint16_t* base, int64_t ld) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0,
                                           (int)(kGroupRows * ld * 2), 0x00020000);
}

template <int NC, bool kPost>
__global__ __launch_bounds__(512) void stats_kernel(PipeArgs a) {
  constexpr int W = 32 * NC;          // slice width (columns of each stream)
  constexpr int UR = W / 8;           // 16-byte units of one stream's slice of a row
  constexpr int UPR = kHC * UR;       // units of one LDS row (four streams)
  constexpr int kFull = NC / 4;       // full wave-wide items
  constexpr bool kHalf = (NC % 4) != 0;  // plus one item in lanes 0-31 (NC % 4 == 2)
  constexpr int kItems = kFull + (kHalf ? 1 : 0);
  constexpr int kLoads = kPost ? kHC + 1 : kHC;
  static_assert(NC % 2 == 0 && NC >= 2 && NC <= 10, "slice geometry");

  __shared__ __attribute__((aligned(16))) u32x4 ring[2][kGroupRows * UPR];
  __shared__ __attribute__((aligned(16))) float epi[2][kHC][kGroupRows][kEpiCols];
  __shared__ __attribute__((aligned(16))) float coef[2][kGroupRows][kCoefs];

  const int S = a.S;
  const int s = blockIdx.x % S;
  const int kb = blockIdx.x / S;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int M = a.M, H = a.H, bps = a.blocks_per_slice;
  const int total = kb < a.groups ? (a.groups - 1 - kb) / bps + 1 : 0;
  if (total == 0) return;  // block-uniform: no barrier is skipped by part of the block
  const int hs = s * W;
  auto group_of = [&](int k) __attribute__((always_inline)) { return k * bps + kb; };

  if (wave < 4) {
    // ===================================== producers ======================================
    // item t of this lane: flat i = 16 NC wave + 64 t + lane over the group's 16 rows x UR
    // units (row i / UR, unit i % UR); the half item is live in lanes 0-31 only
    u32x4 ld0[kItems][kLoads], ld1[kItems][kLoads];
    auto item = [&](int t, int& lr, int& u, bool& live) __attribute__((always_inline)) {
      live = t < kFull || lane < 32;
      const int i = live ? 16 * NC * wave + 64 * t + lane : 16 * NC * wave;
      lr = i / UR;
      u = i - lr * UR;
    };
    // item t of stage k into d[t]; past the last stage the same loads go out with out-of-range
    // offsets in every lane: the instruction stream (and so the in-order wait counts) stays the
    // same, no bytes move
    auto issue_item = [&](int k, int t, u32x4 (&d)[kItems][kLoads]) __attribute__((always_inline)) {
      const bool past = k >= total;
      const int g = group_of(min(k, total - 1));
      const int r0 = g * kGroupRows;
      const __amdgpu_buffer_rsrc_t rR = group_rsrc(a.R + (int64_t)r0 * a.ldR, a.ldR);
      const __amdgpu_buffer_rsrc_t rX = group_rsrc(kPost ? a.x + (int64_t)r0 * a.ldX : a.R, kPost ? a.ldX : a.ldR);
      int lr, u;
      bool live;
      item(t, lr, u, live);
      const int row = min(r0 + lr, M - 1) - r0;  // rows past the end read row M-1
      const bool go = live && !past;
      const uint32_t oR = go ? (uint32_t)((row * a.ldR + hs + 8 * u) * 2) : kOutOfRange;
#pragma unroll
      for (int i = 0; i < kHC; ++i) d[t][i] = buf_load(rR, oR, (uint32_t)(i * H * 2));
      if constexpr (kPost) {
        const uint32_t oX = go ? (uint32_t)((row * a.ldX + hs + 8 * u) * 2) : kOutOfRange;
        d[t][kHC] = buf_load(rX, oX, 0u);
      }
    };
    // stage k from d; right after each item, the same item of stage kn goes out into dn
    auto produce = [&](int k, u32x4 (&d)[kItems][kLoads], int kn, u32x4 (&dn)[kItems][kLoads]) __attribute__((always_inline)) {
      const int r0 = group_of(k) * kGroupRows;
      u32x4* slot = ring[k & 1];
      // (the stats-only form stores nothing; its descriptor is never used)
      const __amdgpu_buffer_rsrc_t rO = group_rsrc(kPost ? a.out + (int64_t)r0 * a.ldOut : a.R, kPost ? a.ldOut : a.ldR);
#pragma unroll
      for (int t = 0; t < kItems; ++t) {
        int lr, u;
        bool live;
        item(t, lr, u, live);
        u32x4 st[kHC];
        if constexpr (kPost) {
          const float* cf = coef[k & 1][lr];
          float pj[kHC], cij[kHC][kHC];
#pragma unroll
          for (int j = 0; j < kHC; ++j) pj[j] = cf[j];
#pragma unroll
          for (int i = 0; i < kHC; ++i)
#pragma unroll
            for (int j = 0; j < kHC; ++j) cij[i][j] = cf[kHC + i * kHC + j];
          float xf[8], rf[kHC][8];
          unpack8(d[t][kHC], xf);
#pragma unroll
          for (int i = 0; i < kHC; ++i) unpack8(d[t][i], rf[i]);
          // same operation order as the standalone hc post kernel: identical bits
#pragma unroll
          for (int j = 0; j < kHC; ++j) {
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              float acc = pj[j] * xf[e];
#pragma unroll
              for (int i = 0; i < kHC; ++i) acc = __fmaf_rn(cij[i][j], rf[i][e], acc);
              o[e] = acc;
            }
            st[j] = pack8(o);
          }
          // rows past the end hold row M-1's inputs and coefficients: they store its bits again
          const int row = min(r0 + lr, M - 1) - r0;
          const uint32_t oO = live ? (uint32_t)((row * a.ldOut + hs + 8 * u) * 2) : kOutOfRange;
#pragma unroll
          for (int j = 0; j < kHC; ++j) buf_store(rO, oO, (uint32_t)(j * H * 2), st[j]);
        } else {
#pragma unroll
          for (int i = 0; i < kHC; ++i) st[i] = d[t][i];
        }
        if (live) {
#pragma unroll
          for (int j = 0; j < kHC; ++j) slot[lr * UPR + ((j * UR + u) ^ lr)] = st[j];
        }
        issue_item(kn, t, dn);
      }
    };

#pragma unroll
    for (int t = 0; t < kItems; ++t) issue_item(0, t, ld0);
    __syncthreads();  // the first group's coefficients are in LDS
    // Stages in pairs (two load buffers in fixed registers); stage k's items were issued one
    // by one during stage k - 1, each as soon as its slot was free, so about one stage of
    // loads is in flight per wave at any time. Every path from one stage to the next issues the
    // same memory operations, so the compiler's in-order wait counts stay exact.
    int k = 0;
    for (; k + 2 <= total; k += 2) {
      produce(k, ld0, k + 1, ld1);
      __syncthreads();
      produce(k + 1, ld1, k + 2, ld0);
      __syncthreads();
    }
    if (k < total) {
      produce(k, ld0, k + 1, ld1);
      __syncthreads();
    }
    __syncthreads();  // the MFMA waves' last stage: total + 2 barriers in all, as theirs
  } else {
    // ===================================== MFMA waves =====================================
    const int q = wave - 4;  // stream
    const int r16 = lane & 15, g = lane >> 4;
    // the slice's fn operands of stream q, kept for the whole call (loaded below)
    u32x4 b[NC][kPackTiles];
    // post / comb of stage k's 16 rows (fused form): 80 of the 256 lanes each load one vector
    // of 4 (16 rows x 5) two iterations before the producers need it, and store it into
    // coefficient slot k & 1 one iteration later, so the load's latency stays off the stage.
    // Every memory operation of these waves is a buffer access that every lane issues in every
    // iteration (lanes and stages without work use out-of-range offsets: no traffic), so the
    // compiler's in-order wait before the coefficient store counts only what was issued after
    // the load instead of draining the partial stores of the stage before.
    const int cv = threadIdx.x - 256;
    const int clr = cv / 5, cc4 = cv - (cv / 5) * 5;
    const bool coef_lane = cv < kGroupRows * 5;
    auto coef_load = [&](int k) __attribute__((always_inline)) {
      const int r0 = group_of(min(k, total - 1)) * kGroupRows;
      const int row = min(r0 + clr, M - 1) - r0;
      const bool go = coef_lane && k < total;
      const __amdgpu_buffer_rsrc_t rP = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(a.post + (int64_t)r0 * kHC), (short)0, kGroupRows * kHC * 4, 0x00020000);
      const __amdgpu_buffer_rsrc_t rC = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(a.comb + (int64_t)r0 * kHC * kHC), (short)0, kGroupRows * kHC * kHC * 4, 0x00020000);
      const uint32_t oP = go && cc4 == 0 ? (uint32_t)(row * kHC * 4) : kOutOfRange;
      const uint32_t oC = go && cc4 != 0 ? (uint32_t)(row * kHC * kHC * 4 + (cc4 - 1) * 16) : kOutOfRange;
      const u32x4 vp = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rP, oP, 0u, 0));
      const u32x4 vc = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rC, oC, 0u, 0));
      return vp | vc;  // the out-of-range one reads zero bits
    };
    auto coef_store = [&](int k, const u32x4& v) __attribute__((always_inline)) {
      if (coef_lane && k < total) *reinterpret_cast<u32x4*>(&coef[k & 1][clr][4 * cc4]) = v;
    };
    // the four streams' accumulators of stage k, summed in stream order, into the partials;
    // k < 0: nothing is stored (the same instructions, out-of-range offsets)
    auto flush = [&](int k) __attribute__((always_inline)) {
      const int kk = max(k, 0);
      const int r0 = group_of(kk) * kGroupRows;
      const auto& ep = epi[kk & 1];
      const __amdgpu_buffer_rsrc_t rO = __builtin_amdgcn_make_buffer_rsrc(
          a.part + ((int64_t)s * M + r0) * kPartStride, (short)0, kGroupRows * kPartStride * 4, 0x00020000);
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int idx = cv + 256 * it;  // 16 rows x 25 values = 400 < 512
        const bool in = idx < kGroupRows * (kMix + 1);
        const int id = in ? idx : 0;
        const int row = id / (kMix + 1);
        const int f = id - row * (kMix + 1);
        float v = 0.0f;
        if (f < 16) {
#pragma unroll
          for (int w = 0; w < kHC; ++w) v += ep[w][row][f];
        } else if (f < kMix) {
#pragma unroll
          for (int w = 0; w < kHC; ++w) v += ep[w][row][f] + ep[w][row][f + 8];
        } else {
#pragma unroll
          for (int w = 0; w < kHC; ++w) v += ep[w][row][32];
        }
        const bool go = k >= 0 && in && r0 + row < M;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rO, go ? (uint32_t)(id * 4) : kOutOfRange, 0u, 0);
      }
    };
    // stage k's MFMAs from its ring slot, accumulators to epilogue slot k & 1 (16x16 layout:
    // lane holds rows 4 (lane / 16) + i of column lane % 16)
    auto mma = [&](int k) __attribute__((always_inline)) {
      const u32x4* slot = ring[k & 1];
      f32x4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = d0, sq = d0;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const bf16x8 xa = __builtin_bit_cast(bf16x8, slot[r16 * UPR + ((q * UR + 4 * c + g) ^ r16)]);
        d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, __builtin_bit_cast(bf16x8, b[c][0]), d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, __builtin_bit_cast(bf16x8, b[c][3]), d1, 0, 0, 0);
        sq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, xa, sq, 0, 0, 0);
        d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, __builtin_bit_cast(bf16x8, b[c][1]), d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, __builtin_bit_cast(bf16x8, b[c][4]), d1, 0, 0, 0);
        d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, __builtin_bit_cast(bf16x8, b[c][2]), d0, 0, 0, 0);
      }
      auto& ep = epi[k & 1][q];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ep[4 * g + i][r16] = d0[i];
        ep[4 * g + i][16 + r16] = d1[i];
        if (r16 == 4 * g + i) ep[r16][32] = sq[i];
      }
    };

    u32x4 cnext = {0u, 0u, 0u, 0u};
    if (kPost) {
      coef_store(0, coef_load(0));
      cnext = coef_load(1);
    }
    // The fn loads go out after the first two stages' coefficients: vector loads complete in
    // order, so the store of stage 0's coefficients, which the producers wait for at the first
    // barrier, does not wait for the 205 KB fill (0.6 us back to back at M = 4096).
    if constexpr (kPost) __builtin_amdgcn_sched_barrier(0);
    {
      const u32x4* src = reinterpret_cast<const u32x4*>(a.fnp) +
                         ((int64_t)(s * kHC + q) * NC) * kPackTiles * 64 + lane;
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int t = 0; t < kPackTiles; ++t) b[c][t] = src[(c * kPackTiles + t) * 64];
    }
    __syncthreads();  // matches the producers' first barrier
    // Iteration i: the coefficients of stage i + 1 into LDS (loaded an iteration earlier) and
    // the load of stage i + 2's, the partials of stage i - 2 (epilogue written in iteration
    // i - 1; none for i < 2), the MFMAs of stage i - 1 (ring slot written by the producers in
    // iteration i - 1); then the block barrier.
    for (int i = 0; i <= total; ++i) {
      if (kPost) {
        coef_store(i + 1, cnext);
        cnext = coef_load(i + 2);
      }
      flush(i - 2);
      if (i >= 1) mma(i - 1);
      __syncthreads();
    }
    flush(total - 1);
  }
}

static int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

static hipError_t launch_pipe(bool fused, PipeArgs args, hipStream_t s) {
  const StatsGeom geo = stats_geom(args.H);
  if (geo.S == 0) return hipErrorInvalidValue;
  args.S = geo.S;
  args.groups = (args.M + kGroupRows - 1) / kGroupRows;
  args.blocks_per_slice = max(1, min(args.groups, device_cus() / geo.S));
  const dim3 grid((unsigned)(args.blocks_per_slice * geo.S)), block(512);
#define HC_STATS_CASE(nc)                                                                        \
  case nc:                                                                                       \
    if (fused)                                                                                   \
      hipLaunchKernelGGL((stats_kernel<nc, true>), grid, block, 0, s, args);                     \
    else                                                                                         \
      hipLaunchKernelGGL((stats_kernel<nc, false>), grid, block, 0, s, args);                    \
    break;
  switch (geo.NC) {
    HC_STATS_CASE(2)
    HC_STATS_CASE(4)
    HC_STATS_CASE(6)
    HC_STATS_CASE(8)
    HC_STATS_CASE(10)
    default: return hipErrorInvalidValue;
  }
#undef HC_STATS_CASE
  return hipGetLastError();
}

hipError_t launch_stats(const uint16_t* R, int64_t ldR, const uint16_t* fn_packed, int M, int H,
                        float* part, hipStream_t s) {
  PipeArgs args{};
  args.R = R;
  args.ldR = ldR;
  args.fnp = fn_packed;
  args.part = part;
  args.M = M;
  args.H = H;
  return launch_pipe(false, args, s);
}

hipError_t launch_post_stats(const uint16_t* x, int64_t ldX, const uint16_t* R, int64_t ldR,
                             const float* post, const float* comb, const uint16_t* fn_packed,
                             int M, int H, uint16_t* out, int64_t ldOut, float* part,
                             hipStream_t s) {
  PipeArgs args{};
  args.x = x;
  args.ldX = ldX;
  args.R = R;
  args.ldR = ldR;
  args.post = post;
  args.comb = comb;
  args.fnp = fn_packed;
  args.out = out;
  args.ldOut = ldOut;
  args.part = part;
  args.M = M;
  args.H = H;
  return launch_pipe(true, args, s);
}

}  // namespace hc
