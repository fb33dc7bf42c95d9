// Mix stats of a residual, alone or fused behind hc post (deepseek_v4.py,
// DeepseekV4DecoderLayer.hc_pre's mix stats; DeepseekV4DecoderLayer.forward's fused
// mhc_fused_post_pre, which takes the previous sublayer's hc post together with the next
// hc pre). Per row x (flattened stream-major, 4H values) the kernel produces, for each of 8
// column slices, the partial dots d[f] = sum_k fn[f, k] x_k (24 of them) and sum_k x_k^2.
// In the fused form x is the bf16 R' = post * y + comb^T R that the kernel also stores.
//
// Arithmetic: the 24 x 4H projection runs on the matrix cores (v_mfma_f32_16x16x32_bf16).
// x is exactly bf16; fn is fp32, split once per weight into three bf16 parts hi + mid + lo
// (each the round-to-nearest-even of what the earlier parts leave). bf16 products are exact
// in fp32 and the three parts carry fn to ~24 significant bits. The 72 (part, row) columns are
// packed into 5 B-operand tiles of 16 feeding two accumulators; sum x^2 is the diagonal of the
// 16x16 Gram tile of x with itself.
//
// Slices: slice s covers columns h in [s*H/8, (s+1)*H/8) of all four streams, so the fused
// kernel produces every stream of R' for its columns. Block b takes slice b % 8: with
// round-robin dispatch each XCD keeps one slice of packed fn (3.3 MB / 8) in its L2.
//
// Work layout (one persistent block of 8 waves per CU):
//  * a tile is 64 rows; a stage is 64 columns of each stream (64 rows x 512 B);
//  * waves 0-3 (producers) stream a stage with wave loads of 8 rows x 128 B (whole cache
//    lines), compute R' in the fused form, store it, and write the bf16 stage into one slot of
//    a two-slot LDS ring; their loads run four stages ahead;
//  * waves 4-7 (consumers) multiply the previous stage: consumer q owns stream q (2 chunks of
//    32 columns) for all 64 rows, so one fn operand load serves 64 rows (128 when two tiles
//    share their stages, see the stage schedule);
//  * one block barrier per stage. Producer and consumer waves keep separate in-order load
//    counters, so a consumer's wait for its fn operands does not count the producers' HBM
//    loads (the operands, L2 hits, can still return behind HBM loads the CU issued earlier,
//    which is why they are loaded two stages ahead).
// The LDS tile stores 16-byte unit u of row r at unit u ^ (r & 15): the consumers' 16-byte
// reads of 16 rows hit 16 distinct bank groups.
//
// Partials go to a workspace [8][M][32] (24 dots, sum of squares); consumers sum their four
// streams' accumulators in stream order. Nothing depends on M or on where a row sits in its
// tile (rows past the end recompute row M-1 and store identical bits), so any row slice of a
// call gives the same bits as the full call. Calls of up to 1024 rows take pipe_small_kernel
// (end of this file) instead, which writes the same partials in one pass.
#include "hc_launch.h"

namespace hc {

constexpr int kPipeH = 64;                         // columns of each stream per stage
constexpr int kRowElems = kHC * kPipeH;            // 256 bf16 per row per stage (512 B)
constexpr int kRowUnits = kRowElems / 8;           // 32 units of 16 B
constexpr int kStageChunks = kRowElems / 32;       // 8 MFMA chunks per stage
constexpr int kSlotElems = kStatsRows * kRowElems; // 16384 bf16 = 32 KB
constexpr int kItemsPerLane = (kStatsRows * (kPipeH / 8)) / 256;  // 2 (row, 8-column) items
constexpr int kEpiCols = 33;                       // 32 accumulator columns + sum of squares
constexpr int kCoefs = kHC + kHC * kHC;            // post(4) + comb(16) per row

// ---- fn packing -------------------------------------------------------------------------------
// Packed index (8-element units): ((s*NCS + c)*5 + t)*64 + lane with NCS = 4*(H/8)/32 chunks
// per slice. Chunk c of slice s is stage p = c / 8, stream j = (c % 8) / 2, half hq = c % 2: it
// covers flattened columns k = j*H + s*(H/8) + 64p + 32hq + [0, 32). Lane (n = lane%16,
// g = lane/16) of tile t holds the 8 columns k0 + 8g + [0..7] of the (part, fn row) the tile
// assigns to n:
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

__device__ __forceinline__ int64_t chunk_col0(int s, int c, int H) {
  const int p = c >> 3, j = (c & 7) >> 1, hq = c & 1;
  return (int64_t)j * H + (int64_t)s * (H / kSlices) + 64 * p + 32 * hq;
}

// fn has `rows` rows (24 for the mixes, 4 for the head); rows past it pack as zeros.
__global__ __launch_bounds__(256) void fn_pack_kernel(const float* __restrict__ fn, int H,
                                                      int rows, uint16_t* __restrict__ out) {
  const int NCS = (int)chunks_per_slice(H);
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
  const int64_t k = chunk_col0(s, c, H) + 8 * (lane >> 4);
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

static bool small_kernel_ready();

hipError_t launch_fn_pack(const float* fn, int H, int rows, uint16_t* fn_packed,
                          hipStream_t s) {
  // Packing runs before any stats call, normally eagerly at set-up: allow the small-batch
  // kernel its LDS here, so that its first call never does it inside a graph capture.
  (void)small_kernel_ready();
  const int64_t total = (int64_t)kSlices * chunks_per_slice(H) * kPackTiles * 64;
  hipLaunchKernelGGL(fn_pack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, fn,
                     H, rows, fn_packed);
  return hipGetLastError();
}

// ---- the pipelined kernel ---------------------------------------------------------------------
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
  float* part;        // [8][M][32]
  int M, H;
  int tiles;          // ceil(M / 64)
  int blocks_per_slice;
};

struct LdsLayout {
  uint16_t ring[2][kSlotElems];                  // 64 KB
  float epi[2][kHC][kStatsRows][kEpiCols];       // 66 KB
  float coef[2][kStatsRows][kCoefs];             // 10 KB: two tiles
};

__device__ __forceinline__ int swz(int row, int unit) { return unit ^ (row & 15); }

template <bool kPost>
__global__ __launch_bounds__(512) void pipe_kernel(PipeArgs a) {
  __shared__ __attribute__((aligned(16))) LdsLayout L;

  const int s = blockIdx.x % kSlices;
  const int kb = blockIdx.x / kSlices;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int M = a.M, H = a.H;
  const int nstage = (H / kSlices) / kPipeH;
  const int my_tiles = kb < a.tiles ? (a.tiles - 1 - kb) / a.blocks_per_slice + 1 : 0;
  const int total = my_tiles * nstage;
  const int hs = s * (H / kSlices);
  if (total == 0) return;  // block-uniform: no barrier is skipped by part of the block

  // Stage schedule. Stats alone: the block's tiles go in pairs (tile iterations 2k, 2k+1)
  // whose stages interleave, (2k, p), (2k+1, p), (2k, p+1), ...: consecutive stages cover the
  // same columns, so the consumers load each stage's fn operands once for two tiles; an odd
  // last tile runs its stages alone. nstage = H / 512 is even, so a paired part is a multiple
  // of four stages. Fused form: the tiles run one after another. It moves five arrays in and
  // four out, and HBM serves that mix faster when the rows in flight at once form a narrower
  // band (64 rows per block instead of 128), which outweighs the doubled fn operand loads.
  constexpr bool kPaired = !kPost;
  const int npair = kPaired ? my_tiles >> 1 : 0;
  const int paired = npair * 2 * nstage;
  auto sched = [&](int sigma, int& ti, int& p) __attribute__((always_inline)) {
    if (sigma < paired) {
      const int k = sigma / (2 * nstage), j = sigma - k * 2 * nstage;
      p = j >> 1;
      ti = 2 * k + (j & 1);
    } else {
      const int r = sigma - paired, u = r / nstage;
      p = r - u * nstage;
      ti = 2 * npair + u;
    }
  };

  if (wave < 4) {
    // ===================================== producers ======================================
    // item it of this lane: row 16*wave + 8*it + lane/8, 8-column group lane%8
    const int hg = lane & 7;
    u32x4 ld0[kItemsPerLane][kHC + 1], ld1[kItemsPerLane][kHC + 1];
    u32x4 ld2[kItemsPerLane][kHC + 1], ld3[kItemsPerLane][kHC + 1];
    // The loop issues loads four stages ahead, also past the last stage, so that it has no
    // branch around them (the in-order load counters then stay exact). Those unused loads read
    // this block's packed fn slice, which the consumers keep in the L2, not HBM. (A slice
    // holds 40H elements; the loads span 3H + 512.)
    const uint16_t* dead = a.fnp + (int64_t)s * chunks_per_slice(H) * kPackTiles * 64 * 8 + lane * 8;
    auto issue = [&](int sigma, u32x4 (&d)[kItemsPerLane][kHC + 1]) __attribute__((always_inline)) {
      const bool live = sigma < total;  // block-uniform
      const int sg = min(sigma, total - 1);
      int ti, p;
      sched(sg, ti, p);
      const int T = kb + ti * a.blocks_per_slice;
      const int h = hs + 64 * p + 8 * hg;
#pragma unroll
      for (int it = 0; it < kItemsPerLane; ++it) {
        const int row = min(T * kStatsRows + 16 * wave + 8 * it + (lane >> 3), M - 1);
        const uint16_t* rr = live ? a.R + (int64_t)row * a.ldR + h : dead;
#pragma unroll
        for (int i = 0; i < kHC; ++i) d[it][i] = ld16_stream(rr + (int64_t)i * H);
        if (kPost) d[it][kHC] = ld16_stream(live ? a.x + (int64_t)row * a.ldX + h : dead);
      }
    };
    auto produce = [&](int sigma, u32x4 (&d)[kItemsPerLane][kHC + 1]) __attribute__((always_inline)) {
      int ti, p;
      sched(sigma, ti, p);
      const int T = kb + ti * a.blocks_per_slice;
      uint16_t* slot = L.ring[sigma & 1];
#pragma unroll
      for (int it = 0; it < kItemsPerLane; ++it) {
        const int lrow = 16 * wave + 8 * it + (lane >> 3);
        u32x4 st[kHC];
        if (kPost) {
          const int row = min(T * kStatsRows + lrow, M - 1);
          const float* cf = L.coef[ti & 1][lrow];
          float pj[kHC], cij[kHC][kHC];
#pragma unroll
          for (int j = 0; j < kHC; ++j) pj[j] = cf[j];
#pragma unroll
          for (int i = 0; i < kHC; ++i)
#pragma unroll
            for (int j = 0; j < kHC; ++j) cij[i][j] = cf[kHC + i * kHC + j];
          float xf[8], rf[kHC][8];
          unpack8(d[it][kHC], xf);
#pragma unroll
          for (int i = 0; i < kHC; ++i) unpack8(d[it][i], rf[i]);
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
          uint16_t* orow = a.out + (int64_t)row * a.ldOut + hs + 64 * p + 8 * hg;
#pragma unroll
          for (int j = 0; j < kHC; ++j) st16(orow + (int64_t)j * H, st[j]);
        } else {
#pragma unroll
          for (int i = 0; i < kHC; ++i) st[i] = d[it][i];
        }
#pragma unroll
        for (int j = 0; j < kHC; ++j)
          *reinterpret_cast<u32x4*>(&slot[lrow * kRowElems + 8 * swz(lrow, 8 * j + hg)]) = st[j];
      }
    };

    issue(0, ld0);
    issue(1, ld1);
    issue(2, ld2);
    issue(3, ld3);
    __syncthreads();  // the consumers' first coefficient tile is in LDS
    // Full trips of four stages (four load buffers in fixed registers); stage sigma's loads
    // were issued four stages earlier. The trip has no branch: every path from one stage to
    // the next issues the same memory operations, so the compiler's in-order wait counts stay
    // exact and each stage waits only for its own loads, not for the three stages behind it.
    auto trip = [&](int sg) __attribute__((always_inline)) {
      produce(sg, ld0);
      issue(sg + 4, ld0);
      __syncthreads();
      produce(sg + 1, ld1);
      issue(sg + 5, ld1);
      __syncthreads();
      produce(sg + 2, ld2);
      issue(sg + 6, ld2);
      __syncthreads();
      produce(sg + 3, ld3);
      issue(sg + 7, ld3);
      __syncthreads();
    };
    // The first trip is peeled: the loop is then entered in the same state it loops back in,
    // so the compiler's wait counts are those of the steady state.
    int sigma = 0;
    if (total >= 4) {
      trip(0);
      for (sigma = 4; sigma + 4 <= total; sigma += 4) trip(sigma);
    }
    // the last total % 4 stages (already loaded), then the barrier that closes the consumers'
    // last stage: total + 2 barriers in all, as the consumers
    const int rest = total - sigma;
    if (rest > 0) {
      produce(sigma, ld0);
      __syncthreads();
    }
    if (rest > 1) {
      produce(sigma + 1, ld1);
      __syncthreads();
    }
    if (rest > 2) {
      produce(sigma + 2, ld2);
      __syncthreads();
    }
    __syncthreads();
  } else {
    // ===================================== consumers ======================================
    const int q = wave - 4;  // stream
    const int r16 = lane & 15, g = lane >> 4;
    const u32x4* bslice = reinterpret_cast<const u32x4*>(a.fnp) + (int64_t)s * chunks_per_slice(H) * kPackTiles * 64 + lane;
    // accumulators of the even (A) and odd (B) tile of a pair
    f32x4 aD0[4], aD1[4], aSq[4], bD0[4], bD1[4], bSq[4];
    auto zero = [&](f32x4 (&v)[4]) __attribute__((always_inline)) {
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) v[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    zero(aD0), zero(aD1), zero(aSq), zero(bD0), zero(bD1), zero(bSq);
    // post / comb of tile iteration ti's 64 rows into coefficient slot ti & 1 (fused form)
    auto load_coef = [&](int ti) __attribute__((always_inline)) {
      if (ti >= my_tiles) return;  // block-uniform
      const int T = kb + ti * a.blocks_per_slice;
      float* dst = &L.coef[ti & 1][0][0];
      for (int v = threadIdx.x - 256; v < kStatsRows * 5; v += 256) {
        const int lr = v / 5, k = v - lr * 5;
        const int row = min(T * kStatsRows + lr, M - 1);
        const float* src = k == 0 ? a.post + (int64_t)row * kHC : a.comb + (int64_t)row * 16 + 4 * (k - 1);
        *reinterpret_cast<f32x4*>(dst + lr * kCoefs + 4 * k) = *reinterpret_cast<const f32x4*>(src);
      }
    };
    // partials of tile iteration ti from epilogue slot ti & 1
    auto flush = [&](int ti) __attribute__((always_inline)) {
      const int T = kb + ti * a.blocks_per_slice;
      const auto& ep = L.epi[ti & 1];
      for (int idx = threadIdx.x - 256; idx < kStatsRows * (kMix + 1); idx += 256) {
        const int row = idx / (kMix + 1);
        const int f = idx - row * (kMix + 1);
        const int grow = T * kStatsRows + row;
        if (grow >= M) continue;
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
        a.part[((int64_t)s * M + grow) * kPartStride + f] = v;
      }
    };
    int pending = -1;  // tile whose epilogue slot waits for its flush

    // fn operands of stage st (clamped to the last stage, so loads past the end read valid
    // memory) for this consumer's two chunks
    auto load_b = [&](int st, u32x4 (&b)[2][kPackTiles]) __attribute__((always_inline)) {
      int ti, p;
      sched(min(st, total - 1), ti, p);
#pragma unroll
      for (int hq = 0; hq < 2; ++hq)
#pragma unroll
        for (int t = 0; t < kPackTiles; ++t)
          b[hq][t] = bslice[((int64_t)(p * kStageChunks + 2 * q + hq) * kPackTiles + t) * 64];
    };
    // the MFMAs of stage st from its ring slot; at a tile's last stage the accumulators go to
    // its epilogue slot (16x16 layout: lane holds rows 4*(lane/16) + i of column lane % 16)
    auto mma = [&](int st, const u32x4 (&b)[2][kPackTiles], f32x4 (&d0)[4], f32x4 (&d1)[4],
                   f32x4 (&sq)[4]) __attribute__((always_inline)) {
      int ti, p;
      sched(st, ti, p);
      const uint16_t* slot = L.ring[st & 1];
#pragma unroll
      for (int hq = 0; hq < 2; ++hq) {
#pragma unroll
        for (int sub = 0; sub < 4; ++sub) {
          const int row = 16 * sub + r16;
          const u32x4 av = *reinterpret_cast<const u32x4*>(&slot[row * kRowElems + 8 * swz(row, 8 * q + 4 * hq + g)]);
          const bf16x8 xa = __builtin_bit_cast(bf16x8, av);
          d0[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, __builtin_bit_cast(bf16x8, b[hq][0]), d0[sub], 0, 0, 0);
          d1[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, __builtin_bit_cast(bf16x8, b[hq][3]), d1[sub], 0, 0, 0);
          sq[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, xa, sq[sub], 0, 0, 0);
          d0[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, __builtin_bit_cast(bf16x8, b[hq][1]), d0[sub], 0, 0, 0);
          d1[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, __builtin_bit_cast(bf16x8, b[hq][4]), d1[sub], 0, 0, 0);
          d0[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, __builtin_bit_cast(bf16x8, b[hq][2]), d0[sub], 0, 0, 0);
        }
      }
      if (p == nstage - 1) {
        auto& ep = L.epi[ti & 1][q];
#pragma unroll
        for (int sub = 0; sub < 4; ++sub) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = sub * 16 + 4 * g + i;
            ep[row][r16] = d0[sub][i];
            ep[row][16 + r16] = d1[sub][i];
            if (r16 == 4 * g + i) ep[sub * 16 + r16][32] = sq[sub][i];
          }
        }
        zero(d0), zero(d1), zero(sq);
        pending = ti;  // flushed in the next iteration, after the barrier
      }
    };
    // start of iteration i: the coefficients of the tile after the one whose stages the
    // producers start now (fused form, where tiles are not paired), and the flush of a
    // finished tile
    auto begin = [&](int i) __attribute__((always_inline)) {
      if (kPost && i % nstage == 0) load_coef(i / nstage + 1);
      if (pending >= 0) {
        flush(pending);
        pending = -1;
      }
    };

    if (kPost) load_coef(0);
    __syncthreads();  // matches the producers' prologue barrier
    // Iteration i multiplies stage i - 1 (written by the producers in iteration i - 1) and ends
    // with the block barrier. Operands: a paired stage couple (2u, 2u + 1) shares the buffer of
    // unit u (bX for even u, bY for odd u); a lone stage st has its own (bX for even st, bY for
    // odd). Each buffer is refilled right after the multiplications that last read it, so
    // its operands are in flight for two iterations: the loads hit the L2 but return behind
    // the HBM loads the producers issued before them.
    u32x4 bX[2][kPackTiles], bY[2][kPackTiles];
    load_b(0, bX);
    for (int i = 0; i < paired; i += 4) {
      begin(i);
      if (i > 0) mma(i - 1, bY, bD0, bD1, bSq);
      load_b(i + 2, bY);
      __syncthreads();
      begin(i + 1);
      mma(i, bX, aD0, aD1, aSq);
      __syncthreads();
      begin(i + 2);
      mma(i + 1, bX, bD0, bD1, bSq);
      load_b(i + 4, bX);  // past the paired part: the first lone stage
      __syncthreads();
      begin(i + 3);
      mma(i + 2, bY, aD0, aD1, aSq);
      __syncthreads();
    }
    // iteration `paired`: the last paired stage; the first lone stage's operands are in bX
    begin(paired);
    if (paired > 0) mma(paired - 1, bY, bD0, bD1, bSq);
    load_b(paired + 1, bY);
    __syncthreads();
    // the unpaired stages: the lone tile of the paired form, all tiles of the fused form
    // (total - paired is even)
    for (int i = paired + 1; i <= total; i += 2) {
      begin(i);
      mma(i - 1, bX, aD0, aD1, aSq);
      load_b(i + 1, bX);
      __syncthreads();
      begin(i + 1);
      mma(i, bY, aD0, aD1, aSq);
      load_b(i + 2, bY);
      __syncthreads();
    }
    if (pending >= 0) flush(pending);
  }
}

// ---- small batches (decode, verify, short prefill) -----------------------------------------------
// The decode and verify steps run the decoder layer's hc pre and post on a handful of rows
// (the engine gates its fused combine-norm on 1..8 rows as on long prefill chunks;
// prefill_sp.py, _combine_norm_fused). Below about a thousand rows the pipelined kernel is
// latency-bound: each block runs a ten-stage pipeline over one or a few 64-row tiles.
// pipe_small_kernel writes the same partials for such batches in one pass per 16-row group
// (one MFMA row tile): block b takes slice b % 8 (so the blocks of a slice share an XCD and its
// L2 copy of the slice's packed fn) and rows [16 (b / 8), +16); wave q < 4 is stream q. Each
// of those waves walks its stream's chunks of the slice in the pipelined kernel's order (stage
// p, then half hq, i.e. chunk c = 2p + hq), with the same A and B operands and the same
// sequence of MFMAs into the same three accumulators, and the four streams' accumulators are
// added in the same order through LDS. Every partial, and so every output of the path, is
// bit-identical to what pipe_kernel gives for these rows, so a call's bits do not depend on
// which kernel its row count selects (a row slice of a large call gives the large call's
// bits). Above about 1024 rows the pipelined kernel is faster (measured crossover).
//
// The block's 8 waves first stage its slice of x (R, or in the fused form R' formed from R and
// the sublayer output with the producers' operation order, and stored) for all rows in LDS, rows
// padded by 16 bytes so that the MFMA operand reads of 8 rows hit distinct banks; waves 0-3
// issue the fn operand loads of their first kSmallAhead chunks before it, so both latencies
// overlap. (Two waves per SIMD halve the staging arithmetic's time; a deeper fn window, 16
// chunks on one wave per SIMD, measured no faster.)
constexpr int kSmallRows = 16;        // rows of one block (one MFMA row tile)
constexpr int kSmallMaxRows = 1024;   // largest batch the one-pass kernel takes
constexpr int kSmallAhead = 8;
constexpr int kStageBatch = 2;
constexpr int kSmallThreads = 512;  // all 8 waves stage the slice; waves 0-3 run the MFMAs

inline int small_row_elems(int H) { return H / kSlices + 8; }
inline size_t small_lds_bytes(int H) {
  return (size_t)kHC * kSmallRows * small_row_elems(H) * 2 +
         (size_t)kHC * kSmallRows * kEpiCols * 4;
}
constexpr size_t kSmallLdsMax = 150 * 1024;

template <bool kPost>
__global__ __launch_bounds__(kSmallThreads) void pipe_small_kernel(PipeArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char small_lds[];
  const int M = a.M, H = a.H;
  const int W = H / kSlices;               // slice width (columns of each stream)
  const int LR = W + 8;                    // LDS row stride in elements
  uint16_t* xs = reinterpret_cast<uint16_t*>(small_lds);  // [4 streams][16 rows][LR]
  float(*ep)[kSmallRows][kEpiCols] =
      reinterpret_cast<float(*)[kSmallRows][kEpiCols]>(small_lds + (size_t)kHC * kSmallRows * LR * 2);
  const int s = blockIdx.x % kSlices;      // slice: the blocks of a slice share an XCD's L2
  const int r0 = (blockIdx.x / kSlices) * kSmallRows;  // this block's 16-row group
  const int Mg = min(kSmallRows, M - r0);  // its rows
  const int q = threadIdx.x >> 6;          // waves 0-3: the stream of this wave's MFMAs
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int nch = 2 * (W / kPipeH);        // chunks of one stream in a slice (multiple of 4)
  const int hs = s * W;
  const u32x4* bq = reinterpret_cast<const u32x4*>(a.fnp) +
                    (int64_t)s * chunks_per_slice(H) * kPackTiles * 64 + lane;
  u32x4 fb[kSmallAhead][kPackTiles];
  auto issue = [&](int c, u32x4 (&d)[kPackTiles]) __attribute__((always_inline)) {
    const int p = c >> 1, hq = c & 1;
#pragma unroll
    for (int t = 0; t < kPackTiles; ++t)
      d[t] = bq[((int64_t)(p * kStageChunks + 2 * q + hq) * kPackTiles + t) * 64];
  };
  const bool mma_wave = q < kHC;  // wave-uniform
  if (mma_wave) {
#pragma unroll
    for (int u = 0; u < kSmallAhead; ++u)
      if (u < nch) issue(u, fb[u]);
  }

  // stage the slice: item = (row, 8-column group), groups of a row on consecutive threads; the
  // loads of kStageBatch items per thread go out together
  const int groups = W / 8;
  const int items = Mg * groups;
  constexpr int kLoads = kPost ? kHC + 1 : kHC;  // R's streams (and the sublayer output)
  for (int it0 = threadIdx.x; it0 < items; it0 += kSmallThreads * kStageBatch) {
    u32x4 ld[kStageBatch][kLoads];
#pragma unroll
    for (int bi = 0; bi < kStageBatch; ++bi) {
      const int it = it0 + kSmallThreads * bi;
      if (it < items) {
        const int r = it / groups;
        const int h = hs + 8 * (it - r * groups);
        const uint16_t* Rr = a.R + (int64_t)(r0 + r) * a.ldR + h;
#pragma unroll
        for (int i = 0; i < kHC; ++i) ld[bi][i] = ld16(Rr + (int64_t)i * H);
        if (kPost) ld[bi][kLoads - 1] = ld16(a.x + (int64_t)(r0 + r) * a.ldX + h);
      }
    }
#pragma unroll
    for (int bi = 0; bi < kStageBatch; ++bi) {
      const int it = it0 + kSmallThreads * bi;
      if (it < items) {
        const int r = it / groups;
        const int h = hs + 8 * (it - r * groups);
        u32x4 v[kHC];
        if (kPost) {
          float xf[8], rf[kHC][8];
          unpack8(ld[bi][kLoads - 1], xf);
#pragma unroll
          for (int i = 0; i < kHC; ++i) unpack8(ld[bi][i], rf[i]);
          const float* cf = a.comb + (int64_t)(r0 + r) * kHC * kHC;
#pragma unroll
          for (int j = 0; j < kHC; ++j) {
            const float pj = a.post[(int64_t)(r0 + r) * kHC + j];
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              float acc = pj * xf[e];
#pragma unroll
              for (int i = 0; i < kHC; ++i) acc = __fmaf_rn(cf[i * kHC + j], rf[i][e], acc);
              o[e] = acc;
            }
            v[j] = pack8(o);
            st16(a.out + (int64_t)(r0 + r) * a.ldOut + (int64_t)j * H + h, v[j]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < kHC; ++i) v[i] = ld[bi][i];
        }
#pragma unroll
        for (int i = 0; i < kHC; ++i)
          *reinterpret_cast<u32x4*>(&xs[((size_t)i * kSmallRows + r) * LR + (h - hs)]) = v[i];
      }
    }
  }
  __syncthreads();

  if (mma_wave) {
    // rows past the end repeat row M-1 (their results are not written)
    const uint16_t* arow = xs + ((size_t)q * kSmallRows + min(r16, Mg - 1)) * LR + 8 * g;
    f32x4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = d0, sq = d0;
    for (int c0 = 0; c0 < nch; c0 += kSmallAhead) {
#pragma unroll
      for (int u = 0; u < kSmallAhead; ++u) {
        const int c = c0 + u;
        if (c < nch) {
          const bf16x8 xa = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(arow + 32 * c));
          const u32x4(&b)[kPackTiles] = fb[u];
          d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, __builtin_bit_cast(bf16x8, b[0]), d0, 0, 0, 0);
          d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, __builtin_bit_cast(bf16x8, b[3]), d1, 0, 0, 0);
          sq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, xa, sq, 0, 0, 0);
          d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, __builtin_bit_cast(bf16x8, b[1]), d0, 0, 0, 0);
          d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, __builtin_bit_cast(bf16x8, b[4]), d1, 0, 0, 0);
          d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, __builtin_bit_cast(bf16x8, b[2]), d0, 0, 0, 0);
          if (c + kSmallAhead < nch) issue(c + kSmallAhead, fb[u]);
        }
      }
    }
    // the pipelined kernel's epilogue layout: lane holds rows 4g + i of column r16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ep[q][4 * g + i][r16] = d0[i];
      ep[q][4 * g + i][16 + r16] = d1[i];
      if (r16 == 4 * g + i) ep[q][r16][32] = sq[i];
    }
  }
  __syncthreads();
  // and its flush: streams added in order, f 16..23 as (hi + lo) + mid
  for (int idx = threadIdx.x; idx < Mg * (kMix + 1); idx += kSmallThreads) {
    const int r = idx / (kMix + 1);
    const int f = idx - r * (kMix + 1);
    float v = 0.0f;
    if (f < 16) {
#pragma unroll
      for (int w = 0; w < kHC; ++w) v += ep[w][r][f];
    } else if (f < kMix) {
#pragma unroll
      for (int w = 0; w < kHC; ++w) v += ep[w][r][f] + ep[w][r][f + 8];
    } else {
#pragma unroll
      for (int w = 0; w < kHC; ++w) v += ep[w][r][32];
    }
    a.part[((int64_t)s * M + r0 + r) * kPartStride + f] = v;
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

// The small-batch kernel takes more than 64 KB of dynamic LDS: allow it once per device.
static bool small_kernel_ready() {
  static signed char ok[64] = {0};  // 0 unknown, 1 ready, -1 failed
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  if (ok[dev] == 0) {
    const int bytes = (int)kSmallLdsMax;
    const bool good =
        hipFuncSetAttribute(reinterpret_cast<const void*>(&pipe_small_kernel<true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess &&
        hipFuncSetAttribute(reinterpret_cast<const void*>(&pipe_small_kernel<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess;
    if (!good) (void)hipGetLastError();  // the pipelined kernel serves instead: no error left
    ok[dev] = good ? 1 : -1;
  }
  return ok[dev] > 0;
}

static hipError_t launch_pipe(bool fused, PipeArgs args, hipStream_t s) {
  const size_t small_lds = small_lds_bytes(args.H);
  if (args.M >= 1 && args.M <= kSmallMaxRows && small_lds <= kSmallLdsMax && small_kernel_ready()) {
    // small batches: same bits in one pass per 16-row group (H up to 8192 fits a slice in LDS)
    const dim3 grid((unsigned)(kSlices * ((args.M + kSmallRows - 1) / kSmallRows)));
    if (fused)
      hipLaunchKernelGGL(pipe_small_kernel<true>, grid, dim3(kSmallThreads), small_lds, s, args);
    else
      hipLaunchKernelGGL(pipe_small_kernel<false>, grid, dim3(kSmallThreads), small_lds, s, args);
    return hipGetLastError();
  }
  args.tiles = (args.M + kStatsRows - 1) / kStatsRows;
  args.blocks_per_slice = max(1, min(args.tiles, device_cus() / kSlices));
  const dim3 grid((unsigned)(args.blocks_per_slice * kSlices)), block(512);
  if (fused)
    hipLaunchKernelGGL(pipe_kernel<true>, grid, block, 0, s, args);
  else
    hipLaunchKernelGGL(pipe_kernel<false>, grid, block, 0, s, args);
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
