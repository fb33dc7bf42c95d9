// Device-side helpers shared by the gfx950 kernels of the mHC pre/post path.
//
// Layout facts used throughout:
//  * the residual R is bf16 [M, 4, H]; a row's flattened index is k = i*H + h (stream-major),
//    as the decoder layer's hc_pre flattens it (deepseek_v4.py, DeepseekV4DecoderLayer.hc_pre);
//  * mixes are 24 fp32 per row, ordered pre(4) | post(4) | res(16), res row-major [i][j]
//    with i the source stream and j the destination stream;
//  * a wavefront is 64 lanes; 16-byte (8 x bf16) vector accesses are the unit of HBM traffic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hc {

constexpr int kHC = 4;
constexpr int kMix = (2 + kHC) * kHC;  // 24

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---- bf16 <-> fp32 -----------------------------------------------------------------------
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

// 8 bf16 (one 16-byte load) -> 8 fp32.
__device__ __forceinline__ void unpack8(const u32x4& w, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf_lo(w[i]);
    f[2 * i + 1] = bf_hi(w[i]);
  }
}

__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return w;
}

// ---- 16-byte global accesses ------------------------------------------------------------
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
__device__ __forceinline__ void st16_stream(void* p, const u32x4& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// ---- cross-lane reductions (DPP; all lanes end with the result) --------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 CTRL, 0xF, 0xF, false));
}
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]: lane l reads lane l^1
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]: lane l reads lane l^2

// row_ror:N (N = 4k): within each 16-lane row, lane l reads lane (l - N) mod 16
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;
constexpr int kRowRor12 = 0x12C;

// Sum over the 4 lanes of a quad (lanes 4q..4q+3).
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp<kQuadSwap1>(v);
  v += dpp<kQuadSwap2>(v);
  return v;
}
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, dpp<kQuadSwap1>(v));
  v = fmaxf(v, dpp<kQuadSwap2>(v));
  return v;
}
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kQuadSwap1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kQuadSwap2, 0xF, 0xF, false));
  return v;
}
// Sum over the lanes {e, e+4, e+8, e+12} (mod 16) of each 16-lane group, lane e holding row
// i = e / 4 of its column. Every lane forms ((v0 + v1) + (v2 + v3)) over the column's rows
// (up to the order of the operands of each add, which does not change a rounded sum), so the
// four lanes of a column get identical bits. With A = v + v[e-4]: an odd row holds the pair
// (i, i-1) in A and finds the other pair two rows away; an even row reads both pairs from
// its neighbours. DPP only: no LDS round trip.
__device__ __forceinline__ float stride4_sum(float v) {
  const float A = v + dpp<kRowRor4>(v);
  const float odd = A + dpp<kRowRor8>(A);
  const float even = dpp<kRowRor12>(A) + dpp<kRowRor4>(A);
  return ((__lane_id() >> 2) & 1) ? odd : even;
}

// Sum over the whole wavefront, in a fixed order (every lane gets the same value).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ---- split + Sinkhorn, one row spread over 16 lanes -------------------------------------
// Lane e (0..15) of a 16-lane group owns res entry (i, j) = (e / 4, e % 4); lanes e < 4 also
// own pre[e], lanes 4 <= e < 8 own post[e - 4]. mix_a = mixes[e] (used when e < 8),
// mix_c = mixes[8 + e]. The pre/post formulas and the Sinkhorn order follow the split and
// the alternating normalisation of hc_split_sinkhorn as the decoder layer calls it
// (deepseek_v4.py, DeepseekV4DecoderLayer.hc_pre; pre's "+ eps" as in hc_head_torch).
struct SplitParams {
  float s0, s1, s2;  // scale[0..2]
  int iters;
  float pre_eps, sk_eps, post_mult;
};

__device__ __forceinline__ float sigmoidf_(float t) { return 1.0f / (1.0f + expf(-t)); }

// Returns this lane's comb entry; *prepost receives pre[e] (e < 4) or post[e-4] (4 <= e < 8).
__device__ __forceinline__ float split_sinkhorn_lane(int e, float mix_a, float mix_c,
                                                     float base_a, float base_c,
                                                     const SplitParams& sp, float* prepost) {
  if (e < 4) {
    *prepost = sigmoidf_(__fmaf_rn(sp.s0, mix_a, base_a)) + sp.pre_eps;
  } else {
    *prepost = sp.post_mult * sigmoidf_(__fmaf_rn(sp.s1, mix_a, base_a));
  }
  float L = __fmaf_rn(sp.s2, mix_c, base_c);
  // softmax over j (the quad), then + eps on every entry. Each normalisation multiplies by
  // v_rcp_f32 of (sum + eps) (reciprocal within 1 ulp).
  float mx = quad_max(L);
  float ex = expf(L - mx);
  float p = ex * __builtin_amdgcn_rcpf(quad_sum(ex)) + sp.sk_eps;
  // first column step
  p = p * __builtin_amdgcn_rcpf(stride4_sum(p) + sp.sk_eps);
  for (int it = 1; it < sp.iters; ++it) {
    p = p * __builtin_amdgcn_rcpf(quad_sum(p) + sp.sk_eps);     // rows: sum over j
    p = p * __builtin_amdgcn_rcpf(stride4_sum(p) + sp.sk_eps);  // columns: sum over i
  }
  return p;
}

// ---- MXFP8 (OCP MX: e4m3fn elements, one ue8m0 scale per 32 values) -----------------------
// Block exponent from the largest magnitude's bf16 bits (for finite bf16, magnitude order is
// the integer order of the low 15 bits): the smallest e with amax * 2^-e <= 448 = 1.75 * 2^8.
// With amax = (1 + f/128) * 2^(E-127), e = E - 135 + [f > 96] (1 + f/128 > 1.75 exactly when
// f > 96), clamped to [-127, 127]; zero and bf16-subnormal maxima give -127. The scale byte
// is e + 127.
__device__ __forceinline__ int mx_block_exponent(uint32_t amax_bits) {
  const int E = (int)(amax_bits >> 7);
  const int f = (int)(amax_bits & 0x7f);
  const int e = (E == 0) ? -127 : E - 135 + (f > 96 ? 1 : 0);
  return min(max(e, -127), 127);
}

// The block scale 2^e as the divisor the MX conversion takes: the scale byte e + 127 in the
// fp32 exponent field. The conversion reads only that field, so byte 0 (e = -127) stands for
// 2^-127 as in the ue8m0 format, although as an fp32 it is 0.
__device__ __forceinline__ float mx_scale(int e) {
  return __uint_as_float((uint32_t)(e + 127) << 23);
}

// Four bf16 values in two packed words, w0 = (v0, v1) and w1 = (v2, v3), divided by the block
// scale -> four e4m3fn codes in one word, v0 in the low byte: CDNA4's MX conversion
// v_cvt_scalef32_pk_fp8_bf16 (OCP e4m3fn), which takes the bf16 pair as it is, scales it
// exactly by the power of two and rounds to nearest even, keeping the sign of zero, subnormals
// down to 2^-9. On all 65 536 bf16 patterns at twelve exponents from -127 to 120 its results
// matched an fp32 multiply by 2^-e followed by v_cvt_pk_fp8_f32 wherever the scaled value stays
// in range (measured), and the MX scale rule keeps every scaled value within +-448.
__device__ __forceinline__ uint32_t e4m3_word(uint32_t w0, uint32_t w1, float scale) {
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  s16x2 r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2, w0), scale, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2, w1), scale, true);
  return __builtin_bit_cast(uint32_t, r);
}

// Largest magnitude bits (low 15 bits) of 8 packed bf16.
__device__ __forceinline__ uint32_t amax_bits8(const u32x4& w) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = max(m, w[i] & 0x7fffu);
    m = max(m, (w[i] >> 16) & 0x7fffu);
  }
  return m;
}

// mixes[f] = d[f] * rsqrt(sumsq / K + eps): the scale factor of the mix stats
// (K = 4H, the flattened row length).
__device__ __forceinline__ float mix_rscale(float sumsq, float kf, float eps) {
  return 1.0f / sqrtf(sumsq / kf + eps);
}

}  // namespace hc
