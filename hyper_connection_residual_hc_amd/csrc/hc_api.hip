// C ABI of the library (include/hc_mi355x.h): argument validation, then the kernel launches.
// No entry point allocates, frees or synchronises; every check happens before anything is
// enqueued, so an error return leaves the stream untouched.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/hc_mi355x.h"
#include "hc_launch.h"

namespace {

using hc::kHC;
using hc::kMix;

constexpr int64_t kMaxRows = (int64_t)1 << 31;

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// [begin, end) byte ranges of strided row tensors, for overlap checks
struct Span {
  uintptr_t b, e;
};
Span rows_span(const void* p, int64_t M, int64_t ld, int64_t row_elems, int64_t elem_bytes) {
  const uintptr_t b = (uintptr_t)p;
  return {b, b + (uintptr_t)(((M - 1) * ld + row_elems) * elem_bytes)};
}
bool overlaps(Span a, Span b) { return a.b < b.e && b.b < a.e; }

bool finite_nonneg(float v) { return isfinite(v) && v >= 0.0f; }

int check_m(int64_t M) {
  if (M < 0 || M >= kMaxRows) return HC_ERR_ARG;
  return HC_OK;
}

int launched(hipError_t err) { return err == hipSuccess ? HC_OK : HC_ERR_LAUNCH; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

bool stats_h_ok(int32_t H) { return hc::stats_geom(H).S > 0; }  // 512 n <= 8192 but 5632, 6656
bool post_h_ok(int32_t H) { return H > 0 && H % 512 == 0 && H <= (1 << 20); }

// Row strides stay below 2^26 elements (the stats kernels address 16 rows of any array with
// 32-bit byte offsets).
constexpr int64_t kMaxLd = (int64_t)1 << 26;

// R [M, 4, H] bf16 with row stride ldR
int check_residual(const uint16_t* R, int64_t ldR, int32_t H) {
  if (ldR < (int64_t)kHC * H || ldR >= kMaxLd) return HC_ERR_SHAPE;
  if (!al16(R) || (ldR * 2) % 16) return HC_ERR_ALIGN;
  return HC_OK;
}


// Disjointness of outputs from inputs and from each other (empty spans are skipped).
int no_alias(const Span* ins, int nin, const Span* outs, int nout) {
  for (int i = 0; i < nout; ++i) {
    if (outs[i].b == outs[i].e) continue;
    for (int j = 0; j < nin; ++j)
      if (ins[j].b != ins[j].e && overlaps(outs[i], ins[j])) return HC_ERR_ALIAS;
    for (int j = i + 1; j < nout; ++j)
      if (outs[j].b != outs[j].e && overlaps(outs[i], outs[j])) return HC_ERR_ALIAS;
  }
  return HC_OK;
}

// What the finish (split + Sinkhorn + combine + RMSNorm) takes and writes. y is bf16 [M, H];
// with mx, q / sc are y's MXFP8 codes [M, H] and scales [M, H/32] and y may be NULL.
struct Finish {
  const float* scale;
  const float* base;
  const uint16_t* weight;
  float rms_eps, pre_eps, sk_eps;
  int32_t iters;
  float post_mult, norm_eps;
  uint16_t* y;
  int64_t ldY;
  uint8_t* q;
  int64_t ldQ;
  uint8_t* sc;
  int64_t ldS;
  float* pre;
  float* post;
  float* comb;
};

// Scalar checks (before the M == 0 no-op).
int finish_scalars(const Finish& f, int32_t H) {
  if (!stats_h_ok(H) || !hc::combine_h_supported(H)) return HC_ERR_SHAPE;
  if (f.iters < 1 || f.iters > 100000) return HC_ERR_SHAPE;
  if (!finite_nonneg(f.rms_eps) || !finite_nonneg(f.pre_eps) || !finite_nonneg(f.sk_eps) ||
      !finite_nonneg(f.norm_eps) || !isfinite(f.post_mult))
    return HC_ERR_ARG;
  return HC_OK;
}

// Pointer, stride and alignment checks; fills the finish's 3 input and 6 output spans.
int finish_pointers(const Finish& f, int64_t M, int32_t H, bool mx, Span* ins, Span* outs) {
  if (!f.scale || !f.base || !f.weight || !f.post || !f.comb) return HC_ERR_NULL;
  if (!mx && !f.y) return HC_ERR_NULL;
  if (mx && (!f.q || !f.sc)) return HC_ERR_NULL;
  if (f.y && f.ldY < H) return HC_ERR_SHAPE;
  if (mx && (f.ldQ < H || f.ldS < H / 32)) return HC_ERR_SHAPE;
  if (!al16(f.weight)) return HC_ERR_ALIGN;
  if (f.y && (!al16(f.y) || (f.ldY * 2) % 16)) return HC_ERR_ALIGN;
  if (mx && (!al16(f.q) || f.ldQ % 16)) return HC_ERR_ALIGN;
  ins[0] = Span{(uintptr_t)f.scale, (uintptr_t)f.scale + 12};
  ins[1] = Span{(uintptr_t)f.base, (uintptr_t)f.base + kMix * 4};
  ins[2] = Span{(uintptr_t)f.weight, (uintptr_t)f.weight + (uintptr_t)H * 2};
  outs[0] = f.y ? rows_span(f.y, M, f.ldY, H, 2) : Span{0, 0};
  outs[1] = rows_span(f.post, M, kHC, kHC, 4);
  outs[2] = rows_span(f.comb, M, kHC * kHC, kHC * kHC, 4);
  outs[3] = f.pre ? rows_span(f.pre, M, kHC, kHC, 4) : Span{0, 0};
  outs[4] = mx ? rows_span(f.q, M, f.ldQ, H, 1) : Span{0, 0};
  outs[5] = mx ? rows_span(f.sc, M, f.ldS, H / 32, 1) : Span{0, 0};
  return HC_OK;
}

int workspace_ok(const void* ws, size_t bytes, int64_t M, int32_t H) {
  if (!ws || bytes < hc::stats_workspace_bytes(M, H)) return HC_ERR_WORKSPACE;
  if (((uintptr_t)ws & 255u) != 0) return HC_ERR_ALIGN;
  return HC_OK;
}

Span workspace_span(const void* ws, int64_t M, int32_t H) {
  return Span{(uintptr_t)ws, (uintptr_t)ws + hc::stats_workspace_bytes(M, H)};
}

hipError_t launch_finish(const float* part, const uint16_t* R, int64_t ldR, const Finish& f,
                         int64_t M, int32_t H, bool mx, hipStream_t s) {
  return hc::launch_pre_finish(part, R, ldR, f.scale, f.base, f.weight, (int)M, H, f.rms_eps,
                               f.pre_eps, f.sk_eps, f.iters, f.post_mult, f.norm_eps, f.y, f.ldY,
                               mx ? f.q : nullptr, f.ldQ, mx ? f.sc : nullptr, f.ldS, f.pre,
                               f.post, f.comb, s);
}

// hc_pre: stats of R into the workspace, then the finish.
int pre_impl(const uint16_t* R, int64_t ldR, const uint16_t* fn_packed, int64_t M, int32_t H,
             const Finish& f, bool mx, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_m(M);
  if (st) return st;
  if ((st = finish_scalars(f, H))) return st;
  if (M == 0) return HC_OK;
  if (!R || !fn_packed) return HC_ERR_NULL;
  Span ins[5], outs[7];
  if ((st = finish_pointers(f, M, H, mx, ins, outs))) return st;
  if ((st = check_residual(R, ldR, H))) return st;
  if (!al16(fn_packed)) return HC_ERR_ALIGN;
  if ((st = workspace_ok(workspace, workspace_bytes, M, H))) return st;
  ins[3] = rows_span(R, M, ldR, (int64_t)kHC * H, 2);
  ins[4] = Span{(uintptr_t)fn_packed, (uintptr_t)fn_packed + hc_fn_packed_bytes(H)};
  outs[6] = workspace_span(workspace, M, H);
  if ((st = no_alias(ins, 5, outs, 7))) return st;
  float* part = static_cast<float*>(workspace);
  hipStream_t s = as_stream(stream);
  if ((st = launched(hc::launch_stats(R, ldR, fn_packed, (int)M, H, part, s)))) return st;
  return launched(launch_finish(part, R, ldR, f, M, H, mx, s));
}

// hc_pre_finish: the finish from a workspace filled by hc_post_stats.
int finish_impl(const uint16_t* R, int64_t ldR, int64_t M, int32_t H, const Finish& f, bool mx,
                const void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_m(M);
  if (st) return st;
  if ((st = finish_scalars(f, H))) return st;
  if (M == 0) return HC_OK;
  if (!R) return HC_ERR_NULL;
  Span ins[5], outs[6];
  if ((st = finish_pointers(f, M, H, mx, ins, outs))) return st;
  if ((st = check_residual(R, ldR, H))) return st;
  if ((st = workspace_ok(workspace, workspace_bytes, M, H))) return st;
  ins[3] = rows_span(R, M, ldR, (int64_t)kHC * H, 2);
  ins[4] = workspace_span(workspace, M, H);
  if ((st = no_alias(ins, 5, outs, 6))) return st;
  return launched(launch_finish(static_cast<const float*>(workspace), R, ldR, f, M, H, mx,
                                as_stream(stream)));
}

// hc_post_stats's checks; fills its 5 input and 2 output spans.
int post_stats_check(const uint16_t* x, int64_t ldX, const uint16_t* R, int64_t ldR,
                     const float* post, const float* comb, const uint16_t* fn_packed, int64_t M,
                     int32_t H, uint16_t* Rout, int64_t ldOut, const void* workspace,
                     size_t workspace_bytes, Span* ins, Span* outs) {
  int st;
  if (!x || !R || !post || !comb || !fn_packed || !Rout) return HC_ERR_NULL;
  if ((st = check_residual(R, ldR, H))) return st;
  if (ldX < H || ldOut < (int64_t)kHC * H || ldX >= kMaxLd || ldOut >= kMaxLd) return HC_ERR_SHAPE;
  if (!al16(x) || !al16(Rout) || !al16(post) || !al16(comb) || !al16(fn_packed) ||
      (ldX * 2) % 16 || (ldOut * 2) % 16)
    return HC_ERR_ALIGN;
  if ((st = workspace_ok(workspace, workspace_bytes, M, H))) return st;
  ins[0] = rows_span(x, M, ldX, H, 2);
  ins[1] = rows_span(R, M, ldR, (int64_t)kHC * H, 2);
  ins[2] = rows_span(post, M, kHC, kHC, 4);
  ins[3] = rows_span(comb, M, kHC * kHC, kHC * kHC, 4);
  ins[4] = Span{(uintptr_t)fn_packed, (uintptr_t)fn_packed + hc_fn_packed_bytes(H)};
  outs[0] = rows_span(Rout, M, ldOut, (int64_t)kHC * H, 2);
  outs[1] = workspace_span(workspace, M, H);
  return HC_OK;
}

// hc_post_pre: hc_post_stats then the finish on Rout.
int post_pre_impl(const uint16_t* x, int64_t ldX, const uint16_t* R, int64_t ldR,
                  const float* post, const float* comb, const uint16_t* fn_packed, int64_t M,
                  int32_t H, uint16_t* Rout, int64_t ldOut, const Finish& f, bool mx,
                  void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_m(M);
  if (st) return st;
  if (!post_h_ok(H)) return HC_ERR_SHAPE;
  if ((st = finish_scalars(f, H))) return st;
  if (M == 0) return HC_OK;
  Span ins[8], outs[8];
  if ((st = post_stats_check(x, ldX, R, ldR, post, comb, fn_packed, M, H, Rout, ldOut, workspace,
                             workspace_bytes, ins, outs)))
    return st;
  if ((st = finish_pointers(f, M, H, mx, ins + 5, outs + 2))) return st;
  if ((st = no_alias(ins, 8, outs, 8))) return st;
  float* part = static_cast<float*>(workspace);
  hipStream_t s = as_stream(stream);
  if ((st = launched(hc::launch_post_stats(x, ldX, R, ldR, post, comb, fn_packed, (int)M, H, Rout,
                                           ldOut, part, s))))
    return st;
  return launched(launch_finish(part, Rout, ldOut, f, M, H, mx, s));
}

}  // namespace

extern "C" {

HC_API const char* hc_status_string(int status) {
  switch (status) {
    case HC_OK: return "HC_OK";
    case HC_ERR_NULL: return "HC_ERR_NULL";
    case HC_ERR_SHAPE: return "HC_ERR_SHAPE";
    case HC_ERR_ALIGN: return "HC_ERR_ALIGN";
    case HC_ERR_ALIAS: return "HC_ERR_ALIAS";
    case HC_ERR_WORKSPACE: return "HC_ERR_WORKSPACE";
    case HC_ERR_LAUNCH: return "HC_ERR_LAUNCH";
    case HC_ERR_ARG: return "HC_ERR_ARG";
    default: return "HC_ERR_UNKNOWN";
  }
}

HC_API int hc_abi_version(void) { return 100; }

// ---- fn packing --------------------------------------------------------------------------
HC_API size_t hc_fn_packed_bytes(int32_t H) {
  if (!stats_h_ok(H)) return 0;
  return (size_t)hc::packed_fn_elems(H) * 2;
}

HC_API int hc_fn_pack(const float* fn, int32_t H, uint16_t* fn_packed, void* stream) {
  if (!stats_h_ok(H)) return HC_ERR_SHAPE;
  if (!fn || !fn_packed) return HC_ERR_NULL;
  if (!al16(fn_packed)) return HC_ERR_ALIGN;
  const Span in{(uintptr_t)fn, (uintptr_t)fn + (uintptr_t)kMix * 4 * H * 4};
  const Span out{(uintptr_t)fn_packed, (uintptr_t)fn_packed + hc_fn_packed_bytes(H)};
  if (overlaps(in, out)) return HC_ERR_ALIAS;
  return launched(hc::launch_fn_pack(fn, H, kMix, fn_packed, as_stream(stream)));
}

HC_API int hc_head_fn_pack(const float* fn, int32_t H, uint16_t* fn_packed, void* stream) {
  if (!stats_h_ok(H)) return HC_ERR_SHAPE;
  if (!fn || !fn_packed) return HC_ERR_NULL;
  if (!al16(fn_packed)) return HC_ERR_ALIGN;
  const Span in{(uintptr_t)fn, (uintptr_t)fn + (uintptr_t)kHC * 4 * H * 4};
  const Span out{(uintptr_t)fn_packed, (uintptr_t)fn_packed + hc_fn_packed_bytes(H)};
  if (overlaps(in, out)) return HC_ERR_ALIAS;
  return launched(hc::launch_fn_pack(fn, H, kHC, fn_packed, as_stream(stream)));
}

// ---- stage 1 -----------------------------------------------------------------------------
HC_API size_t hc_pre_stats_workspace_bytes(int64_t M, int32_t H) {
  if (M < 0 || !stats_h_ok(H)) return 0;
  return hc::stats_workspace_bytes(M, H);
}

HC_API int hc_pre_stats(const uint16_t* R, int64_t ldR, const uint16_t* fn_packed, int64_t M,
                        int32_t H, float rms_eps, float* mixes, float* sumsq, void* workspace,
                        size_t workspace_bytes, void* stream) {
  int st = check_m(M);
  if (st) return st;
  if (!stats_h_ok(H)) return HC_ERR_SHAPE;
  if (!finite_nonneg(rms_eps)) return HC_ERR_ARG;
  if (M == 0) return HC_OK;
  if (!R || !fn_packed || !mixes) return HC_ERR_NULL;
  if ((st = check_residual(R, ldR, H))) return st;
  if (!al16(fn_packed)) return HC_ERR_ALIGN;
  if (!workspace || workspace_bytes < hc::stats_workspace_bytes(M, H)) return HC_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return HC_ERR_ALIGN;
  const Span r = rows_span(R, M, ldR, (int64_t)kHC * H, 2);
  const Span fp{(uintptr_t)fn_packed, (uintptr_t)fn_packed + hc_fn_packed_bytes(H)};
  const Span mx = rows_span(mixes, M, kMix, kMix, 4);
  const Span ws{(uintptr_t)workspace, (uintptr_t)workspace + hc::stats_workspace_bytes(M, H)};
  if (overlaps(mx, r) || overlaps(mx, fp) || overlaps(ws, r) || overlaps(ws, fp) ||
      overlaps(ws, mx))
    return HC_ERR_ALIAS;
  if (sumsq) {
    const Span sq = rows_span(sumsq, M, 1, 1, 4);
    if (overlaps(sq, r) || overlaps(sq, fp) || overlaps(sq, mx) || overlaps(sq, ws))
      return HC_ERR_ALIAS;
  }
  float* part = static_cast<float*>(workspace);
  hipStream_t s = as_stream(stream);
  if ((st = launched(hc::launch_stats(R, ldR, fn_packed, (int)M, H, part, s)))) return st;
  return launched(hc::launch_stats_reduce(part, (int)M, H, rms_eps, mixes, sumsq, s));
}

// ---- stages 2-3 ----------------------------------------------------------------------------
HC_API int hc_sinkhorn(const float* mixes, int64_t M, const float* scale, const float* base,
                       int32_t iters, float pre_eps, float sinkhorn_eps, float post_mult,
                       float* pre, float* post, float* comb, void* stream) {
  int st = check_m(M);
  if (st) return st;
  if (iters < 1 || iters > 100000) return HC_ERR_SHAPE;
  if (!finite_nonneg(pre_eps) || !finite_nonneg(sinkhorn_eps) || !isfinite(post_mult))
    return HC_ERR_ARG;
  if (M == 0) return HC_OK;
  if (!mixes || !scale || !base || !pre || !post || !comb) return HC_ERR_NULL;
  const Span in = rows_span(mixes, M, kMix, kMix, 4);
  const Span sc{(uintptr_t)scale, (uintptr_t)scale + 12};
  const Span bs{(uintptr_t)base, (uintptr_t)base + kMix * 4};
  const Span outs[3] = {rows_span(pre, M, kHC, kHC, 4), rows_span(post, M, kHC, kHC, 4),
                        rows_span(comb, M, kHC * kHC, kHC * kHC, 4)};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(outs[i], in) || overlaps(outs[i], sc) || overlaps(outs[i], bs)) return HC_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], outs[j])) return HC_ERR_ALIAS;
  }
  return launched(hc::launch_sinkhorn(mixes, (int)M, scale, base, iters, pre_eps, sinkhorn_eps,
                                      post_mult, pre, post, comb, as_stream(stream)));
}

// ---- stage 4 -------------------------------------------------------------------------------
HC_API int hc_combine_norm(const uint16_t* R, int64_t ldR, const float* pre, int64_t ldPre,
                           const uint16_t* weight, int64_t M, int32_t H, float eps, uint16_t* y,
                           int64_t ldY, void* stream) {
  int st = check_m(M);
  if (st) return st;
  if (!hc::combine_h_supported(H)) return HC_ERR_SHAPE;
  if (!finite_nonneg(eps)) return HC_ERR_ARG;
  if (M == 0) return HC_OK;
  if (!R || !pre || !weight || !y) return HC_ERR_NULL;
  if ((st = check_residual(R, ldR, H))) return st;
  if (ldPre < kHC || ldY < H) return HC_ERR_SHAPE;
  if (!al16(weight) || !al16(y) || (ldY * 2) % 16) return HC_ERR_ALIGN;
  const Span out = rows_span(y, M, ldY, H, 2);
  if (overlaps(out, rows_span(R, M, ldR, (int64_t)kHC * H, 2)) ||
      overlaps(out, rows_span(pre, M, ldPre, kHC, 4)) ||
      overlaps(out, Span{(uintptr_t)weight, (uintptr_t)weight + (uintptr_t)H * 2}))
    return HC_ERR_ALIAS;
  return launched(hc::launch_combine_norm(R, ldR, pre, ldPre, weight, (int)M, H, eps, y, ldY,
                                          as_stream(stream)));
}

// ---- stage 5 -------------------------------------------------------------------------------
HC_API int hc_post(const uint16_t* x, int64_t ldX, const uint16_t* R, int64_t ldR,
                   const float* post, const float* comb, int64_t M, int32_t H, uint16_t* Rout,
                   int64_t ldOut, void* stream) {
  int st = check_m(M);
  if (st) return st;
  if (!post_h_ok(H)) return HC_ERR_SHAPE;
  if (M * (H / 512) >= kMaxRows) return HC_ERR_ARG;
  if (M == 0) return HC_OK;
  if (!x || !R || !post || !comb || !Rout) return HC_ERR_NULL;
  if ((st = check_residual(R, ldR, H))) return st;
  if (ldX < H || ldOut < (int64_t)kHC * H) return HC_ERR_SHAPE;
  if (!al16(x) || !al16(Rout) || (ldX * 2) % 16 || (ldOut * 2) % 16) return HC_ERR_ALIGN;
  const Span out = rows_span(Rout, M, ldOut, (int64_t)kHC * H, 2);
  if (overlaps(out, rows_span(x, M, ldX, H, 2)) ||
      overlaps(out, rows_span(R, M, ldR, (int64_t)kHC * H, 2)) ||
      overlaps(out, rows_span(post, M, kHC, kHC, 4)) ||
      overlaps(out, rows_span(comb, M, kHC * kHC, kHC * kHC, 4)))
    return HC_ERR_ALIAS;
  return launched(hc::launch_post(x, ldX, R, ldR, post, comb, (int)M, H, Rout, ldOut,
                                  as_stream(stream)));
}

// ---- MXFP8 -----------------------------------------------------------------------------------
HC_API int mxfp8_quant_rows(const uint16_t* y, int64_t ldY, int64_t M, int32_t K, uint8_t* q,
                            int64_t ldQ, uint8_t* scales, int64_t ldS, void* stream) {
  int st = check_m(M);
  if (st) return st;
  if (K <= 0 || K % 32 || K > (1 << 24)) return HC_ERR_SHAPE;
  if (M * (K / 32) >= kMaxRows * 16) return HC_ERR_ARG;
  if (M == 0) return HC_OK;
  if (!y || !q || !scales) return HC_ERR_NULL;
  if (ldY < K || ldQ < K || ldS < K / 32) return HC_ERR_SHAPE;
  if (!al16(y) || !al16(q) || (ldY * 2) % 16 || ldQ % 16) return HC_ERR_ALIGN;
  const Span in = rows_span(y, M, ldY, K, 2);
  const Span qs = rows_span(q, M, ldQ, K, 1);
  const Span ss = rows_span(scales, M, ldS, K / 32, 1);
  if (overlaps(qs, in) || overlaps(ss, in) || overlaps(qs, ss)) return HC_ERR_ALIAS;
  return launched(hc::launch_mxfp8(y, ldY, (int)M, K, q, ldQ, scales, ldS, as_stream(stream)));
}

// ---- fused pre -------------------------------------------------------------------------------
HC_API size_t hc_pre_workspace_bytes(int64_t M, int32_t H) {
  return hc_pre_stats_workspace_bytes(M, H);
}

HC_API int hc_pre(const uint16_t* R, int64_t ldR, const uint16_t* fn_packed, const float* scale,
                  const float* base, const uint16_t* weight, int64_t M, int32_t H,
                  float rms_eps, float pre_eps, float sinkhorn_eps, int32_t iters,
                  float post_mult, float norm_eps, uint16_t* y, int64_t ldY, float* pre,
                  float* post, float* comb, void* workspace, size_t workspace_bytes,
                  void* stream) {
  const Finish f{scale, base, weight, rms_eps, pre_eps, sinkhorn_eps, iters, post_mult, norm_eps,
                 y, ldY, nullptr, 0, nullptr, 0, pre, post, comb};
  return pre_impl(R, ldR, fn_packed, M, H, f, false, workspace, workspace_bytes, stream);
}

HC_API int hc_pre_mxfp8(const uint16_t* R, int64_t ldR, const uint16_t* fn_packed,
                        const float* scale, const float* base, const uint16_t* weight, int64_t M,
                        int32_t H, float rms_eps, float pre_eps, float sinkhorn_eps,
                        int32_t iters, float post_mult, float norm_eps, uint16_t* y, int64_t ldY,
                        uint8_t* q, int64_t ldQ, uint8_t* scales, int64_t ldS, float* pre,
                        float* post, float* comb, void* workspace, size_t workspace_bytes,
                        void* stream) {
  const Finish f{scale, base, weight, rms_eps, pre_eps, sinkhorn_eps, iters, post_mult, norm_eps,
                 y, ldY, q, ldQ, scales, ldS, pre, post, comb};
  return pre_impl(R, ldR, fn_packed, M, H, f, true, workspace, workspace_bytes, stream);
}

// ---- fused post -> pre -----------------------------------------------------------------------
HC_API size_t hc_post_pre_workspace_bytes(int64_t M, int32_t H) {
  return hc_pre_stats_workspace_bytes(M, H);
}

HC_API int hc_post_pre(const uint16_t* x, int64_t ldX, const uint16_t* R, int64_t ldR,
                       const float* post, const float* comb, const uint16_t* fn_packed,
                       const float* scale, const float* base, const uint16_t* weight,
                       int64_t M, int32_t H, float rms_eps, float pre_eps, float sinkhorn_eps,
                       int32_t iters, float post_mult, float norm_eps, uint16_t* Rout,
                       int64_t ldOut, uint16_t* y, int64_t ldY, float* pre_out,
                       float* post_out, float* comb_out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  const Finish f{scale, base, weight, rms_eps, pre_eps, sinkhorn_eps, iters, post_mult, norm_eps,
                 y, ldY, nullptr, 0, nullptr, 0, pre_out, post_out, comb_out};
  return post_pre_impl(x, ldX, R, ldR, post, comb, fn_packed, M, H, Rout, ldOut, f, false,
                       workspace, workspace_bytes, stream);
}

HC_API int hc_post_pre_mxfp8(const uint16_t* x, int64_t ldX, const uint16_t* R, int64_t ldR,
                             const float* post, const float* comb, const uint16_t* fn_packed,
                             const float* scale, const float* base, const uint16_t* weight,
                             int64_t M, int32_t H, float rms_eps, float pre_eps,
                             float sinkhorn_eps, int32_t iters, float post_mult, float norm_eps,
                             uint16_t* Rout, int64_t ldOut, uint16_t* y, int64_t ldY, uint8_t* q,
                             int64_t ldQ, uint8_t* scales, int64_t ldS, float* pre_out,
                             float* post_out, float* comb_out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  const Finish f{scale, base, weight, rms_eps, pre_eps, sinkhorn_eps, iters, post_mult, norm_eps,
                 y, ldY, q, ldQ, scales, ldS, pre_out, post_out, comb_out};
  return post_pre_impl(x, ldX, R, ldR, post, comb, fn_packed, M, H, Rout, ldOut, f, true,
                       workspace, workspace_bytes, stream);
}

// ---- the two halves of hc_post_pre ---------------------------------------------------------
HC_API int hc_post_stats(const uint16_t* x, int64_t ldX, const uint16_t* R, int64_t ldR,
                         const float* post, const float* comb, const uint16_t* fn_packed,
                         int64_t M, int32_t H, uint16_t* Rout, int64_t ldOut, void* workspace,
                         size_t workspace_bytes, void* stream) {
  int st = check_m(M);
  if (st) return st;
  if (!stats_h_ok(H) || !hc::combine_h_supported(H) || !post_h_ok(H)) return HC_ERR_SHAPE;
  if (M == 0) return HC_OK;
  Span ins[5], outs[2];
  if ((st = post_stats_check(x, ldX, R, ldR, post, comb, fn_packed, M, H, Rout, ldOut, workspace,
                             workspace_bytes, ins, outs)))
    return st;
  if ((st = no_alias(ins, 5, outs, 2))) return st;
  return launched(hc::launch_post_stats(x, ldX, R, ldR, post, comb, fn_packed, (int)M, H, Rout,
                                        ldOut, static_cast<float*>(workspace), as_stream(stream)));
}

HC_API int hc_pre_finish(const uint16_t* R, int64_t ldR, const float* scale, const float* base,
                         const uint16_t* weight, int64_t M, int32_t H, float rms_eps,
                         float pre_eps, float sinkhorn_eps, int32_t iters, float post_mult,
                         float norm_eps, uint16_t* y, int64_t ldY, float* pre, float* post,
                         float* comb, const void* workspace, size_t workspace_bytes,
                         void* stream) {
  const Finish f{scale, base, weight, rms_eps, pre_eps, sinkhorn_eps, iters, post_mult, norm_eps,
                 y, ldY, nullptr, 0, nullptr, 0, pre, post, comb};
  return finish_impl(R, ldR, M, H, f, false, workspace, workspace_bytes, stream);
}

HC_API int hc_pre_finish_mxfp8(const uint16_t* R, int64_t ldR, const float* scale,
                               const float* base, const uint16_t* weight, int64_t M, int32_t H,
                               float rms_eps, float pre_eps, float sinkhorn_eps, int32_t iters,
                               float post_mult, float norm_eps, uint16_t* y, int64_t ldY,
                               uint8_t* q, int64_t ldQ, uint8_t* scales, int64_t ldS,
                               float* pre, float* post, float* comb, const void* workspace,
                               size_t workspace_bytes, void* stream) {
  const Finish f{scale, base, weight, rms_eps, pre_eps, sinkhorn_eps, iters, post_mult, norm_eps,
                 y, ldY, q, ldQ, scales, ldS, pre, post, comb};
  return finish_impl(R, ldR, M, H, f, true, workspace, workspace_bytes, stream);
}

// ---- hc_head ---------------------------------------------------------------------------------
HC_API size_t hc_head_workspace_bytes(int64_t M, int32_t H) {
  return hc_pre_stats_workspace_bytes(M, H);
}

HC_API int hc_head(const uint16_t* R, int64_t ldR, const uint16_t* fn_packed, const float* scale,
                   const float* base, int64_t M, int32_t H, float norm_eps, float hc_eps,
                   uint16_t* y, int64_t ldY, void* workspace, size_t workspace_bytes,
                   void* stream) {
  int st = check_m(M);
  if (st) return st;
  if (!stats_h_ok(H) || !hc::combine_h_supported(H)) return HC_ERR_SHAPE;
  if (!finite_nonneg(norm_eps) || !isfinite(hc_eps)) return HC_ERR_ARG;
  if (M == 0) return HC_OK;
  if (!R || !fn_packed || !scale || !base || !y) return HC_ERR_NULL;
  if ((st = check_residual(R, ldR, H))) return st;
  if (ldY < H) return HC_ERR_SHAPE;
  if (!al16(fn_packed) || !al16(y) || (ldY * 2) % 16) return HC_ERR_ALIGN;
  if ((st = workspace_ok(workspace, workspace_bytes, M, H))) return st;
  const Span ins[4] = {rows_span(R, M, ldR, (int64_t)kHC * H, 2),
                       Span{(uintptr_t)fn_packed, (uintptr_t)fn_packed + hc_fn_packed_bytes(H)},
                       Span{(uintptr_t)scale, (uintptr_t)scale + 4},
                       Span{(uintptr_t)base, (uintptr_t)base + kHC * 4}};
  const Span outs[2] = {rows_span(y, M, ldY, H, 2), workspace_span(workspace, M, H)};
  if ((st = no_alias(ins, 4, outs, 2))) return st;
  float* part = static_cast<float*>(workspace);
  hipStream_t s = as_stream(stream);
  if ((st = launched(hc::launch_stats(R, ldR, fn_packed, (int)M, H, part, s)))) return st;
  return launched(hc::launch_head_finish(part, R, ldR, scale, base, (int)M, H, norm_eps, hc_eps,
                                         y, ldY, s));
}

// ---- hc_post_pre without a caller workspace ----------------------------------------------------
// The stats partials live in a file-scope device array of HC_NOALLOC_SCRATCH_BYTES, one copy per
// GPU for the life of the process. Host code never passes the array's name to a kernel (on the
// host that name is only a stand-in): its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept below.
}  // extern "C"

static constexpr size_t kScratchBytes = (size_t)HC_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch array, or NULL (with *err set) when it cannot be had.
// The stream must belong to the current device: that device's copy is the one its kernels see.
void* scratch_for(void* stream, int* err) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = HC_ERR_LAUNCH;
    return nullptr;
  }
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(as_stream(stream), &sdev) != hipSuccess) {
      *err = HC_ERR_ARG;
      return nullptr;
    }
    if ((int)sdev != dev) {
      *err = HC_ERR_ARG;
      return nullptr;
    }
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      *err = HC_ERR_LAUNCH;
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

HC_API int hc_post_pre_noalloc(const uint16_t* x, int64_t ldX, const uint16_t* R, int64_t ldR,
                               const float* post, const float* comb, const uint16_t* fn_packed,
                               const float* scale, const float* base, const uint16_t* weight,
                               int64_t M, int32_t H, float rms_eps, float pre_eps,
                               float sinkhorn_eps, int32_t iters, float post_mult,
                               float norm_eps, uint16_t* Rout, int64_t ldOut, uint16_t* y,
                               int64_t ldY, float* pre_out, float* post_out, float* comb_out,
                               void* stream) {
  int st = check_m(M);
  if (st) return st;
  if (stats_h_ok(H) && hc::stats_workspace_bytes(M, H) > kScratchBytes)
    return HC_ERR_WORKSPACE;  // more rows than the scratch array holds at this H
  void* ws = nullptr;  // an empty call checks its arguments and never touches the array
  if (M > 0 && !(ws = scratch_for(stream, &st))) return st;
  const Finish f{scale, base, weight, rms_eps, pre_eps, sinkhorn_eps, iters, post_mult, norm_eps,
                 y, ldY, nullptr, 0, nullptr, 0, pre_out, post_out, comb_out};
  return post_pre_impl(x, ldX, R, ldR, post, comb, fn_packed, M, H, Rout, ldOut, f, false, ws,
                       kScratchBytes, stream);
}

// ---- 128x4 scale layout ----------------------------------------------------------------------
HC_API size_t mxfp8_swizzled_bytes(int64_t M, int32_t G) {
  if (M < 0 || M >= kMaxRows || G <= 0 || G % 4 || G > (1 << 20)) return 0;
  return (size_t)((M + 127) / 128) * 128 * (size_t)G;
}

HC_API int mxfp8_swizzle_128x4(const uint8_t* scales, int64_t ldS, int64_t M, int32_t G,
                               uint8_t* out, void* stream) {
  int st = check_m(M);
  if (st) return st;
  if (G <= 0 || G % 4 || G > (1 << 20)) return HC_ERR_SHAPE;
  if (M == 0) return HC_OK;
  if (!scales || !out) return HC_ERR_NULL;
  if (ldS < G) return HC_ERR_SHAPE;
  if (((uintptr_t)out & 3u) != 0) return HC_ERR_ALIGN;
  const Span in = rows_span(scales, M, ldS, G, 1);
  const Span o{(uintptr_t)out, (uintptr_t)out + mxfp8_swizzled_bytes(M, G)};
  if (overlaps(in, o)) return HC_ERR_ALIAS;
  return launched(hc::launch_mx_swizzle(scales, ldS, (int)M, G, out, as_stream(stream)));
}

}  // extern "C"
