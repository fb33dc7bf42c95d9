/*
 * hc_mi355x.h - C ABI of the MI355X (gfx950) library for the manifold hyper-connection (mHC)
 * pre/post path of a DeepSeek-V4-style decoder, on the bf16 [M, 4, H] multi-stream residual.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every data pointer is a DEVICE pointer owned by the caller. The library never allocates
 *   or frees device memory and never synchronises; each call enqueues its kernels on
 *   `stream` (a hipStream_t; NULL means the default stream) and returns. Kernel-execution
 *   errors surface at the caller's next synchronisation.
 * - bf16 tensors are passed as uint16_t bit patterns; fp32 as float.
 * - `ld*` arguments are row strides in ELEMENTS of the pointed-to type; inner strides are 1.
 *   The residual R is [M, 4, H] with the 4 streams of a row contiguous (stream i, column h at
 *   R[m*ldR + i*H + h]), so ldR >= 4*H.
 * - Row pointers and row strides of bf16 / u8 tensors must keep 16-byte alignment
 *   (pointers 16-byte aligned, ld*·sizeof(elem) a multiple of 16).
 * - Outputs must not overlap inputs.
 * - M == 0 is a successful no-op. A row slice [a, b) of a call is the same call with every
 *   row pointer advanced by a rows and M = b - a; the library takes no "logical row count",
 *   and every row's result is bit-identical whether the row is computed in a full call or in
 *   any slice (mxfp8_swizzle_128x4, a layout over the whole of M, is the one exception). One
 *   kernel computes the mix stats at every M (decode-sized calls launch fewer blocks), so no
 *   step of a row's arithmetic depends on M.
 * - Return value: HC_OK (0) or one of the HC_ERR_* codes below; hc_status_string() names it.
 *   An error return means nothing was enqueued.
 *
 * Sources: the three pages the method is taken from, cited by page and section -
 *   "deepseek_v4.py" (sglang's DeepSeek-V4 model file), "prefill_sp.py" (the prefill
 *   sequence-parallel adapter) and "test_prefill_sp_gpu.py" (its one-GPU test).
 */
#ifndef HC_MI355X_H
#define HC_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HC_API __attribute__((visibility("default")))

enum {
  HC_OK = 0,
  HC_ERR_NULL = 1,       /* a required pointer is NULL while M > 0 */
  HC_ERR_SHAPE = 2,      /* unsupported H / K / iters, or a row stride shorter than a row */
  HC_ERR_ALIGN = 3,      /* a pointer or a row stride breaks the 16-byte alignment rule */
  HC_ERR_ALIAS = 4,      /* an output overlaps an input */
  HC_ERR_WORKSPACE = 5,  /* workspace NULL or smaller than the matching *_workspace_bytes() */
  HC_ERR_LAUNCH = 6,     /* HIP reported an error while enqueuing a kernel */
  HC_ERR_ARG = 7         /* any other bad argument (negative M, M >= 2^31, non-finite eps) */
};

/* Name of a status code ("HC_OK", "HC_ERR_SHAPE", ...). Never NULL. */
HC_API const char* hc_status_string(int status);

/* Library ABI version (major*100 + minor). */
HC_API int hc_abi_version(void);

/* ---------------------------------------------------------------------------------------
 * Weight preparation: the mix projection fn, split for the matrix cores.
 *
 * deepseek_v4.py, make_hc_mixing_params: fn is fp32 [(2+hc)*hc, hc*H] = [24, 4H]. The
 * DeepGEMM prenorm path of DeepseekV4DecoderLayer.hc_pre contracts it with the bf16
 * flattened residual. This call rewrites fn once per weight into three bf16 parts
 * (fn = hi + mid + lo, each part the round-to-nearest-even of what the earlier parts leave),
 * laid out in the order hc_pre_stats / hc_pre read them. Like the decoder layer's cached
 * bf16 norm weights (DeepseekV4DecoderLayer.refresh_mhc_norm_weight_cache), it belongs to
 * weight loading, not to each forward.
 *
 * fn:        fp32 [24, 4H] row-major (device).
 * fn_packed: hc_fn_packed_bytes(H) bytes (device, 16-byte aligned), written.
 * H:         a multiple of 512 up to 8192, except 5632 and 6656 (HC_ERR_SHAPE; the column
 *            slices the stats kernel needs do not divide them).
 * ------------------------------------------------------------------------------------- */
HC_API size_t hc_fn_packed_bytes(int32_t H);
HC_API int hc_fn_pack(const float* fn, int32_t H, uint16_t* fn_packed, void* stream);

/* ---------------------------------------------------------------------------------------
 * Stage 1, mix stats. deepseek_v4.py, DeepseekV4DecoderLayer.hc_pre (hc_pre_torch_impl and
 * the DeepGEMM prenorm path): with x = R[m] flattened stream-major (4H values),
 *   sumsq[m] = sum_k x_k^2,  mixes[m, f] = (sum_k fn[f, k] x_k) * rsqrt(sumsq[m] / 4H + rms_eps).
 *
 * R:          bf16 [M, 4, H], row stride ldR >= 4H.
 * fn_packed:  from hc_fn_pack for the same H.
 * mixes:      fp32 [M, 24], contiguous, written.
 * sumsq:      fp32 [M] or NULL, written when given.
 * workspace:  >= hc_pre_stats_workspace_bytes(M, H) bytes of device memory, 256-byte aligned;
 *             its contents on entry do not matter.
 * H:          as hc_fn_pack.
 * ------------------------------------------------------------------------------------- */
HC_API size_t hc_pre_stats_workspace_bytes(int64_t M, int32_t H);
HC_API int hc_pre_stats(const uint16_t* R, int64_t ldR, const uint16_t* fn_packed, int64_t M,
                        int32_t H, float rms_eps, float* mixes, float* sumsq,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Stages 2-3, split + Sinkhorn (deepseek_v4.py, DeepseekV4DecoderLayer.hc_pre's
 * hc_split_sinkhorn call with hc_scale, hc_base, hc_mult = 4, hc_sinkhorn_iters, hc_eps;
 * the post multiplier is _MHC_POST_MULT_VALUE = 2). Per row, with s = scale, b = base:
 *   pre[i]   = sigmoid(s[0]*mixes[i]   + b[i])   + pre_eps                     i = 0..3
 *   post[i]  = post_mult * sigmoid(s[1]*mixes[4+i] + b[4+i])                   i = 0..3
 *   L[i][j]  = s[2]*mixes[8+4i+j] + b[8+4i+j]    (i = source stream, j = destination)
 *   P = softmax_j(L) + sinkhorn_eps; P /= (column sums + sinkhorn_eps);
 *   then iters-1 times: P /= (row sums + eps); P /= (column sums + eps);  comb = P.
 *
 * mixes: fp32 [M, 24]; scale fp32 [3]; base fp32 [24]; iters >= 1.
 * pre, post: fp32 [M, 4]; comb: fp32 [M, 4, 4] (comb[m][i][j]); all contiguous, written.
 * ------------------------------------------------------------------------------------- */
HC_API int hc_sinkhorn(const float* mixes, int64_t M, const float* scale, const float* base,
                       int32_t iters, float pre_eps, float sinkhorn_eps, float post_mult,
                       float* pre, float* post, float* comb, void* stream);

/* ---------------------------------------------------------------------------------------
 * Stage 4, combine + RMSNorm (deepseek_v4.py, DeepseekV4DecoderLayer.hc_pre's pre-combine
 * and the input_layernorm that follows it, fused as the hc_pre docstring describes;
 * prefill_sp.py, hc_combine_norm_rows passes explicit row strides the same way):
 *   c[h] = sum_i pre[m, i] * R[m, i, h]   (fp32)
 *   y[m, h] = bf16_rne( c[h] * rsqrt(mean_h c^2 + eps) * weight[h] )      one rounding.
 *
 * R: bf16 [M, 4, H] (ldR); pre: fp32 [M, 4] with row stride ldPre >= 4 (ldPre*4 bytes,
 * 16-byte aligned); weight: bf16 [H]; y: bf16 [M, H] (ldY >= H), written.
 * H: a multiple of 512 up to 8192 (512 * n, n = 1 .. 16).
 * ------------------------------------------------------------------------------------- */
HC_API int hc_combine_norm(const uint16_t* R, int64_t ldR, const float* pre, int64_t ldPre,
                           const uint16_t* weight, int64_t M, int32_t H, float eps,
                           uint16_t* y, int64_t ldY, void* stream);

/* ---------------------------------------------------------------------------------------
 * Stage 5, hc post (deepseek_v4.py, DeepseekV4DecoderLayer.hc_post, hc_post_torch_impl;
 * the out-parameter form follows the aiter mhc_post call there):
 *   Rout[m, j, h] = bf16_rne( post[m, j] * x[m, h] + sum_i comb[m, i, j] * R[m, i, h] ).
 *
 * x: bf16 [M, H] (ldX >= H); R: bf16 [M, 4, H] (ldR); post fp32 [M, 4], comb fp32 [M, 4, 4],
 * contiguous; Rout: bf16 [M, 4, H] (ldOut >= 4H), written. H: multiple of 512.
 * ------------------------------------------------------------------------------------- */
HC_API int hc_post(const uint16_t* x, int64_t ldX, const uint16_t* R, int64_t ldR,
                   const float* post, const float* comb, int64_t M, int32_t H,
                   uint16_t* Rout, int64_t ldOut, void* stream);

/* ---------------------------------------------------------------------------------------
 * Row-local MXFP8 quantizer (prefill_sp.py, module docstring stage 2 and _mxfp8_quantize /
 * mxfp8_gather: e4m3 values, one ue8m0 scale per row per 32 columns, linear scale layout).
 * Per 32-column block with maximum magnitude amax: e = the smallest integer with
 * amax * 2^-e <= 448, clamped to [-127, 127] (all-zero block: -127); scales[m, g] = e + 127;
 * q[m, k] = e4m3fn round-to-nearest-even of y[m, k] * 2^-e (saturating at +-448, sign of
 * zero kept). Inputs must be finite.
 *
 * y: bf16 [M, K] (ldY >= K); q: u8 [M, K] (ldQ >= K); scales: u8 [M, K/32] (ldS >= K/32,
 * any alignment). K: multiple of 32.
 * ------------------------------------------------------------------------------------- */
HC_API int mxfp8_quant_rows(const uint16_t* y, int64_t ldY, int64_t M, int32_t K,
                            uint8_t* q, int64_t ldQ, uint8_t* scales, int64_t ldS, void* stream);

/* ---------------------------------------------------------------------------------------
 * Fused pre: stages 1-4 in two kernels (deepseek_v4.py, DeepseekV4DecoderLayer.hc_pre with a
 * norm given: mhc_pre(residual, fn, hc_scale, hc_base, rms_eps, hc_pre_eps,
 * hc_sinkhorn_eps, hc_post_mult_value, sinkhorn_repeat, norm_weight, norm_eps) returns
 * (post, comb, y) with y already normalised). Same arithmetic, bit for bit, as
 * hc_pre_stats -> hc_sinkhorn -> hc_combine_norm.
 *
 * pre may be NULL (not written); post fp32 [M, 4], comb fp32 [M, 4, 4], y bf16 [M, H] (ldY).
 * H: as hc_fn_pack (every such H is one hc_combine_norm takes). workspace: >=
 * hc_pre_workspace_bytes(M, H), 256-byte aligned (HC_ERR_ALIGN otherwise).
 * ------------------------------------------------------------------------------------- */
HC_API size_t hc_pre_workspace_bytes(int64_t M, int32_t H);
HC_API int hc_pre(const uint16_t* R, int64_t ldR, const uint16_t* fn_packed,
                  const float* scale, const float* base, const uint16_t* weight,
                  int64_t M, int32_t H, float rms_eps, float pre_eps, float sinkhorn_eps,
                  int32_t iters, float post_mult, float norm_eps,
                  uint16_t* y, int64_t ldY, float* pre, float* post, float* comb,
                  void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Fused hc post -> hc pre across a sublayer boundary (deepseek_v4.py,
 * DeepseekV4DecoderLayer.forward: mhc_fused_post_pre takes the residual, the previous
 * site's post / comb and the sublayer output together with the next site's fn, scale, base and
 * norm weight, and returns the new residual, the next post / comb and the normalised input).
 *   Rout = hc_post(x, R, post, comb)                      (bit-identical to hc_post)
 *   (y, pre_out, post_out, comb_out) = hc_pre(Rout, ...)  (bit-identical to hc_pre on Rout)
 * The post kernel also computes the mix stats of the bf16 Rout it writes, so Rout is read
 * back once (by the combine) instead of twice.
 *
 * x: bf16 [M, H] (ldX); R: bf16 [M, 4, H] (ldR); post fp32 [M, 4], comb fp32 [M, 4, 4],
 * contiguous and 16-byte aligned; fn_packed / scale / base / weight: the next site's, as
 * for hc_pre. Rout: bf16 [M, 4, H] (ldOut); y: bf16 [M, H] (ldY); pre_out (or NULL),
 * post_out fp32 [M, 4], comb_out fp32 [M, 4, 4]: written. H: as hc_pre.
 * workspace: >= hc_post_pre_workspace_bytes(M, H), 256-byte aligned (HC_ERR_ALIGN otherwise).
 * Outputs must not overlap any input.
 * ------------------------------------------------------------------------------------- */
HC_API size_t hc_post_pre_workspace_bytes(int64_t M, int32_t H);
HC_API int hc_post_pre(const uint16_t* x, int64_t ldX, const uint16_t* R, int64_t ldR,
                       const float* post, const float* comb, const uint16_t* fn_packed,
                       const float* scale, const float* base, const uint16_t* weight,
                       int64_t M, int32_t H, float rms_eps, float pre_eps, float sinkhorn_eps,
                       int32_t iters, float post_mult, float norm_eps,
                       uint16_t* Rout, int64_t ldOut, uint16_t* y, int64_t ldY, float* pre_out,
                       float* post_out, float* comb_out, void* workspace,
                       size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * hc_post_pre for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. The same kernels and bits as
 * hc_post_pre; instead of a caller workspace it uses a static device array inside the library
 * (HC_NOALLOC_SCRATCH_BYTES = 32 MiB, one copy per GPU, held until the process ends). It calls
 * no allocating routine. The array's device address is looked up on the first call on each
 * device, so make that first call outside a graph capture.
 *
 * Arguments and outputs as hc_post_pre, without workspace / workspace_bytes. The call must fit
 * the array: hc_post_pre_workspace_bytes(M, H) <= HC_NOALLOC_SCRATCH_BYTES (20 971 rows at
 * H = 5120, 11 983 at 7168, 10 485 at 8192); larger calls return HC_ERR_WORKSPACE. `stream`
 * must belong to the current device (HC_ERR_ARG otherwise). Every partial in the array is
 * written before it is read, so nothing has to start at zero; but all calls on one GPU share
 * the array, so calls that overlap in time on one GPU (other streams, other threads) race and
 * must not be issued.
 * ------------------------------------------------------------------------------------- */
#define HC_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)
HC_API int hc_post_pre_noalloc(const uint16_t* x, int64_t ldX, const uint16_t* R, int64_t ldR,
                               const float* post, const float* comb, const uint16_t* fn_packed,
                               const float* scale, const float* base, const uint16_t* weight,
                               int64_t M, int32_t H, float rms_eps, float pre_eps,
                               float sinkhorn_eps, int32_t iters, float post_mult,
                               float norm_eps, uint16_t* Rout, int64_t ldOut, uint16_t* y,
                               int64_t ldY, float* pre_out, float* post_out, float* comb_out,
                               void* stream);

/* ---------------------------------------------------------------------------------------
 * hc_post_pre in two calls, for callers that place other work between the halves or time
 * them apart. hc_post_stats followed by hc_pre_finish on the same stream, with the same
 * workspace, M and H and with hc_pre_finish's R = hc_post_stats's Rout (same pointer and
 * stride), gives exactly the bits of hc_post_pre.
 *
 * hc_post_stats: Rout = hc_post(x, R, post, comb) (bit-identical to hc_post), and in
 *   `workspace` a record of Rout's mix-stat partial sums under the next site's fn_packed.
 *   Arguments as hc_post_pre. H: as hc_pre.
 * hc_pre_finish: reads that record and Rout; writes y, pre (or NULL), post, comb as hc_pre on
 *   Rout would. The record is opaque; a workspace that no hc_post_stats call with this M and
 *   H filled gives unspecified values (never an out-of-bounds access).
 * workspace: >= hc_post_pre_workspace_bytes(M, H), 256-byte aligned, written by the first
 *   call and read by the second.
 * ------------------------------------------------------------------------------------- */
HC_API int hc_post_stats(const uint16_t* x, int64_t ldX, const uint16_t* R, int64_t ldR,
                         const float* post, const float* comb, const uint16_t* fn_packed,
                         int64_t M, int32_t H, uint16_t* Rout, int64_t ldOut, void* workspace,
                         size_t workspace_bytes, void* stream);
HC_API int hc_pre_finish(const uint16_t* R, int64_t ldR, const float* scale, const float* base,
                         const uint16_t* weight, int64_t M, int32_t H, float rms_eps,
                         float pre_eps, float sinkhorn_eps, int32_t iters, float post_mult,
                         float norm_eps, uint16_t* y, int64_t ldY, float* pre, float* post,
                         float* comb, const void* workspace, size_t workspace_bytes,
                         void* stream);

/* ---------------------------------------------------------------------------------------
 * MXFP8 output of the pre (prefill_sp.py, module docstring stage 2: the attention input is
 * all-gathered as e4m3 bytes plus ue8m0 scales; _mxfp8_quantize / mxfp8_gather quantise each
 * row shard with linear scales). These are hc_pre, hc_post_pre and hc_pre_finish with the
 * normalised input y also written in MXFP8, quantised inside the same pass from the same bf16
 * values: q / scales are bit-identical to mxfp8_quant_rows of the y the bf16 form writes.
 *
 * y: bf16 [M, H] (ldY), or NULL to skip the bf16 form. q: u8 [M, H] e4m3fn codes (ldQ >= H,
 * ldQ % 16 == 0, 16-byte aligned). scales: u8 [M, H/32] linear (ldS >= H/32, any alignment).
 * Every other argument, and the error behaviour, as in the bf16 entry point of the same name.
 * ------------------------------------------------------------------------------------- */
HC_API int hc_pre_mxfp8(const uint16_t* R, int64_t ldR, const uint16_t* fn_packed,
                        const float* scale, const float* base, const uint16_t* weight, int64_t M,
                        int32_t H, float rms_eps, float pre_eps, float sinkhorn_eps,
                        int32_t iters, float post_mult, float norm_eps, uint16_t* y, int64_t ldY,
                        uint8_t* q, int64_t ldQ, uint8_t* scales, int64_t ldS, float* pre,
                        float* post, float* comb, void* workspace, size_t workspace_bytes,
                        void* stream);
HC_API int hc_post_pre_mxfp8(const uint16_t* x, int64_t ldX, const uint16_t* R, int64_t ldR,
                             const float* post, const float* comb, const uint16_t* fn_packed,
                             const float* scale, const float* base, const uint16_t* weight,
                             int64_t M, int32_t H, float rms_eps, float pre_eps,
                             float sinkhorn_eps, int32_t iters, float post_mult, float norm_eps,
                             uint16_t* Rout, int64_t ldOut, uint16_t* y, int64_t ldY, uint8_t* q,
                             int64_t ldQ, uint8_t* scales, int64_t ldS, float* pre_out,
                             float* post_out, float* comb_out, void* workspace,
                             size_t workspace_bytes, void* stream);
HC_API int hc_pre_finish_mxfp8(const uint16_t* R, int64_t ldR, const float* scale,
                               const float* base, const uint16_t* weight, int64_t M, int32_t H,
                               float rms_eps, float pre_eps, float sinkhorn_eps, int32_t iters,
                               float post_mult, float norm_eps, uint16_t* y, int64_t ldY,
                               uint8_t* q, int64_t ldQ, uint8_t* scales, int64_t ldS,
                               float* pre, float* post, float* comb, const void* workspace,
                               size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * 128x4 scale layout (prefill_sp.py, swizzle_128x4: what the attention GEMM takes after the
 * gather). From linear scales [M, G]: rows are zero-padded to a multiple of 128; 128 x 4
 * tiles (m / 128, g / 4) follow in row-tile-major order, 512 bytes each; inside a tile the
 * scale of (m, g) sits at byte (m % 32) * 16 + ((m % 128) / 32) * 4 + g % 4.
 *
 * scales: u8 [M, G] with row stride ldS >= G (device). out: mxfp8_swizzled_bytes(M, G) bytes
 * (device, 4-byte aligned), every byte written. G: multiple of 4 (H / 32 for H % 128 == 0).
 * The layout is over the whole of M: unlike the other entry points, a row slice of a call is
 * not a call on a slice (swizzle the gathered scales, as the pages do).
 * ------------------------------------------------------------------------------------- */
HC_API size_t mxfp8_swizzled_bytes(int64_t M, int32_t G);
HC_API int mxfp8_swizzle_128x4(const uint8_t* scales, int64_t ldS, int64_t M, int32_t G,
                               uint8_t* out, void* stream);

/* ---------------------------------------------------------------------------------------
 * hc_head: the model's last mix of the 4 streams into one (deepseek_v4.py, hc_head_torch and
 * the model's hc_head / fused_hc_head; make_hc_head_params: fn fp32 [4, 4H], base [4],
 * scale [1]). Per row, with x = R[m] flattened stream-major (4H values):
 *   mixes[i] = (sum_k fn[i, k] x_k) * rsqrt(sum x^2 / 4H + norm_eps)        i = 0..3
 *   pre[i]   = sigmoid(mixes[i] * scale[0] + base[i]) + hc_eps
 *   y[m, h]  = bf16_rne( sum_i pre[i] * R[m, i, h] )        (no norm: the model's final
 *                                                            RMSNorm is a separate step)
 * hc_head_fn_pack packs the 4-row fn into the layout of hc_fn_pack (hc_fn_packed_bytes(H)
 * bytes; the other rows are zero), once per weight.
 *
 * R: bf16 [M, 4, H] (ldR); scale fp32 [1]; base fp32 [4]; y: bf16 [M, H] (ldY), written.
 * H: as hc_pre. workspace: >= hc_head_workspace_bytes(M, H), 256-byte aligned.
 * ------------------------------------------------------------------------------------- */
HC_API int hc_head_fn_pack(const float* fn, int32_t H, uint16_t* fn_packed, void* stream);
HC_API size_t hc_head_workspace_bytes(int64_t M, int32_t H);
HC_API int hc_head(const uint16_t* R, int64_t ldR, const uint16_t* fn_packed, const float* scale,
                   const float* base, int64_t M, int32_t H, float norm_eps, float hc_eps,
                   uint16_t* y, int64_t ldY, void* workspace, size_t workspace_bytes,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HC_MI355X_H */
