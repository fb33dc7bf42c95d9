"""CPU oracle of the mHC (manifold hyper-connection) pre/post path.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this module. The HIP library never calls it, and it shares no code with the
HIP library (no kernels, headers, helpers, tables or constants).

Everything is computed in float64 from the inputs' exact values (bf16 bit patterns, fp32
parameters). bf16 outputs are rounded once, to nearest even, from the float64 result.

Sources (the pages' own names; a "page" is one of the three web pages the method is taken
from):

* deepseek_v4.py, ``DeepseekV4DecoderLayer.hc_pre`` (the torch path ``hc_pre_torch_impl`` and
  the DeepGEMM prenorm path): mix stats, then ``hc_split_sinkhorn``, then the pre-combine.
* deepseek_v4.py, ``DeepseekV4DecoderLayer.hc_post`` (``hc_post_torch_impl``): the post update.
* deepseek_v4.py, ``hc_head_torch``: the sigmoid-plus-eps form of ``pre`` and the 4-wide head.
* deepseek_v4.py, ``make_hc_mixing_params`` and the ``_MHC_POST_MULT_VALUE`` constant: the
  24 = (2 + 4) * 4 mixes and the post multiplier 2.
* prefill_sp.py, module docstring (stage 2) and ``_mxfp8_quantize`` / ``mxfp8_gather``: the
  row-local MXFP8 format (e4m3 elements, one ue8m0 scale per 32 columns, linear scales).

Readings where the pages are silent (each one is listed with its reason in the design notes):

1. Split order is pre | post | res, with scale[0], scale[1], scale[2] for the three groups;
   res is row-major [i][j] with i the source stream and j the destination stream.
2. pre = sigmoid(.) + hc_eps, as ``hc_head_torch`` does; post = 2 * sigmoid(.).
3. Sinkhorn: softmax over j plus eps on every entry, then a column step, then (iters - 1)
   times a row step and a column step; each step divides by (sum + eps). So the last step
   normalises columns: every destination stream is a unit-sum mix of the sources.
4. RMSNorm after the combine is the fused form: c * rsqrt(mean(c^2) + eps) * w with one
   rounding to bf16 at the end.
5. MXFP8 scale: the smallest power of two 2^e with amax * 2^-e <= 448 (no element
   saturates), e clamped to [-127, 127], scale byte e + 127, all-zero block -> byte 0.
   Elements round to nearest even into e4m3fn, saturate at +-448, keep the sign of zero.
"""
from __future__ import annotations

import numpy as np

HC = 4
ITERS = 20
RMS_EPS = 1e-6
HC_EPS = 1e-6
POST_MULT = 2.0
MX_BLOCK = 32
E4M3_MAX = 448.0


# ------------------------------------------------------------------------------------------
# bf16 <-> float64
# ------------------------------------------------------------------------------------------
def bf16_to_f64(b) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(b, dtype=np.uint16)
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16(v) -> np.ndarray:
    """Round float64 values to bf16 bit patterns, to nearest with ties to even, in ONE
    rounding (no intermediate float32). bf16 has an 8-bit significand and float32's
    exponent range; results beyond the largest finite bf16 become infinity, NaN becomes
    the canonical quiet NaN 0x7FC0."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    m, e = np.frexp(a)  # a = m * 2**e, m in [0.5, 1)
    # significand quantum 2**(e-8) for normal results, 2**-133 below 2**-126
    qexp = np.maximum(e - 8, -133)
    q = np.rint(np.ldexp(a, -qexp))  # exact scaling by a power of two; rint = ties-to-even
    r = np.ldexp(q, qexp)  # exactly representable in bf16 (or overflows)
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)  # exact: r has <= 8 significant bits
    out = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bf16_max = 0x7F7F
    over = (out > bf16_max) | (r > 3.3895313892515355e38)
    out = np.where(over & ~np.isnan(v), np.uint16(0x7F80), out)
    out = out | np.where(np.signbit(v), np.uint16(0x8000), np.uint16(0))
    out = np.where(np.isnan(v), np.uint16(0x7FC0), out)
    return out.astype(np.uint16)


# ------------------------------------------------------------------------------------------
# stage 1: mix stats  (deepseek_v4.py, DeepseekV4DecoderLayer.hc_pre, torch and prenorm paths)
# ------------------------------------------------------------------------------------------
def hc_mix_stats(R_bits, fn, rms_eps: float = RMS_EPS):
    """mixes[m, :] = (fn @ x_m) * rsqrt(mean(x_m^2) + rms_eps) with x_m = R[m].flatten()
    (stream-major: flat column i*H + h). Returns (mixes [M, mix] float64, sumsq [M])."""
    R_bits = np.asarray(R_bits, dtype=np.uint16)
    M = R_bits.shape[0]
    x = bf16_to_f64(R_bits).reshape(M, -1)
    K = x.shape[1]
    fn64 = np.asarray(fn, dtype=np.float64)
    assert fn64.shape[1] == K
    sumsq = np.sum(x * x, axis=1)
    rs = 1.0 / np.sqrt(sumsq / K + rms_eps)
    d = x @ fn64.T
    return d * rs[:, None], sumsq


# ------------------------------------------------------------------------------------------
# stage 2: split  (hc_split_sinkhorn's first half; readings 1 and 2)
# ------------------------------------------------------------------------------------------
def _sigmoid(t):
    return 1.0 / (1.0 + np.exp(-t))


def hc_split(mixes, scale, base, hc: int = HC, pre_eps: float = HC_EPS,
             post_mult: float = POST_MULT):
    """(pre [M,hc], post [M,hc], res logits [M,hc,hc]) from mixes [M,(2+hc)*hc]."""
    mixes = np.asarray(mixes, dtype=np.float64)
    scale = np.asarray(scale, dtype=np.float64)
    base = np.asarray(base, dtype=np.float64)
    M = mixes.shape[0]
    pre = _sigmoid(scale[0] * mixes[:, :hc] + base[:hc]) + pre_eps
    post = post_mult * _sigmoid(scale[1] * mixes[:, hc:2 * hc] + base[hc:2 * hc])
    logits = (scale[2] * mixes[:, 2 * hc:] + base[2 * hc:]).reshape(M, hc, hc)
    return pre, post, logits


# ------------------------------------------------------------------------------------------
# stage 3: Sinkhorn  (reading 3; Sinkhorn and Knopp's alternating normalisation)
# ------------------------------------------------------------------------------------------
def sinkhorn(logits, iters: int = ITERS, eps: float = HC_EPS):
    """comb[m, i, j] after `iters` row/column rounds, i = source stream, j = destination.

    Round 1: a softmax over j (row-wise), eps added to every entry, then columns divided by
    (column sum + eps). Rounds 2..iters: rows divided by (row sum + eps), then columns."""
    L = np.asarray(logits, dtype=np.float64)
    assert iters >= 1
    z = L - L.max(axis=-1, keepdims=True)
    P = np.exp(z)
    P = P / P.sum(axis=-1, keepdims=True) + eps
    P = P / (P.sum(axis=-2, keepdims=True) + eps)
    for _ in range(iters - 1):
        P = P / (P.sum(axis=-1, keepdims=True) + eps)
        P = P / (P.sum(axis=-2, keepdims=True) + eps)
    return P


def hc_split_sinkhorn(mixes, scale, base, hc: int = HC, iters: int = ITERS,
                      eps: float = HC_EPS, post_mult: float = POST_MULT):
    """(pre, post, comb) from mixes, hc_eps used both as the pre offset and as the
    Sinkhorn eps (the decoder layer passes hc_eps for both)."""
    pre, post, logits = hc_split(mixes, scale, base, hc, eps, post_mult)
    return pre, post, sinkhorn(logits, iters, eps)


# ------------------------------------------------------------------------------------------
# stage 4: combine + RMSNorm  (DeepseekV4DecoderLayer.hc_pre's pre-combine; reading 4)
# ------------------------------------------------------------------------------------------
def hc_combine(R_bits, pre):
    """c[m, h] = sum_i pre[m, i] * R[m, i, h], float64."""
    R = bf16_to_f64(R_bits)
    pre = np.asarray(pre, dtype=np.float64)
    c = np.zeros((R.shape[0], R.shape[2]))
    for i in range(R.shape[1]):
        c += pre[:, i, None] * R[:, i, :]
    return c


def hc_combine_norm(R_bits, pre, w_bits, eps: float = RMS_EPS):
    """(y float64 [M,H], y bf16 bits) with y = c * rsqrt(mean(c^2) + eps) * w."""
    c = hc_combine(R_bits, pre)
    w = bf16_to_f64(w_bits)
    ms = np.mean(c * c, axis=-1, keepdims=True)
    y = c / np.sqrt(ms + eps) * w
    return y, f64_to_bf16(y)


# ------------------------------------------------------------------------------------------
# stage 5: hc post  (DeepseekV4DecoderLayer.hc_post, hc_post_torch_impl)
# ------------------------------------------------------------------------------------------
def hc_post(x_bits, R_bits, post, comb):
    """(R' float64 [M,hc,H], R' bf16 bits) with R'[m,j,:] = post[m,j] * x[m,:]
    + sum_i comb[m,i,j] * R[m,i,:]."""
    x = bf16_to_f64(x_bits)
    R = bf16_to_f64(R_bits)
    post = np.asarray(post, dtype=np.float64)
    comb = np.asarray(comb, dtype=np.float64)
    out = post[:, :, None] * x[:, None, :]
    for i in range(R.shape[1]):  # source stream i feeds every destination j with comb[m, i, j]
        out += comb[:, i, :, None] * R[:, i, None, :]
    return out, f64_to_bf16(out)


# ------------------------------------------------------------------------------------------
# pre (all of stages 1-4) and the chains
# ------------------------------------------------------------------------------------------
def hc_pre(R_bits, fn, scale, base, w_bits, rms_eps: float = RMS_EPS, hc_eps: float = HC_EPS,
           iters: int = ITERS, post_mult: float = POST_MULT, norm_eps: float = RMS_EPS):
    """Stages 1-4. Returns dict(mixes, sumsq, pre, post, comb, y, y_bits).

    Three eps values, each in its own stage as the decoder layer passes them (hc_pre's
    TileLang call: rms_eps to the mix stats, hc_eps to pre and to the Sinkhorn, the norm
    module's own variance epsilon to the RMSNorm after the combine); the model uses 1e-6
    for all three."""
    hc = np.asarray(R_bits).shape[1]
    mixes, sumsq = hc_mix_stats(R_bits, fn, rms_eps)
    pre, post, comb = hc_split_sinkhorn(mixes, scale, base, hc, iters, hc_eps, post_mult)
    y, y_bits = hc_combine_norm(R_bits, pre, w_bits, norm_eps)
    return dict(mixes=mixes, sumsq=sumsq, pre=pre, post=post, comb=comb, y=y, y_bits=y_bits)


def hc_head(R_bits, fn, scale, base, norm_eps: float = RMS_EPS, hc_eps: float = HC_EPS):
    """deepseek_v4.py ``hc_head_torch``: pre = sigmoid(mixes * scale + base) + hc_eps with a
    [hc, hc*H] fn and a one-element scale, then y = sum_i pre_i * R_i (no Sinkhorn, no post).
    Returns (y float64 [M,H], y bf16 bits)."""
    mixes, _ = hc_mix_stats(R_bits, fn, norm_eps)
    scale = np.asarray(scale, dtype=np.float64).reshape(-1)
    pre = _sigmoid(mixes * scale[0] + np.asarray(base, dtype=np.float64)) + hc_eps
    y = hc_combine(R_bits, pre)
    return y, f64_to_bf16(y)


# ------------------------------------------------------------------------------------------
# row-local MXFP8  (prefill_sp.py stage 2; reading 5)
# ------------------------------------------------------------------------------------------
def e4m3_encode(s) -> np.ndarray:
    """float64 values -> e4m3fn codes (uint8): round to nearest even, saturate to +-448,
    sign kept on zero. Exponent bias 7, 3 mantissa bits, subnormal quantum 2^-9."""
    s = np.asarray(s, dtype=np.float64)
    a = np.abs(s)
    code = np.zeros(a.shape, dtype=np.int64)
    # normal range (a >= 2^-6 before rounding): quantum 2^(p-3) with a = f * 2^p, f in [1,2)
    m, e = np.frexp(np.where(a > 0, a, 1.0))
    p = e - 1
    qn = np.rint(np.ldexp(np.where(a > 0, a, 1.0), -(p - 3))).astype(np.int64)  # in [8, 16]
    carry = qn == 16
    p = np.where(carry, p + 1, p)
    qn = np.where(carry, 8, qn)
    E = p + 7
    normal_code = (E << 3) | (qn - 8)
    # subnormal range (a < 2^-6): quantum 2^-9, codes 0..8 (8 is the smallest normal, 0x08)
    qs = np.rint(np.ldexp(a, 9)).astype(np.int64)
    code = np.where(a >= 2.0 ** -6, normal_code, qs)
    code = np.where(a > E4M3_MAX, 0x7E, code)
    code = np.where((a >= 2.0 ** -6) & ((E > 15) | ((E == 15) & (qn - 8 > 6))), 0x7E, code)
    code = code | np.where(np.signbit(s), 0x80, 0)
    return code.astype(np.uint8)


def mxfp8_scale_exponent(amax) -> np.ndarray:
    """Block exponent e (int) for block maxima amax >= 0: the smallest e with
    amax * 2^-e <= 448, clamped to [-127, 127]; amax == 0 gives -127."""
    amax = np.asarray(amax, dtype=np.float64)
    pos = amax > 0
    m, k = np.frexp(np.where(pos, amax, 1.0))  # amax = m * 2^k, m in [0.5, 1)
    m1 = 2.0 * m  # in [1, 2)
    k1 = k - 1
    e = k1 - 8 + (m1 > 1.75).astype(np.int64)  # 448 = 1.75 * 2^8
    e = np.where(pos, e, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def mxfp8_quant_rows(y_bits, block: int = MX_BLOCK):
    """bf16 rows [M, K] -> (q uint8 [M, K] e4m3fn codes, sf uint8 [M, K/block] ue8m0 bytes,
    linear layout)."""
    y_bits = np.asarray(y_bits, dtype=np.uint16)
    M, K = y_bits.shape
    assert K % block == 0
    v = bf16_to_f64(y_bits).reshape(M, K // block, block)
    if np.any(~np.isfinite(v)):
        raise ValueError("mxfp8_quant_rows: inputs must be finite")
    amax = np.abs(v).max(axis=-1)
    e = mxfp8_scale_exponent(amax)
    scaled = np.ldexp(v, -e[:, :, None])  # exact: a power-of-two scaling of a bf16 value
    q = e4m3_encode(scaled).reshape(M, K)
    sf = (e + 127).astype(np.uint8)
    return q, sf


def e4m3_decode(code) -> np.ndarray:
    """e4m3fn codes -> float64 (0x7F / 0xFF are NaN)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    mant = c & 0x7
    val = np.where(E == 0, np.ldexp(mant.astype(np.float64), -9),
                   np.ldexp(1.0 + mant / 8.0, E - 7))
    val = np.where((E == 15) & (mant == 7), np.nan, val)
    return sign * val


def swizzle_128x4(sf):
    """[M, G] linear ue8m0 bytes -> the 128x4 tiled order (prefill_sp.py ``swizzle_128x4``):
    rows zero-padded to a multiple of 128; tiles (m // 128, g // 4) in row-tile-major order;
    inside a tile the byte order is [m % 32][(m % 128) // 32][g % 4]. Returns a flat array."""
    sf = np.asarray(sf, dtype=np.uint8)
    M, G = sf.shape
    assert G % 4 == 0
    mt = (M + 127) // 128
    pad = np.zeros((mt * 128, G), dtype=np.uint8)
    pad[:M] = sf
    out = np.empty(mt * 128 * G, dtype=np.uint8)
    pos = 0
    for tm in range(mt):
        for tg in range(G // 4):
            for r32 in range(32):
                for r4 in range(4):
                    for c in range(4):
                        out[pos] = pad[tm * 128 + r4 * 32 + r32, tg * 4 + c]
                        pos += 1
    return out
