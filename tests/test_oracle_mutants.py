"""Test of the tests: each plausible mistake planted in the oracle (on the CPU, through
monkeypatch) must make at least one pin in test_oracle_pins fail."""
import numpy as np
import pytest

import tests.test_oracle_pins as pins
from oracle import hc_oracle as o

_real_sinkhorn = o.sinkhorn
_real_stats = o.hc_mix_stats
_real_split = o.hc_split
_real_combine_norm = o.hc_combine_norm
_real_post = o.hc_post
_real_e4m3 = o.e4m3_encode
_real_scale_exp = o.mxfp8_scale_exponent


def _sinkhorn_row_last(L, iters=20, eps=1e-6):
    P = np.exp(L - L.max(-1, keepdims=True))
    P = P / P.sum(-1, keepdims=True) + eps
    for _ in range(iters):
        P = P / (P.sum(-2, keepdims=True) + eps)
        P = P / (P.sum(-1, keepdims=True) + eps)
    return P


def _sinkhorn_one_round_short(L, iters=20, eps=1e-6):
    return _real_sinkhorn(L, max(iters - 1, 1), eps)


def _sinkhorn_eps_only_in_denominators(L, iters=20, eps=1e-6):
    P = np.exp(L - L.max(-1, keepdims=True))
    P = P / P.sum(-1, keepdims=True)
    P = P / (P.sum(-2, keepdims=True) + eps)
    for _ in range(iters - 1):
        P = P / (P.sum(-1, keepdims=True) + eps)
        P = P / (P.sum(-2, keepdims=True) + eps)
    return P


def _sinkhorn_transposed(L, iters=20, eps=1e-6):
    return np.swapaxes(_real_sinkhorn(np.swapaxes(L, -1, -2), iters, eps), -1, -2)


def _stats_h_major(R_bits, fn, rms_eps=1e-6):
    R_bits = np.asarray(R_bits)
    return _real_stats(np.ascontiguousarray(np.swapaxes(R_bits, 1, 2)).reshape(R_bits.shape), fn, rms_eps)


def _stats_no_eps(R_bits, fn, rms_eps=1e-6):
    return _real_stats(R_bits, fn, 0.0)


def _split_no_post_mult(mixes, scale, base, hc=4, pre_eps=1e-6, post_mult=2.0):
    return _real_split(mixes, scale, base, hc, pre_eps, 1.0)


def _split_pre_without_eps(mixes, scale, base, hc=4, pre_eps=1e-6, post_mult=2.0):
    return _real_split(mixes, scale, base, hc, 0.0, post_mult)


def _combine_norm_no_eps(R_bits, pre, w_bits, eps=1e-6):
    return _real_combine_norm(R_bits, pre, w_bits, 0.0)


def _post_comb_transposed(x_bits, R_bits, post, comb):
    return _real_post(x_bits, R_bits, post, np.swapaxes(np.asarray(comb), -1, -2))


def _e4m3_truncating(s):
    s = np.asarray(s, dtype=np.float64)
    a = np.abs(s)
    m, e = np.frexp(np.where(a > 0, a, 1.0))
    p = e - 1
    q = np.floor(np.ldexp(np.where(a > 0, a, 1.0), -(p - 3))).astype(np.int64)
    code = np.where(a >= 2.0**-6, ((p + 7) << 3) | (q - 8), np.floor(np.ldexp(a, 9)).astype(np.int64))
    code = np.where(a > 448, 0x7E, code) | np.where(np.signbit(s), 0x80, 0)
    return code.astype(np.uint8)


_real_pre = o.hc_pre
_real_head = o.hc_head
_real_split_sinkhorn = o.hc_split_sinkhorn


def _pre_combine_weighted_by_post(R_bits, fn, scale, base, w_bits, rms_eps=1e-6, hc_eps=1e-6,
                                  iters=20, post_mult=2.0, norm_eps=1e-6):
    d = _real_pre(R_bits, fn, scale, base, w_bits, rms_eps, hc_eps, iters, post_mult, norm_eps)
    d["y"], d["y_bits"] = _real_combine_norm(R_bits, d["post"], w_bits, norm_eps)
    return d


def _pre_combine_streams_reversed(R_bits, fn, scale, base, w_bits, rms_eps=1e-6, hc_eps=1e-6,
                                  iters=20, post_mult=2.0, norm_eps=1e-6):
    d = _real_pre(R_bits, fn, scale, base, w_bits, rms_eps, hc_eps, iters, post_mult, norm_eps)
    d["y"], d["y_bits"] = _real_combine_norm(R_bits, d["pre"][:, ::-1], w_bits, norm_eps)
    return d


def _pre_norm_takes_stats_eps(R_bits, fn, scale, base, w_bits, rms_eps=1e-6, hc_eps=1e-6,
                              iters=20, post_mult=2.0, norm_eps=1e-6):
    return _real_pre(R_bits, fn, scale, base, w_bits, rms_eps, hc_eps, iters, post_mult, rms_eps)


def _head_without_rsqrt(R_bits, fn, scale, base, norm_eps=1e-6, hc_eps=1e-6):
    R = o.bf16_to_f64(R_bits)
    mixes = R.reshape(R.shape[0], -1) @ np.asarray(fn, dtype=np.float64).T
    pre = 1.0 / (1.0 + np.exp(-(mixes * np.asarray(scale).reshape(-1)[0] + base))) + hc_eps
    y = o.hc_combine(R_bits, pre)
    return y, o.f64_to_bf16(y)


def _split_sinkhorn_without_sinkhorn_eps(mixes, scale, base, hc=4, iters=20, eps=1e-6,
                                         post_mult=2.0):
    pre, post, logits = _real_split(mixes, scale, base, hc, eps, post_mult)
    return pre, post, _real_sinkhorn(logits, iters, 0.0)


def _stats_over_h(R_bits, fn, rms_eps=1e-6):
    """The RMS scale over one stream's width H instead of the flattened 4H."""
    R_bits = np.asarray(R_bits)
    H = R_bits.shape[-1]
    mixes, sumsq = _real_stats(R_bits, fn, rms_eps)
    s = np.asarray(sumsq, dtype=np.float64)[:, None]
    return mixes * np.sqrt(s / (4 * H) + rms_eps) / np.sqrt(s / H + rms_eps), sumsq


def _post_without_x(x_bits, R_bits, post, comb):
    """The post-weighted sublayer output term left out."""
    return _real_post(x_bits, R_bits, np.zeros_like(np.asarray(post, dtype=np.float64)), comb)


def _combine_norm_mean_over_4h(R_bits, pre, w_bits, eps=1e-6):
    """The RMSNorm mean taken over 4H columns instead of the combined row's H."""
    c = o.hc_combine(R_bits, pre)
    w = o.bf16_to_f64(w_bits)
    y = c / np.sqrt((c * c).sum(-1, keepdims=True) / (4 * c.shape[-1]) + eps) * w
    return y, o.f64_to_bf16(y)


_real_f64_to_bf16 = o.f64_to_bf16


def _f64_to_bf16_truncating(v):
    """Rounding toward zero instead of to nearest even."""
    v = np.asarray(v, dtype=np.float64)
    b = v.astype(np.float32).view(np.uint32) >> np.uint32(16)
    return np.where(np.isnan(v), np.uint16(0x7FC0), b.astype(np.uint16))


def _f64_to_bf16_through_float32(v):
    """Two roundings: float64 -> float32 -> bf16 (ties can land on the wrong side)."""
    return _real_f64_to_bf16(np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64))


def _split_pre_post_swapped(mixes, scale, base, hc=4, pre_eps=1e-6, post_mult=2.0):
    """pre read from the post group of the mixes and post from the pre group."""
    mixes = np.array(mixes, dtype=np.float64)
    base = np.array(base, dtype=np.float64)
    scale = np.array(scale, dtype=np.float64).reshape(-1)
    mixes[:, 0:4], mixes[:, 4:8] = mixes[:, 4:8].copy(), mixes[:, 0:4].copy()
    base[0:4], base[4:8] = base[4:8].copy(), base[0:4].copy()
    scale[0], scale[1] = scale[1], scale[0]
    return _real_split(mixes, scale, base, hc, pre_eps, post_mult)


def _e4m3_flush_subnormals(s):
    """Values below the smallest normal (2^-6) coded as zero."""
    s = np.asarray(s, dtype=np.float64)
    code = _real_e4m3(s)
    zero = np.where(np.signbit(s), 0x80, 0x00)
    return np.where(np.abs(s) < 2.0**-6, zero, code).astype(np.uint8)


_real_quant = o.mxfp8_quant_rows
_real_swizzle = o.swizzle_128x4


def _quant_block_16(y_bits, block=32):
    return _real_quant(y_bits, 16)


def _quant_scale_bias_128(y_bits, block=32):
    q, sf = _real_quant(y_bits, block)
    return q, (sf.astype(np.int64) + 1).astype(np.uint8)


def _e4m3_nan_on_overflow(s):
    """Overflow to the NaN code instead of saturating to +-448."""
    s = np.asarray(s, dtype=np.float64)
    code = _real_e4m3(np.clip(s, -448.0, 448.0))
    nan = 0x7F | np.where(np.signbit(s), 0x80, 0)
    return np.where(np.abs(s) > 448.0, nan, code).astype(np.uint8)


def _swizzle_inner_swapped(sf):
    """Inside a tile [m % 32][g % 4][(m % 128) // 32] instead of [m % 32][(m % 128) // 32][g % 4]."""
    sf = np.asarray(sf, dtype=np.uint8)
    M, G = sf.shape
    mt = (M + 127) // 128
    pad = np.zeros((mt * 128, G), dtype=np.uint8)
    pad[:M] = sf
    out = np.empty(mt * 128 * G, dtype=np.uint8)
    pos = 0
    for tm in range(mt):
        for tg in range(G // 4):
            for r32 in range(32):
                for c in range(4):
                    for r4 in range(4):
                        out[pos] = pad[tm * 128 + r4 * 32 + r32, tg * 4 + c]
                        pos += 1
    return out


def _scale_exp_floor(amax):
    amax = np.asarray(amax, dtype=np.float64)
    pos = amax > 0
    _, k = np.frexp(np.where(pos, amax, 1.0))
    return np.clip(np.where(pos, k - 1 - 8, -127), -127, 127).astype(np.int64)


def _run_all_pins():
    """Run every pin; return the names of those that failed."""
    failed = []
    calls = [
        ("sink_uniform", pins.test_sinkhorn_uniform_logits_fixed_point, ()),
        ("sink_scaling", pins.test_sinkhorn_matches_scaling_vector_form_round_for_round, ()),
        ("sink_cols", pins.test_sinkhorn_ends_on_columns, ()),
        ("sink_eps", pins.test_sinkhorn_eps_is_added_to_entries, ()),
        ("sink_perm", pins.test_sinkhorn_permutation_dominant, ()),
        ("split_zero", pins.test_split_with_zero_scale_is_sigmoid_of_base, ()),
        ("split_groups", pins.test_split_scales_go_to_their_groups, ()),
        ("post_perm", pins.test_post_identity_and_permutation_are_exact, ()),
        ("post_loops", pins.test_post_brute_force_loops, ()),
        ("cn_onehot", pins.test_combine_norm_one_hot_pre_is_rms_norm, (3,)),
        ("e4m3_torch", pins.test_e4m3_encode_matches_torch_cast_over_all_bf16_patterns, ()),
        ("mx_minimal", pins.test_mxfp8_scale_exponent_is_minimal_and_safe, ()),
        ("pre_zero_scale", pins.test_hc_pre_zero_scale_closed_form, ()),
        ("pre_two_streams", pins.test_hc_pre_two_streams_share_a_column, ()),
        ("split_sinkhorn_uniform", pins.test_split_sinkhorn_zero_scale_uniform_logits_closed_form, ()),
        ("post_only", pins.test_post_only_post_term, ()),
        ("bf16_torch", pins.test_bf16_rounding_matches_torch_on_float32_inputs, ()),
        ("bf16_single", pins.test_bf16_rounding_is_single_rounding_from_float64, ()),
        ("cn_zero", pins.test_combine_norm_zero_input_gives_zero, ()),
        ("e4m3_sat", pins.test_e4m3_saturates, ()),
        ("mx_block", pins.test_mxfp8_block_is_32_columns_wide, ()),
        ("swz_layout", pins.test_swizzle_128x4_places_every_byte_by_the_stated_layout, (130, 8)),
        ("swz_hand", pins.test_swizzle_128x4_hand_positions, ()),
    ]
    for i0, h0 in [(0, 0), (2, 5), (3, 7)]:
        calls.append((f"pre_onehot_{i0}_{h0}", pins.test_hc_pre_one_nonzero_row_closed_form, (i0, h0)))
    for i0, h0 in [(1, 3), (3, 0)]:
        calls.append((f"head_onehot_{i0}_{h0}", pins.test_hc_head_one_nonzero_row_closed_form, (i0, h0)))
    for case in pins._golden_sinkhorn():
        calls.append((f"sink_golden_{case[0]}", pins.test_sinkhorn_doubly_stochastic_rownorm_closed_form, (case,)))
    for sh in [(1, 3), (2, 5)]:
        calls.append((f"stats_onehot_{sh}", pins.test_stats_one_nonzero_closed_form, sh))
    for case in pins._golden_mx():
        calls.append((f"mx_hand_{case[2]!r}", pins.test_mxfp8_hand_cases, (case,)))
    for name, fn, args in calls:
        try:
            with np.errstate(all="ignore"):  # a planted mistake may divide by zero
                fn(*args)
        except AssertionError:
            failed.append(name)
    return failed


MUTANTS = [
    ("sinkhorn", _sinkhorn_row_last, "sink_"),
    ("sinkhorn", _sinkhorn_one_round_short, "sink_scaling"),
    ("sinkhorn", _sinkhorn_eps_only_in_denominators, "sink_eps"),
    ("sinkhorn", _sinkhorn_transposed, "sink_"),
    ("hc_mix_stats", _stats_h_major, "stats_onehot"),
    ("hc_mix_stats", _stats_no_eps, "stats_onehot"),
    ("hc_split", _split_no_post_mult, "split_"),
    ("hc_split", _split_pre_without_eps, "split_"),
    ("hc_combine_norm", _combine_norm_no_eps, "cn_onehot"),
    ("hc_post", _post_comb_transposed, "post_"),
    ("e4m3_encode", _e4m3_truncating, "e4m3_torch"),
    ("mxfp8_scale_exponent", _scale_exp_floor, "mx_"),
    ("hc_pre", _pre_combine_weighted_by_post, "pre_"),
    ("hc_pre", _pre_combine_streams_reversed, "pre_"),
    ("hc_pre", _pre_norm_takes_stats_eps, "pre_"),
    ("hc_head", _head_without_rsqrt, "head_onehot"),
    ("hc_split_sinkhorn", _split_sinkhorn_without_sinkhorn_eps, "split_sinkhorn"),
    ("hc_mix_stats", _stats_over_h, "stats_onehot"),
    ("hc_post", _post_without_x, "post_"),
    ("hc_combine_norm", _combine_norm_mean_over_4h, "cn_onehot"),
    ("mxfp8_quant_rows", _quant_block_16, "mx_block"),
    ("mxfp8_quant_rows", _quant_scale_bias_128, "mx_"),
    ("e4m3_encode", _e4m3_nan_on_overflow, "e4m3_sat"),
    ("swizzle_128x4", _swizzle_inner_swapped, "swz_"),
    ("f64_to_bf16", _f64_to_bf16_truncating, "bf16_"),
    ("f64_to_bf16", _f64_to_bf16_through_float32, "bf16_single"),
    ("hc_split", _split_pre_post_swapped, "split_"),
    ("e4m3_encode", _e4m3_flush_subnormals, "e4m3_torch"),
]


def test_unmutated_oracle_passes_every_pin():
    assert _run_all_pins() == []


@pytest.mark.parametrize("attr,mutant,expect", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, attr, mutant, expect):
    monkeypatch.setattr(o, attr, mutant)
    failed = _run_all_pins()
    assert any(f.startswith(expect) for f in failed), failed
