"""The tolerance helpers the GPU tests use, checked on the CPU against the oracle itself: the
bound for comparing the GPU's chain with the oracle's whole chain must cover what one bf16
rounding of R' can do to the next pre, and must not be vacuous."""
import numpy as np

from hyper_connection_residual_hc_amd import inputs
from oracle import hc_oracle as o
from tests import gpu_util as gu


def _one_ulp_apart(bits: np.ndarray, seed: int) -> np.ndarray:
    """Every bf16 element moved by one ulp in a random direction (away from zero where the
    magnitude is 0, so no pattern wraps into the sign or NaN range)."""
    rng = np.random.default_rng(seed)
    step = rng.choice(np.array([-1, 1], dtype=np.int32), size=bits.shape)
    step[(bits & 0x7FFF) == 0] = 1
    return (bits.astype(np.int32) + step).astype(np.uint16)


def test_chain_y_slack_covers_a_one_ulp_residual_shift():
    """Two pre calls on R' bits that differ by one ulp in every element (the worst case of
    two independent bf16 roundings of one R'): y stays within the bf16 bar plus chain_y_slack,
    the coefficients within the chain coefficient bar, and the slack is a small fraction of the
    row's rms (median under 2 %, so the comparison still has teeth)."""
    M = 128
    R = inputs.residual(M, 4107)
    x = inputs.sublayer_out(M, 4108)
    fa, sa, ba = inputs.hc_params(inputs.SEED_ATTN)
    wa = inputs.norm_weight(inputs.SEED_NORM_ATTN)
    ff, sff, bff = inputs.hc_params(inputs.SEED_FFN)
    wf = inputs.norm_weight(inputs.SEED_NORM_FFN)
    ref1 = o.hc_pre(inputs.bits(R), fa.numpy(), sa.numpy(), ba.numpy(), inputs.bits(wa))
    _, Rb = o.hc_post(inputs.bits(x), inputs.bits(R), ref1["post"], ref1["comb"])
    alt = _one_ulp_apart(Rb, 7)
    assert np.all(np.isfinite(o.bf16_to_f64(alt)))
    ra = o.hc_pre(Rb, ff.numpy(), sff.numpy(), bff.numpy(), inputs.bits(wf))
    rb = o.hc_pre(alt, ff.numpy(), sff.numpy(), bff.numpy(), inputs.bits(wf))
    for k in ("pre", "post", "comb"):
        assert np.abs(ra[k] - rb[k]).max() <= gu.CHAIN_COEF_ABS
    slack = gu.chain_y_slack(Rb, ra["pre"], wf)
    gu.assert_bf16_close(rb["y_bits"], ra["y"], "y one ulp of R' apart", extra=slack)
    # without the slack the plain bar does not hold: the slack is needed, not decoration
    g = o.bf16_to_f64(rb["y_bits"])
    rms = np.sqrt(np.mean(ra["y"] ** 2, axis=-1, keepdims=True))
    plain = gu.BF16_REL * np.abs(ra["y"]) + gu.BF16_ROW_ABS * rms
    assert (np.abs(g - ra["y"]) > plain).any()
    assert np.median(slack / rms) < 0.02
