"""hc_head (deepseek_v4.py, hc_head_torch: the model's last mix of the 4 streams) against the
oracle, its packed operands, row-slice invariance and the zero-scale case."""
import numpy as np
import pytest
import torch

from hyper_connection_residual_hc_amd import inputs, ops
from oracle import hc_oracle as o
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def head():
    fn, scale, base = inputs.hc_head_params(inputs.SEED_HEAD)
    return dict(fn=fn, scale=scale, base=base, fnp=ops.head_fn_pack(gu.dev(fn)),
                scale_d=gu.dev(scale), base_d=gu.dev(base))


def _oracle(hp, R_bits, scale=None):
    sc = hp["scale"].numpy() if scale is None else scale
    return o.hc_head(R_bits, hp["fn"].numpy(), sc, hp["base"].numpy())


def test_head_fn_pack_holds_four_rows(head):
    """Rows 0..3 of the packed layout reconstruct the head fn (hi + mid + lo); every other
    (row, part) slot is zero."""
    p = o.bf16_to_f64(head["fnp"].cpu().numpy().view(np.uint16))
    k_idx, S, NC = gu.packed_columns(gu.H)
    k_idx = k_idx.reshape(-1)
    p = p.reshape(S, 4, NC, 5, 4, 16, 8)  # s, q, c, t, g, n, e
    fn = head["fn"].numpy().astype(np.float64)
    recon = np.zeros_like(fn)
    for t in range(3):  # tiles 0..2 hold part t of fn rows 0..15 in lane column n
        for n in range(16):
            blk = p[:, :, :, t, :, n, :].reshape(-1)
            if n < 4:
                recon[n, k_idx] += blk
            else:
                assert not blk.any()
    assert not p[:, :, :, 3:].any()  # rows 16..23 and the padding
    np.testing.assert_allclose(recon, fn, rtol=2.0**-22, atol=0)


@pytest.mark.parametrize("M", [1, 65, 300])
def test_head_matches_oracle(head, M):
    gu.say(f"hc_head M={M}")
    R = inputs.residual(M, M + 55)
    y = ops.head(gu.dev(R), head["fnp"], head["scale_d"], head["base_d"])
    want, _ = _oracle(head, inputs.bits(R))
    gu.assert_bf16_close(gu.bits_of(y), want, "head y")


def test_head_full_size_every_row(head):
    """hc_head at M = 4096, H = 5120 (the launch of a full prefill step) against the oracle on
    all 4096 rows."""
    M = 4096
    gu.say(f"hc_head M={M} every row")
    R = inputs.residual(M, M)
    y = ops.head(gu.dev(R), head["fnp"], head["scale_d"], head["base_d"])
    want, _ = _oracle(head, inputs.bits(R))
    gu.assert_bf16_close(gu.bits_of(y), want, "head y")
    assert torch.isfinite(y.float()).all()


def test_head_zero_scale_and_slices(head):
    M = 1500
    R = gu.dev(inputs.residual(M, M))
    zero = torch.zeros(1, device=gu.DEV)
    y0 = ops.head(R, head["fnp"], zero, head["base_d"])
    want, _ = _oracle(head, inputs.bits(inputs.residual(M, M))[:64], scale=np.zeros(1))
    gu.assert_bf16_close(gu.bits_of(y0)[:64], want, "head y, scale 0")
    full = ops.head(R, head["fnp"], head["scale_d"], head["base_d"])
    for lo, hi in [(0, 375), (375, 750), (1, 18), (63, 192), (M - 5, M)]:
        part = ops.head(R[lo:hi], head["fnp"], head["scale_d"], head["base_d"])
        assert torch.equal(part.view(torch.int16), full[lo:hi].view(torch.int16)), (lo, hi)


@pytest.mark.parametrize("Hs,M", [(3072, 130), (6144, 70), (1024, 1100), (2560, 90), (7680, 40)])
def test_head_other_widths(Hs, M):
    """Other row widths against the oracle: 5 to 15 column blocks per lane in the head's
    finish, at H = 1024 8 slices of 128 columns per stream (32 blocks per slice running 2 or 3
    stages at 1100 rows), and the odd multiples 2560 and 7680 (NC = 10, 8 and 24 slices)."""
    gu.say(f"hc_head H={Hs} M={M}")
    fn, scale, base = inputs.hc_head_params(inputs.SEED_HEAD + 1, H=Hs)
    R = inputs.residual(M, M + 7, H=Hs)
    y = ops.head(gu.dev(R), ops.head_fn_pack(gu.dev(fn)), gu.dev(scale), gu.dev(base))
    want, _ = o.hc_head(inputs.bits(R), fn.numpy(), scale.numpy(), base.numpy())
    gu.assert_bf16_close(gu.bits_of(y), want, "head y")
