"""Row-slice bit invariance: for every entry point, a call on rows [a, b) gives exactly the
bits of rows [a, b) of the full-M call (the key invariant of the row-sharded prefill path in
prefill_sp.py, checked there per kernel in test_prefill_sp_gpu.py's _kernels_at). Shards of
the configurations: M=2048 in 4 x 512 and M=1500 in 4 x 375, plus odd offsets."""
import pytest
import torch

from hyper_connection_residual_hc_amd import inputs, ops
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _eq(a, b):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    return torch.equal(a, b)


def _flip_one_bit(t: torch.Tensor) -> torch.Tensor:
    u = t.clone().view(torch.int16 if t.element_size() == 2 else torch.int32)
    u.view(-1)[u.numel() // 2] ^= 1
    return u.view(t.dtype)


@pytest.fixture(scope="module")
def attn():
    return gu.Site(inputs.SEED_ATTN, inputs.SEED_NORM_ATTN)


@pytest.mark.parametrize("M,W", [(2048, 4), (1500, 4)])
def test_row_slices_are_bit_identical(attn, M, W):
    gu.say(f"slice invariance M={M} W={W}")
    R = gu.dev(inputs.residual(M, M))
    x = gu.dev(inputs.sublayer_out(M, M + 1))
    full = {}
    full["pre"] = ops.pre(R, attn.fnp, attn.scale_d, attn.base_d, attn.w_d, want_pre=True)
    full["stats"] = ops.pre_stats(R, attn.fnp)
    y, post, comb, pre = full["pre"]
    mixes = full["stats"][0]
    full["sinkhorn"] = ops.sinkhorn(mixes, attn.scale_d, attn.base_d)
    full["combine"] = (ops.combine_norm(R, pre, attn.w_d),)
    full["post"] = (ops.post(x, R, post, comb),)
    full["mxfp8"] = ops.mxfp8_quant_rows(y)
    full["post_pre"] = ops.post_pre(x, R, post, comb, attn.fnp, attn.scale_d, attn.base_d,
                                    attn.w_d, want_pre=True)

    def run(lo, hi):
        sl = slice(lo, hi)
        return {
            "pre": ops.pre(R[sl], attn.fnp, attn.scale_d, attn.base_d, attn.w_d, want_pre=True),
            "stats": ops.pre_stats(R[sl], attn.fnp),
            "sinkhorn": ops.sinkhorn(mixes[sl], attn.scale_d, attn.base_d),
            "combine": (ops.combine_norm(R[sl], pre[sl], attn.w_d),),
            "post": (ops.post(x[sl], R[sl], post[sl], comb[sl]),),
            "mxfp8": ops.mxfp8_quant_rows(y[sl]),
            "post_pre": ops.post_pre(x[sl], R[sl], post[sl], comb[sl], attn.fnp, attn.scale_d,
                                     attn.base_d, attn.w_d, want_pre=True),
        }

    shards = [(r * M // W, (r + 1) * M // W) for r in range(W)]
    shards += [(1, 18), (63, 63 + 129), (M - 5, M), (375, 376)]
    for lo, hi in shards:
        got = run(lo, hi)
        for name, outs in got.items():
            for k, (g, f) in enumerate(zip(outs, full[name])):
                if g is None:
                    continue
                assert _eq(g, f[lo:hi]), f"{name}[{k}] differs on rows [{lo}, {hi})"

    # the comparison can see a single flipped bit (test of the test)
    assert not _eq(_flip_one_bit(full["pre"][0][:8]), full["pre"][0][:8])
    assert not _eq(_flip_one_bit(full["stats"][0][:8]), full["stats"][0][:8])
