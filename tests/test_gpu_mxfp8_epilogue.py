"""MXFP8 written by the pre's own finish (the attention input of prefill_sp.py's stage 2,
quantised inside the combine + RMSNorm pass) and the 128x4 scale layout of swizzle_128x4.

The fused bytes must be exactly what the standalone quantizer gives for the bf16 y of the same
call, and what the oracle's MXFP8 gives for those bf16 bits; the swizzled scales must match
the oracle's layout byte for byte."""
import numpy as np
import pytest
import torch

from hyper_connection_residual_hc_amd import inputs, ops
from oracle import hc_oracle as o
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sites():
    return (gu.Site(inputs.SEED_ATTN, inputs.SEED_NORM_ATTN),
            gu.Site(inputs.SEED_FFN, inputs.SEED_NORM_FFN))


def _poison_u8(*shape):
    return torch.full(shape, 0xA5, dtype=torch.uint8, device=gu.DEV)


def _bits_equal(a, b):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    return torch.equal(a, b)


@pytest.mark.parametrize("M", [1, 65, 300, 4096])
def test_pre_mxfp8_equals_pre_then_quantizer(sites, M):
    attn, _ = sites
    gu.say(f"hc_pre_mxfp8 M={M}")
    R = gu.dev(inputs.residual(M, M + 21))
    y, post, comb, pre = ops.pre(R, attn.fnp, attn.scale_d, attn.base_d, attn.w_d, want_pre=True)
    q_ref, s_ref = ops.mxfp8_quant_rows(y)
    out = (None, _poison_u8(M, gu.H), _poison_u8(M, gu.H // 32),
           torch.empty_like(post), torch.empty_like(comb), torch.empty_like(pre))
    y2, q, sc, post2, comb2, pre2 = ops.pre_mxfp8(R, attn.fnp, attn.scale_d, attn.base_d,
                                                   attn.w_d, want_pre=True)
    assert _bits_equal(y2, y)
    assert torch.equal(q, q_ref) and torch.equal(sc, s_ref)
    assert torch.equal(post2, post) and torch.equal(comb2, comb) and torch.equal(pre2, pre)
    # without the bf16 form: same bytes
    _, q3, s3, post3, _, _ = ops.pre_mxfp8(R, attn.fnp, attn.scale_d, attn.base_d, attn.w_d,
                                           want_pre=True, out=out)
    assert torch.equal(q3, q_ref) and torch.equal(s3, s_ref) and torch.equal(post3, post)


@pytest.mark.parametrize("M", [63, 2112])
def test_post_pre_mxfp8_equals_post_pre_then_quantizer(sites, M):
    attn, ffn = sites
    gu.say(f"hc_post_pre_mxfp8 M={M}")
    R = gu.dev(inputs.residual(M, M + 31))
    x = gu.dev(inputs.sublayer_out(M, M + 32))
    _, post, comb, _ = ops.pre(R, attn.fnp, attn.scale_d, attn.base_d, attn.w_d)
    Rn, y, post2, comb2, _ = ops.post_pre(x, R, post, comb, ffn.fnp, ffn.scale_d, ffn.base_d,
                                          ffn.w_d)
    q_ref, s_ref = ops.mxfp8_quant_rows(y)
    Rm, (ym, qm, sm, postm, combm, _) = ops.post_pre_mxfp8(
        x, R, post, comb, ffn.fnp, ffn.scale_d, ffn.base_d, ffn.w_d)
    assert _bits_equal(Rm, Rn) and _bits_equal(ym, y)
    assert torch.equal(qm, q_ref) and torch.equal(sm, s_ref)
    assert torch.equal(postm, post2) and torch.equal(combm, comb2)
    # the two-call form with the MXFP8 finish and no bf16 y
    R3, ws = ops.post_stats(x, R, post, comb, ffn.fnp)
    _, q3, s3, _, _, _ = ops.pre_finish_mxfp8(R3, ws, ffn.scale_d, ffn.base_d, ffn.w_d,
                                             want_y=False)
    assert torch.equal(q3, q_ref) and torch.equal(s3, s_ref)


def test_pre_mxfp8_matches_oracle_on_the_gpu_y(sites):
    """The bytes are the oracle's MXFP8 of the bf16 y the same call writes (config 4 style
    rows: the first 64 columns of every stream x 40 drive some block maxima far up)."""
    attn, _ = sites
    M = 257
    R = gu.dev(inputs.residual(M, 4321))
    y, q, sc, _, _, _ = ops.pre_mxfp8(R, attn.fnp, attn.scale_d, attn.base_d, attn.w_d)
    oq, osc = o.mxfp8_quant_rows(gu.bits_of(y))
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(sc.cpu().numpy(), osc)
    # and y itself is the oracle's y to the bf16 bar
    ref = attn.oracle_pre(inputs.bits(inputs.residual(M, 4321)))
    gu.assert_bf16_close(gu.bits_of(y), ref["y"], "y")


def test_pre_mxfp8_row_slices_are_bit_identical(sites):
    attn, _ = sites
    M = 1500
    R = gu.dev(inputs.residual(M, M))
    full = ops.pre_mxfp8(R, attn.fnp, attn.scale_d, attn.base_d, attn.w_d)
    for lo, hi in [(0, 375), (375, 750), (1, 18), (63, 192), (M - 5, M)]:
        part = ops.pre_mxfp8(R[lo:hi], attn.fnp, attn.scale_d, attn.base_d, attn.w_d)
        for k in (0, 1, 2, 3, 4):
            assert _bits_equal(part[k], full[k][lo:hi]), (k, lo, hi)


@pytest.mark.parametrize("Hs,M", [(1024, 70), (1536, 50), (3072, 33), (4608, 21), (6144, 130), (8192, 17)])
def test_mxfp8_epilogue_at_other_widths(Hs, M):
    """The finish's MXFP8 epilogue compiled for other row widths (2 to 16 column blocks of 512
    per lane; 32 to 256 scale blocks per row): the fused pre and the fused post -> pre give
    the standalone quantizer's bytes of their own bf16 y, and those are the oracle's MXFP8 of
    that y."""
    gu.say(f"MXFP8 epilogue H={Hs} M={M}")
    site = gu.Site(41, 42, H_=Hs)
    nxt = gu.Site(43, 44, H_=Hs)
    R = gu.dev(inputs.residual(M, 45, H=Hs))
    x = gu.dev(inputs.sublayer_out(M, 46, H=Hs))
    y, post, comb, _ = ops.pre(R, site.fnp, site.scale_d, site.base_d, site.w_d)
    y2, q, sc, post2, comb2, _ = ops.pre_mxfp8(R, site.fnp, site.scale_d, site.base_d, site.w_d)
    assert _bits_equal(y2, y) and torch.equal(post2, post) and torch.equal(comb2, comb)
    q_ref, s_ref = ops.mxfp8_quant_rows(y)
    assert torch.equal(q, q_ref) and torch.equal(sc, s_ref)
    oq, osc = o.mxfp8_quant_rows(gu.bits_of(y))
    assert np.array_equal(q.cpu().numpy(), oq) and np.array_equal(sc.cpu().numpy(), osc)
    Rn, yn, _, _, _ = ops.post_pre(x, R, post, comb, nxt.fnp, nxt.scale_d, nxt.base_d, nxt.w_d)
    Rm, (ym, qm, sm, _, _, _) = ops.post_pre_mxfp8(x, R, post, comb, nxt.fnp, nxt.scale_d,
                                                   nxt.base_d, nxt.w_d)
    assert _bits_equal(Rm, Rn) and _bits_equal(ym, yn)
    oq2, osc2 = o.mxfp8_quant_rows(gu.bits_of(yn))
    assert np.array_equal(qm.cpu().numpy(), oq2) and np.array_equal(sm.cpu().numpy(), osc2)


def test_mxfp8_epilogue_argument_checks(sites):
    attn, _ = sites
    M = 8
    R = gu.dev(inputs.residual(M, 5))
    with pytest.raises(ValueError):  # q of the wrong width
        ops.pre_mxfp8(R, attn.fnp, attn.scale_d, attn.base_d, attn.w_d,
                      out=(None, _poison_u8(M, gu.H - 32), _poison_u8(M, gu.H // 32),
                           torch.empty(M, 4, device=gu.DEV), torch.empty(M, 4, 4, device=gu.DEV),
                           None))
    from hyper_connection_residual_hc_amd import _lib
    with pytest.raises(_lib.HCError) as ei:  # q overlapping the residual
        out = (None, R.reshape(M, -1).view(torch.uint8)[:, :gu.H], _poison_u8(M, gu.H // 32),
               torch.empty(M, 4, device=gu.DEV), torch.empty(M, 4, 4, device=gu.DEV), None)
        ops.pre_mxfp8(R, attn.fnp, attn.scale_d, attn.base_d, attn.w_d, out=out)
    assert ei.value.status_name == "HC_ERR_ALIAS"


@pytest.mark.parametrize("M,G", [(1, 160), (130, 160), (4096, 160), (300, 8)])
def test_swizzle_128x4_matches_oracle(M, G):
    gu.say(f"mxfp8_swizzle_128x4 M={M} G={G}")
    rng = np.random.default_rng(M + G)
    sc = rng.integers(0, 256, size=(M, G), dtype=np.uint8)
    out = ops.mxfp8_swizzle_128x4(gu.dev(torch.from_numpy(sc)))
    want = o.swizzle_128x4(sc) if M <= 300 else None
    got = out.cpu().numpy()
    if want is not None:
        assert np.array_equal(got, want)
    else:  # large M: every byte at the stated position (vectorised), padding zero
        m = np.arange(M)[:, None]
        g = np.arange(G)[None, :]
        pos = ((m // 128) * (G // 4) + g // 4) * 512 + (m % 32) * 16 + ((m % 128) // 32) * 4 + g % 4
        assert np.array_equal(got[pos], sc)
        mask = np.ones(got.shape, dtype=bool)
        mask[pos.ravel()] = False
        assert not got[mask].any()


def test_swizzle_of_strided_scales_and_of_gathered_shards(sites):
    """Shard-wise linear scales, concatenated, then swizzled == the swizzle of the full call's
    linear scales (prefill_sp.py: quantise each shard, gather, swizzle)."""
    attn, _ = sites
    M, W = 1500, 4
    R = gu.dev(inputs.residual(M, M))
    _, _, s_full, _, _, _ = ops.pre_mxfp8(R, attn.fnp, attn.scale_d, attn.base_d, attn.w_d,
                                          want_y=False)
    parts = [ops.pre_mxfp8(R[r * M // W:(r + 1) * M // W], attn.fnp, attn.scale_d, attn.base_d,
                           attn.w_d, want_y=False)[2] for r in range(W)]
    sw_full = ops.mxfp8_swizzle_128x4(s_full)
    sw_gath = ops.mxfp8_swizzle_128x4(torch.cat(parts))
    assert torch.equal(sw_full, sw_gath)
    # a strided view of wider scale rows
    wide = torch.zeros(M, 200, dtype=torch.uint8, device=gu.DEV)
    wide[:, :160] = s_full
    assert torch.equal(ops.mxfp8_swizzle_128x4(wide[:, :160]), sw_full)
    assert np.array_equal(sw_full.cpu().numpy(), o.swizzle_128x4(s_full.cpu().numpy()))
