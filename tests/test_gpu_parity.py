"""GPU parity of every C-ABI entry point against the CPU oracle, element by element, on seeded
inputs with the workload's distributions (several tiles plus a ragged tail), and the edge
cases: empty calls, single rows, zero rows, poisoned outputs, untouched inputs."""
import numpy as np
import pytest
import torch

from hyper_connection_residual_hc_amd import inputs, ops
from oracle import hc_oracle as o
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def attn():
    return gu.Site(inputs.SEED_ATTN, inputs.SEED_NORM_ATTN)


def _poison_f32(*shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device=gu.DEV)


def _poison_bf16(*shape):
    return torch.full(shape, -1, dtype=torch.int16, device=gu.DEV).view(torch.bfloat16)


# ------------------------------------------------------------------------------------------
def _pack_slot(t, n):
    """(fn row, part) carried by lane column n of packed tile t (part 0/1/2 = hi/mid/lo), as
    the packed layout documents it; (-1, 2) is padding."""
    if t < 3:
        return n, t
    if t == 3:
        return (16 + n, 0) if n < 8 else (8 + n, 1)
    return (16 + n, 2) if n < 8 else (-1, 2)


def test_fn_pack_reconstructs_fn(attn):
    """The packed hi/mid/lo parts sum back to fn within 2^-22 relative, every (row, part)
    appears exactly once, the padding is zero, and the parts decrease in magnitude."""
    gu.say("fn_pack H=5120 seed=11")
    p = o.bf16_to_f64(attn.fnp.cpu().numpy().view(np.uint16))
    k_idx, S, NC = gu.packed_columns(gu.H)
    p = p.reshape(S, 4, NC, 5, 4, 16, 8)  # s, q, c, t, g, n, e
    assert (S, NC) == (16, 10)
    fn = attn.fn.numpy().astype(np.float64)
    parts = np.zeros((3,) + fn.shape)
    seen = set()
    for t in range(5):
        for n in range(16):
            f, part = _pack_slot(t, n)
            blk = p[:, :, :, t, :, n, :]  # s, q, c, g, e
            if f < 0:
                assert np.all(blk == 0)
                continue
            assert (f, part) not in seen
            seen.add((f, part))
            parts[part, f, k_idx.reshape(-1)] = blk.reshape(-1)
    assert len(seen) == 72
    np.testing.assert_allclose(parts.sum(0), fn, rtol=2.0**-22, atol=0)
    assert np.all(np.abs(parts[1]) <= np.abs(fn) * 2.0**-8) and np.all(np.abs(parts[2]) <= np.abs(fn) * 2.0**-16)


@pytest.mark.parametrize("M", [128, 300, 1500])
def test_pre_stats_matches_oracle(attn, M):
    gu.say(f"hc_pre_stats M={M} seed={M}")
    R = inputs.residual(M, M)
    mixes, sumsq = ops.pre_stats(gu.dev(R), attn.fnp, mixes=_poison_f32(M, 24),
                                 sumsq=_poison_f32(M))
    om, osq = o.hc_mix_stats(inputs.bits(R), attn.fn.numpy())
    gu.assert_mixes_close(gu.f32_np(mixes), om)
    np.testing.assert_allclose(gu.f32_np(sumsq), osq, rtol=2e-6)


@pytest.mark.parametrize("M", [1, 77, 1024])
def test_sinkhorn_matches_oracle(attn, M):
    gu.say(f"hc_sinkhorn M={M}")
    R = inputs.residual(M, M + 7)
    om, _ = o.hc_mix_stats(inputs.bits(R), attn.fn.numpy())
    mixes32 = torch.from_numpy(om.astype(np.float32))
    pre, post, comb = ops.sinkhorn(gu.dev(mixes32), attn.scale_d, attn.base_d,
                                   out=(_poison_f32(M, 4), _poison_f32(M, 4), _poison_f32(M, 4, 4)))
    opre, opost, ocomb = o.hc_split_sinkhorn(mixes32.numpy(), attn.scale.numpy(), attn.base.numpy())
    gu.assert_coef_close(gu.f32_np(pre), opre, "pre")
    gu.assert_coef_close(gu.f32_np(post), opost, "post")
    gu.assert_coef_close(gu.f32_np(comb), ocomb, "comb")


ARG_SETS = [  # iters, rms_eps, pre_eps, sinkhorn_eps, post_mult, norm_eps
    (1, 1e-6, 1e-6, 1e-6, 2.0, 1e-6),
    (2, 1e-4, 1e-3, 1e-5, 1.5, 1e-5),
    (7, 0.0, 0.0, 0.0, 2.0, 1e-3),
    (50, 1e-6, 1e-6, 1e-2, 2.0, 1e-6),
]


def _oracle_pre_args(site, R_bits, iters, rms_eps, pre_eps, sk_eps, post_mult, norm_eps):
    mixes, _ = o.hc_mix_stats(R_bits, site.fn.numpy(), rms_eps)
    pre, post, logits = o.hc_split(mixes, site.scale.numpy(), site.base.numpy(), pre_eps=pre_eps,
                                   post_mult=post_mult)
    comb = o.sinkhorn(logits, iters, sk_eps)
    y, _ = o.hc_combine_norm(R_bits, pre, inputs.bits(site.w), norm_eps)
    return dict(mixes=mixes, pre=pre, post=post, comb=comb, y=y)


@pytest.mark.parametrize("args", ARG_SETS, ids=[f"iters{a[0]}" for a in ARG_SETS])
def test_non_default_arguments_match_oracle(attn, ffn, args):
    """Every argument the entry points take besides the tensors, away from the decoder layer's
    values: 1, 2, 7 and 50 Sinkhorn rounds, pre and Sinkhorn eps that differ (zero included),
    other rms / norm eps and post multipliers. hc_sinkhorn on the oracle's mixes, hc_pre, and
    the pre half of hc_post_pre (on the GPU's own R'), each against the oracle's stages called
    with the same values, M = 300 (19 row groups, the last one ragged)."""
    iters, rms_eps, pre_eps, sk_eps, post_mult, norm_eps = args
    M = 300
    gu.say(f"non-default arguments {args} M={M}")
    R = inputs.residual(M, 300 + iters)
    ref = _oracle_pre_args(attn, inputs.bits(R), *args)
    mixes32 = torch.from_numpy(ref["mixes"].astype(np.float32))
    pre, post, comb = ops.sinkhorn(gu.dev(mixes32), attn.scale_d, attn.base_d, iters=iters,
                                   pre_eps=pre_eps, sinkhorn_eps=sk_eps, post_mult=post_mult)
    # the oracle on the same fp32 mixes the kernel read
    opre, opost, ologits = o.hc_split(mixes32.numpy(), attn.scale.numpy(), attn.base.numpy(),
                                      pre_eps=pre_eps, post_mult=post_mult)
    gu.assert_coef_close(gu.f32_np(pre), opre, "sinkhorn pre")
    gu.assert_coef_close(gu.f32_np(post), opost, "sinkhorn post")
    gu.assert_coef_close(gu.f32_np(comb), o.sinkhorn(ologits, iters, sk_eps), "sinkhorn comb")
    kw = dict(rms_eps=rms_eps, pre_eps=pre_eps, sinkhorn_eps=sk_eps, iters=iters,
              post_mult=post_mult, norm_eps=norm_eps)
    y, post1, comb1, pre1 = ops.pre(gu.dev(R), attn.fnp, attn.scale_d, attn.base_d, attn.w_d,
                                    want_pre=True, **kw)
    for name, g in (("pre", pre1), ("post", post1), ("comb", comb1)):
        gu.assert_coef_close(gu.f32_np(g), ref[name], f"hc_pre {name}")
    gu.assert_bf16_close(gu.bits_of(y), ref["y"], "hc_pre y")
    x = inputs.sublayer_out(M, 301 + iters)
    Rn, y2, post2, comb2, pre2 = ops.post_pre(gu.dev(x), gu.dev(R), post1, comb1, ffn.fnp,
                                              ffn.scale_d, ffn.base_d, ffn.w_d, want_pre=True,
                                              **kw)
    oR, _ = o.hc_post(inputs.bits(x), inputs.bits(R), gu.f32_np(post1), gu.f32_np(comb1))
    gu.assert_bf16_close(gu.bits_of(Rn), oR, "hc_post_pre R'")
    ref2 = _oracle_pre_args(ffn, gu.bits_of(Rn), *args)
    for name, g in (("pre", pre2), ("post", post2), ("comb", comb2)):
        gu.assert_coef_close(gu.f32_np(g), ref2[name], f"hc_post_pre {name}")
    gu.assert_bf16_close(gu.bits_of(y2), ref2["y"], "hc_post_pre y")


@pytest.mark.parametrize("M", [1, 130, 1500])
def test_combine_norm_matches_oracle(attn, M):
    gu.say(f"hc_combine_norm M={M}")
    R = inputs.residual(M, M + 11)
    pre = torch.rand(M, 4, generator=torch.Generator().manual_seed(M)) + 1e-6
    y = ops.combine_norm(gu.dev(R), gu.dev(pre), attn.w_d, out=_poison_bf16(M, gu.H))
    oy, _ = o.hc_combine_norm(inputs.bits(R), pre.numpy(), inputs.bits(attn.w))
    gu.assert_bf16_close(gu.bits_of(y), oy, "y")


def test_combine_norm_strided_pre(attn):
    M = 64
    R = inputs.residual(M, 5)
    pre_wide = torch.rand(M, 8, generator=torch.Generator().manual_seed(3))
    y = ops.combine_norm(gu.dev(R), gu.dev(pre_wide)[:, 2:6], attn.w_d)
    oy, _ = o.hc_combine_norm(inputs.bits(R), pre_wide[:, 2:6].numpy(), inputs.bits(attn.w))
    gu.assert_bf16_close(gu.bits_of(y), oy, "y (strided pre)")


@pytest.mark.parametrize("M", [1, 333, 4096])
def test_post_matches_oracle(attn, M):
    """Config 2 at M=4096: post and comb from the config-0-style parameters on R."""
    gu.say(f"hc_post M={M} seed={M}")
    R = inputs.residual(M, M)
    x = inputs.sublayer_out(M, M + 1)
    ref = attn.oracle_pre(inputs.bits(R))
    post32 = torch.from_numpy(ref["post"].astype(np.float32))
    comb32 = torch.from_numpy(ref["comb"].astype(np.float32))
    out = ops.post(gu.dev(x), gu.dev(R), gu.dev(post32), gu.dev(comb32),
                   out=_poison_bf16(M, 4, gu.H))
    oR, _ = o.hc_post(inputs.bits(x), inputs.bits(R), post32.numpy(), comb32.numpy())
    gu.assert_bf16_close(gu.bits_of(out), oR, "R'")


@pytest.mark.parametrize("M", [128, 2048])
def test_fused_pre_matches_oracle_and_unfused(attn, M):
    """Config 0 (M=128) and config 1 (M=2048): the fused pre against the oracle, and bit for
    bit against the chain of the separate entry points."""
    gu.say(f"hc_pre fused M={M} seed={M}")
    R = inputs.residual(M, M)
    Rd = gu.dev(R)
    y, post, comb, pre = ops.pre(Rd, attn.fnp, attn.scale_d, attn.base_d, attn.w_d, want_pre=True,
                                 out=(_poison_bf16(M, gu.H), _poison_f32(M, 4),
                                      _poison_f32(M, 4, 4), _poison_f32(M, 4)))
    ref = attn.oracle_pre(inputs.bits(R))
    gu.assert_coef_close(gu.f32_np(pre), ref["pre"], "pre")
    gu.assert_coef_close(gu.f32_np(post), ref["post"], "post")
    gu.assert_coef_close(gu.f32_np(comb), ref["comb"], "comb")
    gu.assert_bf16_close(gu.bits_of(y), ref["y"], "y")
    # separate entry points give the same bits
    mixes, _ = ops.pre_stats(Rd, attn.fnp)
    pre2, post2, comb2 = ops.sinkhorn(mixes, attn.scale_d, attn.base_d)
    y2 = ops.combine_norm(Rd, pre2, attn.w_d)
    assert torch.equal(pre, pre2) and torch.equal(post, post2) and torch.equal(comb, comb2)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_sinkhorn_outputs_are_column_stochastic(attn):
    M = 512
    R = inputs.residual(M, 99)
    _, _, comb, _ = ops.pre(gu.dev(R), attn.fnp, attn.scale_d, attn.base_d, attn.w_d)
    col = comb.double().sum(dim=1)
    assert torch.all((col - 1).abs() < 1e-5)
    assert torch.all(comb > 0)


# ------------------------------------------------------------------------------------------
# edge cases
# ------------------------------------------------------------------------------------------
def test_empty_calls_are_noops(attn):
    R = torch.empty(0, 4, gu.H, dtype=torch.bfloat16, device=gu.DEV)
    y, post, comb, _ = ops.pre(R, attn.fnp, attn.scale_d, attn.base_d, attn.w_d)
    assert y.shape == (0, gu.H) and post.shape == (0, 4) and comb.shape == (0, 4, 4)
    out = ops.post(torch.empty(0, gu.H, dtype=torch.bfloat16, device=gu.DEV), R,
                   torch.empty(0, 4, device=gu.DEV), torch.empty(0, 4, 4, device=gu.DEV))
    assert out.shape == (0, 4, gu.H)
    q, s = ops.mxfp8_quant_rows(torch.empty(0, gu.H, dtype=torch.bfloat16, device=gu.DEV))
    assert q.shape == (0, gu.H) and s.shape == (0, gu.H // 32)
    torch.cuda.synchronize()


def test_zero_rows(attn):
    """An all-zero residual row: mixes 0, so pre/post/comb come from base alone and y = 0."""
    M = 20
    R = inputs.residual(M, 31)
    R[3] = 0
    R[17] = 0
    y, post, comb, pre = ops.pre(gu.dev(R), attn.fnp, attn.scale_d, attn.base_d, attn.w_d,
                                 want_pre=True)
    ref = attn.oracle_pre(inputs.bits(R))
    assert np.all(ref["mixes"][[3, 17]] == 0)
    gu.assert_coef_close(gu.f32_np(pre), ref["pre"], "pre")
    gu.assert_coef_close(gu.f32_np(comb), ref["comb"], "comb")
    yb = gu.bits_of(y)
    assert np.all((yb[[3, 17]] & 0x7FFF) == 0)
    gu.assert_bf16_close(yb, ref["y"], "y")


def test_inputs_are_not_modified(attn):
    M = 257
    R = gu.dev(inputs.residual(M, 41))
    x = gu.dev(inputs.sublayer_out(M, 42))
    R0, x0 = R.clone(), x.clone()
    fnp0 = attn.fnp.clone()
    y, post, comb, _ = ops.pre(R, attn.fnp, attn.scale_d, attn.base_d, attn.w_d)
    ops.post(x, R, post, comb)
    ops.mxfp8_quant_rows(y)
    torch.cuda.synchronize()
    assert torch.equal(R.view(torch.int16), R0.view(torch.int16))
    assert torch.equal(x.view(torch.int16), x0.view(torch.int16))
    assert torch.equal(attn.fnp, fnp0)


def test_error_codes_reach_python(attn):
    from hyper_connection_residual_hc_amd._lib import HCError
    R = gu.dev(inputs.residual(8, 1))
    with pytest.raises(HCError, match="HC_ERR_ALIAS"):
        ops.combine_norm(R, gu.dev(torch.rand(8, 4)), attn.w_d,
                         out=R.view(8, -1)[:, : gu.H])
    raw = torch.empty(8 * 4 * gu.H + 8, dtype=torch.bfloat16, device=gu.DEV)
    Rmis = raw[1:1 + 8 * 4 * gu.H].view(8, 4, gu.H)  # 2-byte offset: not 16-byte aligned
    with pytest.raises(HCError, match="HC_ERR_ALIGN"):
        ops.combine_norm(Rmis, gu.dev(torch.rand(8, 4)), attn.w_d)
    with pytest.raises(HCError, match="HC_ERR_SHAPE"):
        ops.post(gu.dev(inputs.sublayer_out(2, 1, H=640)), gu.dev(inputs.residual(2, 1, H=640)),
                 gu.dev(torch.rand(2, 4)), gu.dev(torch.rand(2, 4, 4)))


def test_small_hidden_size():
    """H = 1024: 8 stats slices of 128 columns per stream (one 1 KB stage per slice row)
    and two column blocks per lane in the combine and post kernels."""
    Hs = 1024
    site = gu.Site(5, 6, H_=Hs)
    M = 70
    R = inputs.residual(M, 8, H=Hs)
    y, post, comb, pre = ops.pre(gu.dev(R), site.fnp, site.scale_d, site.base_d, site.w_d,
                                 want_pre=True)
    ref = site.oracle_pre(inputs.bits(R))
    gu.assert_coef_close(gu.f32_np(comb), ref["comb"], "comb")
    gu.assert_bf16_close(gu.bits_of(y), ref["y"], "y")
    x = inputs.sublayer_out(M, 9, H=Hs)
    post32 = torch.from_numpy(ref["post"].astype(np.float32))
    comb32 = torch.from_numpy(ref["comb"].astype(np.float32))
    out = ops.post(gu.dev(x), gu.dev(R), gu.dev(post32), gu.dev(comb32))
    oR, _ = o.hc_post(inputs.bits(x), inputs.bits(R), post32.numpy(), comb32.numpy())
    gu.assert_bf16_close(gu.bits_of(out), oR, "R'")


# ------------------------------------------------------------------------------------------
# fused post -> pre (hc_post_pre)
# ------------------------------------------------------------------------------------------
@pytest.fixture(scope="module")
def ffn():
    return gu.Site(inputs.SEED_FFN, inputs.SEED_NORM_FFN)


@pytest.mark.parametrize("M", [1, 63, 65, 300, 2112, 4096, 6144])
def test_fused_post_pre_equals_post_then_pre(attn, ffn, M):
    """hc_post_pre gives the bits of hc_post followed by hc_pre on its output. M covers one
    partial tile, tile edges, fewer tiles than blocks, and more tiles than blocks (2112 rows =
    33 tiles: one block per slice takes a tile pair, the others a lone tile; 6144 rows = 96
    tiles: three per block on 256 CUs, a pair then a lone tile)."""
    gu.say(f"hc_post_pre fused M={M}")
    R = gu.dev(inputs.residual(M, M + 5))
    x = gu.dev(inputs.sublayer_out(M, M + 6))
    _, post, comb, _ = ops.pre(R, attn.fnp, attn.scale_d, attn.base_d, attn.w_d)
    Rn, y, post2, comb2, pre2 = ops.post_pre(
        x, R, post, comb, ffn.fnp, ffn.scale_d, ffn.base_d, ffn.w_d, want_pre=True,
        out=(_poison_bf16(M, 4, gu.H), _poison_bf16(M, gu.H), _poison_f32(M, 4),
             _poison_f32(M, 4, 4), _poison_f32(M, 4)))
    Rn_ref = ops.post(x, R, post, comb)
    y_ref, post_ref, comb_ref, pre_ref = ops.pre(Rn_ref, ffn.fnp, ffn.scale_d, ffn.base_d,
                                                 ffn.w_d, want_pre=True)
    assert torch.equal(Rn.view(torch.int16), Rn_ref.view(torch.int16))
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    assert torch.equal(post2, post_ref) and torch.equal(comb2, comb_ref) and torch.equal(pre2, pre_ref)


def test_fused_post_pre_matches_oracle(attn, ffn):
    """Config 3 (M = 1500) through the fused op, against the oracle's own chain."""
    M = 1500
    gu.say(f"hc_post_pre vs oracle M={M}")
    R = inputs.residual(M, M)
    x = inputs.sublayer_out(M, M + 1)
    ref1 = attn.oracle_pre(inputs.bits(R))
    post32 = torch.from_numpy(ref1["post"].astype(np.float32))
    comb32 = torch.from_numpy(ref1["comb"].astype(np.float32))
    Rn, y, post2, comb2, pre2 = ops.post_pre(gu.dev(x), gu.dev(R), gu.dev(post32), gu.dev(comb32),
                                             ffn.fnp, ffn.scale_d, ffn.base_d, ffn.w_d,
                                             want_pre=True)
    oR1, oR1_bits = o.hc_post(inputs.bits(x), inputs.bits(R), post32.numpy(), comb32.numpy())
    gu.assert_bf16_close(gu.bits_of(Rn), oR1, "R'")
    # the pre half on the GPU's own R' bits: per-stage bars (coefficients 1e-5)
    ref2g = ffn.oracle_pre(gu.bits_of(Rn))
    gu.assert_bf16_close(gu.bits_of(y), ref2g["y"], "y ffn")
    for name, g in (("pre", pre2), ("post", post2), ("comb", comb2)):
        gu.assert_coef_close(gu.f32_np(g), ref2g[name], f"{name} ffn")
    # and against the oracle's whole chain (its own R'), one bf16 rounding of R' apart
    ref2 = ffn.oracle_pre(oR1_bits)
    gu.assert_bf16_close(gu.bits_of(y), ref2["y"], "y ffn (oracle chain)",
                         extra=gu.chain_y_slack(oR1_bits, ref2["pre"], ffn.w))
    for name, g in (("pre", pre2), ("post", post2), ("comb", comb2)):
        err = np.abs(gu.f32_np(g) - ref2[name]).max()
        assert err <= gu.CHAIN_COEF_ABS, f"{name} ffn (oracle chain): {err}"


@pytest.mark.parametrize("M", [65, 4096])
def test_post_stats_then_pre_finish_equals_post_pre(attn, ffn, M):
    """The two-call form gives the bits of hc_post_pre, also with unrelated work on the stream
    between the halves (here: an hc_post of other rows into another buffer)."""
    gu.say(f"hc_post_stats + hc_pre_finish M={M}")
    R = gu.dev(inputs.residual(M, M + 7))
    x = gu.dev(inputs.sublayer_out(M, M + 8))
    _, post, comb, _ = ops.pre(R, attn.fnp, attn.scale_d, attn.base_d, attn.w_d)
    full = ops.post_pre(x, R, post, comb, ffn.fnp, ffn.scale_d, ffn.base_d, ffn.w_d,
                        want_pre=True)
    Rn, ws = ops.post_stats(x, R, post, comb, ffn.fnp, out=_poison_bf16(M, 4, gu.H))
    other = ops.post(x, R, post, comb)
    y, post2, comb2, pre2 = ops.pre_finish(Rn, ws, ffn.scale_d, ffn.base_d, ffn.w_d,
                                           want_pre=True,
                                           out=(_poison_bf16(M, gu.H), _poison_f32(M, 4),
                                                _poison_f32(M, 4, 4), _poison_f32(M, 4)))
    assert torch.equal(Rn.view(torch.int16), full[0].view(torch.int16))
    assert torch.equal(other.view(torch.int16), full[0].view(torch.int16))
    assert torch.equal(y.view(torch.int16), full[1].view(torch.int16))
    assert torch.equal(post2, full[2]) and torch.equal(comb2, full[3]) and torch.equal(pre2, full[4])


def test_binding_rejects_short_outputs(attn, ffn):
    """The binding checks every output's shape against the inputs before the call (the C ABI
    receives bare pointers and cannot)."""
    M = 64
    R = gu.dev(inputs.residual(M, 3))
    x = gu.dev(inputs.sublayer_out(M, 4))
    _, post, comb, _ = ops.pre(R, attn.fnp, attn.scale_d, attn.base_d, attn.w_d)
    short_y = torch.empty(M - 1, gu.H, dtype=torch.bfloat16, device=R.device)
    with pytest.raises(ValueError):
        ops.pre(R, attn.fnp, attn.scale_d, attn.base_d, attn.w_d,
                out=(short_y, post.clone(), comb.clone(), None))
    with pytest.raises(ValueError):
        ops.post(x, R, post, comb, out=torch.empty(M - 1, 4, gu.H, dtype=torch.bfloat16,
                                                   device=R.device))
    with pytest.raises(ValueError):
        ops.combine_norm(R, post, attn.w_d, out=short_y)
    with pytest.raises(ValueError):
        ops.pre_stats(R, attn.fnp[:-8])
    with pytest.raises(ValueError):  # a host workspace would be a bad device pointer
        ops.pre(R, attn.fnp, attn.scale_d, attn.base_d, attn.w_d,
                workspace=torch.empty(ops.pre_workspace_bytes(M, gu.H), dtype=torch.uint8))
    with pytest.raises(ValueError):  # so would a host weight
        ops.combine_norm(R, post, attn.w_d.cpu())
    R1, ws = ops.post_stats(x, R, post, comb, ffn.fnp)
    spread = torch.empty(2 * ws.numel(), dtype=torch.uint8, device=R.device)
    with pytest.raises(ValueError):  # a strided workspace: its byte count is not its extent
        ops.pre_finish(R1, spread[::2], ffn.scale_d, ffn.base_d, ffn.w_d)
    with pytest.raises(ValueError):
        ops.pre_finish_mxfp8(R1, spread[::2], ffn.scale_d, ffn.base_d, ffn.w_d)


@pytest.mark.parametrize("Hs", [512, 1536, 2048, 2560, 3072, 3584, 4096, 4608, 6144, 7168, 7680, 8192])
def test_wider_hidden_sizes(Hs):
    """Other row widths: 1 to 16 column blocks of 512 per lane in the finish, and every stats
    geometry: 8 to 32 column slices of 64 (NC = 2, H = 512) to 320 (NC = 10) columns per
    stream, the odd multiples of 512 included. The pre and the post vs the oracle, the fused op
    vs post then pre."""
    gu.say(f"H={Hs}")
    site = gu.Site(15, 16, H_=Hs)
    nxt = gu.Site(17, 18, H_=Hs)
    M = 130
    R = inputs.residual(M, 19, H=Hs)
    y, post, comb, pre = ops.pre(gu.dev(R), site.fnp, site.scale_d, site.base_d, site.w_d,
                                 want_pre=True)
    ref = site.oracle_pre(inputs.bits(R))
    gu.assert_mixes_close(gu.f32_np(ops.pre_stats(gu.dev(R), site.fnp)[0]), ref["mixes"])
    gu.assert_coef_close(gu.f32_np(comb), ref["comb"], "comb")
    gu.assert_bf16_close(gu.bits_of(y), ref["y"], "y")
    x = gu.dev(inputs.sublayer_out(M, 20, H=Hs))
    Rd = gu.dev(R)
    full = ops.post_pre(x, Rd, post, comb, nxt.fnp, nxt.scale_d, nxt.base_d, nxt.w_d)
    Rn = ops.post(x, Rd, post, comb)
    y2, post2, comb2, _ = ops.pre(Rn, nxt.fnp, nxt.scale_d, nxt.base_d, nxt.w_d)
    assert torch.equal(full[0].view(torch.int16), Rn.view(torch.int16))
    assert torch.equal(full[1].view(torch.int16), y2.view(torch.int16))
    assert torch.equal(full[2], post2) and torch.equal(full[3], comb2)
    oR, oR_bits = o.hc_post(inputs.bits(x.cpu()), inputs.bits(R), gu.f32_np(post), gu.f32_np(comb))
    gu.assert_bf16_close(gu.bits_of(Rn), oR, "R'")
    ref2 = nxt.oracle_pre(gu.bits_of(Rn))
    gu.assert_coef_close(gu.f32_np(comb2), ref2["comb"], "comb (next site)")
    gu.assert_bf16_close(gu.bits_of(y2), ref2["y"], "y (next site)")


@pytest.mark.parametrize("Hs", [512, 1536, 2560, 3584, 4608, 5632, 6656, 7680])
def test_combine_norm_and_post_at_odd_block_counts(Hs):
    """Row widths that are odd multiples of 512 (1 to 15 column blocks per lane): the combine +
    norm and the post vs the oracle, on rows with a ragged tail of waves. The mix stats take
    all of them but 5632 and 6656, whose fn the binding refuses to pack."""
    gu.say(f"combine_norm / post H={Hs}")
    M = 37
    R = inputs.residual(M, 30, H=Hs)
    x = inputs.sublayer_out(M, 31, H=Hs)
    w = inputs.norm_weight(32, H=Hs)
    rng = np.random.default_rng(Hs)
    pre = torch.from_numpy(rng.random((M, 4)).astype(np.float32) + 1e-6)
    post = torch.from_numpy((2 * rng.random((M, 4))).astype(np.float32))
    comb = torch.from_numpy(rng.dirichlet(np.ones(4), size=(M, 4)).astype(np.float32))
    y = ops.combine_norm(gu.dev(R), gu.dev(pre), gu.dev(w))
    oy, _ = o.hc_combine_norm(inputs.bits(R), pre.numpy(), inputs.bits(w))
    gu.assert_bf16_close(gu.bits_of(y), oy, "y")
    Rn = ops.post(gu.dev(x), gu.dev(R), gu.dev(post), gu.dev(comb))
    oR, _ = o.hc_post(inputs.bits(x), inputs.bits(R), post.numpy(), comb.numpy())
    gu.assert_bf16_close(gu.bits_of(Rn), oR, "R'")
    if Hs in (5632, 6656):
        with pytest.raises(ValueError):
            ops.fn_pack(gu.dev(inputs.hc_params(1, H=Hs)[0]))


def test_narrow_hidden_size_two_stages_per_slice():
    """H = 1024, a narrow width with mix stats: 8 column slices of 128 columns per stream
    (NC = 4, one full wave-wide item per array and producer wave), 32 blocks per slice. At
    M = 6161 (386 row groups, the last one ragged) the blocks run 12 or 13 stages each: the pre
    vs the oracle on sampled rows, and the fused op vs post then pre, bit for bit."""
    Hs, M = 1024, 6161
    gu.say(f"H={Hs} M={M}")
    site = gu.Site(21, 22, H_=Hs)
    nxt = gu.Site(23, 24, H_=Hs)
    R = inputs.residual(M, 25, H=Hs)
    Rd = gu.dev(R)
    y, post, comb, pre = ops.pre(Rd, site.fnp, site.scale_d, site.base_d, site.w_d,
                                 want_pre=True)
    rng = np.random.default_rng(6161)
    rows = np.unique(np.concatenate([np.arange(70), np.arange(M - 70, M),
                                     rng.choice(M, 200, replace=False)]))
    ref = site.oracle_pre(inputs.bits(R)[rows])
    ridx = torch.from_numpy(rows).to(gu.DEV)
    gu.assert_coef_close(gu.f32_np(comb[ridx]), ref["comb"], "comb")
    gu.assert_coef_close(gu.f32_np(pre[ridx]), ref["pre"], "pre")
    gu.assert_bf16_close(gu.bits_of(y[ridx]), ref["y"], "y")
    x = gu.dev(inputs.sublayer_out(M, 26, H=Hs))
    full = ops.post_pre(x, Rd, post, comb, nxt.fnp, nxt.scale_d, nxt.base_d, nxt.w_d)
    Rn = ops.post(x, Rd, post, comb)
    y2, post2, comb2, _ = ops.pre(Rn, nxt.fnp, nxt.scale_d, nxt.base_d, nxt.w_d)
    assert torch.equal(full[0].view(torch.int16), Rn.view(torch.int16))
    assert torch.equal(full[1].view(torch.int16), y2.view(torch.int16))
    assert torch.equal(full[2], post2) and torch.equal(full[3], comb2)


def test_widest_hidden_size_many_stages():
    """H = 8192, the widest width with mix stats: 32 column slices of 256 columns per stream,
    8 blocks per slice. At M = 2500 (157 row groups, the last one of 4 rows) every block runs
    19 or 20 stages: the fused op vs post then pre bit for bit, and the pre and the post vs the
    oracle on sampled rows (every group's edges at both ends, random rows)."""
    Hs, M = 8192, 2500
    gu.say(f"H={Hs} M={M}")
    site = gu.Site(51, 52, H_=Hs)
    nxt = gu.Site(53, 54, H_=Hs)
    R = inputs.residual(M, 55, H=Hs)
    x = inputs.sublayer_out(M, 56, H=Hs)
    Rd, xd = gu.dev(R), gu.dev(x)
    y, post, comb, pre = ops.pre(Rd, site.fnp, site.scale_d, site.base_d, site.w_d,
                                 want_pre=True)
    full = ops.post_pre(xd, Rd, post, comb, nxt.fnp, nxt.scale_d, nxt.base_d, nxt.w_d)
    Rn = ops.post(xd, Rd, post, comb)
    y2, post2, comb2, _ = ops.pre(Rn, nxt.fnp, nxt.scale_d, nxt.base_d, nxt.w_d)
    assert torch.equal(full[0].view(torch.int16), Rn.view(torch.int16))
    assert torch.equal(full[1].view(torch.int16), y2.view(torch.int16))
    assert torch.equal(full[2], post2) and torch.equal(full[3], comb2)
    rng = np.random.default_rng(8192)
    rows = np.unique(np.concatenate([np.arange(0, 160, 16), np.arange(15, 160, 16),
                                     np.arange(M - 40, M), rng.choice(M, 60, replace=False)]))
    ridx = torch.from_numpy(rows).to(gu.DEV)
    ref = site.oracle_pre(inputs.bits(R)[rows])
    gu.assert_coef_close(gu.f32_np(pre[ridx]), ref["pre"], "pre")
    gu.assert_coef_close(gu.f32_np(comb[ridx]), ref["comb"], "comb")
    gu.assert_bf16_close(gu.bits_of(y[ridx]), ref["y"], "y")
    oR, _ = o.hc_post(inputs.bits(x)[rows], inputs.bits(R)[rows], gu.f32_np(post)[rows],
                      gu.f32_np(comb)[rows])
    gu.assert_bf16_close(gu.bits_of(Rn[ridx]), oR, "R'")
    ref2 = nxt.oracle_pre(gu.bits_of(Rn[ridx]))
    gu.assert_coef_close(gu.f32_np(comb2[ridx]), ref2["comb"], "comb (next site)")
    gu.assert_coef_close(gu.f32_np(post2[ridx]), ref2["post"], "post (next site)")
    gu.assert_bf16_close(gu.bits_of(y2[ridx]), ref2["y"], "y (next site)")


def test_graph_capture_replays_match_eager(attn, ffn):
    """The fused step captured in a HIP graph (the entry points allocate nothing and clear no
    memory, so they capture as plain kernel nodes): three replays, with unrelated eager work
    and a synchronisation between them, each give the eager result."""
    M = 1024
    R = gu.dev(inputs.residual(M, 31))
    x = gu.dev(inputs.sublayer_out(M, 32))
    _, post, comb, _ = ops.pre(R, attn.fnp, attn.scale_d, attn.base_d, attn.w_d)
    outs = (torch.empty_like(R), torch.empty(M, gu.H, dtype=torch.bfloat16, device=gu.DEV),
            torch.empty(M, 4, device=gu.DEV), torch.empty(M, 4, 4, device=gu.DEV), None)
    ws = torch.empty(ops.post_pre_workspace_bytes(M, gu.H), dtype=torch.uint8, device=gu.DEV)

    def step():
        ops.post_pre(x, R, post, comb, ffn.fnp, ffn.scale_d, ffn.base_d, ffn.w_d, out=outs,
                     workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs[:4]]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = gu.dev(inputs.residual(M, 33))
    for rep in range(3):
        for t in outs[:4]:
            t.view(torch.uint8).fill_(0xA5)
        ops.post(x, other, post, comb)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(outs[:4], ref)):
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), (rep, k)



def _wide_bf16(M, inner, pad):
    """(whole [M, inner + pad] buffer filled with -7, the [M, inner] view of its row heads)."""
    b = torch.full((M, inner + pad), -7.0, dtype=torch.bfloat16, device=gu.DEV)
    return b, b[:, :inner]


def test_padded_row_strides_fused_and_separate(attn, ffn):
    """Every bf16 row argument of hc_pre, hc_post and hc_post_pre as a view into wider rows
    (a different pad for each), at a size where the stats blocks run 16 or 17 stages of 16 rows
    and the last group is ragged (M = 4177: 261 full groups and one row): the same bits as the
    contiguous calls, and no pad byte written."""
    M, H = 4177, gu.H
    gu.say(f"padded strides M={M}")
    R = gu.dev(inputs.residual(M, 91))
    x = gu.dev(inputs.sublayer_out(M, 92))
    y_c, post_c, comb_c, _ = ops.pre(R, attn.fnp, attn.scale_d, attn.base_d, attn.w_d)
    ref_post = ops.post(x, R, post_c, comb_c)
    ref = ops.post_pre(x, R, post_c, comb_c, ffn.fnp, ffn.scale_d, ffn.base_d, ffn.w_d)

    Rb, Rv = _wide_bf16(M, 4 * H, 512)
    Rv.copy_(R.reshape(M, 4 * H))
    Rs = Rv.view(M, 4, H)
    xb, xs = _wide_bf16(M, H, 64)
    xs.copy_(x)
    Rb0, xb0 = Rb.clone(), xb.clone()

    yb, ys = _wide_bf16(M, H, 128)
    y2, post2, comb2, _ = ops.pre(Rs, attn.fnp, attn.scale_d, attn.base_d, attn.w_d,
                                  out=(ys, _poison_f32(M, 4), _poison_f32(M, 4, 4), None))
    assert torch.equal(y2, y_c) and torch.equal(post2, post_c) and torch.equal(comb2, comb_c)
    assert bool((yb[:, H:] == -7.0).all())

    ob, ov = _wide_bf16(M, 4 * H, 256)
    assert torch.equal(ops.post(xs, Rs, post_c, comb_c, out=ov.view(M, 4, H)), ref_post)
    assert bool((ob[:, 4 * H:] == -7.0).all())

    Rnb, Rnv = _wide_bf16(M, 4 * H, 1024)
    ynb, ynv = _wide_bf16(M, H, 32)
    got = ops.post_pre(xs, Rs, post_c, comb_c, ffn.fnp, ffn.scale_d, ffn.base_d, ffn.w_d,
                       out=(Rnv.view(M, 4, H), ynv, _poison_f32(M, 4), _poison_f32(M, 4, 4),
                            None))
    for a, b, what in zip(got[:4], ref[:4], ("R'", "y", "post", "comb")):
        assert torch.equal(a, b), what
    assert bool((Rnb[:, 4 * H:] == -7.0).all()) and bool((ynb[:, H:] == -7.0).all())
    assert torch.equal(Rb, Rb0) and torch.equal(xb, xb0)  # inputs, pads included, untouched


def test_rows_past_32_bit_offsets(attn, ffn):
    """M = 131072 rows at H = 5120: R takes 5.4 GB, so row offsets pass 2^31 bytes (from row
    52429) and 2^31 elements (from row 104858). The batch is 32 copies of one seeded 4096-row
    block, copy k rolled by 37 k rows, so an address that wraps or truncates reads a row other
    than the one its output stands for. Every entry point's outputs for copy k must equal those
    of the block alone rolled the same way, bit for bit: the fused step, post then pre, the
    MXFP8 form with the quantizer, and the head. (The block's own parity with the oracle is the
    full-size test below.)"""
    B, K = 4096, 32
    M = B * K
    assert M * 4 * gu.H > 2**31
    gu.say(f"rows past 32-bit offsets M={M}")
    shifts = [37 * k for k in range(K)]

    def tile(t):
        return torch.cat([torch.roll(t, sh, dims=0) for sh in shifts])

    def check(big, small, what):
        if big.dtype == torch.bfloat16:
            big, small = big.view(torch.int16), small.view(torch.int16)
        for k, sh in enumerate(shifts):
            assert torch.equal(big[k * B:(k + 1) * B], torch.roll(small, sh, dims=0)), \
                f"{what}: copy {k} (rows {k * B}..{(k + 1) * B - 1})"

    R0 = gu.dev(inputs.residual(B, 4096 + 11))
    x0 = gu.dev(inputs.sublayer_out(B, 4096 + 12))
    _, p0, c0, _ = ops.pre(R0, attn.fnp, attn.scale_d, attn.base_d, attn.w_d)
    small = ops.post_pre(x0, R0, p0, c0, ffn.fnp, ffn.scale_d, ffn.base_d, ffn.w_d,
                         want_pre=True)
    R, x, post_, comb = tile(R0), tile(x0), tile(p0), tile(c0)
    full = ops.post_pre(x, R, post_, comb, ffn.fnp, ffn.scale_d, ffn.base_d, ffn.w_d,
                        want_pre=True)
    for what, big, sm in zip(("R'", "y", "post", "comb", "pre"), full, small):
        check(big, sm, f"hc_post_pre {what}")
    # post then pre on the same batch: the fused op's bits
    Rn = ops.post(x, R, post_, comb)
    assert torch.equal(Rn.view(torch.int16), full[0].view(torch.int16))
    y2, post2, comb2, _ = ops.pre(Rn, ffn.fnp, ffn.scale_d, ffn.base_d, ffn.w_d)
    assert torch.equal(y2.view(torch.int16), full[1].view(torch.int16))
    assert torch.equal(post2, full[2]) and torch.equal(comb2, full[3])
    del Rn, y2, post2, comb2
    # the MXFP8 form and the quantizer over the whole batch
    Rq, (yq, q, sf, _, _, _) = ops.post_pre_mxfp8(x, R, post_, comb, ffn.fnp, ffn.scale_d,
                                                  ffn.base_d, ffn.w_d)
    assert torch.equal(Rq.view(torch.int16), full[0].view(torch.int16))
    assert torch.equal(yq.view(torch.int16), full[1].view(torch.int16))
    del Rq, yq
    q0, sf0 = ops.mxfp8_quant_rows(small[1])
    check(q, q0, "q")
    check(sf, sf0, "scales")
    q2, sf2 = ops.mxfp8_quant_rows(full[1])
    assert torch.equal(q2, q) and torch.equal(sf2, sf)
    del q, sf, q2, sf2, full, x, post_, comb
    # the head over the same residual
    hf, hs, hb = inputs.hc_head_params(inputs.SEED_HEAD)
    hfp, hs_d, hb_d = ops.head_fn_pack(gu.dev(hf)), gu.dev(hs), gu.dev(hb)
    check(ops.head(R, hfp, hs_d, hb_d), ops.head(R0, hfp, hs_d, hb_d), "head y")


def test_full_size_post_pre_matches_oracle_on_every_row(attn, ffn):
    """The measured step itself: hc_post_pre at M = 4096, H = 5120 in the launch the throughput
    benchmark times (256 blocks, 16 per column slice, each running 16 stages of one 16-row
    group), against the oracle's post followed by its pre on all 4096 rows. post and comb come
    from the oracle's pre of the attention site."""
    M = 4096
    gu.say(f"hc_post_pre full size M={M} every row")
    R = inputs.residual(M, 4096 + 11)
    x = inputs.sublayer_out(M, 4096 + 12)
    ref1 = attn.oracle_pre(inputs.bits(R))
    post32 = torch.from_numpy(ref1["post"].astype(np.float32))
    comb32 = torch.from_numpy(ref1["comb"].astype(np.float32))
    Rn, y, post2, comb2, pre2 = ops.post_pre(
        gu.dev(x), gu.dev(R), gu.dev(post32), gu.dev(comb32), ffn.fnp, ffn.scale_d,
        ffn.base_d, ffn.w_d, want_pre=True,
        out=(_poison_bf16(M, 4, gu.H), _poison_bf16(M, gu.H), _poison_f32(M, 4),
             _poison_f32(M, 4, 4), _poison_f32(M, 4)))
    oR1, oR1_bits = o.hc_post(inputs.bits(x), inputs.bits(R), post32.numpy(), comb32.numpy())
    gRn = gu.bits_of(Rn)
    gu.assert_bf16_close(gRn, oR1, "R'")
    del oR1
    # the pre half on the GPU's own R' bits: per-stage bars (coefficients 1e-5)
    ref2g = ffn.oracle_pre(gRn)
    gy = gu.bits_of(y)
    gu.assert_bf16_close(gy, ref2g["y"], "y")
    for name, g in (("pre", pre2), ("post", post2), ("comb", comb2)):
        gu.assert_coef_close(gu.f32_np(g), ref2g[name], name)
    del ref2g
    # and against the oracle's whole chain (its own R'), one bf16 rounding of R' apart: y also
    # moves by what that rounding and the 2e-3 coefficient bar can shift where the combine cancels
    ref2 = ffn.oracle_pre(oR1_bits)
    gu.assert_bf16_close(gy, ref2["y"], "y (oracle chain)",
                         extra=gu.chain_y_slack(oR1_bits, ref2["pre"], ffn.w))
    for name, g in (("pre", pre2), ("post", post2), ("comb", comb2)):
        err = np.abs(gu.f32_np(g) - ref2[name]).max()
        assert err <= gu.CHAIN_COEF_ABS, f"{name} (oracle chain): {err}"
    # properties that hold at any size
    gu.assert_coef_properties(pre2, post2, comb2)
    assert torch.isfinite(y.float()).all() and torch.isfinite(Rn.float()).all()
