"""Small batches: calls of 1 to 1024 rows (decode, verify, short prefill; the decode and verify
steps of the decoder layer run hc pre / post on a few rows, and prefill_sp.py,
_combine_norm_fused gates the engine's fused combine-norm on 1..8 rows) go through the same
stats kernel as large calls, with fewer blocks per slice. Every output of a row slice must be
the full call's bits: checked here as row slices of 1100-row calls at eight hidden sizes (every
stats geometry: 8 to 32 slices of 4, 8 or 10 chunks), for every entry point that computes mix
stats, and against the oracle at small sizes."""
import numpy as np
import pytest
import torch

from hyper_connection_residual_hc_amd import inputs, ops
from oracle import hc_oracle as o
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

M_BIG = 1100  # several row groups on every block of a slice
# slices of 1 .. 1024 rows: one and several 16-row groups, ragged last groups, group boundaries,
# odd offsets, the last rows
SLICES = [(0, 1), (0, 16), (3, 5), (7, 15), (31, 39), (48, 64), (63, 65), (1, 18), (70, 177),
          (333, 433), (5, 1029), (76, 1100), (1099, 1100)]


def _eq(a, b):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    return torch.equal(a, b)


@pytest.mark.parametrize("H", [5120, 512, 1024, 2048, 3072, 3584, 4096, 4608, 6144, 7168, 8192])
def test_small_batch_slices_match_the_full_call(H):
    gu.say(f"small-batch slices H={H}")
    attn = gu.Site(inputs.SEED_ATTN, inputs.SEED_NORM_ATTN, H_=H)
    ffn = gu.Site(inputs.SEED_FFN, inputs.SEED_NORM_FFN, H_=H)
    fh, sh, bh = inputs.hc_head_params(inputs.SEED_HEAD, H=H)
    hfnp, sh, bh = ops.head_fn_pack(gu.dev(fh)), gu.dev(sh), gu.dev(bh)
    R = gu.dev(inputs.residual(M_BIG, M_BIG, H=H))
    x = gu.dev(inputs.sublayer_out(M_BIG, M_BIG + 1, H=H))
    _, post, comb, _ = ops.pre(R, attn.fnp, attn.scale_d, attn.base_d, attn.w_d)

    def run(sl):
        Rs, xs, ps, cs = R[sl], x[sl], post[sl], comb[sl]
        pp = ops.post_pre(xs, Rs, ps, cs, ffn.fnp, ffn.scale_d, ffn.base_d, ffn.w_d,
                          want_pre=True)
        ppm = ops.post_pre_mxfp8(xs, Rs, ps, cs, ffn.fnp, ffn.scale_d, ffn.base_d, ffn.w_d,
                                 want_y=False)
        R1, ws = ops.post_stats(xs, Rs, ps, cs, ffn.fnp)
        return {
            "pre_stats": ops.pre_stats(Rs, ffn.fnp),
            "pre": ops.pre(Rs, ffn.fnp, ffn.scale_d, ffn.base_d, ffn.w_d, want_pre=True),
            "pre_mxfp8": ops.pre_mxfp8(Rs, ffn.fnp, ffn.scale_d, ffn.base_d, ffn.w_d),
            "post_pre": pp,
            "post_pre_mxfp8": ppm,
            "halves": (R1,) + ops.pre_finish(R1, ws, ffn.scale_d, ffn.base_d, ffn.w_d),
            "head": (ops.head(Rs, hfnp, sh, bh),),
        }

    full = run(slice(0, M_BIG))
    for lo, hi in SLICES:
        got = run(slice(lo, hi))
        for name, outs in got.items():
            for k, (g, f) in enumerate(zip(outs, full[name])):
                if g is None or not isinstance(g, torch.Tensor):
                    continue
                assert _eq(g, f[lo:hi]), f"H={H} {name}[{k}] differs on rows [{lo}, {hi})"


@pytest.mark.parametrize("M", [1, 5, 16, 100])
def test_small_batch_post_pre_matches_oracle(M):
    """hc post (attention site) then hc pre (FFN site) at small sizes against the oracle."""
    gu.say(f"small-batch post_pre vs oracle M={M}")
    attn = gu.Site(inputs.SEED_ATTN, inputs.SEED_NORM_ATTN)
    ffn = gu.Site(inputs.SEED_FFN, inputs.SEED_NORM_FFN)
    R_h = inputs.residual(M, 7 + M)
    x_h = inputs.sublayer_out(M, 8 + M)
    R, x = gu.dev(R_h), gu.dev(x_h)
    _, post, comb, _ = ops.pre(R, attn.fnp, attn.scale_d, attn.base_d, attn.w_d)
    R1, y, post2, comb2, pre2 = ops.post_pre(x, R, post, comb, ffn.fnp, ffn.scale_d,
                                             ffn.base_d, ffn.w_d, want_pre=True)
    mixes = ops.pre_stats(R1, ffn.fnp)[0]
    # post against the oracle on the GPU's own coefficients
    oR1, _ = o.hc_post(inputs.bits(x_h), inputs.bits(R_h), gu.f32_np(post).astype(np.float32),
                       gu.f32_np(comb).astype(np.float32))
    gu.assert_bf16_close(gu.bits_of(R1), oR1, "R'")
    # pre against the oracle on the GPU's R'
    ref = ffn.oracle_pre(gu.bits_of(R1))
    gu.assert_mixes_close(gu.f32_np(mixes), ref["mixes"])
    gu.assert_coef_close(gu.f32_np(pre2), ref["pre"], "pre")
    gu.assert_coef_close(gu.f32_np(post2), ref["post"], "post")
    gu.assert_coef_close(gu.f32_np(comb2), ref["comb"], "comb")
    gu.assert_bf16_close(gu.bits_of(y), ref["y"], "y")


def test_small_batch_graph_replays_and_padded_strides():
    """hc_post_pre at 7 rows captured in a HIP graph: three replays, with eager work and a
    synchronisation between them, each give the eager bits; and every bf16 row argument as a
    view into wider rows gives the contiguous call's bits and writes no pad byte."""
    gu.say("small-batch graph replays and padded strides M=7")
    M, H = 7, gu.H
    attn = gu.Site(inputs.SEED_ATTN, inputs.SEED_NORM_ATTN)
    ffn = gu.Site(inputs.SEED_FFN, inputs.SEED_NORM_FFN)
    R = gu.dev(inputs.residual(M, 41))
    x = gu.dev(inputs.sublayer_out(M, 42))
    _, post, comb, _ = ops.pre(R, attn.fnp, attn.scale_d, attn.base_d, attn.w_d)
    outs = (torch.empty_like(R), torch.empty(M, H, dtype=torch.bfloat16, device=gu.DEV),
            torch.empty(M, 4, device=gu.DEV), torch.empty(M, 4, 4, device=gu.DEV), None)
    ws = torch.empty(ops.post_pre_workspace_bytes(M, H), dtype=torch.uint8, device=gu.DEV)

    def step():
        ops.post_pre(x, R, post, comb, ffn.fnp, ffn.scale_d, ffn.base_d, ffn.w_d, out=outs,
                     workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs[:4]]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = gu.dev(inputs.residual(M, 43))
    for rep in range(3):
        for t in outs[:4]:
            t.view(torch.uint8).fill_(0xA5)
        ops.pre(other, ffn.fnp, ffn.scale_d, ffn.base_d, ffn.w_d)  # eager work in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(outs[:4], ref)):
            assert _eq(a, b), (rep, k)

    # padded row strides: R, x, R' and y as views into wider rows, each with its own pad
    def wide(inner, pad, src=None):
        b = torch.full((M, inner + pad), -7.0, dtype=torch.bfloat16, device=gu.DEV)
        v = b[:, :inner]
        if src is not None:
            v.copy_(src.reshape(M, inner))
        return b, v

    Rb, Rv = wide(4 * H, 512, R)
    xb, xv = wide(H, 256, x)
    R1b, R1v = wide(4 * H, 1024)
    yb, yv = wide(H, 128)
    got = ops.post_pre(xv, Rv.view(M, 4, H), post, comb, ffn.fnp, ffn.scale_d, ffn.base_d,
                       ffn.w_d, out=(R1v.view(M, 4, H), yv, torch.empty_like(outs[2]),
                                     torch.empty_like(outs[3]), None))
    torch.cuda.synchronize()
    assert _eq(R1v.reshape(M, 4, H), ref[0]) and _eq(yv, ref[1])
    assert _eq(got[2], ref[2]) and _eq(got[3], ref[3])
    for b, inner in ((R1b, 4 * H), (yb, H)):
        assert bool((b[:, inner:] == -7.0).all()), "a pad byte was written"
