"""hc_post_pre_noalloc: the fused post -> pre with the library's static scratch array instead
of a caller workspace. Called through the C ABI and checked bit for bit against hc_post_pre
(same kernels), on two calls in a row, the second with fewer rows, so the second reuses the
array the first one left behind; then the size limit and an empty call."""
import ctypes

import pytest
import torch

from hyper_connection_residual_hc_amd import _lib, inputs, ops
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sites():
    return (gu.Site(inputs.SEED_ATTN, inputs.SEED_NORM_ATTN),
            gu.Site(inputs.SEED_FFN, inputs.SEED_NORM_FFN))


def _outs(M, poison):
    H = gu.H
    bf = lambda *s: torch.full(s, poison, dtype=torch.int16, device=gu.DEV).view(torch.bfloat16)  # noqa: E731
    f32 = lambda *s: torch.full(s, float("nan"), dtype=torch.float32, device=gu.DEV)  # noqa: E731
    return (bf(M, 4, H), bf(M, H), f32(M, 4), f32(M, 4, 4), f32(M, 4))


def _case(attn, ffn, M, seed):
    gu.say(f"hc_post_pre_noalloc M={M} seed={seed}")
    R = gu.dev(inputs.residual(M, seed))
    x = gu.dev(inputs.sublayer_out(M, seed + 1))
    _, post, comb, _ = ops.pre(R, attn.fnp, attn.scale_d, attn.base_d, attn.w_d)
    ref = ops.post_pre(x, R, post, comb, ffn.fnp, ffn.scale_d, ffn.base_d, ffn.w_d,
                       want_pre=True, out=_outs(M, -3))
    got = ops.post_pre_noalloc(x, R, post, comb, ffn.fnp, ffn.scale_d, ffn.base_d, ffn.w_d,
                               out=_outs(M, -1))
    torch.cuda.synchronize()
    for a, b, what in zip(got, ref, ("R'", "y", "post", "comb", "pre")):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                           b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16)), what
    return got


def test_noalloc_matches_post_pre_on_two_calls(sites):
    attn, ffn = sites
    # first call: several tiles per block plus a ragged tail; second call: fewer rows, so it
    # reads partials only where it wrote them over the first call's contents
    _case(attn, ffn, 4177, 71)
    _case(attn, ffn, 1500, 72)
    _case(attn, ffn, 7, 73)


def test_noalloc_limits(sites):
    attn, ffn = sites
    L = _lib.lib()
    H = gu.H
    M = ops.noalloc_max_rows(H) + 1
    stream = torch.cuda.current_stream().cuda_stream
    # too many rows: refused before anything is enqueued (no buffer is read, so none is passed
    # beyond pointers that are never dereferenced)
    dummy = torch.empty(16, dtype=torch.uint8, device=gu.DEV)
    p = dummy.data_ptr()
    st = L.hc_post_pre_noalloc(p, H, p, 4 * H, p, p, ffn.fnp.data_ptr(), p, p, p, M, H, 1e-6,
                               1e-6, 1e-6, 20, 2.0, 1e-6, p, 4 * H, p, H, None, p, p,
                               ctypes.c_void_p(stream))
    assert L.hc_status_string(st).decode() == "HC_ERR_WORKSPACE"
    # an empty call is a no-op
    st = L.hc_post_pre_noalloc(p, H, p, 4 * H, p, p, ffn.fnp.data_ptr(), p, p, p, 0, H, 1e-6,
                               1e-6, 1e-6, 20, 2.0, 1e-6, p, 4 * H, p, H, None, p, p,
                               ctypes.c_void_p(stream))
    assert st == 0
    # and the array still serves a call afterwards
    _case(attn, ffn, 300, 74)
