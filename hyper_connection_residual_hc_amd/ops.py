"""Python binding of the mHC pre/post library: argument marshalling only.

Every function takes and returns torch tensors on a ROCm device, passes their device
pointers and row strides to the C ABI (include/hc_mi355x.h) and enqueues on torch's current
stream. All arithmetic happens in the HIP kernels. Output tensors are allocated with torch
when the caller does not pass them.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib

HC = 4
MIX = 24
RMS_EPS = 1e-6
HC_EPS = 1e-6
ITERS = 20
POST_MULT = 2.0


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a ROCm device, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if t.numel() and t.stride(-1) != 1:
        raise ValueError(f"{name} needs a unit inner stride")


def _residual(R: torch.Tensor):
    _need(R, "R", torch.bfloat16, 3)
    M, hc, H = R.shape
    if hc != HC:
        raise ValueError(f"R must be [M, {HC}, H], got {tuple(R.shape)}")
    if M and R.stride(1) != H:
        raise ValueError("R's streams must be contiguous inside a row")
    return M, H, (R.stride(0) if M else HC * H)


def _shaped(t: torch.Tensor, name: str, dtype: torch.dtype, shape) -> None:
    """A row-strided tensor of exactly `shape` (the kernels write every element of it)."""
    _need(t, name, dtype, len(shape))
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {tuple(shape)}, got {tuple(t.shape)}")


def _packed(fn_packed: torch.Tensor, H: int) -> None:
    if not isinstance(fn_packed, torch.Tensor) or fn_packed.device.type != "cuda":
        raise ValueError("fn_packed must be a device tensor from fn_pack")
    if not fn_packed.is_contiguous() or fn_packed.numel() * fn_packed.element_size() < fn_packed_bytes(H):
        raise ValueError(f"fn_packed is smaller than fn_pack's output for H={H}")


def _rows(t: torch.Tensor, width: int) -> int:
    return t.stride(0) if t.shape[0] else width


def _contig(t: torch.Tensor, name: str, dtype: torch.dtype, shape) -> None:
    _need(t, name, dtype, len(shape))
    if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {tuple(shape)} tensor, got {tuple(t.shape)}")


# ---- weight preparation -------------------------------------------------------------------
def fn_packed_bytes(H: int) -> int:
    return int(_lib.lib().hc_fn_packed_bytes(H))


def fn_pack(fn: torch.Tensor) -> torch.Tensor:
    """fp32 fn [24, 4H] -> the packed bf16 hi/mid/lo form hc_pre_stats and hc_pre read."""
    _need(fn, "fn", torch.float32, 2)
    if fn.shape[0] != MIX or fn.shape[1] % HC or not fn.is_contiguous():
        raise ValueError(f"fn must be a contiguous [{MIX}, 4H] tensor, got {tuple(fn.shape)}")
    H = fn.shape[1] // HC
    nbytes = fn_packed_bytes(H)
    if nbytes == 0:
        raise ValueError(f"unsupported H={H}")
    out = torch.empty(nbytes // 2, dtype=torch.int16, device=fn.device)
    _one_device(fn, out)
    _lib.call("hc_fn_pack", fn.data_ptr(), H, out.data_ptr(), _stream(fn))
    return out


# ---- stage 1 ---------------------------------------------------------------------------------
def stats_workspace_bytes(M: int, H: int) -> int:
    return int(_lib.lib().hc_pre_stats_workspace_bytes(M, H))


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    if workspace is None:
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor) or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return workspace


def _one_device(*ts) -> None:
    """Every tensor argument of a call on the same ROCm device (the kernels run on that
    device's stream and read every pointer there)."""
    devs = {t.device for t in ts if isinstance(t, torch.Tensor)}
    if len(devs) != 1 or next(iter(devs)).type != "cuda":
        raise ValueError(f"all tensors of a call must be on one ROCm device, got {sorted(map(str, devs))}")


def pre_stats(R: torch.Tensor, fn_packed: torch.Tensor, rms_eps: float = RMS_EPS,
              mixes: Optional[torch.Tensor] = None, sumsq: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, want_sumsq: bool = True):
    """(mixes fp32 [M, 24], sumsq fp32 [M] or None)."""
    M, H, ldR = _residual(R)
    _packed(fn_packed, H)
    if mixes is None:
        mixes = torch.empty(M, MIX, dtype=torch.float32, device=R.device)
    _contig(mixes, "mixes", torch.float32, (M, MIX))
    if sumsq is None and want_sumsq:
        sumsq = torch.empty(M, dtype=torch.float32, device=R.device)
    if sumsq is not None:
        _contig(sumsq, "sumsq", torch.float32, (M,))
    ws = _workspace(stats_workspace_bytes(M, H), R.device, workspace)
    _one_device(R, fn_packed, mixes, sumsq, ws)
    _lib.call("hc_pre_stats", R.data_ptr(), ldR, fn_packed.data_ptr(), M, H, rms_eps,
              mixes.data_ptr(), _ptr(sumsq), ws.data_ptr(), ws.numel() * ws.element_size(),
              _stream(R))
    return mixes, sumsq


# ---- stages 2-3 ------------------------------------------------------------------------------
def sinkhorn(mixes: torch.Tensor, scale: torch.Tensor, base: torch.Tensor, iters: int = ITERS,
             pre_eps: float = HC_EPS, sinkhorn_eps: float = HC_EPS, post_mult: float = POST_MULT,
             out=None):
    """(pre [M, 4], post [M, 4], comb [M, 4, 4]) fp32."""
    M = mixes.shape[0]
    _contig(mixes, "mixes", torch.float32, (M, MIX))
    _contig(scale, "scale", torch.float32, (3,))
    _contig(base, "base", torch.float32, (MIX,))
    if out is None:
        out = (torch.empty(M, HC, dtype=torch.float32, device=mixes.device),
               torch.empty(M, HC, dtype=torch.float32, device=mixes.device),
               torch.empty(M, HC, HC, dtype=torch.float32, device=mixes.device))
    pre, post, comb = out
    _contig(pre, "pre", torch.float32, (M, HC))
    _contig(post, "post", torch.float32, (M, HC))
    _contig(comb, "comb", torch.float32, (M, HC, HC))
    _one_device(mixes, scale, base, pre, post, comb)
    _lib.call("hc_sinkhorn", mixes.data_ptr(), M, scale.data_ptr(), base.data_ptr(), iters,
              pre_eps, sinkhorn_eps, post_mult, pre.data_ptr(), post.data_ptr(), comb.data_ptr(),
              _stream(mixes))
    return pre, post, comb


# ---- stage 4 ---------------------------------------------------------------------------------
def combine_norm(R: torch.Tensor, pre: torch.Tensor, weight: torch.Tensor,
                 eps: float = RMS_EPS, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y bf16 [M, H] = RMSNorm(sum_i pre_i R_i) * weight."""
    M, H, ldR = _residual(R)
    _need(pre, "pre", torch.float32, 2)
    if tuple(pre.shape) != (M, HC):
        raise ValueError(f"pre must be [{M}, {HC}]")
    _contig(weight, "weight", torch.bfloat16, (H,))
    if out is None:
        out = torch.empty(M, H, dtype=torch.bfloat16, device=R.device)
    _shaped(out, "out", torch.bfloat16, (M, H))
    _one_device(R, pre, weight, out)
    _lib.call("hc_combine_norm", R.data_ptr(), ldR, pre.data_ptr(), _rows(pre, HC),
              weight.data_ptr(), M, H, eps, out.data_ptr(), _rows(out, H), _stream(R))
    return out


# ---- stage 5 ---------------------------------------------------------------------------------
def post(x: torch.Tensor, R: torch.Tensor, post_: torch.Tensor, comb: torch.Tensor,
         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """R' bf16 [M, 4, H] = post * x + comb^T R (per row)."""
    M, H, ldR = _residual(R)
    _need(x, "x", torch.bfloat16, 2)
    if tuple(x.shape) != (M, H):
        raise ValueError(f"x must be [{M}, {H}]")
    _contig(post_, "post", torch.float32, (M, HC))
    _contig(comb, "comb", torch.float32, (M, HC, HC))
    if out is None:
        out = torch.empty(M, HC, H, dtype=torch.bfloat16, device=R.device)
    _shaped(out, "out", torch.bfloat16, (M, HC, H))
    _residual(out)
    _one_device(x, R, post_, comb, out)
    _lib.call("hc_post", x.data_ptr(), _rows(x, H), R.data_ptr(), ldR, post_.data_ptr(),
              comb.data_ptr(), M, H, out.data_ptr(), _rows(out, HC * H), _stream(R))
    return out


# ---- MXFP8 -----------------------------------------------------------------------------------
def mxfp8_quant_rows(y: torch.Tensor, q: Optional[torch.Tensor] = None,
                     scales: Optional[torch.Tensor] = None):
    """(q uint8 [M, K] e4m3fn codes, scales uint8 [M, K/32] ue8m0, linear)."""
    _need(y, "y", torch.bfloat16, 2)
    M, K = y.shape
    if q is None:
        q = torch.empty(M, K, dtype=torch.uint8, device=y.device)
    if scales is None:
        scales = torch.empty(M, K // 32, dtype=torch.uint8, device=y.device)
    _shaped(q, "q", torch.uint8, (M, K))
    _shaped(scales, "scales", torch.uint8, (M, K // 32))
    _one_device(y, q, scales)
    _lib.call("mxfp8_quant_rows", y.data_ptr(), _rows(y, K), M, K, q.data_ptr(), _rows(q, K),
              scales.data_ptr(), _rows(scales, K // 32), _stream(y))
    return q, scales


# ---- fused pre -------------------------------------------------------------------------------
def pre_workspace_bytes(M: int, H: int) -> int:
    return int(_lib.lib().hc_pre_workspace_bytes(M, H))


def pre(R: torch.Tensor, fn_packed: torch.Tensor, scale: torch.Tensor, base: torch.Tensor,
        weight: torch.Tensor, rms_eps: float = RMS_EPS, pre_eps: float = HC_EPS,
        sinkhorn_eps: float = HC_EPS, iters: int = ITERS, post_mult: float = POST_MULT,
        norm_eps: float = RMS_EPS, want_pre: bool = False, out=None,
        workspace: Optional[torch.Tensor] = None):
    """Fused stages 1-4: (y bf16 [M, H], post [M, 4], comb [M, 4, 4], pre [M, 4] or None)."""
    M, H, ldR = _residual(R)
    _contig(scale, "scale", torch.float32, (3,))
    _contig(base, "base", torch.float32, (MIX,))
    _contig(weight, "weight", torch.bfloat16, (H,))
    dev = R.device
    if out is None:
        out = (torch.empty(M, H, dtype=torch.bfloat16, device=dev),
               torch.empty(M, HC, dtype=torch.float32, device=dev),
               torch.empty(M, HC, HC, dtype=torch.float32, device=dev),
               torch.empty(M, HC, dtype=torch.float32, device=dev) if want_pre else None)
    y, post_, comb, pre_ = out
    _packed(fn_packed, H)
    _shaped(y, "y", torch.bfloat16, (M, H))
    _contig(post_, "post", torch.float32, (M, HC))
    _contig(comb, "comb", torch.float32, (M, HC, HC))
    if pre_ is not None:
        _contig(pre_, "pre", torch.float32, (M, HC))
    ws = _workspace(pre_workspace_bytes(M, H), dev, workspace)
    _one_device(R, fn_packed, scale, base, weight, y, post_, comb, pre_, ws)
    _lib.call("hc_pre", R.data_ptr(), ldR, fn_packed.data_ptr(), scale.data_ptr(),
              base.data_ptr(), weight.data_ptr(), M, H, rms_eps, pre_eps, sinkhorn_eps, iters,
              post_mult, norm_eps, y.data_ptr(), _rows(y, H), _ptr(pre_), post_.data_ptr(),
              comb.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(), _stream(R))
    return y, post_, comb, pre_


# ---- fused post -> pre -----------------------------------------------------------------------
def post_pre_workspace_bytes(M: int, H: int) -> int:
    return int(_lib.lib().hc_post_pre_workspace_bytes(M, H))


def post_pre(x: torch.Tensor, R: torch.Tensor, post_: torch.Tensor, comb: torch.Tensor,
             fn_packed: torch.Tensor, scale: torch.Tensor, base: torch.Tensor,
             weight: torch.Tensor, rms_eps: float = RMS_EPS, pre_eps: float = HC_EPS,
             sinkhorn_eps: float = HC_EPS, iters: int = ITERS, post_mult: float = POST_MULT,
             norm_eps: float = RMS_EPS, want_pre: bool = False, out=None,
             workspace: Optional[torch.Tensor] = None):
    """hc post of one site fused with hc pre of the next:
    (R' [M, 4, H], y [M, H], post' [M, 4], comb' [M, 4, 4], pre' [M, 4] or None)."""
    M, H, ldR = _residual(R)
    _need(x, "x", torch.bfloat16, 2)
    if tuple(x.shape) != (M, H):
        raise ValueError(f"x must be [{M}, {H}]")
    _contig(post_, "post", torch.float32, (M, HC))
    _contig(comb, "comb", torch.float32, (M, HC, HC))
    _contig(scale, "scale", torch.float32, (3,))
    _contig(base, "base", torch.float32, (MIX,))
    _contig(weight, "weight", torch.bfloat16, (H,))
    dev = R.device
    if out is None:
        out = (torch.empty(M, HC, H, dtype=torch.bfloat16, device=dev),
               torch.empty(M, H, dtype=torch.bfloat16, device=dev),
               torch.empty(M, HC, dtype=torch.float32, device=dev),
               torch.empty(M, HC, HC, dtype=torch.float32, device=dev),
               torch.empty(M, HC, dtype=torch.float32, device=dev) if want_pre else None)
    Rn, y, post_o, comb_o, pre_o = out
    _packed(fn_packed, H)
    _shaped(Rn, "R_out", torch.bfloat16, (M, HC, H))
    _, _, ldOut = _residual(Rn)
    _shaped(y, "y", torch.bfloat16, (M, H))
    _contig(post_o, "post_out", torch.float32, (M, HC))
    _contig(comb_o, "comb_out", torch.float32, (M, HC, HC))
    if pre_o is not None:
        _contig(pre_o, "pre_out", torch.float32, (M, HC))
    ws = _workspace(post_pre_workspace_bytes(M, H), dev, workspace)
    _one_device(x, R, post_, comb, fn_packed, scale, base, weight, Rn, y, post_o, comb_o, pre_o, ws)
    _lib.call("hc_post_pre", x.data_ptr(), _rows(x, H), R.data_ptr(), ldR, post_.data_ptr(),
              comb.data_ptr(), fn_packed.data_ptr(), scale.data_ptr(), base.data_ptr(),
              weight.data_ptr(), M, H, rms_eps, pre_eps, sinkhorn_eps, iters, post_mult,
              norm_eps, Rn.data_ptr(), ldOut, y.data_ptr(), _rows(y, H), _ptr(pre_o),
              post_o.data_ptr(), comb_o.data_ptr(), ws.data_ptr(),
              ws.numel() * ws.element_size(), _stream(R))
    return Rn, y, post_o, comb_o, pre_o


NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024  # HC_NOALLOC_SCRATCH_BYTES


def noalloc_max_rows(H: int) -> int:
    """Most rows post_pre_noalloc takes at row width H (its partials must fit the scratch)."""
    return NOALLOC_SCRATCH_BYTES // post_pre_workspace_bytes(1, H)


def post_pre_noalloc(x: torch.Tensor, R: torch.Tensor, post_: torch.Tensor, comb: torch.Tensor,
                     fn_packed: torch.Tensor, scale: torch.Tensor, base: torch.Tensor,
                     weight: torch.Tensor, out, rms_eps: float = RMS_EPS,
                     pre_eps: float = HC_EPS, sinkhorn_eps: float = HC_EPS, iters: int = ITERS,
                     post_mult: float = POST_MULT, norm_eps: float = RMS_EPS):
    """post_pre with the library's static scratch array instead of a workspace (at most
    noalloc_max_rows(H) rows; calls on one GPU must not overlap). The caller passes every
    output: out = (R' [M, 4, H], y [M, H], post' [M, 4], comb' [M, 4, 4], pre' [M, 4] or
    None); nothing is allocated here either."""
    M, H, ldR = _residual(R)
    _need(x, "x", torch.bfloat16, 2)
    if tuple(x.shape) != (M, H):
        raise ValueError(f"x must be [{M}, {H}]")
    _contig(post_, "post", torch.float32, (M, HC))
    _contig(comb, "comb", torch.float32, (M, HC, HC))
    _contig(scale, "scale", torch.float32, (3,))
    _contig(base, "base", torch.float32, (MIX,))
    _contig(weight, "weight", torch.bfloat16, (H,))
    Rn, y, post_o, comb_o, pre_o = out
    _packed(fn_packed, H)
    _shaped(Rn, "R_out", torch.bfloat16, (M, HC, H))
    _, _, ldOut = _residual(Rn)
    _shaped(y, "y", torch.bfloat16, (M, H))
    _contig(post_o, "post_out", torch.float32, (M, HC))
    _contig(comb_o, "comb_out", torch.float32, (M, HC, HC))
    if pre_o is not None:
        _contig(pre_o, "pre_out", torch.float32, (M, HC))
    _one_device(x, R, post_, comb, fn_packed, scale, base, weight, Rn, y, post_o, comb_o, pre_o)
    _lib.call("hc_post_pre_noalloc", x.data_ptr(), _rows(x, H), R.data_ptr(), ldR,
              post_.data_ptr(), comb.data_ptr(), fn_packed.data_ptr(), scale.data_ptr(),
              base.data_ptr(), weight.data_ptr(), M, H, rms_eps, pre_eps, sinkhorn_eps, iters,
              post_mult, norm_eps, Rn.data_ptr(), ldOut, y.data_ptr(), _rows(y, H), _ptr(pre_o),
              post_o.data_ptr(), comb_o.data_ptr(), _stream(R))
    return Rn, y, post_o, comb_o, pre_o


# ---- the two halves of the fused post -> pre ----------------------------------------------------
def post_stats(x: torch.Tensor, R: torch.Tensor, post_: torch.Tensor, comb: torch.Tensor,
               fn_packed: torch.Tensor, out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None):
    """First half of post_pre: (R' [M, 4, H], workspace holding R''s mix-stat partials under
    the next site's fn_packed). Pass both to pre_finish."""
    M, H, ldR = _residual(R)
    _need(x, "x", torch.bfloat16, 2)
    if tuple(x.shape) != (M, H):
        raise ValueError(f"x must be [{M}, {H}]")
    _contig(post_, "post", torch.float32, (M, HC))
    _contig(comb, "comb", torch.float32, (M, HC, HC))
    _packed(fn_packed, H)
    if out is None:
        out = torch.empty(M, HC, H, dtype=torch.bfloat16, device=R.device)
    _shaped(out, "out", torch.bfloat16, (M, HC, H))
    _, _, ldOut = _residual(out)
    ws = _workspace(post_pre_workspace_bytes(M, H), R.device, workspace)
    _one_device(x, R, post_, comb, fn_packed, out, ws)
    _lib.call("hc_post_stats", x.data_ptr(), _rows(x, H), R.data_ptr(), ldR, post_.data_ptr(),
              comb.data_ptr(), fn_packed.data_ptr(), M, H, out.data_ptr(), ldOut, ws.data_ptr(),
              ws.numel() * ws.element_size(), _stream(R))
    return out, ws


def pre_finish(R: torch.Tensor, workspace: torch.Tensor, scale: torch.Tensor,
               base: torch.Tensor, weight: torch.Tensor, rms_eps: float = RMS_EPS,
               pre_eps: float = HC_EPS, sinkhorn_eps: float = HC_EPS, iters: int = ITERS,
               post_mult: float = POST_MULT, norm_eps: float = RMS_EPS, want_pre: bool = False,
               out=None):
    """Second half of post_pre, on post_stats's (R', workspace):
    (y bf16 [M, H], post [M, 4], comb [M, 4, 4], pre [M, 4] or None)."""
    M, H, ldR = _residual(R)
    _contig(scale, "scale", torch.float32, (3,))
    _contig(base, "base", torch.float32, (MIX,))
    _contig(weight, "weight", torch.bfloat16, (H,))
    dev = R.device
    if out is None:
        out = (torch.empty(M, H, dtype=torch.bfloat16, device=dev),
               torch.empty(M, HC, dtype=torch.float32, device=dev),
               torch.empty(M, HC, HC, dtype=torch.float32, device=dev),
               torch.empty(M, HC, dtype=torch.float32, device=dev) if want_pre else None)
    y, post_o, comb_o, pre_o = out
    _shaped(y, "y", torch.bfloat16, (M, H))
    _contig(post_o, "post", torch.float32, (M, HC))
    _contig(comb_o, "comb", torch.float32, (M, HC, HC))
    if pre_o is not None:
        _contig(pre_o, "pre", torch.float32, (M, HC))
    _workspace(0, dev, workspace)  # a contiguous tensor: its byte count is its extent
    _one_device(R, workspace, scale, base, weight, y, post_o, comb_o, pre_o)
    _lib.call("hc_pre_finish", R.data_ptr(), ldR, scale.data_ptr(), base.data_ptr(),
              weight.data_ptr(), M, H, rms_eps, pre_eps, sinkhorn_eps, iters, post_mult,
              norm_eps, y.data_ptr(), _rows(y, H), _ptr(pre_o), post_o.data_ptr(),
              comb_o.data_ptr(), workspace.data_ptr(),
              workspace.numel() * workspace.element_size(), _stream(R))
    return y, post_o, comb_o, pre_o


# ---- MXFP8 output of the pre ------------------------------------------------------------------
def _mx_outputs(M: int, H: int, dev, want_y: bool, want_pre: bool, out):
    """(y or None, q, scales, post, comb, pre or None), allocated unless given, then checked."""
    if out is None:
        out = (torch.empty(M, H, dtype=torch.bfloat16, device=dev) if want_y else None,
               torch.empty(M, H, dtype=torch.uint8, device=dev),
               torch.empty(M, H // 32, dtype=torch.uint8, device=dev),
               torch.empty(M, HC, dtype=torch.float32, device=dev),
               torch.empty(M, HC, HC, dtype=torch.float32, device=dev),
               torch.empty(M, HC, dtype=torch.float32, device=dev) if want_pre else None)
    y, q, sc, post_o, comb_o, pre_o = out
    if y is not None:
        _shaped(y, "y", torch.bfloat16, (M, H))
    _shaped(q, "q", torch.uint8, (M, H))
    _shaped(sc, "scales", torch.uint8, (M, H // 32))
    _contig(post_o, "post", torch.float32, (M, HC))
    _contig(comb_o, "comb", torch.float32, (M, HC, HC))
    if pre_o is not None:
        _contig(pre_o, "pre", torch.float32, (M, HC))
    return out


def _mx_args(out, H):
    y, q, sc, post_o, comb_o, pre_o = out
    return (_ptr(y), _rows(y, H) if y is not None else H, q.data_ptr(), _rows(q, H),
            sc.data_ptr(), _rows(sc, H // 32), _ptr(pre_o), post_o.data_ptr(), comb_o.data_ptr())


def pre_mxfp8(R: torch.Tensor, fn_packed: torch.Tensor, scale: torch.Tensor, base: torch.Tensor,
              weight: torch.Tensor, rms_eps: float = RMS_EPS, pre_eps: float = HC_EPS,
              sinkhorn_eps: float = HC_EPS, iters: int = ITERS, post_mult: float = POST_MULT,
              norm_eps: float = RMS_EPS, want_y: bool = True, want_pre: bool = False, out=None,
              workspace: Optional[torch.Tensor] = None):
    """hc_pre with y also in MXFP8: (y bf16 or None, q u8 [M, H], scales u8 [M, H/32] linear,
    post, comb, pre or None)."""
    M, H, ldR = _residual(R)
    _packed(fn_packed, H)
    _contig(scale, "scale", torch.float32, (3,))
    _contig(base, "base", torch.float32, (MIX,))
    _contig(weight, "weight", torch.bfloat16, (H,))
    out = _mx_outputs(M, H, R.device, want_y, want_pre, out)
    ws = _workspace(pre_workspace_bytes(M, H), R.device, workspace)
    _one_device(R, fn_packed, scale, base, weight, ws, *[t for t in out if t is not None])
    _lib.call("hc_pre_mxfp8", R.data_ptr(), ldR, fn_packed.data_ptr(), scale.data_ptr(),
              base.data_ptr(), weight.data_ptr(), M, H, rms_eps, pre_eps, sinkhorn_eps, iters,
              post_mult, norm_eps, *_mx_args(out, H), ws.data_ptr(),
              ws.numel() * ws.element_size(), _stream(R))
    return out


def post_pre_mxfp8(x: torch.Tensor, R: torch.Tensor, post_: torch.Tensor, comb: torch.Tensor,
                   fn_packed: torch.Tensor, scale: torch.Tensor, base: torch.Tensor,
                   weight: torch.Tensor, rms_eps: float = RMS_EPS, pre_eps: float = HC_EPS,
                   sinkhorn_eps: float = HC_EPS, iters: int = ITERS,
                   post_mult: float = POST_MULT, norm_eps: float = RMS_EPS,
                   want_y: bool = True, want_pre: bool = False, R_out=None, out=None,
                   workspace: Optional[torch.Tensor] = None):
    """hc_post_pre with y also in MXFP8: (R', (y or None, q, scales, post', comb', pre' or None))."""
    M, H, ldR = _residual(R)
    _need(x, "x", torch.bfloat16, 2)
    if tuple(x.shape) != (M, H):
        raise ValueError(f"x must be [{M}, {H}]")
    _contig(post_, "post", torch.float32, (M, HC))
    _contig(comb, "comb", torch.float32, (M, HC, HC))
    _packed(fn_packed, H)
    _contig(scale, "scale", torch.float32, (3,))
    _contig(base, "base", torch.float32, (MIX,))
    _contig(weight, "weight", torch.bfloat16, (H,))
    if R_out is None:
        R_out = torch.empty(M, HC, H, dtype=torch.bfloat16, device=R.device)
    _shaped(R_out, "R_out", torch.bfloat16, (M, HC, H))
    _, _, ldOut = _residual(R_out)
    out = _mx_outputs(M, H, R.device, want_y, want_pre, out)
    ws = _workspace(post_pre_workspace_bytes(M, H), R.device, workspace)
    _one_device(x, R, post_, comb, fn_packed, scale, base, weight, R_out, ws, *[t for t in out if t is not None])
    _lib.call("hc_post_pre_mxfp8", x.data_ptr(), _rows(x, H), R.data_ptr(), ldR,
              post_.data_ptr(), comb.data_ptr(), fn_packed.data_ptr(), scale.data_ptr(),
              base.data_ptr(), weight.data_ptr(), M, H, rms_eps, pre_eps, sinkhorn_eps, iters,
              post_mult, norm_eps, R_out.data_ptr(), ldOut, *_mx_args(out, H), ws.data_ptr(),
              ws.numel() * ws.element_size(), _stream(R))
    return R_out, out


def pre_finish_mxfp8(R: torch.Tensor, workspace: torch.Tensor, scale: torch.Tensor,
                     base: torch.Tensor, weight: torch.Tensor, rms_eps: float = RMS_EPS,
                     pre_eps: float = HC_EPS, sinkhorn_eps: float = HC_EPS, iters: int = ITERS,
                     post_mult: float = POST_MULT, norm_eps: float = RMS_EPS,
                     want_y: bool = True, want_pre: bool = False, out=None):
    """Second half of post_pre_mxfp8, on post_stats's (R', workspace)."""
    M, H, ldR = _residual(R)
    _contig(scale, "scale", torch.float32, (3,))
    _contig(base, "base", torch.float32, (MIX,))
    _contig(weight, "weight", torch.bfloat16, (H,))
    out = _mx_outputs(M, H, R.device, want_y, want_pre, out)
    _workspace(0, R.device, workspace)  # a contiguous tensor: its byte count is its extent
    _one_device(R, workspace, scale, base, weight, *[t for t in out if t is not None])
    _lib.call("hc_pre_finish_mxfp8", R.data_ptr(), ldR, scale.data_ptr(), base.data_ptr(),
              weight.data_ptr(), M, H, rms_eps, pre_eps, sinkhorn_eps, iters, post_mult,
              norm_eps, *_mx_args(out, H), workspace.data_ptr(),
              workspace.numel() * workspace.element_size(), _stream(R))
    return out


def mxfp8_swizzle_128x4(scales: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Linear ue8m0 scales [M, G] -> the 128x4 tiled layout, flat uint8 of
    ceil(M / 128) * 128 * G bytes (padded rows zero)."""
    _need(scales, "scales", torch.uint8, 2)
    M, G = scales.shape
    nbytes = int(_lib.lib().mxfp8_swizzled_bytes(M, G))
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=scales.device)
    _shaped(out, "out", torch.uint8, (nbytes,))
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    _one_device(scales, out)
    _lib.call("mxfp8_swizzle_128x4", scales.data_ptr(), _rows(scales, G), M, G, out.data_ptr(),
              _stream(scales))
    return out


# ---- hc_head ----------------------------------------------------------------------------------
def head_fn_pack(fn: torch.Tensor) -> torch.Tensor:
    """fp32 head fn [4, 4H] -> the packed operands hc_head reads."""
    _need(fn, "fn", torch.float32, 2)
    if fn.shape[0] != HC or fn.shape[1] % HC or not fn.is_contiguous():
        raise ValueError(f"fn must be a contiguous [{HC}, 4H] tensor, got {tuple(fn.shape)}")
    H = fn.shape[1] // HC
    nbytes = fn_packed_bytes(H)
    if nbytes == 0:
        raise ValueError(f"unsupported H={H}")
    out = torch.empty(nbytes // 2, dtype=torch.int16, device=fn.device)
    _one_device(fn, out)
    _lib.call("hc_head_fn_pack", fn.data_ptr(), H, out.data_ptr(), _stream(fn))
    return out


def head(R: torch.Tensor, fn_packed: torch.Tensor, scale: torch.Tensor, base: torch.Tensor,
         norm_eps: float = RMS_EPS, hc_eps: float = HC_EPS, out: Optional[torch.Tensor] = None,
         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y bf16 [M, H] = sum_i pre_i R_i with pre = sigmoid(mixes * scale + base) + hc_eps."""
    M, H, ldR = _residual(R)
    _packed(fn_packed, H)
    _contig(scale, "scale", torch.float32, (1,))
    _contig(base, "base", torch.float32, (HC,))
    if out is None:
        out = torch.empty(M, H, dtype=torch.bfloat16, device=R.device)
    _shaped(out, "out", torch.bfloat16, (M, H))
    ws = _workspace(int(_lib.lib().hc_head_workspace_bytes(M, H)), R.device, workspace)
    _one_device(R, fn_packed, scale, base, out, ws)
    _lib.call("hc_head", R.data_ptr(), ldR, fn_packed.data_ptr(), scale.data_ptr(),
              base.data_ptr(), M, H, norm_eps, hc_eps, out.data_ptr(), _rows(out, H),
              ws.data_ptr(), ws.numel() * ws.element_size(), _stream(R))
    return out
