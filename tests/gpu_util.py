"""Helpers shared by the GPU tests: device transfer, oracle-side tolerance checks and the
workload recipes (shapes, seeds, distributions of the five configurations)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from hyper_connection_residual_hc_amd import inputs
from oracle import hc_oracle as o

DEV = "cuda"
H = inputs.H

# tolerances: bf16 outputs |g - o| <= 2e-2 |o| + 1e-3 rms(o_row); fp32 mixes per-row
# normwise max|g - o| / max|o| <= 1e-5; pre / post / comb max |g - o| <= 1e-5
BF16_REL = 2e-2
BF16_ROW_ABS = 1e-3
STATS_NORMWISE = 1e-5
COEF_ABS = 1e-5


def say(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.to(DEV, non_blocking=False).contiguous()


def bits_of(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a (device or host) bf16 tensor."""
    return inputs.bits(t.detach().cpu())


def f32_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float64)


def assert_bf16_close(gpu_bits: np.ndarray, oracle: np.ndarray, what: str,
                      extra: np.ndarray | None = None) -> None:
    """|g - o| <= 2e-2 |o| + 1e-3 rms(o_row) (+ extra, an elementwise bound that a comparison
    across differently rounded inputs derives, where it applies)."""
    g = o.bf16_to_f64(gpu_bits)
    rms = np.sqrt(np.mean(oracle * oracle, axis=-1, keepdims=True))
    bound = BF16_REL * np.abs(oracle) + BF16_ROW_ABS * rms
    if extra is not None:
        bound = bound + extra
    err = np.abs(g - oracle)
    bad = err > bound
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of tolerance; worst "
                           f"{float((err - bound).max()):.3g} at {np.unravel_index(np.argmax(err - bound), err.shape)}")


def assert_mixes_close(gpu: np.ndarray, oracle: np.ndarray, what: str = "mixes") -> None:
    err = np.max(np.abs(gpu - oracle), axis=-1)
    scale = np.max(np.abs(oracle), axis=-1)
    rel = err / np.maximum(scale, 1e-30)
    assert np.all(rel <= STATS_NORMWISE), f"{what}: worst normwise {rel.max():.3g} (row {rel.argmax()})"


def assert_coef_close(gpu: np.ndarray, oracle: np.ndarray, what: str) -> None:
    err = np.abs(gpu - oracle)
    assert np.all(err <= COEF_ABS), f"{what}: worst abs {err.max():.3g}"


CHAIN_COEF_ABS = 2e-3


def chain_y_slack(R_bits: np.ndarray, pre: np.ndarray, w: torch.Tensor,
                  coef_abs: float = CHAIN_COEF_ABS) -> np.ndarray:
    """Elementwise bound on how far the pre's y moves between two residuals that are each a
    bf16 rounding of the same R' (at most one ulp, 2^-7 relative, apart) read with pre weights
    up to coef_abs apart. The combine c = sum_i pre_i R'_i then moves by up to
    sum_i (pre_i 2^-7 + coef_abs) |R'_i|, which the norm scales by |w| rsqrt(mean(c^2) + eps);
    the norm factor itself moves by up to 2^-7 relative. R_bits is one of the two residuals,
    pre the oracle's pre on it."""
    Ra = np.abs(o.bf16_to_f64(R_bits))
    pre = np.asarray(pre, dtype=np.float64)
    c = o.hc_combine(R_bits, pre)
    rstd = 1.0 / np.sqrt(np.mean(c * c, axis=-1, keepdims=True) + o.RMS_EPS)
    wa = np.abs(w.double().numpy())[None, :]
    dc = np.einsum("mi,mih->mh", pre * 2.0**-7 + coef_abs, Ra)
    return wa * rstd * (dc + 2.0**-7 * np.abs(c))


class Site:
    """One hc site's parameters on host and device (fn, scale, base, norm weight, packed fn)."""

    def __init__(self, param_seed: int, norm_seed: int, H_: int = H):
        from hyper_connection_residual_hc_amd import ops
        self.fn, self.scale, self.base = inputs.hc_params(param_seed, H=H_)
        self.w = inputs.norm_weight(norm_seed, H=H_)
        self.fn_d, self.scale_d, self.base_d, self.w_d = map(dev, (self.fn, self.scale, self.base, self.w))
        self.fnp = ops.fn_pack(self.fn_d)

    def oracle_pre(self, R_bits):
        return o.hc_pre(R_bits, self.fn.numpy(), self.scale.numpy(), self.base.numpy(),
                        inputs.bits(self.w))


def assert_coef_properties(pre, post, comb, eps: float = 1e-6) -> None:
    """What every row's coefficients satisfy, checked on all rows on the device: pre in
    [eps, 1 + eps] (sigmoid + eps), post in [0, 2] (2 sigmoid), comb positive with every
    destination column summing to 1 within 1e-5 (the last Sinkhorn step normalises the
    columns: s / (s + eps))."""
    slack = 1e-6
    for t in (pre, post, comb):
        assert t is None or torch.isfinite(t).all()
    if pre is not None:
        assert (pre >= eps - slack).all() and (pre <= 1 + eps + slack).all()
    assert (post >= 0).all() and (post <= 2).all()
    assert (comb > 0).all()
    colsum = comb.double().sum(dim=1)  # comb[m, i, j] over the sources i
    assert (colsum - 1).abs().max().item() <= 1e-5


def assert_mxfp8_bits_match_oracle(y: torch.Tensor, q: torch.Tensor, sf: torch.Tensor,
                                   chunk: int = 1024) -> None:
    """q / sf equal, byte for byte on every row, the oracle's MXFP8 of the bf16 y the GPU wrote
    (rows taken in chunks to bound host memory)."""
    M = y.shape[0]
    for a in range(0, M, chunk):
        gy = bits_of(y[a:a + chunk])
        oq, osf = o.mxfp8_quant_rows(gy)
        gq = q[a:a + chunk].cpu().numpy()
        gs = sf[a:a + chunk].cpu().numpy()
        bad = np.nonzero(np.any(oq != gq, axis=1) | np.any(osf != gs, axis=1))[0]
        assert len(bad) == 0, f"MXFP8 rows differing from the oracle: {a + bad[:8]}"


def stats_geom(H):
    """(slices S, 32-column chunks per stream per slice NC) of the stats kernels at width H, as
    the packed layout documents it: the largest even NC <= 10 with S = H / 32 NC a multiple of
    4 and at least 8."""
    for nc in (10, 8, 6, 4, 2):
        if H % (32 * nc) == 0 and (H // (32 * nc)) % 4 == 0 and H // (32 * nc) >= 8:
            return H // (32 * nc), nc
    raise ValueError(H)


def packed_columns(H):
    """Flattened fn column of every packed element, as an array shaped like the packed layout
    [slice][stream][chunk][tile][k-group g][lane column n][8] (without the tile and n axes)."""
    S, NC = stats_geom(H)
    W = H // S
    s = np.arange(S)[:, None, None, None, None]
    q = np.arange(4)[None, :, None, None, None]
    c = np.arange(NC)[None, None, :, None, None]
    g = np.arange(4)[None, None, None, :, None]
    e = np.arange(8)[None, None, None, None, :]
    return (q * H + s * W + 32 * c + 8 * g + e), S, NC
