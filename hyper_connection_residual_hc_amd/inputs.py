"""Seeded synthetic inputs for the mHC pre/post path.

This module only draws random numbers. It holds none of the method's arithmetic, so both the
HIP path and the CPU oracle can take their inputs from it. Everything is drawn on the host
with a CPU ``torch.Generator``, so a seed gives the same bits on every machine.

Distributions follow the one-GPU test page of the prefill sequence-parallel adapter
(test_prefill_sp_gpu.py, helpers ``_hc_params``, ``_residual`` and ``_norm``):

* ``fn``    fp32 ``[24, 4*H]``, standard normal times 0.0225
* ``base``  fp32 ``[24]``, standard normal times 3
* ``scale`` fp32 ``[3]``, uniform on [0.01, 0.06)
* ``R``     bf16 ``[M, 4, H]``, standard normal (drawn in bf16) times 0.5, then the first 64
  columns of every stream times 40 (in bf16, in that order)
* ``w``     bf16 ``[H]``, 1 + 0.1 * standard normal, rounded to bf16
* ``x``     bf16 ``[M, H]``, standard normal (the stand-in for the sublayer output)

Parameter tensors for one site are drawn from one generator in the order fn, base, scale,
as the test page does. Seeds: attention-site parameters 11, FFN-site parameters 61 (= 11+50),
norm weights 12 and 13, residual seed M, sublayer output seed M+1. The head mix (fn [4, 4H],
base [4], scale [1]; the test page draws none) uses the same distributions with seed 71.
"""
from __future__ import annotations

import numpy as np
import torch

H = 5120
HC = 4
MIX = (2 + HC) * HC  # 24 mixes per row: pre(4) | post(4) | res(16)

SEED_ATTN = 11
SEED_FFN = 61
SEED_NORM_ATTN = 12
SEED_NORM_FFN = 13
SEED_HEAD = 71


def hc_params(seed: int, H: int = H, hc: int = HC):
    """(fn fp32 [mix, hc*H], scale fp32 [3], base fp32 [mix]) for one hc site."""
    mix = (2 + hc) * hc
    g = torch.Generator().manual_seed(seed)
    fn = torch.randn(mix, hc * H, generator=g) * 0.0225
    base = torch.randn(mix, generator=g) * 3
    scale = torch.rand(3, generator=g) * 0.05 + 0.01
    return fn.contiguous(), scale.contiguous(), base.contiguous()


def hc_head_params(seed: int, H: int = H, hc: int = HC):
    """(fn fp32 [hc, hc*H], scale fp32 [1], base fp32 [hc]) for the head mix, with the
    distributions of the site parameters, drawn in the order fn, base, scale."""
    g = torch.Generator().manual_seed(seed)
    fn = torch.randn(hc, hc * H, generator=g) * 0.0225
    base = torch.randn(hc, generator=g) * 3
    scale = torch.rand(1, generator=g) * 0.05 + 0.01
    return fn.contiguous(), scale.contiguous(), base.contiguous()


def residual(M: int, seed: int, H: int = H, hc: int = HC) -> torch.Tensor:
    """bf16 [M, hc, H] multi-stream residual."""
    g = torch.Generator().manual_seed(seed)
    r = torch.randn(M, hc, H, generator=g, dtype=torch.bfloat16) * 0.5
    r[:, :, :64] *= 40
    return r.contiguous()


def norm_weight(seed: int, H: int = H) -> torch.Tensor:
    """bf16 [H] RMSNorm weight."""
    g = torch.Generator().manual_seed(seed)
    return (1 + 0.1 * torch.randn(H, generator=g)).to(torch.bfloat16).contiguous()


def sublayer_out(M: int, seed: int, H: int = H, std: float = 1.0) -> torch.Tensor:
    """bf16 [M, H] stand-in for the attention / MoE output that hc post consumes."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, H, generator=g, dtype=torch.bfloat16)
    if std != 1.0:
        x = x * std
    return x.contiguous()


def mxfp8_rows(M: int, seed: int, K: int = H) -> torch.Tensor:
    """bf16 [M, K] rows for the MXFP8 quantizer (standard normal times 0.5, first 64
    columns times 40), the distribution of the page's shard-vs-full MXFP8 test."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, K, generator=g, dtype=torch.bfloat16) * 0.5
    x[:, :64] *= 40
    return x.contiguous()


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a CPU bf16 tensor as a uint16 numpy array (no copy of values)."""
    assert t.dtype == torch.bfloat16 and t.device.type == "cpu"
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)
