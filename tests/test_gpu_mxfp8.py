"""Row-local MXFP8 quantizer: bit-exact bytes and scales against the oracle, over every finite
bf16 pattern under every reachable block exponent, the hand-derived cases and rows with the
distribution of the page's MXFP8 test (randn * 0.5, first 64 columns x 40)."""
import os

import numpy as np
import pytest
import torch

from hyper_connection_residual_hc_amd import inputs, ops
from oracle import hc_oracle as o
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
K = 5120


def _gpu_quant(bits: np.ndarray):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    q, s = ops.mxfp8_quant_rows(gu.dev(t))
    return q.cpu().numpy(), s.cpu().numpy()


def _exhaustive_rows():
    """One row per block exponent e in [-127, 120]: every block starts with amax = 448 * 2^e
    (so the block exponent is e) followed by bf16 patterns with |v| in [2^(e-11), amax],
    both signs, which scale into the whole e4m3 range including the subnormals and ties."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    allv = o.bf16_to_f64(allb)
    finite = np.isfinite(allv)
    rows = []
    for e in range(-127, 121):
        amax = 448.0 * 2.0**e
        if amax > 3.3e38:
            continue
        sel = finite & (np.abs(allv) <= amax) & (np.abs(allv) >= 2.0 ** (e - 11))
        vals = allb[sel]
        G = K // 32
        for start in range(0, len(vals), G * 31):
            take = vals[start:start + G * 31]
            blocks = np.zeros((G, 32), dtype=np.uint16)
            blocks[:, 0] = o.f64_to_bf16(np.array(amax))
            flat = np.zeros(G * 31, dtype=np.uint16)
            flat[: len(take)] = take
            blocks[:, 1:] = flat.reshape(G, 31)
            rows.append(blocks.reshape(-1))
    return np.stack(rows)


def test_mxfp8_exhaustive_patterns_bit_exact():
    gu.say("mxfp8 exhaustive bf16 patterns")
    rows = _exhaustive_rows()
    q, s = _gpu_quant(rows)
    oq, osf = o.mxfp8_quant_rows(rows)
    assert np.array_equal(s, osf)
    bad = np.argwhere(q != oq)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}"


def test_mxfp8_every_pattern_under_largest_scale():
    # a block maximum at the largest finite bf16 puts every finite pattern into one scale
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = o.bf16_to_f64(allb)
    vals = allb[np.isfinite(v)]
    n = -(-len(vals) // 31)
    blocks = np.zeros((n, 32), dtype=np.uint16)
    blocks[:, 0] = 0x7F7F
    flat = np.zeros(n * 31, dtype=np.uint16)
    flat[: len(vals)] = vals
    blocks[:, 1:] = flat.reshape(n, 31)
    rows = blocks.reshape(-1)
    rows = np.concatenate([rows, np.zeros((-len(rows)) % K, np.uint16)]).reshape(-1, K)
    q, s = _gpu_quant(rows)
    oq, osf = o.mxfp8_quant_rows(rows)
    assert np.array_equal(s, osf) and np.array_equal(q, oq)


def test_mxfp8_hand_cases_on_gpu():
    path = os.path.join(os.path.dirname(__file__), "golden", "mxfp8_hand_cases.txt")
    cases = []
    with open(path) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if line:
                a, byte, v, code = line.split()
                cases.append((float.fromhex(a), int(byte), float.fromhex(v), int(code, 16)))
    rows = np.zeros((len(cases), 64), dtype=np.uint16)
    for r, (a, _, v, _) in enumerate(cases):
        rows[r, 0] = o.f64_to_bf16(np.array(a))
        rows[r, 1] = o.f64_to_bf16(np.array(v))
    q, s = _gpu_quant(rows)
    for r, (_, byte, _, code) in enumerate(cases):
        assert int(s[r, 0]) == byte, (r, cases[r])
        assert int(q[r, 1]) == code, (r, cases[r])


@pytest.mark.parametrize("M", [128, 1500, 3152])
def test_mxfp8_workload_rows_bit_exact(M):
    gu.say(f"mxfp8 rows M={M}")
    y = inputs.mxfp8_rows(M, M)
    q, s = _gpu_quant(inputs.bits(y))
    oq, osf = o.mxfp8_quant_rows(inputs.bits(y))
    assert np.array_equal(s, osf) and np.array_equal(q, oq)


def test_mxfp8_strided_rows():
    M = 40
    y = inputs.mxfp8_rows(M, 7, K=2 * K)
    yd = gu.dev(y)[:, :K]  # row stride 2K
    q = torch.zeros(M, K + 64, dtype=torch.uint8, device=gu.DEV)[:, :K]
    s = torch.zeros(M, K // 32 + 3, dtype=torch.uint8, device=gu.DEV)[:, : K // 32]
    ops.mxfp8_quant_rows(yd, q, s)
    oq, osf = o.mxfp8_quant_rows(inputs.bits(y)[:, :K])
    assert np.array_equal(q.cpu().numpy(), oq) and np.array_equal(s.cpu().numpy(), osf)
