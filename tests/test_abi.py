"""The C-ABI library loads without a GPU, exports every entry point include/hc_mi355x.h
declares, and its host-side argument checks return the documented status codes. None of these
calls reaches a kernel launch (each fails validation or is an M = 0 no-op)."""
import ctypes
import os

import pytest

from hyper_connection_residual_hc_amd import _lib


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from hyper_connection_residual_hc_amd import build
        build.build()
    return _lib.lib()


def test_every_header_symbol_is_exported(L):
    names = _lib.header_symbols()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_no_extra_exports_beyond_the_header(L):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    ours = {n for n in exported if n.startswith(("hc_", "mxfp8_"))}
    assert ours == set(_lib.header_symbols())


def test_status_strings(L):
    assert L.hc_status_string(0) == b"HC_OK"
    assert L.hc_status_string(2) == b"HC_ERR_SHAPE"
    assert L.hc_status_string(99) == b"HC_ERR_UNKNOWN"
    assert L.hc_abi_version() == 100


def test_sizes(L):
    H = 5120
    assert L.hc_fn_packed_bytes(H) == 8 * (4 * (H // 8) // 32) * 5 * 64 * 8 * 2
    assert L.hc_fn_packed_bytes(512) == 4 * 512 * 5 * 16 * 2
    assert L.hc_fn_packed_bytes(5632) == 0  # no slice count fits 5632 or 6656
    assert L.hc_fn_packed_bytes(6656) == 0
    assert L.hc_fn_packed_bytes(1000) == 0
    assert L.hc_fn_packed_bytes(100) == 0
    # partial records: 16 slices x 25 floats per row at H = 5120; 28 slices at 7168
    assert L.hc_pre_stats_workspace_bytes(4096, H) == 16 * 4096 * 25 * 4
    assert L.hc_pre_stats_workspace_bytes(10, 7168) == 28 * 10 * 25 * 4
    assert L.hc_pre_stats_workspace_bytes(10, 9216) == 0  # the stats stop at 8192
    # slices at the odd multiples of 512: 8 at 512, 1536, 2560; 28 at 3584; 24 at 4608, 7680
    for Hs, S in ((512, 8), (1536, 8), (2560, 8), (3584, 28), (4608, 24), (7680, 24)):
        assert L.hc_pre_stats_workspace_bytes(10, Hs) == S * 10 * 25 * 4
    assert L.hc_pre_workspace_bytes(0, H) == 0
    assert L.hc_pre_stats_workspace_bytes(-1, H) == 0


def test_validation_codes(L):
    H = 5120
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation
    # M = 0 is a no-op, even with NULL pointers
    assert L.hc_post(None, 0, None, 0, None, None, 0, H, None, 0, None) == 0
    assert L.hc_combine_norm(None, 0, None, 0, None, 0, H, 1e-6, None, 0, None) == 0
    assert L.mxfp8_quant_rows(None, 0, 0, H, None, 0, None, 0, None) == 0
    # NULL pointers with M > 0
    assert L.hc_post(None, H, None, 4 * H, None, None, 5, H, None, 4 * H, None) == 1
    assert L.hc_sinkhorn(None, 3, None, None, 20, 1e-6, 1e-6, 2.0, None, None, None, None) == 1
    # shapes
    assert L.hc_post(fake, H, fake, 4 * H, fake, fake, 5, 640, fake, 4 * H, None) == 2
    assert L.hc_combine_norm(fake, 4 * H, fake, 4, fake, 5, 17 * 512, 1e-6, fake, H, None) == 2  # > 8192
    assert L.hc_combine_norm(fake, 4 * H, fake, 4, fake, 5, 3 * 256, 1e-6, fake, H, None) == 2  # not 512 n
    assert L.hc_sinkhorn(fake, 3, fake, fake, 0, 1e-6, 1e-6, 2.0, fake, fake, fake, None) == 2
    assert L.mxfp8_quant_rows(fake, 40, 2, 40, fake, 40, fake, 1, None) == 2
    assert L.hc_post(fake, H, fake, 4 * H - 8, fake, fake, 5, H, fake, 4 * H, None) == 2
    # arguments
    assert L.hc_post(fake, H, fake, 4 * H, fake, fake, -1, H, fake, 4 * H, None) == 7
    assert L.hc_combine_norm(fake, 4 * H, fake, 4, fake, 5, H, float("nan"), fake, H, None) == 7
    # alignment: a 2-byte offset pointer
    mis = ctypes.c_void_p(0x10002)
    assert L.hc_post(mis, H, fake, 4 * H, fake, fake, 5, H, fake, 4 * H, None) == 3
    # aliasing: output over the input residual
    assert L.hc_post(ctypes.c_void_p(0x900000), H, fake, 4 * H, ctypes.c_void_p(0xA00000),
                     ctypes.c_void_p(0xB00000), 5, H, fake, 4 * H, None) == 4
    # workspace too small
    assert L.hc_pre_stats(fake, 4 * H, fake, 5, H, 1e-6, ctypes.c_void_p(0x800000), None,
                          ctypes.c_void_p(0x700000), 16, None) == 5


def test_validation_codes_of_the_post_pre_halves(L):
    H = 5120
    fake = ctypes.c_void_p(0x10000)
    a, b, c, d = (ctypes.c_void_p(v) for v in (0x1000000, 0x2000000, 0x3000000, 0x4000000))
    ws = ctypes.c_void_p(0x5000000)
    need = L.hc_post_pre_workspace_bytes(7, H)
    assert need == 16 * 7 * 25 * 4  # 16 slices x 25 floats per row at H = 5120
    # M = 0 no-ops
    assert L.hc_post_stats(None, 0, None, 0, None, None, None, 0, H, None, 0, None, 0, None) == 0
    assert L.hc_pre_finish(None, 0, None, None, None, 0, H, 1e-6, 1e-6, 1e-6, 20, 2.0, 1e-6,
                           None, 0, None, None, None, None, 0, None) == 0
    # NULL, shape, workspace, alias
    assert L.hc_post_stats(None, H, fake, 4 * H, fake, fake, fake, 7, H, fake, 4 * H, ws, need,
                           None) == 1
    assert L.hc_post_stats(a, H, b, 4 * H, c, c, d, 7, 512 * 11, fake, 4 * H, ws, need, None) == 2
    assert L.hc_post_stats(a, H, b, 4 * H, c, c, d, 7, H, fake, 4 * H, ws, need - 4, None) == 5
    assert L.hc_post_stats(a, H, b, 4 * H, c, ctypes.c_void_p(0x3000040), d, 7, H, b, 4 * H, ws,
                           need, None) == 4
    assert L.hc_pre_finish(a, 4 * H, b, c, d, 7, H, 1e-6, 1e-6, 1e-6, 0, 2.0, 1e-6, fake, H,
                           None, fake, fake, ws, need, None) == 2
    assert L.hc_pre_finish(a, 4 * H, b, c, d, 7, H, 1e-6, 1e-6, 1e-6, 20, 2.0, 1e-6, fake, H,
                           None, fake, fake, None, need, None) == 5
    # the workspace is an input of the second half: y over it is an alias
    assert L.hc_pre_finish(a, 4 * H, b, c, d, 7, H, 1e-6, 1e-6, 1e-6, 20, 2.0, 1e-6, ws, H,
                           None, fake, ctypes.c_void_p(0x6000000), ws, need, None) == 4


def test_mxfp8_epilogue_and_swizzle_checks(L):
    H = 5120
    assert L.mxfp8_swizzled_bytes(130, 160) == 256 * 160
    assert L.mxfp8_swizzled_bytes(128, 160) == 128 * 160
    assert L.mxfp8_swizzled_bytes(0, 160) == 0
    assert L.mxfp8_swizzled_bytes(5, 6) == 0  # G must be a multiple of 4
    a, b = ctypes.c_void_p(0x1000000), ctypes.c_void_p(0x2000000)
    assert L.mxfp8_swizzle_128x4(a, 160, 5, 6, b, None) == 2
    assert L.mxfp8_swizzle_128x4(a, 100, 5, 160, b, None) == 2  # ldS < G
    assert L.mxfp8_swizzle_128x4(a, 160, 5, 160, ctypes.c_void_p(0x2000002), None) == 3
    assert L.mxfp8_swizzle_128x4(a, 160, 5, 160, ctypes.c_void_p(0x1000010), None) == 4
    assert L.mxfp8_swizzle_128x4(None, 160, 0, 160, None, None) == 0
    # hc_pre_mxfp8: q is required, y is not; q row stride must keep 16-byte rows
    fake = ctypes.c_void_p(0x10000)
    ws = ctypes.c_void_p(0x5000000)
    need = L.hc_pre_workspace_bytes(7, H)
    args = [a, 4 * H, fake, fake, fake, fake, 7, H, 1e-6, 1e-6, 1e-6, 20, 2.0, 1e-6]
    assert L.hc_pre_mxfp8(*args, None, H, None, H, fake, H // 32, None, fake, fake, ws, need,
                          None) == 1
    assert L.hc_pre_mxfp8(*args, None, H, b, H + 8, fake, H // 32, None, fake, fake, ws, need,
                          None) == 3
    assert L.hc_pre_mxfp8(*args, None, H, b, H - 16, fake, H // 32, None, fake, fake, ws, need,
                          None) == 2
