"""Host-side checks of the layer, GEMM and conv entry points: defaults,
workspace sizing and argument validation (every case is rejected before any
launch, so no GPU is needed)."""
from __future__ import annotations

import ctypes
import os

import pytest

from gated_deltanet_linear_04_amd import binding as B

P = 0x7f0000100000  # fake, aligned device addresses (never dereferenced)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libgdn.so is not built; run __graft_entry__.build()")
    return B.load()


def test_layer_desc_defaults_and_workspace(lib):
    d = B.make_layer_desc(1, 2048, 2560, 16, 32, 4)
    assert (d.hidden, d.conv_width) == (2560, 4)
    assert (d.op.hk, d.op.hv, d.op.dk, d.op.dv, d.op.dtype) == (16, 32, 128, 128, B.GDN_BF16)
    ws = B.layer_workspace_size(d)
    # P (8192 cols) + z (4096) + b, a (32 each) + q, k (2048 each) + v (4096)
    # + y (4096), bf16, plus the prefill's workspace
    inter = 2048 * 2 * (8192 + 4096 + 32 + 32 + 2048 + 2048 + 4096 + 4096)
    assert ws >= inter + B.workspace_size(B.make_desc(1, 2048, 16, 32, B.GDN_BF16))
    assert ws % 256 == 0
    assert B.layer_workspace_size(B.make_layer_desc(1, 4096, 2560, 16, 32, 4)) > ws
    # any value-head count that is a multiple of the key heads is planned
    # (the in_proj segments b | a may then start off the 8-column grid)
    for hk, hv in ((1, 1), (3, 6), (4, 12), (8, 24), (2, 10)):
        assert B.layer_workspace_size(B.make_layer_desc(1, 300, 512, hk, hv, 4)) > 0, (hk, hv)


def _layer_call(lib, d, **kw):
    args = dict(x=P, W_in=P + 0x1000000, conv_w=P + 0x2000000, A_log=P + 0x3000000,
                dt_bias=P + 0x3100000, norm_w=P + 0x3200000, W_out=P + 0x4000000,
                state_in=None, conv_in=None, cu=None, out=P + 0x5000000, state_out=None,
                conv_out=None, ws=P + 0x10000000,
                ws_bytes=B.layer_workspace_size(d) if d else 0)
    args.update(kw)
    order = ["x", "W_in", "conv_w", "A_log", "dt_bias", "norm_w", "W_out",
             "state_in", "conv_in", "cu", "out", "state_out", "conv_out", "ws"]
    ptrs = [None if args[n] is None else ctypes.c_void_p(args[n]) for n in order]
    return lib.gdn_layer_prefill(ctypes.byref(d) if d is not None else None, *ptrs,
                                 ctypes.c_size_t(args["ws_bytes"]), None)


def _ld(**kw):
    d = B.make_layer_desc(kw.pop("N", 1), kw.pop("T", 128), kw.pop("hidden", 256),
                          kw.pop("hk", 16), kw.pop("hv", 32), kw.pop("W", 4))
    for key, val in kw.items():
        if key in ("hidden", "conv_width"):
            setattr(d, key, val)
        else:
            setattr(d.op, key, val)
    return d


@pytest.mark.parametrize("case,expect", [
    ("null_desc", B.GDN_ERR_INVALID),
    ("fp32", B.GDN_ERR_UNSUPPORTED),
    ("hidden_not_32", B.GDN_ERR_UNSUPPORTED),
    ("conv_width_5", B.GDN_ERR_UNSUPPORTED),
    ("conv_width_0", B.GDN_ERR_UNSUPPORTED),
    ("null_W_in", B.GDN_ERR_INVALID),
    ("null_norm_w", B.GDN_ERR_INVALID),
    ("misaligned_x", B.GDN_ERR_INVALID),
    ("misaligned_conv_state", B.GDN_ERR_INVALID),
    ("conv_state_partial_overlap", B.GDN_ERR_INVALID),
    ("no_cu_multi_seq", B.GDN_ERR_INVALID),
    ("small_workspace", B.GDN_ERR_WORKSPACE),
    ("dk64", B.GDN_ERR_UNSUPPORTED),
])
def test_layer_validation_rejects(lib, case, expect):
    calls = {
        "null_desc": lambda: _layer_call(lib, None, ws_bytes=1 << 30),
        "fp32": lambda: _layer_call(lib, _ld(dtype=B.GDN_F32), ws_bytes=1 << 30),
        "hidden_not_32": lambda: _layer_call(lib, _ld(hidden=100), ws_bytes=1 << 30),
        "conv_width_5": lambda: _layer_call(lib, _ld(conv_width=5), ws_bytes=1 << 30),
        "conv_width_0": lambda: _layer_call(lib, _ld(conv_width=0), ws_bytes=1 << 30),
        "null_W_in": lambda: _layer_call(lib, _ld(), W_in=None),
        "null_norm_w": lambda: _layer_call(lib, _ld(), norm_w=None),
        "misaligned_x": lambda: _layer_call(lib, _ld(), x=P + 8),
        "misaligned_conv_state": lambda: _layer_call(lib, _ld(), conv_in=P + 0x6000008),
        "conv_state_partial_overlap": lambda: _layer_call(
            lib, _ld(), conv_in=P + 0x6000000, conv_out=P + 0x6000000 + 4096),
        "no_cu_multi_seq": lambda: _layer_call(lib, _ld(N=2)),
        "small_workspace": lambda: _layer_call(lib, _ld(), ws_bytes=B.layer_workspace_size(_ld()) - 256),
        "dk64": lambda: _layer_call(lib, _ld(dk=64), ws_bytes=1 << 30),
    }
    st = calls[case]()
    assert st == expect, (case, B.status_string(st), B.last_error())
    assert B.last_error() != ""


def test_gemm_and_conv_validation(lib):
    vp = ctypes.c_void_p
    # K not a multiple of 32
    assert lib.gdn_gemm_bf16(64, 64, 40, vp(P), 40, vp(P), 40, vp(P), 64, None) == B.GDN_ERR_UNSUPPORTED
    assert lib.gdn_gemm_bf16(-1, 64, 32, vp(P), 32, vp(P), 32, vp(P), 64, None) == B.GDN_ERR_INVALID
    assert lib.gdn_gemm_bf16(64, 64, 32, None, 32, vp(P), 32, vp(P), 64, None) == B.GDN_ERR_INVALID
    assert lib.gdn_gemm_bf16(64, 64, 32, vp(P + 8), 32, vp(P), 32, vp(P), 64, None) == B.GDN_ERR_INVALID
    assert lib.gdn_gemm_bf16(64, 64, 32, vp(P), 16, vp(P), 32, vp(P), 64, None) == B.GDN_ERR_INVALID
    # empty products launch nothing
    assert lib.gdn_gemm_bf16(0, 64, 32, None, 32, None, 32, None, 64, None) == B.GDN_OK
    # conv: width, channel multiple, sequences
    conv = lambda T, C, W, x, ldx, w, hi, cu, N, y, ho: lib.gdn_conv_silu_bf16(
        T, C, W, x, ldx, w, hi, cu, N, y, ho, None)
    assert conv(16, 64, 5, vp(P), 64, vp(P), None, None, 1, vp(P), None) == B.GDN_ERR_UNSUPPORTED
    assert conv(16, 60, 4, vp(P), 64, vp(P), None, None, 1, vp(P), None) == B.GDN_ERR_UNSUPPORTED
    assert conv(16, 64, 4, vp(P), 64, vp(P), None, None, 2, vp(P), None) == B.GDN_ERR_INVALID
    assert conv(16, 64, 4, None, 64, vp(P), None, None, 1, vp(P), None) == B.GDN_ERR_INVALID
    assert conv(0, 64, 4, None, 64, None, None, None, 1, None, None) == B.GDN_OK
    # history buffers: alignment and partial overlap
    assert conv(16, 64, 4, vp(P), 64, vp(P), vp(P + 8), None, 1, vp(P), None) == B.GDN_ERR_INVALID
    assert conv(16, 64, 4, vp(P), 64, vp(P), None, None, 1, vp(P), vp(P + 8)) == B.GDN_ERR_INVALID
    assert conv(16, 64, 4, vp(P), 64, vp(P), vp(P + 0x100000), None, 1, vp(P),
                vp(P + 0x100000 + 16)) == B.GDN_ERR_INVALID
