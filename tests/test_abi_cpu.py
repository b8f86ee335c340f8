"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects every invalid argument on the host before any
launch (each case below fails validation, so nothing reaches a device)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

from gated_deltanet_linear_04_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libgdn.so is not built; run __graft_entry__.build()")
    return B.load()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert "gdn_prefill" in names and "gdn_prefill_workspace_size" in names
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (gdn_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(lib, n)


def test_desc_defaults_and_version(lib):
    d = B.make_desc(1, 2048, 16, 32, B.GDN_BF16)
    assert (d.hq, d.hk, d.hv, d.dk, d.dv) == (16, 16, 32, 128, 128)
    assert d.scale == pytest.approx(128 ** -0.5)
    assert d.qk_l2_eps == pytest.approx(1e-6) and d.norm_eps == pytest.approx(1e-6)
    assert d.short_tokens == 8
    assert lib.gdn_version() >= 100
    assert lib.gdn_desc_init(None, 1, 1, 1, 1, 128, 128, 1) == B.GDN_ERR_INVALID


def test_workspace_size(lib):
    d = B.make_desc(1, 2048, 16, 32, B.GDN_BF16)
    ws = B.workspace_size(d)
    assert ws > 0 and ws % 256 == 0
    # grows with tokens and sequences; fp32 needs more than bf16
    assert B.workspace_size(B.make_desc(1, 4096, 16, 32, B.GDN_BF16)) > ws
    assert B.workspace_size(B.make_desc(8, 2048, 16, 32, B.GDN_BF16)) > ws
    assert B.workspace_size(B.make_desc(1, 2048, 16, 32, B.GDN_F32)) > ws
    # T = 0 still needs the sequence table
    assert B.workspace_size(B.make_desc(3, 0, 16, 32, B.GDN_BF16)) > 0
    # invalid shapes report 0
    assert B.workspace_size(B.make_desc(1, 64, 16, 24, B.GDN_BF16)) == 0
    assert B.workspace_size(B.make_desc(1, 64, 16, 32, B.GDN_BF16, dk=64)) == 0
    assert lib.gdn_prefill_workspace_size(None) == 0


# Fake, aligned device addresses: never dereferenced, because every call
# below is rejected by the host-side validation.
P = 0x7f0000100000


def _call(lib, d, **kw):
    args = dict(q=P, k=P + 0x100000, v=P + 0x200000, a=P + 0x300000,
                b=P + 0x400000, A_log=P + 0x500000, dt_bias=P + 0x600000,
                z=None, norm_w=None, state_in=None, cu=None, o=P + 0x700000,
                state_out=None, ws=None, ws_bytes=0)
    args.update(kw)
    order = ["q", "k", "v", "a", "b", "A_log", "dt_bias", "z", "norm_w",
             "state_in", "cu", "o", "state_out", "ws"]
    ptrs = [None if args[n] is None else ctypes.c_void_p(args[n]) for n in order]
    st = lib.gdn_prefill(ctypes.byref(d) if d is not None else None, *ptrs,
                         ctypes.c_size_t(args["ws_bytes"]), None)
    return st


def _d(**kw):
    d = B.make_desc(kw.pop("N", 1), kw.pop("T", 128), kw.pop("hk", 2),
                    kw.pop("hv", 4), kw.pop("dtype", B.GDN_BF16),
                    kw.pop("dk", 128), kw.pop("dv", 128))
    for key, val in kw.items():
        setattr(d, key, val)
    return d


@pytest.mark.parametrize("case,expect", [
    ("null_desc", B.GDN_ERR_INVALID),
    ("num_seqs0", B.GDN_ERR_INVALID),
    ("neg_tokens", B.GDN_ERR_INVALID),
    ("hv_not_multiple", B.GDN_ERR_INVALID),
    ("bad_dtype", B.GDN_ERR_INVALID),
    ("dk64", B.GDN_ERR_UNSUPPORTED),
    ("dv256", B.GDN_ERR_UNSUPPORTED),
    ("hq_ne_hk", B.GDN_ERR_UNSUPPORTED),
    ("neg_eps", B.GDN_ERR_INVALID),
    ("nan_scale", B.GDN_ERR_INVALID),
    ("neg_short_tokens", B.GDN_ERR_INVALID),
    ("no_cu_multi_seq", B.GDN_ERR_INVALID),
    ("z_without_w", B.GDN_ERR_INVALID),
    ("w_without_z", B.GDN_ERR_INVALID),
    ("null_q", B.GDN_ERR_INVALID),
    ("null_o", B.GDN_ERR_INVALID),
    ("null_alog", B.GDN_ERR_INVALID),
    ("misaligned_q", B.GDN_ERR_INVALID),
    ("misaligned_state", B.GDN_ERR_INVALID),
    ("misaligned_a", B.GDN_ERR_INVALID),
    ("state_partial_overlap", B.GDN_ERR_INVALID),
    ("no_workspace", B.GDN_ERR_WORKSPACE),
    ("small_workspace", B.GDN_ERR_WORKSPACE),
    ("misaligned_workspace", B.GDN_ERR_INVALID),
])
def test_validation_rejects(lib, case, expect):
    need = B.workspace_size(_d())
    good_ws = dict(ws=P + 0x10000000, ws_bytes=need)
    calls = {
        "null_desc": lambda: _call(lib, None, **good_ws),
        "num_seqs0": lambda: _call(lib, _d(num_seqs=0), **good_ws),
        "neg_tokens": lambda: _call(lib, _d(total_tokens=-1), **good_ws),
        "hv_not_multiple": lambda: _call(lib, _d(hv=5), **good_ws),
        "bad_dtype": lambda: _call(lib, _d(dtype=7), **good_ws),
        "dk64": lambda: _call(lib, _d(dk=64), **good_ws),
        "dv256": lambda: _call(lib, _d(dv=256), **good_ws),
        "hq_ne_hk": lambda: _call(lib, _d(hq=4), **good_ws),
        "neg_eps": lambda: _call(lib, _d(qk_l2_eps=-1.0), **good_ws),
        "nan_scale": lambda: _call(lib, _d(scale=float("nan")), **good_ws),
        "neg_short_tokens": lambda: _call(lib, _d(short_tokens=-1), **good_ws),
        "no_cu_multi_seq": lambda: _call(lib, _d(N=2), **good_ws),
        "z_without_w": lambda: _call(lib, _d(), z=P + 0x800000, **good_ws),
        "w_without_z": lambda: _call(lib, _d(), norm_w=P + 0x800000, **good_ws),
        "null_q": lambda: _call(lib, _d(), q=None, **good_ws),
        "null_o": lambda: _call(lib, _d(), o=None, **good_ws),
        "null_alog": lambda: _call(lib, _d(), A_log=None, **good_ws),
        "misaligned_q": lambda: _call(lib, _d(), q=P + 8, **good_ws),
        "misaligned_state": lambda: _call(lib, _d(), state_in=P + 0x900004,
                                          **good_ws),
        "misaligned_a": lambda: _call(lib, _d(), a=P + 1, **good_ws),
        "state_partial_overlap": lambda: _call(
            lib, _d(), state_in=P + 0x900000, state_out=P + 0x900000 + 4096,
            **good_ws),
        "no_workspace": lambda: _call(lib, _d()),
        "small_workspace": lambda: _call(lib, _d(), ws=P + 0x10000000,
                                         ws_bytes=need - 256),
        "misaligned_workspace": lambda: _call(lib, _d(), ws=P + 0x10000010,
                                              ws_bytes=need),
    }
    st = calls[case]()
    assert st == expect, (case, B.status_string(st), B.last_error())
    assert B.last_error() != ""


def test_status_strings(lib):
    for code, name in [(0, "GDN_OK"), (-1, "GDN_ERR_INVALID"),
                       (-2, "GDN_ERR_UNSUPPORTED"), (-3, "GDN_ERR_WORKSPACE"),
                       (-4, "GDN_ERR_HIP"), (-99, "GDN_ERR_UNKNOWN")]:
        assert B.status_string(code) == name


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(4, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        B.prefill(x, x, torch.zeros(4, 4, 128, dtype=torch.bfloat16),
                  torch.zeros(4, 4, dtype=torch.bfloat16),
                  torch.zeros(4, 4, dtype=torch.bfloat16),
                  torch.zeros(4), torch.zeros(4))


def test_stage_timing_api_without_gpu(lib):
    # disabling and reading with nothing recorded are host-only
    B.stage_timing_enable(0)
    stages, calls = B.stage_timing_read()
    assert calls == 0
    assert list(stages) == ["prep", "chain", "out", "short"]


def test_no_process_wide_routing_state(lib):
    # which kernels compute a call is set by its descriptor alone: the
    # library exports no setter of global routing state
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    assert "set_short" not in out
    assert B.workspace_size(_d(short_tokens=0)) == B.workspace_size(_d())


def test_noalloc_refuses_calls_beyond_its_array_on_the_host(lib):
    # the size check comes before any device call: a T = 4096 call at the 4B
    # geometry needs more than the 96 MiB array and is refused
    d = _d(T=4096, hk=16, hv=32)
    assert B.workspace_size(d) > B.NOALLOC_SCRATCH_BYTES
    ptrs = [ctypes.c_void_p(P + i * 0x1000000) for i in range(7)] + [None] * 4 + [
        ctypes.c_void_p(P + 0x8000000), None]
    st = lib.gdn_prefill_noalloc(ctypes.byref(d), *ptrs, None)
    assert st == B.GDN_ERR_WORKSPACE, B.last_error()
    assert "gdn_prefill_noalloc" in B.last_error()
    assert lib.gdn_prefill_noalloc(None, *([None] * 13), None) == B.GDN_ERR_INVALID


@pytest.mark.parametrize("N,hk,hv,short", [(1 << 17, 16, 16, 0), (1 << 20, 16, 32, 8)])
def test_prefill_refuses_a_grid_past_the_dispatch_limit(lib, N, hk, hv, short):
    # one token per sequence.  Chunked (short = 0): the chain's 320-thread
    # blocks over 2^21 (sequence, head) units x 8 column blocks make 5.4e9
    # work-items.  Recurrent (short = 8): 2^25 256-thread blocks make 8.6e9.
    # Both exceed the dispatch packet's 32-bit grid size and are refused on
    # the host, with the workspace the call asks for.
    d = _d(N=N, T=N, hk=hk, hv=hv, short_tokens=short)
    need = B.workspace_size(d)
    assert need > 0
    st = _call(lib, d, cu=P + 0x20000000, ws=P + 0x40000000, ws_bytes=need)
    assert st == B.GDN_ERR_UNSUPPORTED, (B.status_string(st), B.last_error())
    assert "work-items" in B.last_error()
