"""Host-side checks of the decode entry point: every invalid argument is
rejected before any launch, so no GPU is needed."""
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


def _desc(Bn=4, T=None, hk=16, hv=32, dtype=B.GDN_BF16, **kw):
    d = B.make_desc(Bn, Bn if T is None else T, hk, hv, dtype)
    for key, val in kw.items():
        setattr(d, key, val)
    return d


def _call(lib, d, **kw):
    args = dict(q=P, k=P + 0x100000, v=P + 0x200000, a=P + 0x300000,
                b=P + 0x310000, A_log=P + 0x320000, dt_bias=P + 0x330000,
                z=P + 0x400000, norm_w=P + 0x500000, cache=P + 0x1000000,
                num_slots=8, slots=P + 0x600000, o=P + 0x700000)
    args.update(kw)
    order = ["q", "k", "v", "a", "b", "A_log", "dt_bias", "z", "norm_w",
             "cache"]
    ptrs = [None if args[n] is None else ctypes.c_void_p(args[n]) for n in order]
    slots = None if args["slots"] is None else ctypes.c_void_p(args["slots"])
    o = None if args["o"] is None else ctypes.c_void_p(args["o"])
    return lib.gdn_decode(ctypes.byref(d) if d is not None else None, *ptrs,
                          ctypes.c_int64(args["num_slots"]), slots, o, None)


@pytest.mark.parametrize("case,expect", [
    ("null_desc", B.GDN_ERR_INVALID),
    ("tokens_ne_requests", B.GDN_ERR_INVALID),
    ("zero_slots", B.GDN_ERR_INVALID),
    ("null_slots_too_few", B.GDN_ERR_INVALID),
    ("z_without_w", B.GDN_ERR_INVALID),
    ("null_q", B.GDN_ERR_INVALID),
    ("null_cache", B.GDN_ERR_INVALID),
    ("null_A_log", B.GDN_ERR_INVALID),
    ("misaligned_q", B.GDN_ERR_INVALID),
    ("misaligned_cache", B.GDN_ERR_INVALID),
    ("misaligned_slots", B.GDN_ERR_INVALID),
    ("misaligned_a_f32", B.GDN_ERR_INVALID),
    ("dk_64", B.GDN_ERR_UNSUPPORTED),
    ("hq_ne_hk", B.GDN_ERR_UNSUPPORTED),
    ("hv_not_multiple", B.GDN_ERR_INVALID),
    ("cache_overflow", B.GDN_ERR_UNSUPPORTED),
])
def test_decode_validation_rejects(lib, case, expect):
    calls = {
        "null_desc": lambda: _call(lib, None),
        "tokens_ne_requests": lambda: _call(lib, _desc(4, T=5)),
        "zero_slots": lambda: _call(lib, _desc(), num_slots=0),
        "null_slots_too_few": lambda: _call(lib, _desc(4), slots=None, num_slots=3),
        "z_without_w": lambda: _call(lib, _desc(), norm_w=None),
        "null_q": lambda: _call(lib, _desc(), q=None),
        "null_cache": lambda: _call(lib, _desc(), cache=None),
        "null_A_log": lambda: _call(lib, _desc(), A_log=None),
        "misaligned_q": lambda: _call(lib, _desc(), q=P + 8),
        "misaligned_cache": lambda: _call(lib, _desc(), cache=P + 0x1000004),
        "misaligned_slots": lambda: _call(lib, _desc(), slots=P + 0x600002),
        "misaligned_a_f32": lambda: _call(lib, _desc(dtype=B.GDN_F32), a=P + 0x300002),
        "dk_64": lambda: _call(lib, _desc(dk=64)),
        "hq_ne_hk": lambda: _call(lib, _desc(hq=8)),
        "hv_not_multiple": lambda: _call(lib, _desc(hv=33)),
        "cache_overflow": lambda: _call(lib, _desc(), num_slots=1 << 60),
    }
    st = calls[case]()
    assert st == expect, (case, B.status_string(st), B.last_error())
    assert B.last_error() != ""


def test_decode_empty_batch_rejected(lib):
    # a batch holds at least one request (num_seqs >= 1, as every descriptor)
    d = _desc(1)
    d.num_seqs = 0
    d.total_tokens = 0
    assert _call(lib, d) == B.GDN_ERR_INVALID


def test_decode_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(2, 16, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        B.decode(x, x, torch.zeros(2, 32, 128, dtype=torch.bfloat16),
                 torch.zeros(2, 32, dtype=torch.bfloat16),
                 torch.zeros(2, 32, dtype=torch.bfloat16),
                 torch.zeros(32), torch.zeros(32),
                 torch.zeros(2, 32, 128, 128))


def test_decode_refuses_a_grid_past_the_dispatch_limit(lib):
    # 2^20 requests over 32 value heads: one 256-thread block per (request,
    # head) is 2^33 work-items, past the dispatch packet's 32-bit grid size
    # (a small slot cache makes such a batch fit in memory)
    d = _desc(Bn=1 << 20)
    st = _call(lib, d, num_slots=1)
    assert st == B.GDN_ERR_UNSUPPORTED, B.last_error()
    assert "work-items" in B.last_error()
