"""Thin ctypes binding of ``libgdn.so`` (declared in ``include/gdn.h``).

Argument marshalling only: it checks dtypes/devices/contiguity of torch
tensors, allocates outputs and the workspace with torch's allocator when the
caller does not pass them, and hands raw device pointers plus the current
HIP stream to the C ABI.  Every step of the operator runs in the library's
HIP kernels; there is no fallback path, and loading fails loudly when the
library has not been built.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgdn.so")

GDN_OK = 0
GDN_ERR_INVALID = -1
GDN_ERR_UNSUPPORTED = -2
GDN_ERR_WORKSPACE = -3
GDN_ERR_HIP = -4
GDN_F32 = 0
GDN_BF16 = 1

_DTYPES = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}


class GdnDesc(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("total_tokens", ctypes.c_int64),
        ("hq", ctypes.c_int32),
        ("hk", ctypes.c_int32),
        ("hv", ctypes.c_int32),
        ("dk", ctypes.c_int32),
        ("dv", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("qk_l2_eps", ctypes.c_float),
        ("norm_eps", ctypes.c_float),
        ("short_tokens", ctypes.c_int32),
        ("chain_segments", ctypes.c_int32),
    ]


class GdnLayerDesc(ctypes.Structure):
    _fields_ = [
        ("op", GdnDesc),
        ("hidden", ctypes.c_int32),
        ("conv_width", ctypes.c_int32),
        ("conv_fused", ctypes.c_int32),
    ]


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (status_string(status), message))
        self.status = status


_lock = threading.Lock()
_lib = None
_vp = ctypes.c_void_p


def load(path: str = LIB_PATH):
    """Load libgdn.so; raises if it is missing (no fallback exists)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                "libgdn.so is not built (%s); run "
                "`python -m gated_deltanet_linear_04_amd.build`" % path)
        lib = ctypes.CDLL(path)
        lib.gdn_desc_init.restype = ctypes.c_int
        lib.gdn_desc_init.argtypes = [
            ctypes.POINTER(GdnDesc), ctypes.c_int32, ctypes.c_int64,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32]
        lib.gdn_prefill_workspace_size.restype = ctypes.c_size_t
        lib.gdn_prefill_workspace_size.argtypes = [ctypes.POINTER(GdnDesc)]
        lib.gdn_prefill.restype = ctypes.c_int
        lib.gdn_prefill.argtypes = [ctypes.POINTER(GdnDesc)] + [_vp] * 14 + [
            ctypes.c_size_t, _vp]
        lib.gdn_prefill_noalloc.restype = ctypes.c_int
        lib.gdn_prefill_noalloc.argtypes = [ctypes.POINTER(GdnDesc)] + [_vp] * 14
        lib.gdn_decode.restype = ctypes.c_int
        lib.gdn_decode.argtypes = [ctypes.POINTER(GdnDesc)] + [_vp] * 10 + [
            ctypes.c_int64, _vp, _vp, _vp]
        lib.gdn_mfma_probe.restype = ctypes.c_int
        lib.gdn_mfma_probe.argtypes = [ctypes.c_int64, ctypes.c_int32, _vp, _vp]
        lib.gdn_status_string.restype = ctypes.c_char_p
        lib.gdn_status_string.argtypes = [ctypes.c_int]
        lib.gdn_last_error.restype = ctypes.c_char_p
        lib.gdn_last_error.argtypes = []
        lib.gdn_version.restype = ctypes.c_int32
        lib.gdn_version.argtypes = []
        lib.gdn_stage_timing_enable.restype = ctypes.c_int
        lib.gdn_stage_timing_enable.argtypes = [ctypes.c_int32]
        lib.gdn_stage_timing_read.restype = ctypes.c_int32
        lib.gdn_stage_timing_read.argtypes = [
            ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_char_p),
            ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
        lib.gdn_layer_desc_init.restype = ctypes.c_int
        lib.gdn_layer_desc_init.argtypes = [
            ctypes.POINTER(GdnLayerDesc), ctypes.c_int32, ctypes.c_int64,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
        lib.gdn_layer_workspace_size.restype = ctypes.c_size_t
        lib.gdn_layer_workspace_size.argtypes = [ctypes.POINTER(GdnLayerDesc)]
        lib.gdn_layer_prefill.restype = ctypes.c_int
        lib.gdn_layer_prefill.argtypes = [ctypes.POINTER(GdnLayerDesc)] + \
            [_vp] * 14 + [ctypes.c_size_t, _vp]
        lib.gdn_gemm_bf16.restype = ctypes.c_int
        lib.gdn_gemm_bf16.argtypes = [
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _vp, ctypes.c_int64,
            _vp, ctypes.c_int64, _vp, ctypes.c_int64, _vp]
        lib.gdn_conv_silu_bf16.restype = ctypes.c_int
        lib.gdn_conv_silu_bf16.argtypes = [
            ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_int64,
            _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp]
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load().gdn_status_string(int(status)).decode()


def last_error() -> str:
    return load().gdn_last_error().decode()


def _check(status: int):
    if status != GDN_OK:
        raise GdnError(status, last_error())


def make_desc(num_seqs, total_tokens, hk, hv, dtype, dk=128, dv=128,
              scale=None, l2_eps=1e-6, norm_eps=1e-6, hq=None,
              short_tokens=None, chain_segments=None) -> GdnDesc:
    d = GdnDesc()
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    _check(load().gdn_desc_init(ctypes.byref(d), int(num_seqs),
                                int(total_tokens), int(hk), int(hv), int(dk),
                                int(dv), code))
    if hq is not None:
        d.hq = int(hq)
    if scale is not None:
        d.scale = float(scale)
    d.qk_l2_eps = float(l2_eps)
    d.norm_eps = float(norm_eps)
    if short_tokens is not None:
        d.short_tokens = int(short_tokens)
    if chain_segments is not None:
        d.chain_segments = int(chain_segments)
    return d


def workspace_size(desc: GdnDesc) -> int:
    return int(load().gdn_prefill_workspace_size(ctypes.byref(desc)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype, device, shape=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s"
                         % (name, tuple(t.shape), tuple(shape)))


def prefill(q, k, v, a, b, A_log, dt_bias, z=None, norm_w=None,
            state_in=None, cu_seqlens=None, *, scale=None, l2_eps=1e-6,
            norm_eps=1e-6, out=None, state_out=None, workspace=None,
            output_final_state=True, stream=None, short_tokens=None,
            chain_segments=None):
    """Gated delta rule prefill on the GPU (see include/gdn.h).

    q, k: [T, Hk, 128]; v: [T, Hv, 128]; a, b: [T, Hv] (all bf16 or all
    fp32); A_log, dt_bias: [Hv] fp32; z: [T, Hv, 128] and norm_w: [128] fp32
    (both or neither); state_in: [N, Hv, 128, 128] fp32 or None;
    cu_seqlens: int32 [N+1] on the device, or None for one sequence.
    Returns (o [T, Hv, 128], state_out [N, Hv, 128, 128] fp32 or None).
    ``state_out`` may be passed as ``state_in`` for an in-place update.
    ``short_tokens`` sets the descriptor's bound for the single-kernel form
    and ``chain_segments`` how the state chain runs (None: the library's
    defaults).
    """
    device = q.device
    if device.type != "cuda":
        raise ValueError("tensors must be on a GPU device, got %s" % device)
    dt = q.dtype
    if dt not in _DTYPES:
        raise TypeError("q must be bfloat16 or float32")
    T, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
    _need(q, "q", dt, device, (T, Hk, Dk))
    _need(k, "k", dt, device, (T, Hk, Dk))
    _need(v, "v", dt, device, (T, Hv, Dv))
    _need(a, "a", dt, device, (T, Hv))
    _need(b, "b", dt, device, (T, Hv))
    _need(A_log, "A_log", torch.float32, device, (Hv,))
    _need(dt_bias, "dt_bias", torch.float32, device, (Hv,))
    _need(z, "z", dt, device, (T, Hv, Dv))
    _need(norm_w, "norm_w", torch.float32, device, (Dv,))
    _need(state_in, "state_in", torch.float32, device, (N, Hv, Dv, Dk))
    _need(cu_seqlens, "cu_seqlens", torch.int32, device, (N + 1,))
    desc = make_desc(N, T, Hk, Hv, dt, Dk, Dv, scale, l2_eps, norm_eps,
                     short_tokens=short_tokens, chain_segments=chain_segments)
    if out is None:
        out = torch.empty((T, Hv, Dv), dtype=dt, device=device)
    _need(out, "out", dt, device, (T, Hv, Dv))
    if state_out is None and output_final_state:
        state_out = torch.empty((N, Hv, Dv, Dk), dtype=torch.float32,
                                device=device)
    _need(state_out, "state_out", torch.float32, device, (N, Hv, Dv, Dk))
    ws_bytes = workspace_size(desc)
    if ws_bytes == 0:
        # the shape itself is rejected: let the library report why (it
        # validates the descriptor before looking at any pointer)
        _check(load().gdn_prefill(ctypes.byref(desc), *([None] * 14), 0, None))
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
    if stream is None:
        stream = torch.cuda.current_stream(device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    with torch.cuda.device(device):
        st = load().gdn_prefill(
            ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
            _ptr(A_log), _ptr(dt_bias), _ptr(z), _ptr(norm_w), _ptr(state_in),
            _ptr(cu_seqlens), _ptr(out), _ptr(state_out), _ptr(workspace),
            ctypes.c_size_t(workspace.numel() * workspace.element_size()),
            ctypes.c_void_p(handle))
    _check(st)
    return out, state_out


NOALLOC_SCRATCH_BYTES = 96 << 20


def prefill_noalloc(q, k, v, a, b, A_log, dt_bias, z=None, norm_w=None,
                    state_in=None, cu_seqlens=None, *, out, state_out,
                    scale=None, l2_eps=1e-6, norm_eps=1e-6, stream=None,
                    short_tokens=None):
    """gdn_prefill_noalloc: the prefill with its scratch in the library's
    static per-GPU array (no workspace argument).  The caller passes out and
    state_out (or None for state_out), so this call allocates nothing."""
    device = q.device
    if device.type != "cuda":
        raise ValueError("tensors must be on a GPU device, got %s" % device)
    dt = q.dtype
    if dt not in _DTYPES:
        raise TypeError("q must be bfloat16 or float32")
    T, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
    for t, name, tdt, shape in ((q, "q", dt, (T, Hk, Dk)), (k, "k", dt, (T, Hk, Dk)),
                                (v, "v", dt, (T, Hv, Dv)), (a, "a", dt, (T, Hv)),
                                (b, "b", dt, (T, Hv)), (A_log, "A_log", torch.float32, (Hv,)),
                                (dt_bias, "dt_bias", torch.float32, (Hv,)),
                                (z, "z", dt, (T, Hv, Dv)), (norm_w, "norm_w", torch.float32, (Dv,)),
                                (state_in, "state_in", torch.float32, (N, Hv, Dv, Dk)),
                                (cu_seqlens, "cu_seqlens", torch.int32, (N + 1,)),
                                (out, "out", dt, (T, Hv, Dv)),
                                (state_out, "state_out", torch.float32, (N, Hv, Dv, Dk))):
        _need(t, name, tdt, device, shape)
    desc = make_desc(N, T, Hk, Hv, dt, Dk, Dv, scale, l2_eps, norm_eps,
                     short_tokens=short_tokens)
    if stream is None:
        stream = torch.cuda.current_stream(device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    with torch.cuda.device(device):
        st = load().gdn_prefill_noalloc(
            ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
            _ptr(A_log), _ptr(dt_bias), _ptr(z), _ptr(norm_w), _ptr(state_in),
            _ptr(cu_seqlens), _ptr(out), _ptr(state_out), ctypes.c_void_p(handle))
    _check(st)
    return out, state_out


def decode(q, k, v, a, b, A_log, dt_bias, state_cache, slot_idx=None,
           z=None, norm_w=None, *, scale=None, l2_eps=1e-6, norm_eps=1e-6,
           out=None, stream=None):
    """One decode step for B requests on a slot-addressed state cache (see
    gdn_decode in include/gdn.h).

    q, k: [B, Hk, 128]; v: [B, Hv, 128]; a, b: [B, Hv] (all bf16 or all
    fp32); A_log, dt_bias: [Hv] fp32; state_cache: [num_slots, Hv, 128, 128]
    fp32, updated in place; slot_idx: int32 [B] on the device or None
    (request i uses slot i); z: [B, Hv, 128] and norm_w: [128] fp32 (both or
    neither).  Returns o [B, Hv, 128].
    """
    device = q.device
    if device.type != "cuda":
        raise ValueError("tensors must be on a GPU device, got %s" % device)
    dt = q.dtype
    if dt not in _DTYPES:
        raise TypeError("q must be bfloat16 or float32")
    B, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    if state_cache is None or state_cache.dim() != 4:
        raise ValueError("state_cache must be [num_slots, Hv, Dv, Dk]")
    S = state_cache.shape[0]
    _need(q, "q", dt, device, (B, Hk, Dk))
    _need(k, "k", dt, device, (B, Hk, Dk))
    _need(v, "v", dt, device, (B, Hv, Dv))
    _need(a, "a", dt, device, (B, Hv))
    _need(b, "b", dt, device, (B, Hv))
    _need(A_log, "A_log", torch.float32, device, (Hv,))
    _need(dt_bias, "dt_bias", torch.float32, device, (Hv,))
    _need(z, "z", dt, device, (B, Hv, Dv))
    _need(norm_w, "norm_w", torch.float32, device, (Dv,))
    _need(state_cache, "state_cache", torch.float32, device, (S, Hv, Dv, Dk))
    _need(slot_idx, "slot_idx", torch.int32, device, (B,))
    desc = make_desc(B, B, Hk, Hv, dt, Dk, Dv, scale, l2_eps, norm_eps)
    if out is None:
        out = torch.empty((B, Hv, Dv), dtype=dt, device=device)
    _need(out, "out", dt, device, (B, Hv, Dv))
    handle = _stream_handle(stream, device)
    with torch.cuda.device(device):
        st = load().gdn_decode(
            ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
            _ptr(A_log), _ptr(dt_bias), _ptr(z), _ptr(norm_w),
            _ptr(state_cache), ctypes.c_int64(S), _ptr(slot_idx), _ptr(out),
            ctypes.c_void_p(handle))
    _check(st)
    return out


def _stream_handle(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def make_layer_desc(num_seqs, total_tokens, hidden, hk, hv, conv_width=4,
                    scale=None, l2_eps=1e-6, norm_eps=1e-6,
                    conv_fused=None) -> GdnLayerDesc:
    d = GdnLayerDesc()
    _check(load().gdn_layer_desc_init(ctypes.byref(d), int(num_seqs),
                                      int(total_tokens), int(hidden), int(hk),
                                      int(hv), int(conv_width)))
    if scale is not None:
        d.op.scale = float(scale)
    d.op.qk_l2_eps = float(l2_eps)
    d.op.norm_eps = float(norm_eps)
    if conv_fused is not None:
        d.conv_fused = int(conv_fused)
    return d


def layer_workspace_size(desc: GdnLayerDesc) -> int:
    return int(load().gdn_layer_workspace_size(ctypes.byref(desc)))


def layer_prefill(x, W_in, conv_w, A_log, dt_bias, norm_w, W_out, Hk, Hv,
                  state_in=None, cu_seqlens=None, *, conv_state_in=None,
                  conv_state_out=None, scale=None, l2_eps=1e-6, norm_eps=1e-6,
                  out=None, state_out=None, workspace=None, stream=None,
                  conv_fused=None):
    """Full GDN layer prefill on the GPU (see include/gdn.h).

    x: [T, hidden] bf16; W_in: [2*Hk*128 + 2*Hv*128 + 2*Hv, hidden] bf16
    ([out, in] layout; output columns q|k|v|z|b|a); conv_w:
    [2*Hk*128 + Hv*128, W] bf16; A_log, dt_bias: [Hv] fp32; norm_w: [128]
    fp32; W_out: [hidden, Hv*128] bf16; conv_state_in / conv_state_out:
    [N, W - 1, 2*Hk*128 + Hv*128] bf16 or None (the conv history carried
    between calls; conv_state_out may be conv_state_in).  Returns
    (out [T, hidden] bf16, state_out [N, Hv, 128, 128] fp32).
    ``conv_fused`` (None: the library's default) selects whether the conv
    runs inside the prefill's first kernel or as a kernel of its own.
    """
    device = x.device
    if device.type != "cuda":
        raise ValueError("tensors must be on a GPU device, got %s" % device)
    bf = torch.bfloat16
    T, hidden = x.shape
    Wq, Wv = Hk * 128, Hv * 128
    Wp = 2 * Wq + 2 * Wv + 2 * Hv
    N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
    conv_width = conv_w.shape[1]
    _need(x, "x", bf, device, (T, hidden))
    _need(W_in, "W_in", bf, device, (Wp, hidden))
    _need(conv_w, "conv_w", bf, device, (2 * Wq + Wv, conv_width))
    _need(A_log, "A_log", torch.float32, device, (Hv,))
    _need(dt_bias, "dt_bias", torch.float32, device, (Hv,))
    _need(norm_w, "norm_w", torch.float32, device, (128,))
    _need(W_out, "W_out", bf, device, (hidden, Wv))
    _need(state_in, "state_in", torch.float32, device, (N, Hv, 128, 128))
    _need(cu_seqlens, "cu_seqlens", torch.int32, device, (N + 1,))
    hist_shape = (N, conv_width - 1, 2 * Wq + Wv)
    _need(conv_state_in, "conv_state_in", bf, device, hist_shape)
    _need(conv_state_out, "conv_state_out", bf, device, hist_shape)
    desc = make_layer_desc(N, T, hidden, Hk, Hv, conv_width, scale, l2_eps,
                           norm_eps, conv_fused=conv_fused)
    if out is None:
        out = torch.empty((T, hidden), dtype=bf, device=device)
    _need(out, "out", bf, device, (T, hidden))
    if state_out is None:
        state_out = torch.empty((N, Hv, 128, 128), dtype=torch.float32,
                                device=device)
    _need(state_out, "state_out", torch.float32, device, (N, Hv, 128, 128))
    ws_bytes = layer_workspace_size(desc)
    if ws_bytes == 0:
        _check(load().gdn_layer_prefill(ctypes.byref(desc), *([None] * 14), 0,
                                        None))
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
    with torch.cuda.device(device):
        st = load().gdn_layer_prefill(
            ctypes.byref(desc), _ptr(x), _ptr(W_in), _ptr(conv_w), _ptr(A_log),
            _ptr(dt_bias), _ptr(norm_w), _ptr(W_out), _ptr(state_in),
            _ptr(conv_state_in), _ptr(cu_seqlens), _ptr(out), _ptr(state_out),
            _ptr(conv_state_out), _ptr(workspace),
            ctypes.c_size_t(workspace.numel() * workspace.element_size()),
            ctypes.c_void_p(_stream_handle(stream, device)))
    _check(st)
    return out, state_out


def gemm(A, B, out=None, stream=None):
    """C = A @ B^T on the GPU: A [M, K], B [N, K] bf16 (K a multiple of 32),
    fp32 accumulation, C [M, N] bf16."""
    device = A.device
    M, K = A.shape
    N = B.shape[0]
    _need(A, "A", torch.bfloat16, device, (M, K))
    _need(B, "B", torch.bfloat16, device, (N, K))
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=device)
    _need(out, "out", torch.bfloat16, device, (M, N))
    with torch.cuda.device(device):
        _check(load().gdn_gemm_bf16(M, N, K, _ptr(A), K, _ptr(B), K, _ptr(out),
                                    N, ctypes.c_void_p(_stream_handle(stream, device))))
    return out


def conv_silu(x, w, cu_seqlens=None, out=None, hist_in=None, hist_out=None,
              stream=None):
    """Depthwise causal conv + SiLU on the GPU: x [T, C], w [C, W] bf16;
    before each sequence of cu_seqlens (None: one sequence) the rows of
    hist_in [N, W - 1, C] (None: zeros); hist_out [N, W - 1, C] (or None)
    receives each sequence's last W - 1 input rows."""
    device = x.device
    T, C = x.shape
    W = w.shape[1]
    N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
    _need(x, "x", torch.bfloat16, device, (T, C))
    _need(w, "w", torch.bfloat16, device, (C, W))
    _need(cu_seqlens, "cu_seqlens", torch.int32, device, (N + 1,))
    _need(hist_in, "hist_in", torch.bfloat16, device, (N, W - 1, C))
    _need(hist_out, "hist_out", torch.bfloat16, device, (N, W - 1, C))
    if out is None:
        out = torch.empty((T, C), dtype=torch.bfloat16, device=device)
    _need(out, "out", torch.bfloat16, device, (T, C))
    with torch.cuda.device(device):
        _check(load().gdn_conv_silu_bf16(T, C, W, _ptr(x), C, _ptr(w), _ptr(hist_in),
                                         _ptr(cu_seqlens), N, _ptr(out), _ptr(hist_out),
                                         ctypes.c_void_p(_stream_handle(stream, device))))
    return out


def mfma_probe(iters, blocks, out, stream=None):
    """Measurement only: launches the bf16 MFMA rate probe (see
    gdn_mfma_probe); out is a float32 tensor of blocks * 256 elements."""
    _need(out, "out", torch.float32, out.device, (blocks * 256,))
    with torch.cuda.device(out.device):
        _check(load().gdn_mfma_probe(int(iters), int(blocks), _ptr(out),
                                     ctypes.c_void_p(_stream_handle(stream, out.device))))
    return out


def stage_timing_enable(max_calls: int):
    _check(load().gdn_stage_timing_enable(int(max_calls)))


def stage_timing_read():
    """Returns ({stage: summed ms}, calls) for the calls timed so far."""
    cap = 8
    ms = (ctypes.c_double * cap)()
    names = (ctypes.c_char_p * cap)()
    calls = ctypes.c_int32(0)
    n = load().gdn_stage_timing_read(ms, names, cap, ctypes.byref(calls))
    if n < 0:
        _check(n)
    return {names[i].decode(): ms[i] for i in range(n)}, calls.value
