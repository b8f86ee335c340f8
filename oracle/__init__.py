"""fp64 CPU oracle for the gated delta rule prefill (and the full GDN layer).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
library never imports, links or calls it, and it shares no code with the HIP
path.

The arithmetic lives in ``gdn_oracle.c`` (plain C, fp64, OpenMP over
(sequence, value head) units).  This module only converts arrays to fp64,
calls the C code through ctypes, and, for the full layer, strings the C steps
together with numpy float64 matmuls for the two projections.

Sources (page title, section): "Add opt-in fused Qwen3.5 inference kernels",
Summary (gate from A_log/dt_bias, beta sigmoid, q/k L2 norm, grouped value
heads, gated RMSNorm after, four input projections as one GEMM);
"feat(qwen35): add SM120 FlashInfer GDN prefill candidate", Correctness (the
16/16/32/128 geometry, chunked vs unchunked prefill, the FP64 oracle).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")
_lock = threading.Lock()
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into ``oracle/libgdn_oracle.so``."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.gdn_oracle_softplus.restype = ctypes.c_double
        lib.gdn_oracle_softplus.argtypes = [ctypes.c_double]
        lib.gdn_oracle_sigmoid.restype = ctypes.c_double
        lib.gdn_oracle_sigmoid.argtypes = [ctypes.c_double]
        lib.gdn_oracle_delta_core.restype = None
        lib.gdn_oracle_delta_core.argtypes = [
            ctypes.c_int64, ctypes.c_int, ctypes.c_int, _dp, _dp,
            _dp, ctypes.c_int64, _dp, ctypes.c_int64, _dp, ctypes.c_int64,
            _dp, _dp, ctypes.c_int64]
        lib.gdn_oracle_gated_rmsnorm_row.restype = None
        lib.gdn_oracle_gated_rmsnorm_row.argtypes = [
            ctypes.c_int, _dp, _dp, _dp, ctypes.c_double, _dp]
        lib.gdn_oracle_prefill.restype = ctypes.c_int
        lib.gdn_oracle_prefill.argtypes = [
            ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int,
            _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
            ctypes.POINTER(ctypes.c_int32),
            ctypes.c_double, ctypes.c_double, ctypes.c_double,
            _dp, _dp, ctypes.c_int]
        lib.gdn_oracle_delta_core_terms.restype = None
        lib.gdn_oracle_delta_core_terms.argtypes = [
            ctypes.c_int64, ctypes.c_int, ctypes.c_int, _dp, _dp,
            _dp, ctypes.c_int64, _dp, ctypes.c_int64, _dp, ctypes.c_int64,
            _dp, _dp, ctypes.c_int64, _dp, ctypes.c_int64]
        lib.gdn_oracle_prefill_ex.restype = ctypes.c_int
        lib.gdn_oracle_prefill_ex.argtypes = [
            ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int,
            _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
            ctypes.POINTER(ctypes.c_int32),
            ctypes.c_double, ctypes.c_double, ctypes.c_double,
            _dp, _dp, _dp, _dp, ctypes.c_int]
        lib.gdn_oracle_causal_conv_silu.restype = None
        lib.gdn_oracle_causal_conv_silu.argtypes = [
            ctypes.c_int64, ctypes.c_int, ctypes.c_int, _dp, _dp, _dp]
        _lib = lib
        return lib


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(_dp)


def softplus(x: float) -> float:
    return _load().gdn_oracle_softplus(float(x))


def sigmoid(x: float) -> float:
    return _load().gdn_oracle_sigmoid(float(x))


def delta_core(alpha, beta, kn, qn, v, S0, terms=False):
    """The recurrence on prepared inputs: alpha, beta [T]; kn, qn [T,Dk];
    v [T,Dv]; S0 [Dv,Dk].  Returns (o [T,Dv], S_T [Dv,Dk]), and with
    terms=True also rss [T,Dv]: the root-sum-square of the Dk products
    S_t[i,j] qn_t[j] that sum to o_t[i] (the size of the terms of each
    output element, a diagnostic for the tests' error bounds)."""
    alpha, beta, kn, qn, v = map(_f64, (alpha, beta, kn, qn, v))
    S = _f64(S0).copy()
    T, Dk = kn.shape
    Dv = v.shape[1]
    o = np.zeros((T, Dv), dtype=np.float64)
    rss = np.zeros((T, Dv), dtype=np.float64) if terms else None
    _load().gdn_oracle_delta_core_terms(T, Dk, Dv, _ptr(alpha), _ptr(beta),
                                        _ptr(kn), Dk, _ptr(qn), Dk, _ptr(v), Dv,
                                        _ptr(S), _ptr(o), Dv, _ptr(rss), Dv)
    return (o, S, rss) if terms else (o, S)


def gated_rmsnorm(o, z, w, eps=1e-6):
    """Row-wise y = o / sqrt(mean(o^2)+eps) * w * silu(z) over the last dim."""
    o = _f64(o)
    z = _f64(z)
    w = _f64(w)
    D = o.shape[-1]
    of = o.reshape(-1, D)
    zf = z.reshape(-1, D)
    y = np.empty_like(of)
    lib = _load()
    for i in range(of.shape[0]):
        lib.gdn_oracle_gated_rmsnorm_row(D, _ptr(of[i]), _ptr(zf[i]), _ptr(w),
                                         float(eps), _ptr(y[i]))
    return y.reshape(o.shape)


def prefill(q, k, v, a, b, A_log, dt_bias, z=None, norm_w=None,
            state_in=None, cu_seqlens=None, scale=None, l2_eps=1e-6,
            norm_eps=1e-6, num_threads=0, terms=False):
    """fp64 gated delta rule prefill.

    q, k: [T, Hk, Dk]; v: [T, Hv, Dv]; a, b: [T, Hv]; A_log, dt_bias: [Hv];
    z: [T, Hv, Dv] or None; norm_w: [Dv] or None; state_in: [N, Hv, Dv, Dk]
    or None (zeros); cu_seqlens: int [N+1] or None (one sequence).
    Inputs of any float dtype are converted exactly to float64 first.
    Returns (o [T, Hv, Dv], state_out [N, Hv, Dv, Dk]) as float64.  With
    terms=True it returns (o, state_out, o_raw, rss): o_raw [T, Hv, Dv] is
    the output before the gated norm and rss [T, Hv, Dv] the size of the
    terms of each o_raw element (see delta_core).
    """
    q, k, v, a, b, A_log, dt_bias = map(_f64, (q, k, v, a, b, A_log, dt_bias))
    z = _f64(z)
    norm_w = _f64(norm_w)
    state_in = _f64(state_in)
    T, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    if scale is None:
        scale = Dk ** -0.5
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        N = cu.shape[0] - 1
        cu_p = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    else:
        cu = None
        N = 1
        cu_p = None
    o = np.zeros((T, Hv, Dv), dtype=np.float64)
    S = np.zeros((N, Hv, Dv, Dk), dtype=np.float64)
    o_raw = np.zeros((T, Hv, Dv), dtype=np.float64) if terms else None
    rss = np.zeros((T, Hv, Dv), dtype=np.float64) if terms else None
    rc = _load().gdn_oracle_prefill_ex(
        N, T, Hk, Hv, Dk, Dv, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
        _ptr(A_log), _ptr(dt_bias), _ptr(z), _ptr(norm_w), _ptr(state_in),
        cu_p, float(scale), float(l2_eps), float(norm_eps), _ptr(o), _ptr(S),
        _ptr(o_raw), _ptr(rss), int(num_threads))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
    return (o, S, o_raw, rss) if terms else (o, S)


def decode(q, k, v, a, b, A_log, dt_bias, cache, slots=None, z=None,
           norm_w=None, scale=None, l2_eps=1e-6, norm_eps=1e-6):
    """fp64 decode step on a slot-addressed state cache.

    Request i brings one token (q[i], k[i], v[i], a[i], b[i], z[i]) of the
    sequence whose state is cache[slots[i]] (cache: [num_slots, Hv, Dv, Dk]);
    the step is, by definition, the prefill of that one-token sequence from
    that state (the recurrence of "Add opt-in fused Qwen3.5 inference
    kernels", Summary, for a single token).  slots=None means request i uses
    slot i.  A slot outside [0, num_slots) marks a padding entry: its output
    row is zero and no state changes.  Live entries must name distinct
    slots.  Returns (o [B, Hv, Dv], new cache) as float64; the cache passed
    in is not modified.
    """
    cache = _f64(cache)
    B = np.asarray(q).shape[0]
    Hv, Dv = np.asarray(v).shape[1], np.asarray(v).shape[2]
    S = cache.shape[0]
    slots = np.arange(B) if slots is None else np.asarray(slots, dtype=np.int64)
    live = [i for i in range(B) if 0 <= slots[i] < S]
    if len({int(slots[i]) for i in live}) != len(live):
        raise ValueError("live requests must name distinct slots")
    new = cache.copy()
    o = np.zeros((B, Hv, Dv), dtype=np.float64)
    for i in live:
        s = int(slots[i])
        zi = None if z is None else np.asarray(z)[i:i + 1]
        o_i, S_i = prefill(np.asarray(q)[i:i + 1], np.asarray(k)[i:i + 1],
                           np.asarray(v)[i:i + 1], np.asarray(a)[i:i + 1],
                           np.asarray(b)[i:i + 1], A_log, dt_bias, zi, norm_w,
                           state_in=cache[s:s + 1], scale=scale, l2_eps=l2_eps,
                           norm_eps=norm_eps)
        o[i] = o_i[0]
        new[s] = S_i[0]
    return o, new


def causal_conv_silu(x, w, history=None):
    """Depthwise causal conv + SiLU.  x: [T, C]; w: [C, W].

    history: [W-1, C] input rows that precede x (oldest first), or None for
    zeros.  The conv with a history is, by definition, the zero-history conv
    of the rows [history; x] with its first W-1 outputs dropped.
    """
    x = _f64(x)
    w = _f64(w)
    T, C = x.shape
    W = w.shape[1]
    if history is not None and W > 1:
        xe = np.concatenate([_f64(history).reshape(W - 1, C), x], axis=0)
        return causal_conv_silu(xe, w)[W - 1:]
    y = np.empty_like(x)
    _load().gdn_oracle_causal_conv_silu(T, C, W, _ptr(x), _ptr(w), _ptr(y))
    return y


def conv_history(x, W, history=None):
    """The last W-1 rows of [history; x] (history None = zeros): the conv
    history a following call continues from.  x: [T, C]."""
    x = _f64(x)
    C = x.shape[1]
    h = np.zeros((W - 1, C)) if history is None else _f64(history).reshape(W - 1, C)
    return np.concatenate([h, x], axis=0)[x.shape[0]:]


# Column order of the packed input projection output: q | k | v | z | b | a.
def layer_split_widths(Hk, Hv, D):
    return [Hk * D, Hk * D, Hv * D, Hv * D, Hv, Hv]


def layer(x, W_in, conv_w, A_log, dt_bias, norm_w, W_out, Hk, Hv, D=128,
          scale=None, l2_eps=1e-6, norm_eps=1e-6, num_threads=0,
          state_in=None, conv_state=None, return_conv_state=False):
    """Full GDN layer in fp64 for one sequence.

    x [T, hidden] @ W_in [hidden, 2*Hk*D + 2*Hv*D + 2*Hv] -> q|k|v|z|b|a;
    causal conv (width conv_w.shape[1]) + SiLU over the q|k|v channels,
    continuing from conv_state [W-1, 2*Hk*D + Hv*D] (None: zero history);
    gated delta rule prefill with gated RMSNorm from state_in [1, Hv, D, D]
    (None: zeros); y [T, Hv*D] @ W_out.
    Returns (out [T, hidden_out], state_out [1, Hv, D, D]) and, with
    return_conv_state, the new conv history [W-1, 2*Hk*D + Hv*D] as a third
    element.
    """
    x, W_in, conv_w, W_out = map(_f64, (x, W_in, conv_w, W_out))
    T = x.shape[0]
    P = x @ W_in
    wq, wk, wv, wz, wb, wa = layer_split_widths(Hk, Hv, D)
    c0 = 0
    qkv = P[:, : wq + wk + wv]
    c0 = wq + wk + wv
    zz = P[:, c0: c0 + wz]
    c0 += wz
    bb = P[:, c0: c0 + wb]
    c0 += wb
    aa = P[:, c0: c0 + wa]
    W = conv_w.shape[1]
    new_hist = conv_history(qkv, W, conv_state) if return_conv_state else None
    qkv = causal_conv_silu(qkv, conv_w, conv_state)
    q = qkv[:, :wq].reshape(T, Hk, D)
    k = qkv[:, wq: wq + wk].reshape(T, Hk, D)
    v = qkv[:, wq + wk:].reshape(T, Hv, D)
    y, S = prefill(q, k, v, aa, bb, A_log, dt_bias, z=zz.reshape(T, Hv, D),
                   norm_w=norm_w, state_in=state_in, scale=scale,
                   l2_eps=l2_eps, norm_eps=norm_eps, num_threads=num_threads)
    out = y.reshape(T, Hv * D) @ W_out
    if return_conv_state:
        return out, S, new_hist
    return out, S
