"""Helpers shared by the GPU tests: host<->device conversion of the seeded
cases, the oracle call on the same values, and the parity metric.

Parity metric (fixed before any kernel existed): for each (sequence, value
head) slice of the output and of the final state, rel = ||x - ref||_2 /
||ref||_2; the case passes when the largest rel over all slices is at most
1e-4 for fp32 inputs and 2e-2 for bf16 inputs.  Taking the maximum over
slices keeps a small head from hiding behind a large one.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from gated_deltanet_linear_04_amd import binding, synth

TOL = {synth.F32: 1e-4, synth.BF16: 2e-2}


def to_dev(arr, device):
    if arr is None:
        return None
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        t = torch.from_numpy(arr.view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(arr.copy())
    return t.to(device)


def to_f64(t):
    if t is None:
        return None
    return t.detach().float().cpu().numpy().astype(np.float64)


def device_case(case, device):
    keys = ("q", "k", "v", "a", "b", "A_log", "dt_bias", "z", "norm_w",
            "state_in", "cu_seqlens")
    return {k: to_dev(case[k], device) for k in keys}


def run_gpu(case, device, **kw):
    d = device_case(case, device)
    o, S = binding.prefill(d["q"], d["k"], d["v"], d["a"], d["b"],
                           d["A_log"], d["dt_bias"], z=d["z"],
                           norm_w=d["norm_w"], state_in=d["state_in"],
                           cu_seqlens=d["cu_seqlens"], **kw)
    torch.cuda.synchronize(device)
    return o, S


def run_oracle(case, **kw):
    c = synth.case_f64(case)
    return oracle.prefill(c["q"], c["k"], c["v"], c["a"], c["b"], c["A_log"],
                          c["dt_bias"], z=c["z"], norm_w=c["norm_w"],
                          state_in=c["state_in"], cu_seqlens=c["cu_seqlens"],
                          **kw)


def slices(case):
    cu = case["cu_seqlens"]
    if cu is None:
        return [(0, 0, case["T"])]
    return [(n, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]


def parity(case, o, S, o_ref, S_ref):
    """Returns (max rel over output slices, max rel over state slices,
    elementwise stats of the state error)."""
    o = np.asarray(o, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    rel_o = 0.0
    rel_s = 0.0
    Hv = o_ref.shape[1]
    for n, t0, t1 in slices(case):
        for h in range(Hv):
            if t1 > t0:
                ref = o_ref[t0:t1, h]
                den = np.linalg.norm(ref)
                num = np.linalg.norm(o[t0:t1, h] - ref)
                rel_o = max(rel_o, num / den if den > 0 else num)
            ref = S_ref[n, h]
            den = np.linalg.norm(ref)
            num = np.linalg.norm(S[n, h] - ref)
            rel_s = max(rel_s, num / den if den > 0 else num)
    err = np.abs(S - S_ref)
    stats = dict(max_abs=float(err.max()) if err.size else 0.0,
                 mean_abs=float(err.mean()) if err.size else 0.0,
                 p99_abs=float(np.percentile(err, 99)) if err.size else 0.0)
    return rel_o, rel_s, stats


def check_parity(case, device, label="", **kw):
    o, S = run_gpu(case, device, **kw)
    okw = {k: v for k, v in kw.items() if k in ("scale", "l2_eps", "norm_eps")}
    o_ref, S_ref = run_oracle(case, **okw)
    rel_o, rel_s, stats = parity(case, to_f64(o), to_f64(S), o_ref, S_ref)
    tol = TOL[case["dtype"]]
    print("[parity] %s T=%d Hk=%d Hv=%d N=%d dtype=%s rel_o=%.3e rel_state=%.3e "
          "state max/mean/p99 abs=%.2e/%.2e/%.2e" % (
              label, case["T"], case["Hk"], case["Hv"], case["N"],
              case["dtype"], rel_o, rel_s, stats["max_abs"],
              stats["mean_abs"], stats["p99_abs"]), flush=True)
    assert rel_o <= tol, (label, rel_o, tol)
    assert rel_s <= tol, (label, rel_s, tol)
    return o, S, rel_o, rel_s, stats
