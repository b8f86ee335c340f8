"""Benchmark of the gated delta rule prefill on one MI355X.

Workload: one gdn_prefill call at the Qwen3.5-4B GDN geometry
(Hq/Hk/Hv/D = 16/16/32/128), one sequence of T = 2048 tokens, bf16 inputs,
fp32 random initial state, gated RMSNorm on -- the T = 2048 single-request
prefill of "feat(qwen35): add SM120 FlashInfer GDN prefill candidate"
(pegainfer PR #862), Performance, at the geometry of its Correctness section.
Synthetic inputs (seeded, i.i.d.) stand in for real prompts.

A step is one full call (all kernels: prep, chain, out) on inputs
already resident in HBM.  Inputs and outputs rotate over several buffer sets
so that the 256 MB last-level cache cannot serve a step from the previous
one.  Prints one JSON line.  Beside the headline it reports the full GDN
layer at T = 2048, hidden 2560 ("layer": time per call and the projection
GEMMs against the bf16 MFMA peak) unless --no-layer is given, and one
decode step for batches of 16 and 128 requests on a slot-addressed state
cache ("decode", against the HBM peak) unless --no-decode is given, and the
other prefill workloads ("configs": T=2048 in four calls carrying the
state, a packed batch of 8 short sequences, Hv=48, and the latency-bound
short cases) unless --no-configs is given.  "call_us" gives the median,
p10 and p90 of single calls beside the K-step average.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--no-layer] [--no-decode] [--no-configs]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, TFLOP/s
T_TOK, HK, HV, D = 2048, 16, 32, 128
ELEM = 2  # bf16
# q, k (Hk x D each), v, z, y (Hv x D each), a, b (Hv each), bf16
TOKEN_BYTES = ELEM * (2 * HK * D + 3 * HV * D + 2 * HV)


def algorithmic_bytes(T, Hk, Hv, Dh, N=1, norm=True):
    """Bytes the operator must move at minimum: its inputs and outputs once
    (q, k, v, a, b, z in; y out; fp32 state in and out; the per-head
    parameters), every intermediate kept on chip."""
    per_tok = ELEM * (2 * Hk * Dh + Hv * Dh + 2 * Hv + Hv * Dh)  # q k v a b o
    if norm:
        per_tok += ELEM * Hv * Dh  # z
    params = 4 * (2 * Hv + (Dh if norm else 0))
    state = 2 * N * Hv * Dh * Dh * 4
    return T * per_tok + state + params


def stage_bytes(T, Hk, Hv, Dh, N=1):
    """The operator's algorithmic bytes split over its kernels, each input
    and output counted once, in the first kernel that reads it (or the
    kernel that writes it): the parts add up to algorithmic_bytes (less the
    per-head parameters).  The workspace is intermediate traffic, and the
    re-reads of q and k by later kernels are not counted."""
    return {
        "prep": T * ELEM * (2 * Hk * Dh + 2 * Hv),              # q, k, a, b
        "chain": T * ELEM * (Hv * Dh)                           # v
        + 2 * N * Hv * Dh * Dh * 4,                             # state in/out
        "out": T * ELEM * (2 * Hv * Dh),                        # z; y
    }


KERNEL_SOURCES = ("gdn_prefill.hip", "gdn_frag.hpp", "gdn_internal.hpp", "gdn_math.hpp")
# every file the library is built from, plus this script: the source tree a
# result belongs to, on a box with no git checkout
TREE_SOURCES = ("gated_deltanet_linear_04_amd/csrc", "include",
                "gated_deltanet_linear_04_amd/binding.py", "bench.py")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles",
                               "gdn_prefill_T2048_4b_fabric_traffic.md")


def kernel_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_deltanet_linear_04_amd", "csrc")
    for f in KERNEL_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(kernel):
    """L2-to-fabric bytes per launch of `kernel` from the committed
    rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE, scaled by a plain
    copy's reading; they include hits in the last-level cache, so they
    bound the HBM bytes from above), or None when that summary was taken on
    other kernel sources."""
    try:
        lines = open(TRAFFIC_PROFILE).read().splitlines()
    except OSError:
        return None
    sha, vals = None, {}
    for ln in lines:
        parts = ln.split()
        if len(parts) == 2 and parts[0] == "kernel_sources_sha256":
            sha = parts[1]
        elif len(parts) == 3 and parts[0] == "traffic_bytes_per_launch":
            vals[parts[1]] = float(parts[2])
    if sha is None or sha != kernel_sources_sha256():
        return None
    return vals.get(kernel)


def algorithmic_flops(T, Hk, Hv, Dh, C=64):
    """Chunked (WY) form: Gram products per key head (K K^T, Q K^T), per
    value head the inverse (~C^3/3 per chunk), Tb R, MP V', and the three
    state products (K H, Q H, K^T V')."""
    nch = math.ceil(T / C)
    gram = nch * Hk * 2 * (2 * C * C * Dh)
    inv = nch * Hv * (C ** 3 / 3) * 2
    per_vh = nch * Hv * (2 * C * C * Dh * 2          # Tb R, MP V'
                         + 3 * 2 * C * Dh * Dh)      # K H, Q H, K^T V'
    return gram + inv + per_vh


def git_info():
    """(short revision, dirty) of the checkout, or (None, None) when the tree
    is not a git checkout (then nothing is known about its state)."""
    try:
        p = subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT,
                           capture_output=True, text=True)
        rev = p.stdout.strip()
        if p.returncode != 0 or not rev:
            return None, None
        st = subprocess.run(["git", "status", "--porcelain"], cwd=ROOT,
                            capture_output=True, text=True)
        if st.returncode != 0:
            return rev, None
        return rev, bool(st.stdout.strip())
    except Exception:
        return None, None


def tree_sources_sha256():
    """sha256 over the library's sources, its header and this script (file
    names and contents, in sorted order)."""
    import hashlib
    h = hashlib.sha256()
    files = []
    for rel in TREE_SOURCES:
        path = os.path.join(ROOT, rel)
        if os.path.isdir(path):
            files += [os.path.join(rel, f) for f in sorted(os.listdir(path))
                      if os.path.isfile(os.path.join(path, f))]
        else:
            files.append(rel)
    for rel in sorted(files):
        h.update(rel.encode() + b"\0")
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def platform_info():
    """ROCm version and the GPU's current engine clock, as far as this
    process can read them without privileges."""
    info = {"rocm_version": None, "sclk_mhz": None}
    try:
        with open("/opt/rocm/.info/version") as fh:
            info["rocm_version"] = fh.read().strip()
    except OSError:
        pass
    try:
        import glob
        for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
            for ln in open(f).read().splitlines():
                if ln.strip().endswith("*"):
                    info["sclk_mhz"] = ln.split(":", 1)[1].strip().rstrip("*").strip()
                    break
            if info["sclk_mhz"]:
                break
    except OSError:
        pass
    return info


def cpu_baseline(target_s=12.0):
    """The fp64 oracle on this host's cores, on the same workload (T=2048,
    4B geometry, gated norm on), repeated to ~target_s seconds."""
    import oracle
    from gated_deltanet_linear_04_amd import synth

    case = synth.case_f64(synth.config2_case())
    try:
        cores = len(os.sched_getaffinity(0))
    except Exception:
        cores = os.cpu_count() or 1
    threads = max(1, min(cores, HV))
    args = (case["q"], case["k"], case["v"], case["a"], case["b"],
            case["A_log"], case["dt_bias"])
    kw = dict(z=case["z"], norm_w=case["norm_w"], state_in=case["state_in"],
              num_threads=threads)
    oracle.prefill(*args, **kw)  # warm (thread pool, pages)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.prefill(*args, **kw)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 1000:
            break
    # the same call on one thread: the median of three
    kw["num_threads"] = 1
    one = []
    for _ in range(3):
        t1 = time.perf_counter()
        oracle.prefill(*args, **kw)
        one.append(time.perf_counter() - t1)
    one_s = float(np.median(one))
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": reps * T_TOK / el, "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "host_cpu": model, "host_nproc": os.cpu_count(),
            "sample": "%d full calls of the T=2048 workload (fp64, %d threads, "
                      "%.1f s)" % (reps, threads, el),
            "single_thread": {"value": T_TOK / one_s, "unit": "tokens/s",
                              "sample": "median of 3 full calls on 1 thread "
                                        "(%.2f s each)" % one_s}}


def layer_measure(torch, binding, synth, dev, steps=20, warmup=10):
    """The full GDN layer at T=2048, hidden 2560 (4B geometry): time per
    call, and the two projection GEMMs on their own against the bf16 MFMA
    peak.  Random-init weights of the layer's shapes (synthetic)."""
    import numpy as np
    c = synth.layer_case(synth.seed_for(4, 0), T=T_TOK)

    def to_dev(x):
        return to_device(torch, x, dev)

    x = to_dev(c["x"])
    W_in = to_dev(np.ascontiguousarray(c["W_in"].T))
    W_out = to_dev(np.ascontiguousarray(c["W_out"].T))
    args = (x, W_in, to_dev(c["conv_w"]), to_dev(c["A_log"]),
            to_dev(c["dt_bias"]), to_dev(c["norm_w"]), W_out, HK, HV)
    desc = binding.make_layer_desc(1, T_TOK, c["hidden"], HK, HV, 4)
    ws = torch.empty(binding.layer_workspace_size(desc), dtype=torch.uint8,
                     device=dev)
    out = torch.empty(T_TOK, c["hidden"], dtype=torch.bfloat16, device=dev)
    S = torch.empty(1, HV, D, D, dtype=torch.float32, device=dev)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return 1000.0 * e0.elapsed_time(e1) / steps

    # the library's default (the conv a kernel of its own) and the conv
    # applied inside the prefill's first kernel (conv_fused = 1), timed in
    # alternating rounds: medians of five each, so that clock and cache
    # drift between the two do not decide their order
    # the clocks ramp over the first tens of milliseconds of a sustained
    # load: run the layer for about that long before the timed rounds
    for _ in range(60):
        binding.layer_prefill(*args, out=out, state_out=S, workspace=ws)
    torch.cuda.synchronize()
    sep, fus = [], []
    for _ in range(5):
        sep.append(timed(lambda: binding.layer_prefill(*args, out=out, state_out=S,
                                                       workspace=ws)))
        fus.append(timed(lambda: binding.layer_prefill(*args, out=out, state_out=S,
                                                       workspace=ws, conv_fused=1)))
    us, us_fused = float(np.median(sep)), float(np.median(fus))
    res = {"workload": "GDN layer T=2048 hidden=2560 Hk/Hv/D=16/32/128 bf16: "
                       "in_proj GEMM 2560->12352, conv1d(4)+SiLU, gdn_prefill "
                       "with gated RMSNorm, out_proj 4096->2560; zero state",
           "us_per_call": us, "tokens_per_s": T_TOK / (us * 1e-6),
           "conv": "a kernel of its own (the library's default)",
           "us_per_call_fused_conv": us_fused,
           "rounds_us": {"separate_conv": sep, "fused_conv": fus}}
    for name, (M, N, K) in (("in_proj", (T_TOK, W_in.shape[0], c["hidden"])),
                            ("out_proj", (T_TOK, c["hidden"], HV * D))):
        A = torch.randn(M, K, device=dev).to(torch.bfloat16)
        B = (0.02 * torch.randn(N, K, device=dev)).to(torch.bfloat16)
        C = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        # median of five rounds after a warm-up of its own, as for the
        # layer: the clocks drift under a sustained matrix load
        for _ in range(100):
            binding.gemm(A, B, out=C)
        torch.cuda.synchronize()
        g_rounds = [timed(lambda: binding.gemm(A, B, out=C)) for _ in range(5)]
        g_us = float(np.median(g_rounds))
        tf = 2.0 * M * N * K / (g_us * 1e-6) / 1e12
        res[name] = {"M": M, "N": N, "K": K, "us": g_us, "tflops": tf,
                     "mfma_frac": tf / BF16_PEAK_TFLOPS, "rounds_us": g_rounds}
    return res


def measured_peaks(torch, binding, dev):
    """Peaks measured on this device, reported beside the datasheet ones:
    HBM bandwidth of a plain device copy of 1 GiB (bytes read + written per
    second), and the bf16 rate of the library's MFMA probe (register-only
    MFMA loop on every SIMD)."""
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    t_copy = timed(lambda: dst.copy_(src), 10)
    del src, dst
    blocks, iters = 256 * 8, 20000
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    t_mfma = timed(lambda: binding.mfma_probe(iters, blocks, out), 3)
    flop = 2.0 * 16 * 16 * 32 * 8 * iters * blocks * 4
    return {"hbm_copy_GBs": 2.0 * (1 << 30) / t_copy / 1e9,
            "mfma_bf16_TFLOPs": flop / t_mfma / 1e12,
            "how": "1 GiB device copy (read + write); MFMA probe "
                   "(2048 blocks x 4 waves x 20000 rounds of 8 "
                   "16x16x32 bf16 MFMAs)"}


def decode_measure(torch, binding, synth, dev, batches=(16, 128), reps=3):
    """gdn_decode on the 4B geometry (bf16, gated norm on): one step for B
    requests, each on its own slot of a state cache.  The cache holds
    `nsets` disjoint batches of slots (more than the 256 MB last-level
    cache), and one HIP graph steps each batch once in turn, so every step
    reads its states from HBM.  Algorithmic bytes per request: the state
    read and written (2 x Hv x 128 x 128 x 4) plus the token's q, k, v, a,
    b, z in and y out (32,896 B)."""
    import numpy as np
    res = []
    for B in batches:
        per_set = B * HV * D * D * 4
        nsets = max(2, int(math.ceil(384e6 / per_set)))
        c = synth.decode_case(synth.seed_for(5, B), B, HK, HV, 1,
                              identity_slots=True)

        def to_dev(x):
            return to_device(torch, x, dev)

        t = {k: to_dev(c[k]) for k in ("q", "k", "v", "a", "b", "A_log",
                                       "dt_bias", "z", "norm_w")}
        cache = 0.02 * torch.randn(nsets * B, HV, D, D, device=dev)
        slots = [torch.arange(j * B, (j + 1) * B, dtype=torch.int32,
                              device=dev) for j in range(nsets)]
        out = torch.empty(B, HV, D, dtype=torch.bfloat16, device=dev)

        def step(j):
            binding.decode(t["q"], t["k"], t["v"], t["a"], t["b"], t["A_log"],
                           t["dt_bias"], cache, slots[j], z=t["z"],
                           norm_w=t["norm_w"], out=out)

        for j in range(nsets):
            step(j)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for j in range(nsets):
                    step(j)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = 1000.0 * e0.elapsed_time(e1) / (reps * nsets)
        nbytes = B * (2 * HV * D * D * 4 + TOKEN_BYTES)
        gbs = nbytes / (us * 1e-6) / 1e9
        res.append({"workload": "gdn_decode B=%d Hk/Hv/D=16/32/128 bf16, "
                                "gated RMSNorm on, states in HBM" % B,
                    "B": B, "us_per_step": us,
                    "algorithmic_bytes": nbytes, "achieved_GBs": gbs,
                    "frac_hbm": gbs / HBM_PEAK_GBS})
        del cache
    return res


def to_device(torch, x, dev):
    """numpy storage array (float32, int32, or uint16 bf16 bits) -> device
    tensor; None stays None."""
    if x is None:
        return None
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)
                                .copy()).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def per_call_us(torch, unit, reps, warmup=3):
    """Device time of each of `reps` consecutive calls of unit(i), from HIP
    events recorded between them on the current stream (the stream the
    library launches on): median, p10 and p90 in microseconds."""
    for i in range(warmup):
        unit(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        unit(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    d = np.array([1000.0 * ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])
    return {"median_us": float(np.median(d)),
            "p10_us": float(np.percentile(d, 10)),
            "p90_us": float(np.percentile(d, 90)), "calls": reps}


def graph_call_us(torch, unit, calls, replays=15):
    """Device time per call of unit(i) with host submission taken out: the
    calls unit(0) .. unit(calls - 1) are captured into one HIP graph, the
    graph is replayed `replays` times with HIP events between replays, and
    each replay's time is divided by `calls`.  Median, p10 and p90 over the
    replays, in microseconds."""
    for i in range(calls):
        unit(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(calls):
                unit(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(replays + 1)]
    ev[0].record()
    for r in range(replays):
        g.replay()
        ev[r + 1].record()
    torch.cuda.synchronize()
    d = np.array([1000.0 * ev[r].elapsed_time(ev[r + 1]) / calls
                  for r in range(replays)])
    del g
    return {"median_us": float(np.median(d)),
            "p10_us": float(np.percentile(d, 10)),
            "p90_us": float(np.percentile(d, 90)),
            "timing": "HIP graph of %d calls, %d replays" % (calls, replays)}


def configs_measure(torch, binding, synth, dev, reps=30):
    """The other prefill workloads, each timed per call (median, p10, p90),
    with inputs and outputs rotated over enough buffer sets to exceed the
    256 MB last-level cache where the workload is HBM-bound:
      * T=2048 as four 512-token calls carrying the state (the state of one
        call is the next call's state_in, updated in place);
      * a packed batch of 8 sequences of 32..128 tokens, one state each;
      * Hv=48 (three value heads per key head) at T=128;
      * one long prompt on one GPU's share of the heads at 8-way head
        sharding (Hk/Hv = 2/4, T = 16,384, bf16 and fp32), with the state
        chain as the library runs it (a sequence-parallel scan) and as one
        pass (chain_segments = 1), on weak-decay heads (A_log from -6 to
        -1, dt_bias -2) so that the state carries across the sequence;
      * latency only: the per-GPU share at 8-way head sharding (fp32, T=64,
        Hk=2, Hv=4, no state, no norm) and single sequences of 1..128
        tokens at the 4B geometry.
    The HBM-bound ones report their algorithmic bytes against 8 TB/s.
    Times come from HIP graph replays (host submission excluded: through
    the Python binding, one call costs about 30 us of host time, more than
    the device time of the short cases); "eager_median_us" is the same call
    issued from Python, one event pair per call."""
    res = {}

    def dev_sets(case, nsets):
        keys = ("q", "k", "v", "a", "b", "A_log", "dt_bias", "z", "norm_w",
                "state_in", "cu_seqlens")
        base = {k: to_device(torch, case[k], dev) for k in keys}
        sets = []
        for i in range(nsets):
            st = {k: (v.clone() if (i and v is not None) else v)
                  for k, v in base.items()}
            sets.append(st)
        return sets

    def nsets_for(nbytes):
        return int(min(64, max(2, math.ceil(384e6 / nbytes))))

    def call(st, sl=None, state_in=None, state_out=None, ws=None, **kw):
        r = slice(None) if sl is None else sl
        binding.prefill(st["q"][r], st["k"][r], st["v"][r], st["a"][r],
                        st["b"][r], st["A_log"], st["dt_bias"],
                        z=None if st["z"] is None else st["z"][r],
                        norm_w=st["norm_w"],
                        state_in=st["state_in"] if state_in is None else state_in,
                        cu_seqlens=st["cu_seqlens"], out=st["o"][r],
                        state_out=state_out, workspace=ws, **kw)

    def add_outputs(sets, case):
        dt = torch.bfloat16 if case["dtype"] == synth.BF16 else torch.float32
        for st in sets:
            st["o"] = torch.empty(case["T"], case["Hv"], D, dtype=dt, device=dev)
            st["S"] = torch.empty(case["N"], case["Hv"], D, D,
                                  dtype=torch.float32, device=dev)

    def timed(unit, nsets):
        t = graph_call_us(torch, unit, nsets * int(math.ceil(16 / nsets)))
        t["eager_median_us"] = per_call_us(torch, unit, reps)["median_us"]
        return t

    def report(name, workload, case, t, nbytes=None):
        r = {"workload": workload, "tokens": case["T"], "sequences": case["N"]}
        r.update(t)
        r["tokens_per_s"] = case["T"] / (t["median_us"] * 1e-6)
        if nbytes is not None:
            r["algorithmic_bytes"] = nbytes
            r["t_roofline_us"] = nbytes / (HBM_PEAK_GBS * 1e3)
            r["frac_hbm"] = r["t_roofline_us"] / t["median_us"]
        res[name] = r

    # T=2048 in four 512-token calls, state carried through S
    case = synth.config2_case()
    part = 512
    nb = 4 * algorithmic_bytes(part, HK, HV, D)
    sets = dev_sets(case, nsets_for(nb))
    add_outputs(sets, case)
    ws = torch.empty(binding.workspace_size(binding.make_desc(
        1, part, HK, HV, torch.bfloat16)), dtype=torch.uint8, device=dev)

    def chunked(i):
        st = sets[i % len(sets)]
        for j in range(4):
            call(st, slice(j * part, (j + 1) * part),
                 state_in=st["state_in"] if j == 0 else st["S"],
                 state_out=st["S"], ws=ws)

    report("chunked_4x512", "gdn_prefill T=2048 as 4 calls of 512 tokens "
           "carrying the state, 4B geometry, bf16, gated RMSNorm on", case,
           timed(chunked, len(sets)), nb)

    # packed varlen batch and the Hv=48 case
    for name, case, what in (
            ("varlen_8", synth.config3_case(),
             "gdn_prefill 8 packed sequences of 32..128 tokens (cu_seqlens), "
             "one random state each, 4B geometry, bf16, gated RMSNorm on"),
            ("hv48_T128", synth.config3_hv48_case(),
             "gdn_prefill T=128 Hk/Hv/D=16/48/128, bf16, random state, "
             "gated RMSNorm on")):
        nb = algorithmic_bytes(case["T"], case["Hk"], case["Hv"], D, N=case["N"])
        sets = dev_sets(case, nsets_for(nb))
        add_outputs(sets, case)
        dt = torch.bfloat16
        ws = torch.empty(binding.workspace_size(binding.make_desc(
            case["N"], case["T"], case["Hk"], case["Hv"], dt)),
            dtype=torch.uint8, device=dev)

        def unit(i, sets=sets, ws=ws):
            st = sets[i % len(sets)]
            call(st, state_out=st["S"], ws=ws)

        report(name, what + " (%d tokens)" % case["T"], case,
               timed(unit, len(sets)), nb)

    # one long prompt on few heads: the scan against one pass
    for dtype, dname in ((synth.BF16, "bf16"), (synth.F32, "fp32")):
        case = synth.make_case(96_500, 16_384, 2, 4, dtype=dtype)
        case["A_log"] = np.linspace(-6.0, -1.0, 4).astype(np.float32)
        case["dt_bias"] = np.full(4, -2.0, dtype=np.float32)
        dt = torch.bfloat16 if dtype == synth.BF16 else torch.float32
        nb = algorithmic_bytes(case["T"], 2, 4, D) * (2 if dtype == synth.F32 else 1)
        sets = dev_sets(case, nsets_for(nb))
        add_outputs(sets, case)
        for segs, tag in ((None, "scan"), (1, "one_pass")):
            desc = binding.make_desc(1, case["T"], 2, 4, dt, chain_segments=segs)
            ws = torch.empty(binding.workspace_size(desc), dtype=torch.uint8, device=dev)

            def unit(i, sets=sets, ws=ws, segs=segs):
                st = sets[i % len(sets)]
                call(st, state_out=st["S"], ws=ws, chain_segments=segs)

            report("head_share_T16384_%s_%s" % (dname, tag),
                   "gdn_prefill T=16384 Hk/Hv/D=2/4/128 %s, random state, gated RMSNorm "
                   "on, weak-decay heads, state chain %s" % (
                       dname, "as the library runs it (scan)" if segs is None else "in one pass"),
                   case, timed(unit, len(sets)), nb)

    # latency-bound cases: time per call only
    small = [("head_share_fp32_T64", synth.config0_case(),
              "gdn_prefill fp32 T=64 Hk/Hv/D=2/4/128, zero state, no norm "
              "(one GPU's share at 8-way head sharding)")]
    for T in synth.CONFIG1_TS:
        small.append(("single_T%d" % T, synth.config1_case(T),
                      "gdn_prefill T=%d 4B geometry bf16, random state, gated "
                      "RMSNorm on" % T))
    for name, case, what in small:
        sets = dev_sets(case, 2)
        add_outputs(sets, case)
        dt = torch.bfloat16 if case["dtype"] == synth.BF16 else torch.float32
        ws = torch.empty(binding.workspace_size(binding.make_desc(
            case["N"], case["T"], case["Hk"], case["Hv"], dt)),
            dtype=torch.uint8, device=dev)

        def unit(i, sets=sets, ws=ws):
            st = sets[i % len(sets)]
            call(st, state_out=st["S"], ws=ws)

        report(name, what, case, timed(unit, len(sets)))
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=6,
                    help="rotated input/output buffer sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-layer", action="store_true",
                    help="skip the full-layer measurement")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-step measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other prefill workloads (chunked, varlen, "
                         "Hv=48, short sequences)")
    ap.add_argument("--copy-calibrate-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB "
                         "(reference kernel for the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU "
              "path (the operator would shard over sequences and heads with "
              "no communication).  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_deltanet_linear_04_amd import binding, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")

    if args.copy_calibrate_mib:
        n = args.copy_calibrate_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n * 4, "launches": 5}))
        return

    binding.load()
    case = synth.config2_case()

    base = {k: to_device(torch, case[k], dev) for k in ("q", "k", "v", "a", "b", "A_log",
                                         "dt_bias", "z", "norm_w",
                                         "state_in")}
    sets = []
    for i in range(args.sets):
        s = {k: (v.clone() if i else v) for k, v in base.items()}
        s["o"] = torch.empty(T_TOK, HV, D, dtype=torch.bfloat16, device=dev)
        s["S"] = torch.empty(1, HV, D, D, dtype=torch.float32, device=dev)
        sets.append(s)
    desc = binding.make_desc(1, T_TOK, HK, HV, torch.bfloat16)
    ws_bytes = binding.workspace_size(desc)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def step(i):
        s = sets[i % len(sets)]
        binding.prefill(s["q"], s["k"], s["v"], s["a"], s["b"], s["A_log"],
                        s["dt_bias"], z=s["z"], norm_w=s["norm_w"],
                        state_in=s["state_in"], out=s["o"], state_out=s["S"],
                        workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly K steps, no per-stage events
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / args.steps

    # second pass of K steps with the library's per-kernel HIP events (on
    # the stream the kernels run on), for the per-kernel roofline
    binding.stage_timing_enable(args.steps)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    stage_ms, calls = binding.stage_timing_read()
    binding.stage_timing_enable(0)
    # a T = 2048 call runs the three chunked kernels; the single-kernel
    # form's stage stays empty
    stage_avg_us = {k: 1000.0 * v / max(calls, 1) for k, v in stage_ms.items()
                    if k in ("prep", "chain", "out")}

    # third pass: each call's own device time (events between calls), for
    # the median and spread; the headline stays the K-step average above
    call_us = per_call_us(torch, step, args.steps, warmup=0)

    sb = stage_bytes(T_TOK, HK, HV, D)
    dom = max(stage_avg_us, key=lambda k: stage_avg_us[k])
    op_bytes = algorithmic_bytes(T_TOK, HK, HV, D)
    # the headline roofline is the whole operator's: its algorithmic bytes
    # per call over the measured time of a call
    achieved = op_bytes / (ms_step * 1e-3) / 1e9
    traffic_parts = [stored_traffic(k) for k in stage_avg_us]
    traffic = (sum(traffic_parts) if traffic_parts and
               all(t is not None for t in traffic_parts) else None)
    op_flops = algorithmic_flops(T_TOK, HK, HV, D)
    t_roof_us = max(op_bytes / (HBM_PEAK_GBS * 1e3),
                    op_flops / (BF16_PEAK_TFLOPS * 1e6))
    rev, dirty = git_info()
    prop = torch.cuda.get_device_properties(dev)

    line = {
        "metric": "GDN prefill tokens/sec/GPU @ Qwen3.5-4B geom T=2048; "
                  "% MFMA/HBM roofline",
        "value": T_TOK / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gdn_prefill T=2048 Hq/Hk/Hv/D=16/16/32/128 "
                               "bf16, fp32 random initial state, gated "
                               "RMSNorm on, one sequence",
                   "global_batch": 1, "seq_len": T_TOK,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": "gdn_prefill call (%s)"
                     % " + ".join(stage_avg_us),
                     "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "traffic_counts": "L2-to-fabric bytes (rocprofv3 "
                                       "FETCH_SIZE + WRITE_SIZE, scaled by a "
                                       "plain copy's reading), which include "
                                       "last-level-cache hits",
                     "algorithmic_bytes_per_launch": op_bytes,
                     "avg_launch_us": ms_step * 1e3,
                     "dominant_kernel": dom,
                     "dominant_kernel_us": stage_avg_us[dom]},
        "op_roofline": {"bound": "hbm", "algorithmic_bytes": op_bytes,
                        "algorithmic_flops": op_flops,
                        "t_roofline_us": t_roof_us,
                        "t_call_us": ms_step * 1e3,
                        "frac": t_roof_us / (ms_step * 1e3),
                        "achieved_GBs": op_bytes / (ms_step * 1e-3) / 1e9},
        "call_us": call_us,
        "stage_us": stage_avg_us,
        # every prefill kernel against the HBM peak (same definitions as
        # "roofline", which reports the one with the longest launch)
        "kernels": {k: {"avg_launch_us": stage_avg_us[k],
                        "algorithmic_bytes_per_launch": sb[k],
                        "achieved_GBs": sb[k] / (stage_avg_us[k] * 1e-6) / 1e9,
                        "frac": sb[k] / (stage_avg_us[k] * 1e-6) / 1e9 / HBM_PEAK_GBS,
                        "traffic": stored_traffic(k)}
                    for k in stage_avg_us},
        "workspace_bytes": ws_bytes,
        "wall_s_timed": wall,
        "device": prop.name,
        "cus": prop.multi_processor_count,
        "git": rev, "dirty": dirty,
        "kernel_sources_sha256": kernel_sources_sha256(),
        "tree_sources_sha256": tree_sources_sha256(),
        "torch": torch.__version__,
    }
    line.update(platform_info())
    peaks = measured_peaks(torch, binding, dev)
    line["peaks_measured"] = peaks
    line["roofline"]["frac_of_measured_peak"] = achieved / peaks["hbm_copy_GBs"]
    line["op_roofline"]["frac_of_measured_peak"] = (
        op_bytes / (peaks["hbm_copy_GBs"] * 1e3)) / (ms_step * 1e3)
    if not args.no_layer:
        line["layer"] = layer_measure(torch, binding, synth, dev)
        for g in ("in_proj", "out_proj"):
            line["layer"][g]["frac_of_measured_peak"] = (
                line["layer"][g]["tflops"] / peaks["mfma_bf16_TFLOPs"])
    if not args.no_decode:
        line["decode"] = decode_measure(torch, binding, synth, dev)
    if not args.no_configs:
        line["configs"] = configs_measure(torch, binding, synth, dev)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
