"""GPU parity of gdn_decode (one token per request on a slot-addressed state
cache) against the fp64 oracle, called through the C ABI.

Bar: the step runs entirely in fp32 on inputs that the oracle sees exactly
(bf16 -> fp64 is exact), so the only differences are fp32 rounding in
128-term dot products (relative ~1e-6) and, for bf16 outputs, the final
round-to-nearest-even of o (bf16 keeps 8 significant bits: at most 2^-8 =
3.9e-3 relative per element, about 2.3e-3 rms).  Per (request, value head)
slice: rel L2 of o <= 4e-3 (bf16) or 2e-5 (fp32); rel L2 of the updated
state <= 2e-5; and every element within the same bar times (|r| + rms of its
slice) (tests/parity_metrics.py).  Slots the batch does not name, and
padding entries, must leave the cache bit-identical; padding rows of o are
exactly zero.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_linear_04_amd import binding, synth
from tests import gpu_helpers as G
from tests import parity_metrics as PM
from tests.fp32_cases import DECODE_SWEEP_IDS

pytestmark = pytest.mark.gpu

# Bars from the arithmetic of a well-conditioned step: fp32 throughout on
# inputs the oracle sees exactly, plus the final bf16 rounding of o for bf16.
# A (request, head) whose o is small through cancellation (q nearly
# orthogonal to what the state and the new key hold) has a relative error
# set by that cancellation in any fp32 evaluation: a plain fp32 numpy step
# misses 2e-5 there too (1.7e-4 on one such head).  For fp32 the output bar
# is therefore scaled by the condition number kappa = ||S||_F ||q^|| / ||S q^||
# of the step's output product (tests/parity_metrics.py).
TOL_O = {synth.F32: 2e-5, synth.BF16: 4e-3}
TOL_S = 2e-5


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load()
    return torch.device("cuda:0")


def _say(msg):
    print("[case] " + msg, flush=True)


def _run(case, dev, cache_dev=None):
    d = {k: G.to_dev(case[k], dev) for k in
         ("q", "k", "v", "a", "b", "A_log", "dt_bias", "z", "norm_w")}
    if cache_dev is None:
        cache_dev = G.to_dev(case["cache"], dev)
    slots = G.to_dev(case["slots"], dev)
    o = binding.decode(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"],
                       d["dt_bias"], cache_dev, slots, z=d["z"],
                       norm_w=d["norm_w"])
    torch.cuda.synchronize(dev)
    return o, cache_dev


def _oracle(case, cache=None):
    c = synth.case_f64(case)
    return oracle.decode(c["q"], c["k"], c["v"], c["a"], c["b"], c["A_log"],
                         c["dt_bias"],
                         case["cache"] if cache is None else cache,
                         case["slots"], z=c["z"], norm_w=c["norm_w"])


def _rel(x, ref):
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    return num / den if den > 0 else num


def _check(case, o, cache_after, label):
    """Per (request, value head): relative L2 and every element of o and of
    the updated state against the bars (tests/parity_metrics.py).  An fp32
    output's bar is scaled by the conditioning of o = S q^ (one token per
    request)."""
    o_ref, cache_ref = _oracle(case)
    o = G.to_f64(o)
    S = G.to_f64(cache_after)
    B, Hv = o.shape[0], o.shape[1]
    r = Hv // case["Hk"]
    q64 = synth.storage_to_f64(case["q"], case["dtype"])
    z64 = synth.storage_to_f64(case["z"], case["dtype"]) if case["z"] is not None else None
    nslots = case["cache"].shape[0]
    slots = case["slots"] if case["slots"] is not None else np.arange(B)
    live = {int(s) for s in slots if 0 <= s < nslots}
    t_o, t_s = PM.Tally(), PM.Tally()
    for i in range(B):
        s = int(slots[i])
        if not (0 <= s < nslots):
            assert np.all(o[i] == 0.0), (label, "padding row", i)
            continue
        for h in range(Hv):
            kappa = 1.0
            if case["dtype"] == synth.F32:
                kappa = PM.one_token_kappa(cache_ref[s, h],
                                           PM.qhat(q64[i, h // r], 128 ** -0.5))
            gsc = None if z64 is None else PM.gate(case["norm_w"], z64[i, h])
            t_o.add(o[i, h], o_ref[i, h], TOL_O[case["dtype"]], kappa, gsc)
            t_s.add(S[s, h], cache_ref[s, h], TOL_S)
    for s in range(nslots):
        if s not in live:
            assert np.array_equal(S[s], case["cache"][s].astype(np.float64)), \
                (label, "untouched slot changed", s)
    print("[parity] %s | o: %r | state: %r" % (label, t_o, t_s), flush=True)
    G.assert_parity(t_o, t_s, label)


def test_decode_4b_bf16_slots_with_padding(dev):
    _say("decode 4B bf16 B=16 slots=24 pad=2")
    case = synth.decode_case(300, 16, 16, 32, 24, pad=2)
    o, cache = _run(case, dev)
    _check(case, o, cache, "decode-4b-bf16")


def test_decode_fp32_identity_slots_no_norm(dev):
    _say("decode fp32 Hk=2 Hv=4 B=5 identity slots, no norm")
    case = synth.decode_case(301, 5, 2, 4, 5, dtype=synth.F32,
                             with_norm=False, identity_slots=True)
    o, cache = _run(case, dev)
    _check(case, o, cache, "decode-fp32")


def test_decode_hv48(dev):
    _say("decode bf16 Hk=16 Hv=48 B=4")
    case = synth.decode_case(302, 4, 16, 48, 6, pad=1)
    o, cache = _run(case, dev)
    _check(case, o, cache, "decode-hv48")


def test_decode_large_batch(dev):
    _say("decode 4B bf16 B=256 slots=300 pad=8")
    case = synth.decode_case(303, 256, 16, 32, 300, pad=8)
    o, cache = _run(case, dev)
    _check(case, o, cache, "decode-b256")


def test_decode_steps_match_prefill(dev):
    # eight steps of one sequence on slot 2 = the oracle's prefill of the
    # eight tokens from the same initial state
    _say("decode 8 steps vs oracle prefill, 4B bf16")
    T = 8
    pf = synth.make_case(304, T, 16, 32)
    cache0 = np.zeros((4, 32, 128, 128), dtype=np.float32)
    cache0[2] = pf["state_in"][0]
    cache_dev = G.to_dev(cache0, dev)
    slots = torch.tensor([2], dtype=torch.int32, device=dev)
    d = {k: G.to_dev(pf[k], dev) for k in
         ("q", "k", "v", "a", "b", "A_log", "dt_bias", "z", "norm_w")}
    outs = []
    for t in range(T):
        o = binding.decode(d["q"][t:t + 1].contiguous(),
                           d["k"][t:t + 1].contiguous(),
                           d["v"][t:t + 1].contiguous(),
                           d["a"][t:t + 1].contiguous(),
                           d["b"][t:t + 1].contiguous(), d["A_log"],
                           d["dt_bias"], cache_dev, slots,
                           z=d["z"][t:t + 1].contiguous(), norm_w=d["norm_w"])
        outs.append(o)
    torch.cuda.synchronize(dev)
    o_ref, S_ref = G.run_oracle(pf)
    o = G.to_f64(torch.cat(outs))
    S = G.to_f64(cache_dev)
    t_o, t_s = PM.Tally(), PM.Tally()
    z64 = synth.storage_to_f64(pf["z"], pf["dtype"])
    for h in range(32):
        for t in range(T):
            t_o.add(o[t, h], o_ref[t, h], TOL_O[synth.BF16], scale=PM.gate(pf["norm_w"], z64[t, h]))
        t_s.add(S[2, h], S_ref[0, h], TOL_S)
    print("[parity] decode-steps | o: %r | state: %r" % (t_o, t_s), flush=True)
    G.assert_parity(t_o, t_s, "decode-steps")
    for s in (0, 1, 3):
        assert torch.count_nonzero(cache_dev[s]).item() == 0


def test_decode_overwrites_poisoned_output_and_guards(dev):
    _say("decode NaN-poisoned output with guard bands")
    case = synth.decode_case(305, 6, 16, 32, 8, pad=2)
    d = {k: G.to_dev(case[k], dev) for k in
         ("q", "k", "v", "a", "b", "A_log", "dt_bias", "z", "norm_w")}
    cache = G.to_dev(case["cache"], dev)
    slots = G.to_dev(case["slots"], dev)
    n = 6 * 32 * 128
    guard = 4096
    buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.bfloat16,
                     device=dev)
    buf[:guard] = 7.0
    buf[-guard:] = 7.0
    out = buf[guard:guard + n].view(6, 32, 128)
    binding.decode(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"],
                   d["dt_bias"], cache, slots, z=d["z"], norm_w=d["norm_w"],
                   out=out)
    torch.cuda.synchronize(dev)
    assert not torch.isnan(out).any()
    assert torch.all(buf[:guard] == 7.0) and torch.all(buf[-guard:] == 7.0)
    _check(case, out, cache, "decode-poison")


def test_decode_deterministic(dev):
    _say("decode run-to-run determinism")
    case = synth.decode_case(306, 16, 16, 32, 16, pad=0)
    o1, c1 = _run(case, dev)
    o2, c2 = _run(case, dev)
    assert torch.equal(o1, o2) and torch.equal(c1, c2)


def test_prefill_then_decode_matches_one_prefill(dev):
    # the serving flow: prefill a 300-token prompt for two requests (packed,
    # cu_seqlens), place their final states in slots 5 and 2 of a cache,
    # then decode 6 more tokens per request; every output and the final
    # states equal the oracle's prefill of the 306-token sequences
    _say("prefill 2 x 300 tokens, then 6 decode steps per request")
    Tp, Td, Hk, Hv = 300, 6, 16, 32
    cases = [synth.make_case(310 + n, Tp + Td, Hk, Hv) for n in range(2)]
    keys = ("q", "k", "v", "a", "b", "z")
    dv = {k: [G.to_dev(c[k], dev) for c in cases] for k in keys}
    A_log = G.to_dev(cases[0]["A_log"], dev)
    dt_bias = G.to_dev(cases[0]["dt_bias"], dev)
    norm_w = G.to_dev(cases[0]["norm_w"], dev)
    S0 = torch.cat([G.to_dev(c["state_in"], dev) for c in cases])
    cu = torch.tensor([0, Tp, 2 * Tp], dtype=torch.int32, device=dev)
    o_pf, S_pf = binding.prefill(
        *(torch.cat([t[:Tp] for t in dv[k]]) for k in "qkvab"), A_log, dt_bias,
        z=torch.cat([t[:Tp] for t in dv["z"]]), norm_w=norm_w, state_in=S0,
        cu_seqlens=cu)
    cache = torch.zeros(8, Hv, 128, 128, dtype=torch.float32, device=dev)
    slots = torch.tensor([5, 2], dtype=torch.int32, device=dev)
    cache[5] = S_pf[0]
    cache[2] = S_pf[1]
    outs = []
    for t in range(Tp, Tp + Td):
        step = {k: torch.stack([dv[k][n][t] for n in range(2)]) for k in keys}
        outs.append(binding.decode(step["q"], step["k"], step["v"], step["a"], step["b"],
                                   A_log, dt_bias, cache, slots, z=step["z"],
                                   norm_w=norm_w))
    torch.cuda.synchronize()
    o_dec = G.to_f64(torch.stack(outs))  # [Td, 2, Hv, 128]
    o_pf = G.to_f64(o_pf)
    S_end = G.to_f64(cache)
    t_o, t_s = PM.Tally.for_dtype("bf16"), PM.Tally.for_dtype("bf16")
    p64 = synth.case_f64(cases[0])  # the per-head parameters both requests used
    for n, c in enumerate(cases):
        c64 = synth.case_f64(c)
        o_ref, S_ref = G.oracle.prefill(c64["q"], c64["k"], c64["v"], c64["a"], c64["b"],
                                        p64["A_log"], p64["dt_bias"], z=c64["z"],
                                        norm_w=p64["norm_w"], state_in=c64["state_in"])
        got = np.concatenate([o_pf[n * Tp:(n + 1) * Tp], o_dec[:, n]])
        for h in range(Hv):
            t_o.add(got[:, h], o_ref[:, h], PM.TOL["bf16"],
                    scale=PM.gate(p64["norm_w"], c64["z"][:, h]))
            t_s.add(S_end[(5, 2)[n], h], S_ref[0, h], PM.TOL["bf16"])
    print("[parity] prefill+decode | o: %r | state: %r" % (t_o, t_s), flush=True)
    # the prefill part carries bf16 MFMA rounding: the prefill bar applies
    G.assert_parity(t_o, t_s, "prefill+decode")


def decode_sweep_case(i: int):
    """Seeded decode batch i: dtype, 1..16 key heads with 1..4 value heads
    each, 1..40 requests, padding entries, spare slots, identity slots,
    with or without the gated norm, small or unit-scale cache."""
    rng = np.random.default_rng(95_000 + i)
    dtype = synth.F32 if i % 3 == 1 else synth.BF16
    Hk = int(rng.choice([1, 2, 4, 16]))
    Hv = Hk * int(rng.integers(1, 5))
    B = int(rng.integers(1, 41))
    identity = bool(i % 4 == 3)
    pad = 0 if identity else int(rng.integers(0, min(3, B - 1) + 1))
    num_slots = B + int(rng.integers(0, 9))
    return synth.decode_case(96_000 + i, B, Hk, Hv, num_slots, dtype=dtype,
                             with_norm=bool(rng.random() < 0.7), pad=pad,
                             state_std=float(rng.choice([0.02, 1.0])),
                             identity_slots=identity)


@pytest.mark.parametrize("i", range(12))
def test_decode_sweep(dev, i):
    case = decode_sweep_case(i)
    _say("decode sweep %d dtype=%s Hk=%d Hv=%d B=%d slots=%d identity=%s norm=%s" % (
        i, case["dtype"], case["Hk"], case["Hv"], case["T"], case["cache"].shape[0],
        case["slots"] is None, case["z"] is not None))
    o, cache = _run(case, dev)
    _check(case, o, cache, "decode-sweep%d" % i)


@pytest.mark.parametrize("i", DECODE_SWEEP_IDS)
def test_decode_fp32_cancellation_cases(dev, i):
    # fp32 decode batches in which a (request, head) output is small through
    # cancellation (found by a randomized sweep; a plain fp32 numpy step
    # misses the plain 2e-5 bar on them, tests/test_parity_bound_cpu.py):
    # held to the conditioned bar
    case = decode_sweep_case(i)
    _say("decode fp32 cancellation case %d Hk=%d Hv=%d B=%d" % (
        i, case["Hk"], case["Hv"], case["T"]))
    o, cache = _run(case, dev)
    _check(case, o, cache, "decode-cancel%d" % i)


def test_decode_graph_replay_matches_eager_steps(dev):
    # A serving loop replays one captured decode step.  The step updates the
    # cache in place, so three replays on one cache must equal three eager
    # steps on a copy of it, output and cache bitwise, with eager work and
    # synchronisation between the replays.
    _say("decode graph capture/replay, 4B bf16 B=8 slots=12 pad=1")
    case = synth.decode_case(310, 8, 16, 32, 12, pad=1)
    d = {k: G.to_dev(case[k], dev) for k in
         ("q", "k", "v", "a", "b", "A_log", "dt_bias", "z", "norm_w")}
    slots = G.to_dev(case["slots"], dev)
    cache_g = G.to_dev(case["cache"], dev)
    cache_e = cache_g.clone()
    o_g = torch.empty(8, 32, 128, dtype=torch.bfloat16, device=dev)
    o_e = torch.empty_like(o_g)

    def step(cache, o):
        binding.decode(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                       cache, slots, z=d["z"], norm_w=d["norm_w"], out=o)

    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):  # capture records the step without running it
        step(cache_g, o_g)
    for rep in range(3):
        o_g.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(cache_e, o_e)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), rep
        assert torch.equal(cache_g, cache_e), rep
