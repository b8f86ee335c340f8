"""The sequence-parallel scan of the state chain (gdn_desc.chain_segments)
against the fp64 oracle and against the one-pass chain, through the C ABI.

Workload: one GPU's share of the 4B geometry at 8-way head sharding (Hk/Hv
= 2/4, the head counts of the fp32 per-rank case) over one long prompt,
T = 16,384 tokens (256 chunks): the chain grid is 32 blocks, so the one
pass leaves most of the GPU idle and the library scans it.  Cases: the
library's own choice (bf16 and fp32), forced segment counts (2: no
composition step; 3; 7 with a ragged last segment), an in-place state, and
agreement with the one-pass result within the operator's bar.

Decay.  With the usual gate distributions (exp(A_log) >= 1) the state decays
by e^-45 or more per chunk, so a segment's start state is below fp32
resolution by the next segment and the scan reproduces the one pass bit for
bit.  The composition of segment maps is only exercised when the state
carries: most cases here use weak-decay heads (A_log from -6 to -1,
dt_bias -2: about e^-0.7 over 2048 tokens on the weakest head).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gated_deltanet_linear_04_amd import binding, synth
from tests import gpu_helpers as G
from tests import parity_metrics as PM

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load()
    return torch.device("cuda:0")


def _say(msg):
    print("[case] " + msg, flush=True)


def weak_decay(case):
    Hv = case["Hv"]
    case["A_log"] = np.linspace(-6.0, -1.0, Hv).astype(np.float32)
    case["dt_bias"] = np.full(Hv, -2.0, dtype=np.float32)
    return case


@pytest.fixture(scope="module")
def long_cases():
    return {dt: weak_decay(synth.make_case(96_001 if dt == synth.BF16 else 96_002, 16_384, 2, 4,
                                           dtype=dt))
            for dt in (synth.BF16, synth.F32)}


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32])
def test_scan_matches_oracle_and_one_pass(dev, long_cases, dtype):
    case = long_cases[dtype]
    _say("scan T=16384 Hk/Hv=2/4 %s (library's choice) vs oracle and one pass" % dtype)
    o_s, S_s, rel_o, rel_s, _ = G.check_parity(case, dev, "scan-auto-%s" % dtype)
    o_1, S_1, _, _, _ = G.check_parity(case, dev, "one-pass-%s" % dtype, chain_segments=1)
    # the two forms differ only by rounding (and with weak decay they do
    # differ: the segment maps carry the state across segments)
    assert not torch.equal(S_s, S_1)
    bar = PM.TOL[dtype]
    t_o, t_s = PM.Tally.for_dtype(dtype), PM.Tally.for_dtype(dtype)
    c64 = synth.case_f64(case)
    for h in range(4):
        t_o.add(G.to_f64(o_s[:, h]), G.to_f64(o_1[:, h]), bar,
                scale=PM.gate(case["norm_w"], c64["z"][:, h]))
        t_s.add(G.to_f64(S_s[0, h]), G.to_f64(S_1[0, h]), bar)
    print("[parity] scan vs one pass %s | o: %r | state: %r" % (dtype, t_o, t_s), flush=True)
    G.assert_parity(t_o, t_s, "scan-vs-one-pass")
    if dtype == synth.F32:
        assert rel_o <= 1e-5 and rel_s <= 1e-5, (rel_o, rel_s)


@pytest.mark.parametrize("segs,T", [(2, 4096), (3, 5000), (7, 6000)])
def test_forced_segment_counts(dev, segs, T):
    _say("scan forced G=%d T=%d Hk/Hv=2/4 bf16" % (segs, T))
    case = weak_decay(synth.make_case(96_100 + segs, T, 2, 4))
    G.check_parity(case, dev, "scan-G%d" % segs, chain_segments=segs)


def test_scan_in_place_state_and_fp32_forced(dev):
    _say("scan in place, fp32 G=4 T=3000 Hk/Hv=1/2 no norm")
    case = weak_decay(synth.make_case(96_200, 3000, 1, 2, dtype=synth.F32, with_norm=False))
    o_ref, S_ref = G.run_gpu(case, dev, chain_segments=4)
    d = G.device_case(case, dev)
    st = d["state_in"].clone()
    o, S = binding.prefill(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"],
                           d["dt_bias"], state_in=st, state_out=st, chain_segments=4)
    torch.cuda.synchronize()
    assert S.data_ptr() == st.data_ptr()
    assert torch.equal(o, o_ref) and torch.equal(st, S_ref)
    G.check_parity(case, dev, "scan-fp32-G4", chain_segments=4)


def test_strong_decay_scan_equals_one_pass(dev):
    # usual gates: the state does not survive a chunk, so the scan's start
    # states equal the one pass's to the bit
    _say("scan strong decay T=8192 Hk/Hv=2/4 bf16, auto vs one pass")
    case = synth.make_case(96_400, 8192, 2, 4)
    o_s, S_s = G.run_gpu(case, dev)
    o_1, S_1 = G.run_gpu(case, dev, chain_segments=1)
    assert torch.equal(o_s, o_1) and torch.equal(S_s, S_1)


def test_scan_refused_for_several_sequences(dev):
    case = synth.make_case(96_300, 200, 2, 4, seqlens=[100, 100])
    with pytest.raises(binding.GdnError) as e:
        G.run_gpu(case, dev, chain_segments=3)
    assert e.value.status == binding.GDN_ERR_UNSUPPORTED
