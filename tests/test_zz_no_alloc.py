"""gdn_prefill_noalloc (the prefill with its scratch in the library's static
per-GPU array) against gdn_prefill on the same inputs, through the C ABI:
two calls in a row, the second smaller than the first, each bitwise equal
to gdn_prefill's result (the same kernels on the same inputs; what the
scratch held before does not matter).  A call that needs more scratch than
the array holds is refused on the host."""
from __future__ import annotations

import pytest
import torch

from gated_deltanet_linear_04_amd import binding, synth
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load()
    return torch.device("cuda:0")


def _both(case, dev):
    d = G.device_case(case, dev)
    args = (d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"])
    kw = dict(z=d["z"], norm_w=d["norm_w"], state_in=d["state_in"],
              cu_seqlens=d["cu_seqlens"])
    o_ref, S_ref = binding.prefill(*args, **kw)
    dt = d["q"].dtype
    o = torch.full_like(o_ref, float("nan"))
    S = torch.full_like(S_ref, float("nan"))
    binding.prefill_noalloc(*args, **kw, out=o, state_out=S)
    torch.cuda.synchronize(dev)
    assert o.dtype == dt
    return o, S, o_ref, S_ref


def test_noalloc_matches_prefill_on_two_calls(dev):
    # first call: two packed sequences, 2048 tokens at the 4B geometry (34
    # workspace slots x 32 value heads, within the 96 MiB array)
    lens = [1300, 748]
    first = synth.make_case(8801, sum(lens), 16, 32, seqlens=lens)
    need = binding.workspace_size(binding.make_desc(2, 2048, 16, 32, torch.bfloat16))
    assert need <= binding.NOALLOC_SCRATCH_BYTES
    print("[case] noalloc call 1: lens=%s workspace=%d" % (lens, need), flush=True)
    o, S, o_ref, S_ref = _both(first, dev)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    # second call, smaller: one sequence of 130 tokens, fp32 state chain of
    # the same kernels on the array the first call left behind
    second = synth.make_case(8802, 130, 16, 32)
    print("[case] noalloc call 2: T=130", flush=True)
    o, S, o_ref, S_ref = _both(second, dev)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    # and the second call against the oracle, to the operator's bar
    t_o, t_s, _ = G.parity(second, G.to_f64(o), G.to_f64(S), *G.run_oracle(second))
    G.assert_parity(t_o, t_s, "noalloc-130")


def test_noalloc_refuses_calls_beyond_the_array(dev):
    case = synth.make_case(8803, 4096, 16, 32)
    d = G.device_case(case, dev)
    o = torch.empty(4096, 32, 128, dtype=torch.bfloat16, device=dev)
    S = torch.empty(1, 32, 128, 128, dtype=torch.float32, device=dev)
    with pytest.raises(binding.GdnError) as e:
        binding.prefill_noalloc(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"],
                                d["dt_bias"], z=d["z"], norm_w=d["norm_w"],
                                state_in=d["state_in"], out=o, state_out=S)
    assert e.value.status == binding.GDN_ERR_WORKSPACE
