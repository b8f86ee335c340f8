"""fp32 inputs on which a one-token output is small through cancellation.

They were found by randomized GPU sweeps against the oracle (seeded draws of
the shapes and lengths below); they are kept as fixed regression cases for
the conditioned fp32 bar (tests/parity_metrics.py):

* CANCELLATION_PREFILL: 17 packed sequences of 0-3 tokens, 16 key heads,
  48 value heads, no initial state, gated norm on.  One one-token slice has
  k^ . q^ = 1.7e-5 (relative to unit vectors), so its o = beta (k^ . q^) v is
  small through cancellation.
* decode_cancellation_cases(): decode batches 31, 73, 76, 91 and 94 of the
  decode sweep generator, each with a (request, head) whose output is small
  through cancellation.
"""
from __future__ import annotations

from gated_deltanet_linear_04_amd import synth

PREFILL_LENS = [3, 0, 3, 2, 3, 3, 1, 3, 3, 3, 2, 3, 0, 1, 1, 3, 2]
DECODE_SWEEP_IDS = (31, 73, 76, 91, 94)


def CANCELLATION_PREFILL():
    return synth.make_case(124_166, sum(PREFILL_LENS), 16, 48, dtype=synth.F32,
                           with_state=False, with_norm=True, seqlens=PREFILL_LENS)


def decode_cancellation_cases():
    from tests.test_gpu_decode import decode_sweep_case

    return [(i, decode_sweep_case(i)) for i in DECODE_SWEEP_IDS]
