"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds random draws and dtype casts only -- none of the operator's
arithmetic -- so that the HIP path and the CPU oracle can be fed identical
values without sharing any code that computes the method.

Workload shapes follow the pages (page title, section):
  * "feat(qwen35): add SM120 FlashInfer GDN prefill candidate", Correctness:
    the 4B geometry Hq/Hk/Hv/D = 16/16/32/128, operator tests at
    T = 1, 2, 63, 64, 65, 127, 128, chunked vs unchunked prefill, and the Hv48
    variant at T = 128;  Performance: T = 2048 at concurrency 1 and T = 128
    at concurrency 8.
  * "Add opt-in fused Qwen3.5 inference kernels", Summary: the four input
    projections as one GEMM and the gated RMSNorm after the chunked kernel.
None of the pages' datasets is available; these i.i.d. Gaussian/uniform
tensors stand in for their shapes.

Draws use numpy's PCG64 (``default_rng(seed)``) in float64 in the fixed order
q, k, v, a, b, A_log, dt_bias, state_in, z, norm_w (only those a case uses),
then round to the storage dtype: fp64 -> fp32 with numpy's RNE cast, then
fp32 -> bf16 with round-to-nearest-even on the bit pattern.
"""
from __future__ import annotations

import math

import numpy as np

BF16 = "bf16"
F32 = "f32"

# 4B geometry
HK_4B, HV_4B, D = 16, 32, 128
CONFIG1_TS = (1, 2, 63, 64, 65, 127, 128)


def seed_for(config: int, subcase: int = 0) -> int:
    return 1000 * (config + 1) + subcase


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (RNE); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    u = u.astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 draw -> storage array (float32, or uint16 bf16 bits)."""
    x32 = np.asarray(x64, dtype=np.float32)
    if dtype == F32:
        return x32
    if dtype == BF16:
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def storage_to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact conversion of a storage array back to float64."""
    if x is None:
        return None
    if dtype == BF16 and x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def make_case(seed: int, T: int, Hk: int, Hv: int, Dk: int = D, Dv: int = D,
              dtype: str = BF16, with_state: bool = True,
              with_norm: bool = True, seqlens=None, N: int | None = None):
    """One prefill case.  Returns a dict of numpy arrays in storage form:
    q,k [T,Hk,Dk]; v [T,Hv,Dv]; a,b [T,Hv] (storage dtype); A_log, dt_bias
    [Hv] fp32; state_in [N,Hv,Dv,Dk] fp32 or None; z [T,Hv,Dv] (storage) or
    None; norm_w [Dv] fp32 or None; cu_seqlens int32 [N+1] or None.

    Distributions: q,k,v,a,b,z ~ N(0,1); A_log ~ U(0, ln 16);
    dt_bias ~ U(-1, 1); state ~ N(0, 0.02^2); norm_w ~ 1 + N(0, 0.02^2).
    """
    rng = np.random.default_rng(seed)
    if seqlens is not None:
        seqlens = [int(s) for s in seqlens]
        assert sum(seqlens) == T
        N = len(seqlens)
        cu = np.zeros(N + 1, dtype=np.int32)
        cu[1:] = np.cumsum(seqlens)
    else:
        N = 1 if N is None else N
        cu = None
    out = {"dtype": dtype, "T": T, "Hk": Hk, "Hv": Hv, "Dk": Dk, "Dv": Dv,
           "N": N, "seed": seed}
    out["q"] = to_storage(rng.standard_normal((T, Hk, Dk)), dtype)
    out["k"] = to_storage(rng.standard_normal((T, Hk, Dk)), dtype)
    out["v"] = to_storage(rng.standard_normal((T, Hv, Dv)), dtype)
    out["a"] = to_storage(rng.standard_normal((T, Hv)), dtype)
    out["b"] = to_storage(rng.standard_normal((T, Hv)), dtype)
    out["A_log"] = rng.uniform(0.0, math.log(16.0), Hv).astype(np.float32)
    out["dt_bias"] = rng.uniform(-1.0, 1.0, Hv).astype(np.float32)
    if with_state:
        out["state_in"] = (0.02 * rng.standard_normal((N, Hv, Dv, Dk))
                           ).astype(np.float32)
    else:
        out["state_in"] = None
    if with_norm:
        out["z"] = to_storage(rng.standard_normal((T, Hv, Dv)), dtype)
        out["norm_w"] = (1.0 + 0.02 * rng.standard_normal(Dv)).astype(
            np.float32)
    else:
        out["z"] = None
        out["norm_w"] = None
    out["cu_seqlens"] = cu
    return out


def case_f64(case: dict) -> dict:
    """The same case as exact float64 arrays (what the oracle consumes)."""
    dt = case["dtype"]
    res = dict(case)
    for key in ("q", "k", "v", "a", "b", "z"):
        res[key] = storage_to_f64(case[key], dt)
    for key in ("A_log", "dt_bias", "state_in", "norm_w"):
        res[key] = None if case[key] is None else case[key].astype(np.float64)
    return res


# ---- the configured workloads -------------------------------------------

def config0_case():
    """Per-rank share at 8-way head sharding: fp32, T=64, Hk=2, Hv=4, zero
    state, no gated norm."""
    return make_case(seed_for(0), 64, 2, 4, dtype=F32, with_state=False,
                     with_norm=False)


def config1_case(T: int, subcase: int | None = None):
    """4B geometry, bf16, random state, gated norm on."""
    sc = CONFIG1_TS.index(T) if subcase is None else subcase
    return make_case(seed_for(1, sc), T, HK_4B, HV_4B)


def config2_case(T: int = 2048, subcase: int = 0):
    """4B geometry, bf16, T=2048, random state, gated norm on."""
    return make_case(seed_for(2, subcase), T, HK_4B, HV_4B)


def config3_lengths(subcase: int = 0, n: int = 8):
    rng = np.random.default_rng(seed_for(3, 100 + subcase))
    return [int(x) for x in rng.integers(32, 129, n)]


def config3_case(subcase: int = 0):
    """Packed varlen batch of 8 sequences, lengths U{32..128}."""
    lens = config3_lengths(subcase)
    return make_case(seed_for(3, subcase), sum(lens), HK_4B, HV_4B,
                     seqlens=lens)


def config3_hv48_case():
    """Hv=48 (3 value heads per key head) at T=128."""
    return make_case(seed_for(3, 50), 128, HK_4B, 48)


def layer_case(seed: int, T: int = 2048, hidden: int = 2560, Hk: int = HK_4B,
               Hv: int = HV_4B, Dh: int = D, conv_width: int = 4):
    """Full-layer inputs: x ~ N(0,1) [T, hidden] bf16; W_in [hidden, 2*Hk*D +
    2*Hv*D + 2*Hv], conv_w [3 q|k|v channels, width], W_out [Hv*D, hidden]
    ~ N(0, 0.02^2) bf16; A_log, dt_bias, norm_w as for the op (fp32)."""
    rng = np.random.default_rng(seed)
    width = 2 * Hk * Dh + 2 * Hv * Dh + 2 * Hv
    conv_ch = 2 * Hk * Dh + Hv * Dh
    out = {"T": T, "hidden": hidden, "Hk": Hk, "Hv": Hv, "D": Dh,
           "width": width, "conv_ch": conv_ch, "seed": seed}
    out["x"] = to_storage(rng.standard_normal((T, hidden)), BF16)
    out["W_in"] = to_storage(0.02 * rng.standard_normal((hidden, width)), BF16)
    out["conv_w"] = to_storage(0.02 * rng.standard_normal((conv_ch, conv_width)),
                               BF16)
    out["W_out"] = to_storage(0.02 * rng.standard_normal((Hv * Dh, hidden)),
                              BF16)
    out["A_log"] = rng.uniform(0.0, math.log(16.0), Hv).astype(np.float32)
    out["dt_bias"] = rng.uniform(-1.0, 1.0, Hv).astype(np.float32)
    out["norm_w"] = (1.0 + 0.02 * rng.standard_normal(Dh)).astype(np.float32)
    return out


def decode_case(seed: int, B: int, Hk: int, Hv: int, num_slots: int,
                dtype: str = BF16, with_norm: bool = True, pad: int = 0,
                state_std: float = 1.0, identity_slots: bool = False):
    """One decode batch: B one-token requests on a [num_slots, Hv, D, D]
    fp32 state cache.  Token inputs as make_case (with T = B); the cache is
    N(0, state_std^2) (unit scale, as a cache that has absorbed many tokens);
    slots are B - pad distinct slots drawn without replacement, plus `pad`
    padding entries (alternately -1 and num_slots, both outside the cache),
    shuffled; identity_slots gives slot i to request i instead (no padding).
    """
    case = make_case(seed, B, Hk, Hv, dtype=dtype, with_state=False,
                     with_norm=with_norm)
    rng = np.random.default_rng(seed + 7919)
    case["cache"] = (state_std * rng.standard_normal((num_slots, Hv, D, D))
                     ).astype(np.float32)
    if identity_slots:
        case["slots"] = None
    else:
        live = rng.choice(num_slots, size=B - pad, replace=False)
        pads = [-1 if i % 2 == 0 else num_slots for i in range(pad)]
        slots = np.concatenate([live, np.array(pads, dtype=np.int64)])
        case["slots"] = rng.permutation(slots).astype(np.int32)
    return case

