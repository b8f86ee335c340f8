"""Pins of the fp64 oracle against what the mathematics fixes (CPU only).

Each test checks the oracle against something other than itself: a closed
form, an exact rational expansion, a library routine, or an invariant of the
operator.  Together they are chosen so that a plausible slip in the oracle (a
dropped term, a wrong sign or index, a transposed operand, a wrong head map)
fails at least one of them.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.signal
import scipy.special
import torch

import oracle
from oracle import brute
from gated_deltanet_linear_04_amd import synth
from tests import wy_model

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(seed, T, Hk, Hv, Dk, Dv, N=1, with_state=True, with_norm=True):
    rng = np.random.default_rng(seed)
    c = dict(
        q=rng.standard_normal((T, Hk, Dk)), k=rng.standard_normal((T, Hk, Dk)),
        v=rng.standard_normal((T, Hv, Dv)), a=rng.standard_normal((T, Hv)),
        b=rng.standard_normal((T, Hv)),
        A_log=rng.uniform(0, math.log(16), Hv), dt_bias=rng.uniform(-1, 1, Hv))
    c["state_in"] = (0.02 * rng.standard_normal((N, Hv, Dv, Dk))
                     if with_state else None)
    if with_norm:
        c["z"] = rng.standard_normal((T, Hv, Dv))
        c["norm_w"] = 1 + 0.02 * rng.standard_normal(Dv)
    return c


# ---- P12: scalar special values and library cross-checks -----------------

def test_softplus_sigmoid_special_values():
    assert oracle.softplus(0.0) == pytest.approx(math.log(2.0), abs=1e-16)
    assert oracle.sigmoid(0.0) == 0.5
    xs = np.linspace(-60, 60, 241)
    sp = np.array([oracle.softplus(x) for x in xs])
    sg = np.array([oracle.sigmoid(x) for x in xs])
    np.testing.assert_allclose(sp, np.logaddexp(0.0, xs), rtol=1e-15, atol=0)
    np.testing.assert_allclose(sg, scipy.special.expit(xs), rtol=1e-15, atol=0)
    # saturation: no overflow, exact limits
    assert oracle.sigmoid(-1e4) == 0.0 and oracle.sigmoid(1e4) == 1.0
    assert oracle.softplus(1e4) == 1e4


# ---- P1: T = 1 closed form -------------------------------------------------

def test_single_token_closed_form_zero_state():
    # with S_0 = 0: o = beta (kn . qn) v, S_1 = beta v kn^T
    c = _rand_case(1, 1, 2, 4, 8, 6, with_state=False, with_norm=False)
    o, S = oracle.prefill(**c)
    r = 2
    for h in range(4):
        kh = h // r
        kn = c["k"][0, kh] / np.linalg.norm(c["k"][0, kh])
        qn = c["q"][0, kh] / np.linalg.norm(c["q"][0, kh]) * 8 ** -0.5
        beta = scipy.special.expit(c["b"][0, h])
        # eps = 1e-6 changes norms at the ~1e-8 relative level
        np.testing.assert_allclose(o[0, h], beta * (kn @ qn) * c["v"][0, h],
                                   rtol=1e-6, atol=1e-12)
        np.testing.assert_allclose(S[0, h], beta * np.outer(c["v"][0, h], kn),
                                   rtol=1e-6, atol=1e-12)


def test_single_token_closed_form_with_state():
    # S_1 = alpha S_0 (I - beta kn kn^T) + beta v kn^T with alpha written as
    # (1 + e^x)^(-exp(A_log)), a power form independent of the exp/softplus
    # evaluation in the oracle.
    c = _rand_case(2, 1, 1, 3, 5, 4, with_norm=False)
    o, S = oracle.prefill(**c, l2_eps=0.0)
    for h in range(3):
        x = c["a"][0, h] + c["dt_bias"][h]
        alpha = (1.0 + math.exp(x)) ** (-math.exp(c["A_log"][h]))
        beta = 1.0 / (1.0 + math.exp(-c["b"][0, h]))
        kn = c["k"][0, 0] / np.linalg.norm(c["k"][0, 0])
        qn = c["q"][0, 0] / np.linalg.norm(c["q"][0, 0]) * 5 ** -0.5
        S0 = c["state_in"][0, h]
        S1 = alpha * S0 @ (np.eye(5) - beta * np.outer(kn, kn)) + beta * np.outer(
            c["v"][0, h], kn)
        np.testing.assert_allclose(S[0, h], S1, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(o[0, h], S1 @ qn, rtol=1e-12, atol=1e-15)


# ---- P1b: decode on a slot-addressed cache ----------------------------------

def test_decode_slot_gather_closed_form():
    # each live request follows the one-token closed form (power-form alpha)
    # on its own slot; the padding entry gives zeros; other slots unchanged
    rng = np.random.default_rng(21)
    B, Hk, Hv, Dk, Dv, S = 3, 1, 2, 5, 4, 5
    q = rng.standard_normal((B, Hk, Dk))
    k = rng.standard_normal((B, Hk, Dk))
    v = rng.standard_normal((B, Hv, Dv))
    a = rng.standard_normal((B, Hv))
    b = rng.standard_normal((B, Hv))
    A_log = rng.uniform(0, math.log(16), Hv)
    dt_bias = rng.uniform(-1, 1, Hv)
    cache = rng.standard_normal((S, Hv, Dv, Dk))
    slots = np.array([3, -1, 0])
    o, new = oracle.decode(q, k, v, a, b, A_log, dt_bias, cache, slots,
                           l2_eps=0.0)
    for i, s in ((0, 3), (2, 0)):
        kn = k[i, 0] / np.linalg.norm(k[i, 0])
        qn = q[i, 0] / np.linalg.norm(q[i, 0]) * Dk ** -0.5
        for h in range(Hv):
            x = a[i, h] + dt_bias[h]
            alpha = (1.0 + math.exp(x)) ** (-math.exp(A_log[h]))
            beta = 1.0 / (1.0 + math.exp(-b[i, h]))
            S1 = alpha * cache[s, h] @ (np.eye(Dk) - beta * np.outer(kn, kn)) \
                + beta * np.outer(v[i, h], kn)
            np.testing.assert_allclose(new[s, h], S1, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(o[i, h], S1 @ qn, rtol=1e-12, atol=1e-14)
    assert np.all(o[1] == 0.0)
    for s in (1, 2, 4):
        assert np.array_equal(new[s], cache[s])


def test_decode_steps_equal_prefill():
    # T decode steps on one slot = one prefill of the T tokens (with norm)
    c = _rand_case(22, 6, 2, 4, 8, 8)
    cache = np.zeros((3, 4, 8, 8))
    cache[1] = c["state_in"][0]
    o_pf, S_pf = oracle.prefill(**c)
    outs = []
    for t in range(6):
        o, cache = oracle.decode(
            c["q"][t:t + 1], c["k"][t:t + 1], c["v"][t:t + 1],
            c["a"][t:t + 1], c["b"][t:t + 1], c["A_log"], c["dt_bias"], cache,
            [1], z=c["z"][t:t + 1], norm_w=c["norm_w"])
        outs.append(o[0])
    np.testing.assert_allclose(np.stack(outs), o_pf, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(cache[1], S_pf[0], rtol=1e-12, atol=1e-15)
    assert np.all(cache[0] == 0.0) and np.all(cache[2] == 0.0)


def test_decode_rejects_duplicate_live_slots():
    c = _rand_case(23, 2, 1, 1, 4, 4, with_norm=False)
    with pytest.raises(ValueError):
        oracle.decode(c["q"], c["k"], c["v"], c["a"], c["b"], c["A_log"],
                      c["dt_bias"], np.zeros((2, 1, 4, 4)), [1, 1])


# ---- P2: beta = 0 gives pure decay -----------------------------------------

def test_beta_zero_pure_decay_half_per_token():
    # A_log = a = dt_bias = 0 -> g = -ln 2 -> alpha = 1/2; b = -1e4 -> beta = 0
    T, Hk, Hv, D = 7, 1, 2, 4
    c = _rand_case(3, T, Hk, Hv, D, D, with_norm=False)
    c["A_log"][:] = 0.0
    c["dt_bias"][:] = 0.0
    c["a"][:] = 0.0
    c["b"][:] = -1e4
    o, S = oracle.prefill(**c)
    np.testing.assert_allclose(S, c["state_in"] * 2.0 ** -T, rtol=1e-14, atol=0)
    for t in range(T):
        for h in range(Hv):
            qn = c["q"][t, 0] / math.sqrt((c["q"][t, 0] ** 2).sum() + 1e-6) * D ** -0.5
            ref = 2.0 ** -(t + 1) * c["state_in"][0, h] @ qn
            np.testing.assert_allclose(o[t, h], ref, rtol=1e-13, atol=1e-18)


def test_beta_zero_decay_power_form():
    # beta = 0: S_T = prod_t (1 + e^{x_t})^(-exp(A_log)) S_0
    T, Hk, Hv, D = 9, 2, 4, 3
    c = _rand_case(4, T, Hk, Hv, D, D, with_norm=False)
    c["b"][:] = -1e4
    _, S = oracle.prefill(**c)
    for h in range(Hv):
        x = c["a"][:, h] + c["dt_bias"][h]
        fac = np.prod((1.0 + np.exp(x)) ** (-math.exp(c["A_log"][h])))
        np.testing.assert_allclose(S[0, h], fac * c["state_in"][0, h],
                                   rtol=1e-12, atol=0)


# ---- P3: pure delta rule with orthonormal keys ------------------------------

def test_orthonormal_keys_store_and_overwrite():
    # alpha = 1 (A_log = -200), beta = 1 (b = +1e4), keys are basis vectors
    # (scaled by positive factors; l2_eps = 0 makes kn exact).  Then column
    # pi(t) of S holds v of the last token that wrote key pi(t), and a query
    # along e_j returns scale * that v, or 0 if key j was never written.
    D, T = 6, 10
    rng = np.random.default_rng(5)
    keys = [0, 3, 1, 3, 5, 2, 0, 4, 4, 1]
    queries = [0, 3, 2, 3, 5, 1, 4, 0, 4, 2]
    q = np.zeros((T, 1, D))
    k = np.zeros((T, 1, D))
    for t in range(T):
        k[t, 0, keys[t]] = rng.uniform(0.5, 3.0)
        q[t, 0, queries[t]] = rng.uniform(0.5, 3.0)
    v = rng.standard_normal((T, 1, D))
    a = np.zeros((T, 1))
    b = np.full((T, 1), 1e4)
    scale = 0.25
    o, S = oracle.prefill(q, k, v, a, b, np.array([-200.0]), np.array([0.0]),
                          scale=scale, l2_eps=0.0)
    last = {}
    for t in range(T):
        last[keys[t]] = v[t, 0]
        j = queries[t]
        expect = scale * last[j] if j in last else np.zeros(D)
        np.testing.assert_allclose(o[t, 0], expect, rtol=1e-14, atol=1e-15)
    for j in range(D):
        col = last.get(j, np.zeros(D))
        np.testing.assert_allclose(S[0, 0][:, j], col, rtol=1e-14, atol=1e-15)


# ---- P4: scalar head = first-order linear filter (library routine) ----------

def test_scalar_head_matches_lfilter():
    # D = 1 with constant gates and a constant key: s_t = c s_{t-1} + x_t with
    # c = alpha (1 - beta kn^2), x_t = beta v_t kn -- an IIR filter.
    T = 50
    rng = np.random.default_rng(6)
    kval, qval = 1.7, -0.6
    q = np.full((T, 1, 1), qval)
    k = np.full((T, 1, 1), kval)
    v = rng.standard_normal((T, 1, 1))
    a = np.full((T, 1), 0.3)
    b = np.full((T, 1), -0.2)
    A_log = np.array([0.4])
    dt_bias = np.array([-0.1])
    S0 = np.array([[[[0.37]]]])
    o, S = oracle.prefill(q, k, v, a, b, A_log, dt_bias, state_in=S0,
                          scale=1.0, l2_eps=0.0)
    alpha = (1.0 + math.exp(0.2)) ** (-math.exp(0.4))
    beta = 1.0 / (1.0 + math.exp(0.2))
    kn = 1.0
    qn = -1.0
    cc = alpha * (1 - beta * kn * kn)
    x = beta * v[:, 0, 0] * kn
    s, _ = scipy.signal.lfilter([1.0], [1.0, -cc], x, zi=[cc * 0.37])
    np.testing.assert_allclose(o[:, 0, 0], s * qn, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(S[0, 0, 0, 0], s[-1], rtol=1e-12)


# ---- P5: exact rational brute force on tiny heads ---------------------------

@pytest.mark.parametrize("seed,T,Dk,Dv", [(7, 1, 2, 2), (8, 5, 3, 2),
                                          (9, 8, 4, 3), (10, 6, 2, 4)])
def test_core_matches_exact_product_expansion(seed, T, Dk, Dv):
    rng = np.random.default_rng(seed)
    alpha = rng.uniform(0.2, 1.0, T)
    beta = rng.uniform(0.0, 1.0, T)
    kn = rng.standard_normal((T, Dk))
    kn /= np.linalg.norm(kn, axis=1, keepdims=True)
    qn = rng.standard_normal((T, Dk))
    v = rng.standard_normal((T, Dv))
    S0 = rng.standard_normal((Dv, Dk))
    o, S = oracle.delta_core(alpha, beta, kn, qn, v, S0)
    F = Fraction
    o_ex, S_ex = brute.outputs([F(x) for x in alpha], [F(x) for x in beta],
                               [[F(x) for x in r] for r in kn],
                               [[F(x) for x in r] for r in qn],
                               [[F(x) for x in r] for r in v],
                               [[F(x) for x in r] for r in S0])
    o_ex = np.array([[float(x) for x in r] for r in o_ex])
    S_ex = np.array([[float(x) for x in r] for r in S_ex])
    np.testing.assert_allclose(o, o_ex, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, S_ex, rtol=1e-12, atol=1e-13)


# ---- term sizes: the diagnostic behind the bf16 element bound ---------------

@pytest.mark.parametrize("seed,T,Dk,Dv", [(21, 5, 3, 2), (22, 7, 2, 3)])
def test_term_rss_matches_exact_states(seed, T, Dk, Dv):
    """rss[t, i] is the root-sum-square of S_t[i, j] qn_t[j] with S_t the state
    after token t: checked against the exact rational states of the product
    expansion (a slip to S_{t-1}, to kn, or to a transposed state fails)."""
    rng = np.random.default_rng(seed)
    alpha = rng.uniform(0.2, 1.0, T)
    beta = rng.uniform(0.0, 1.0, T)
    kn = rng.standard_normal((T, Dk))
    kn /= np.linalg.norm(kn, axis=1, keepdims=True)
    qn = rng.standard_normal((T, Dk))
    v = rng.standard_normal((T, Dv))
    S0 = rng.standard_normal((Dv, Dk))
    o, S, rss = oracle.delta_core(alpha, beta, kn, qn, v, S0, terms=True)
    o2, S2 = oracle.delta_core(alpha, beta, kn, qn, v, S0)
    assert np.array_equal(o, o2) and np.array_equal(S, S2)
    F = Fraction
    fa, fb = [F(x) for x in alpha], [F(x) for x in beta]
    fk = [[F(x) for x in r] for r in kn]
    fv = [[F(x) for x in r] for r in v]
    f0 = [[F(x) for x in r] for r in S0]
    for t in range(T):
        St = brute.state_after(t + 1, fa, fb, fk, fv, f0)
        ex = [math.sqrt(float(sum((St[i][j] * F(qn[t][j])) ** 2 for j in range(Dk))))
              for i in range(Dv)]
        np.testing.assert_allclose(rss[t], ex, rtol=1e-12, atol=0)


def test_term_rss_of_a_single_term_is_the_output():
    """With Dk = 1 each output element is one product, so the size of its
    terms is |o|; o_raw is the output before the gated norm, which maps it to
    o (the norm written out here in numpy)."""
    c = _rand_case(24, 40, 1, 3, 1, 5, N=2)
    c["cu_seqlens"] = np.array([0, 17, 40], dtype=np.int32)
    o, S, o_raw, rss = oracle.prefill(**c, terms=True)
    np.testing.assert_allclose(rss, np.abs(o_raw), rtol=1e-15, atol=0)
    z = c["z"]
    ms = np.mean(o_raw * o_raw, axis=-1, keepdims=True)
    y = o_raw / np.sqrt(ms + 1e-6) * c["norm_w"] * z * scipy.special.expit(z)
    np.testing.assert_allclose(o, y, rtol=1e-13, atol=1e-15)
    o_plain, S_plain = oracle.prefill(**{k_: v_ for k_, v_ in c.items()
                                         if k_ not in ("z", "norm_w")})
    assert np.array_equal(o_plain, o_raw) and np.array_equal(S_plain, S)


def test_term_rss_one_token_closed_form():
    """One token from a zero state: S_1 = beta v kn^T, so the terms of o[i]
    are beta v_i kn_j qn_j and their size is beta |v_i| ||kn * qn||."""
    c = _rand_case(23, 1, 2, 4, 8, 5, with_state=False, with_norm=False)
    _, _, _, rss = oracle.prefill(**c, scale=0.7, terms=True)
    for h in range(4):
        kh = h // 2
        q, k = c["q"][0, kh], c["k"][0, kh]
        qn = 0.7 * q / np.sqrt(q @ q + 1e-6)
        kn = k / np.sqrt(k @ k + 1e-6)
        beta = scipy.special.expit(c["b"][0, h])
        want = beta * np.abs(c["v"][0, h]) * np.linalg.norm(kn * qn)
        np.testing.assert_allclose(rss[0, h], want, rtol=1e-13, atol=0)


def test_golden_exact_fixture():
    """Stored exact-rational worked example (tests/golden/delta_rule_tiny.json,
    written by tests/golden/make_golden.py with oracle.brute only)."""
    with open(os.path.join(GOLDEN, "delta_rule_tiny.json")) as f:
        g = json.load(f)
    arr = lambda key: np.array(g[key], dtype=np.float64)
    o, S = oracle.delta_core(arr("alpha"), arr("beta"), arr("kn"), arr("qn"),
                             arr("v"), arr("S0"))
    o_ex = np.array([[float(Fraction(x)) for x in r] for r in g["o_exact"]])
    S_ex = np.array([[float(Fraction(x)) for x in r] for r in g["S_exact"]])
    np.testing.assert_allclose(o, o_ex, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(S, S_ex, rtol=1e-14, atol=1e-15)


# ---- P6 / P7: split-carry and varlen invariants (bitwise) ------------------

def test_split_carry_bitwise():
    c = _rand_case(11, 300, 2, 4, 16, 16)
    o_full, S_full = oracle.prefill(**c)
    S = c["state_in"]
    outs = []
    for t0, t1 in [(0, 64), (64, 65), (65, 200), (200, 300)]:
        part = {k_: (v_[t0:t1] if k_ in ("q", "k", "v", "a", "b", "z") else v_)
                for k_, v_ in c.items()}
        part["state_in"] = S
        o_p, S = oracle.prefill(**part)
        outs.append(o_p)
    assert np.array_equal(np.concatenate(outs), o_full)
    assert np.array_equal(S, S_full)


def test_varlen_equals_separate_calls_bitwise():
    lens = [5, 0, 17, 1, 40]
    T = sum(lens)
    N = len(lens)
    c = _rand_case(12, T, 2, 6, 8, 8, N=N)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o_p, S_p = oracle.prefill(**c, cu_seqlens=cu)
    for n in range(N):
        t0, t1 = cu[n], cu[n + 1]
        part = {k_: (v_[t0:t1] if k_ in ("q", "k", "v", "a", "b", "z") else v_)
                for k_, v_ in c.items()}
        part["state_in"] = c["state_in"][n:n + 1]
        o_n, S_n = oracle.prefill(**part)
        assert np.array_equal(o_p[t0:t1], o_n)
        assert np.array_equal(S_p[n:n + 1], S_n)
    # the zero-length sequence passes its state through
    assert np.array_equal(S_p[1], c["state_in"][1])


def test_null_state_equals_zero_state():
    c = _rand_case(13, 20, 1, 2, 8, 8, with_state=False)
    o1, S1 = oracle.prefill(**c)
    c["state_in"] = np.zeros((1, 2, 8, 8))
    o2, S2 = oracle.prefill(**c)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


# ---- P8: grouped value heads reduce to repeated key heads ------------------

@pytest.mark.parametrize("r", [2, 3])
def test_gva_equals_repeated_heads_bitwise(r):
    Hk = 2
    Hv = Hk * r
    c = _rand_case(14 + r, 33, Hk, Hv, 8, 8)
    o1, S1 = oracle.prefill(**c)
    rep = np.repeat(np.arange(Hk), r)  # blocked: value head h -> key h // r
    c2 = dict(c)
    c2["q"] = c["q"][:, rep]
    c2["k"] = c["k"][:, rep]
    o2, S2 = oracle.prefill(**c2)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
    # and the map is the blocked one: swapping key heads changes the result
    c3 = dict(c)
    c3["q"] = c["q"][:, ::-1].copy()
    c3["k"] = c["k"][:, ::-1].copy()
    o3, _ = oracle.prefill(**c3)
    assert not np.allclose(o1, o3)


# ---- P9: L2 normalisation invariance ----------------------------------------

def test_l2_scale_invariance():
    c = _rand_case(17, 40, 2, 4, 16, 8)
    c2 = dict(c)
    c2["q"] = c["q"] * 3.5
    c2["k"] = c["k"] * 0.25
    # without the epsilon the normalisation is exactly scale-free
    o1, S1 = oracle.prefill(**c, l2_eps=0.0)
    o2, S2 = oracle.prefill(**c2, l2_eps=0.0)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S2, S1, rtol=1e-12, atol=1e-14)
    # with eps = 1e-6 the change is O(eps / |x|^2) (|x|^2 ~ 16 here)
    o1, S1 = oracle.prefill(**c)
    c2["k"] = c["k"] * 2.0
    o2, S2 = oracle.prefill(**c2)
    np.testing.assert_allclose(o2, o1, rtol=1e-5, atol=1e-7)
    np.testing.assert_allclose(S2, S1, rtol=1e-5, atol=1e-7)
    # the q scale multiplies the pre-norm output linearly
    c3 = {k_: v_ for k_, v_ in c.items() if k_ not in ("z", "norm_w")}
    oa, _ = oracle.prefill(**c3, scale=1.0)
    ob, _ = oracle.prefill(**c3, scale=0.125)
    np.testing.assert_allclose(ob, 0.125 * oa, rtol=1e-13, atol=1e-16)


# ---- P10: chunked (WY) algebra equals the token recurrence ------------------

@pytest.mark.parametrize("T", synth.CONFIG1_TS)
@pytest.mark.parametrize("chunk", [64, 16])
def test_chunked_algebra_matches_recurrence(T, chunk):
    c = _rand_case(100 + T, T, 2, 4, 32, 16)
    o1, S1 = oracle.prefill(**c)
    o2, S2 = wy_model.prefill(**c, chunk=chunk)
    np.testing.assert_allclose(o2, o1, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S2, S1, rtol=1e-11, atol=1e-13)


def test_chunked_algebra_varlen_and_strong_gates():
    # varlen with partial chunks, and gates at the distribution's extremes
    lens = [70, 3, 64, 129]
    c = _rand_case(21, sum(lens), 1, 3, 16, 16, N=4)
    c["a"] *= 4.0
    cu = np.concatenate([[0], np.cumsum(lens)])
    o1, S1 = oracle.prefill(**c, cu_seqlens=cu)
    o2, S2 = wy_model.prefill(**c, cu_seqlens=cu)
    np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(S2, S1, rtol=1e-10, atol=1e-13)


# ---- P11: gated RMSNorm ------------------------------------------------------

def test_gated_norm_library_crosscheck():
    rng = np.random.default_rng(22)
    o = rng.standard_normal((5, 3, 16))
    z = rng.standard_normal((5, 3, 16))
    w = 1 + 0.02 * rng.standard_normal(16)
    y = oracle.gated_rmsnorm(o, z, w, 1e-6)
    ot = torch.from_numpy(o)
    ref = torch.nn.functional.rms_norm(ot, (16,), torch.from_numpy(w), 1e-6) * \
        torch.nn.functional.silu(torch.from_numpy(z))
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-13, atol=1e-15)


def test_gated_norm_special_values():
    D = 8
    w = np.linspace(0.5, 1.5, D)
    z = np.linspace(-2, 2, D)
    # z = 0 -> y = 0 exactly
    y0 = oracle.gated_rmsnorm(np.arange(D, dtype=float) + 1, np.zeros(D), w)
    assert np.all(y0 == 0.0)
    # constant o = c: RMSNorm(o) = c / sqrt(c^2 + eps)
    c_, eps = 0.003, 1e-6
    y = oracle.gated_rmsnorm(np.full(D, c_), z, w, eps)
    np.testing.assert_allclose(y, c_ / math.sqrt(c_ * c_ + eps) * w *
                               z * scipy.special.expit(z), rtol=1e-14)
    # linear in w
    y2 = oracle.gated_rmsnorm(np.full(D, c_), z, 2 * w, eps)
    np.testing.assert_allclose(y2, 2 * y, rtol=1e-15)


def test_prefill_applies_gated_norm_after_recurrence():
    c = _rand_case(23, 30, 2, 4, 16, 16)
    y, S = oracle.prefill(**c)
    c2 = {k_: v_ for k_, v_ in c.items() if k_ not in ("z", "norm_w")}
    o, S2 = oracle.prefill(**c2)
    assert np.array_equal(S, S2)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(o), (16,),
                                       torch.from_numpy(c["norm_w"]), 1e-6) * \
        torch.nn.functional.silu(torch.from_numpy(c["z"]))
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-15)


# ---- P13: the full layer's pieces ------------------------------------------

def test_causal_conv_matches_np_convolve():
    rng = np.random.default_rng(24)
    T, C, W = 37, 5, 4
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, W))
    y = oracle.causal_conv_silu(x, w)
    for c_ in range(C):
        # causal: output t uses x[t-3..t]; tap w[c, W-1] on the current token
        full = np.convolve(x[:, c_], w[c_, ::-1])[:T]
        np.testing.assert_allclose(y[:, c_], full * scipy.special.expit(full),
                                   rtol=1e-13, atol=1e-15)


def test_conv_history_closed_form():
    # W = 2, one history row h: y_0 = silu(w0 h + w1 x_0), y_1 = silu(w0 x_0 +
    # w1 x_1); the new history is x's last row
    x = np.array([[0.5, -1.0], [2.0, 0.25]])
    w = np.array([[0.3, -0.7], [1.1, 0.4]])
    h = np.array([[-2.0, 3.0]])
    silu = lambda u: u / (1.0 + np.exp(-u))
    want = np.array([[silu(0.3 * -2.0 - 0.7 * 0.5), silu(1.1 * 3.0 + 0.4 * -1.0)],
                     [silu(0.3 * 0.5 - 0.7 * 2.0), silu(1.1 * -1.0 + 0.4 * 0.25)]])
    np.testing.assert_allclose(oracle.causal_conv_silu(x, w, h), want, rtol=1e-14)
    np.testing.assert_array_equal(oracle.conv_history(x, 2, h), x[1:])
    # a sequence shorter than the history keeps the older history rows
    np.testing.assert_array_equal(
        oracle.conv_history(x[:1], 4, np.arange(6.0).reshape(3, 2)),
        np.array([[2.0, 3.0], [4.0, 5.0], [0.5, -1.0]]))


def test_conv_split_carry_exact():
    rng = np.random.default_rng(31)
    x = rng.standard_normal((23, 16))
    w = rng.standard_normal((16, 4))
    h0 = rng.standard_normal((3, 16))
    full = oracle.causal_conv_silu(x, w, h0)
    for cut in (0, 1, 2, 3, 7, 23):
        h1 = oracle.conv_history(x[:cut], 4, h0)
        parts = np.concatenate([oracle.causal_conv_silu(x[:cut], w, h0),
                                oracle.causal_conv_silu(x[cut:], w, h1)])
        np.testing.assert_allclose(parts, full, rtol=1e-14, atol=1e-15)


def test_layer_split_carry_matches_one_call():
    # two layer calls carrying the recurrent state and the conv history give
    # the one-call result (small geometry: hidden 32, Hk 1, Hv 2, D 8)
    rng = np.random.default_rng(32)
    T, hidden, Hk, Hv, D = 21, 32, 1, 2, 8
    width = 2 * Hk * D + 2 * Hv * D + 2 * Hv
    x = rng.standard_normal((T, hidden))
    W_in = 0.2 * rng.standard_normal((hidden, width))
    conv_w = rng.standard_normal((2 * Hk * D + Hv * D, 4))
    A_log = rng.uniform(0, 1, Hv)
    dt_bias = rng.uniform(-1, 1, Hv)
    w = 1 + 0.1 * rng.standard_normal(D)
    W_out = 0.2 * rng.standard_normal((Hv * D, hidden))
    args = (conv_w, A_log, dt_bias, w, W_out, Hk, Hv, D)
    out, S, hist = oracle.layer(x, W_in, *args, return_conv_state=True)
    for cut in (1, 2, 9):
        o1, S1, h1 = oracle.layer(x[:cut], W_in, *args, return_conv_state=True)
        o2, S2, h2 = oracle.layer(x[cut:], W_in, *args, state_in=S1,
                                  conv_state=h1, return_conv_state=True)
        np.testing.assert_allclose(np.concatenate([o1, o2]), out, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(S2, S, rtol=1e-10, atol=1e-14)
        np.testing.assert_array_equal(h2, hist)


def test_layer_wiring():
    # the layer oracle equals the composition of its documented steps
    Hk, Hv, D, T, hidden = 1, 2, 8, 12, 10
    rng = np.random.default_rng(25)
    width = 2 * Hk * D + 2 * Hv * D + 2 * Hv
    x = rng.standard_normal((T, hidden))
    W_in = 0.3 * rng.standard_normal((hidden, width))
    conv_w = rng.standard_normal((2 * Hk * D + Hv * D, 4))
    W_out = rng.standard_normal((Hv * D, 7))
    A_log = rng.uniform(0, 1, Hv)
    dt_bias = rng.uniform(-1, 1, Hv)
    w = 1 + 0.1 * rng.standard_normal(D)
    out, S = oracle.layer(x, W_in, conv_w, A_log, dt_bias, w, W_out, Hk, Hv, D)
    P = x @ W_in
    qkv = P[:, :32]
    conv = np.stack([np.convolve(qkv[:, c_], conv_w[c_, ::-1])[:T]
                     for c_ in range(32)], 1)
    act = conv * scipy.special.expit(conv)
    q = act[:, :8].reshape(T, 1, 8)
    k = act[:, 8:16].reshape(T, 1, 8)
    v = act[:, 16:32].reshape(T, 2, 8)
    z = P[:, 32:48].reshape(T, 2, 8)
    b = P[:, 48:50]
    a = P[:, 50:52]
    y, S2 = oracle.prefill(q, k, v, a, b, A_log, dt_bias, z=z, norm_w=w)
    np.testing.assert_allclose(out, y.reshape(T, 16) @ W_out, rtol=1e-11,
                               atol=1e-13)
    np.testing.assert_allclose(S, S2, rtol=1e-12, atol=1e-15)


# ---- argument checks ---------------------------------------------------------

def test_oracle_rejects_bad_arguments():
    c = _rand_case(26, 8, 2, 3, 4, 4, with_norm=False)  # Hv % Hk != 0
    with pytest.raises(ValueError):
        oracle.prefill(**c)
    c = _rand_case(27, 8, 1, 2, 4, 4, N=2, with_norm=False)
    with pytest.raises(ValueError):
        oracle.prefill(**c, cu_seqlens=[0, 9, 8])
