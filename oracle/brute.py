"""Exact rational brute force of the gated delta rule on tiny heads.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

This is a second, independent formulation of the recurrence, used to pin the
fp64 oracle: instead of stepping the state, it expands the state after t
tokens as an explicit sum of products of per-token transition matrices,

    S_t = S_0 A_1 A_2 ... A_t + sum_{s<=t} B_s A_{s+1} ... A_t,
    A_r = alpha_r (I - beta_r k_r k_r^T),     B_s = beta_s v_s k_s^T,

where the k_r are the (already normalised) keys.  Each S_t is rebuilt from
scratch with this formula, in exact ``fractions.Fraction`` arithmetic, and
o_t = S_t q_t.  Only tiny D (<= 4) and T (<= 8) are practical.

Source of the operator: "Add opt-in fused Qwen3.5 inference kernels"
(JevAny PR #29), Summary -- the gated delta rule whose ingredients are the
decay gate, the sigmoid beta and normalised keys; the formula itself is the
operator's definition, which the pages do not print.
"""
from __future__ import annotations

from fractions import Fraction


def _eye(n):
    return [[Fraction(int(i == j)) for j in range(n)] for i in range(n)]


def _matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][l] * B[l][j] for l in range(m)), Fraction(0))
             for j in range(p)] for i in range(n)]


def _add(A, B):
    return [[x + y for x, y in zip(ra, rb)] for ra, rb in zip(A, B)]


def _transition(alpha, beta, kvec):
    n = len(kvec)
    return [[alpha * (Fraction(int(i == j)) - beta * kvec[i] * kvec[j])
             for j in range(n)] for i in range(n)]


def _outer(u, w):
    return [[x * y for y in w] for x in u]


def state_after(t, alpha, beta, kn, v, S0):
    """S_t from the explicit expansion (t tokens consumed, 0 <= t <= T)."""
    Dk = len(kn[0]) if kn else len(S0[0])
    # S_0 A_1 ... A_t
    P = _eye(Dk)
    for r in range(t):
        P = _matmul(P, _transition(alpha[r], beta[r], kn[r]))
    S = _matmul(S0, P)
    for s in range(t):
        B = [[beta[s] * x for x in row] for row in _outer(v[s], kn[s])]
        Q = _eye(Dk)
        for r in range(s + 1, t):
            Q = _matmul(Q, _transition(alpha[r], beta[r], kn[r]))
        S = _add(S, _matmul(B, Q))
    return S


def outputs(alpha, beta, kn, qn, v, S0):
    """Returns ([o_1..o_T], S_T) with o_t = S_t q_t, all exact Fractions."""
    T = len(alpha)
    outs = []
    for t in range(1, T + 1):
        S = state_after(t, alpha, beta, kn, v, S0)
        outs.append([sum((S[i][j] * qn[t - 1][j] for j in range(len(qn[0]))),
                         Fraction(0)) for i in range(len(S))])
    return outs, state_after(T, alpha, beta, kn, v, S0)
