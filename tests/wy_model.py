"""Test-only fp64 model of the chunked (WY / UT) form of the gated delta rule.

It is a second, independently structured computation of the same operator:
the token loop of the oracle is replaced by per-chunk dense algebra, exactly
the algebra the HIP kernels evaluate (in lower precision).  Agreement with the
oracle to ~1e-12 pins both the oracle and the chunk algebra.

Derivation (the pages print none; the operator is the gated delta rule named
in "Add opt-in fused Qwen3.5 inference kernels", Summary).  With H = S^T the
Dk x Dv state at chunk entry, gamma_t the in-chunk cumulative log-decay,
K, Q the raw key/query rows and rk, rq their inverse L2 norms (rq includes
the q scale), the per-token delta writes u_t satisfy

    (I + A) U = diag(beta) (V - diag(e^gamma * rk) K H),
    A_ts = beta_t e^{gamma_t - gamma_s} rk_t rk_s (K K^T)_ts   (t > s),
    O    = diag(e^gamma * rq) Q H + MP U,
    MP_ts = e^{gamma_t - gamma_s} rq_t rk_s (Q K^T)_ts          (s <= t),
    H'   = e^{gamma_L} H + K^T diag(e^{gamma_L - gamma} * rk) U.
"""
from __future__ import annotations

import numpy as np
import scipy.linalg


def _softplus(x):
    return np.logaddexp(0.0, x)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def chunk_step(Kc, Qc, Vc, g, beta, rk, rq, H, operand_round=None):
    """One chunk.  Kc, Qc [L, Dk]; Vc [L, Dv]; g, beta, rk, rq [L]; H [Dk, Dv].
    Returns (O [L, Dv], H_next [Dk, Dv]).

    operand_round (a function, or None for plain fp64) rounds the products'
    operands where a reduced-precision matrix unit takes them: the copy of H
    multiplied by K and Q, R = V - diag(e^gamma rk) K H, the explicit
    Tb = (I + A)^-1 diag(beta), the delta writes U as the output's operand,
    diag(fk) U as the state update's operand, and MP.  The raw K, Q, V rows,
    the per-row factors, the sums and the carried H stay in fp64."""
    L = Kc.shape[0]
    gam = np.cumsum(g)
    diff = gam[:, None] - gam[None, :]
    lower_strict = np.tril(np.ones((L, L), dtype=bool), -1)
    lower = np.tril(np.ones((L, L), dtype=bool), 0)
    decay = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
    G = (Kc @ Kc.T) * rk[:, None] * rk[None, :]
    A = np.where(lower_strict, beta[:, None] * decay * G, 0.0)
    P = (Qc @ Kc.T) * rq[:, None] * rk[None, :]
    MP = decay * P
    fk = np.exp(gam[-1] - gam) * rk
    if operand_round is not None:
        rd = operand_round
        Hb = rd(H)
        R = rd(Vc - (np.exp(gam) * rk)[:, None] * (Kc @ Hb))
        Tb = rd(scipy.linalg.solve_triangular(np.eye(L) + A, np.diag(beta),
                                              lower=True, unit_diagonal=True))
        U = Tb @ R
        O = (np.exp(gam) * rq)[:, None] * (Qc @ Hb) + rd(MP) @ rd(U)
        Hn = np.exp(gam[-1]) * H + Kc.T @ rd(fk[:, None] * U)
        return O, Hn
    R = Vc - (np.exp(gam) * rk)[:, None] * (Kc @ H)
    U = scipy.linalg.solve_triangular(np.eye(L) + A, beta[:, None] * R,
                                      lower=True, unit_diagonal=True)
    O = (np.exp(gam) * rq)[:, None] * (Qc @ H) + MP @ U
    Hn = np.exp(gam[-1]) * H + Kc.T @ (fk[:, None] * U)
    return O, Hn


def prefill(q, k, v, a, b, A_log, dt_bias, z=None, norm_w=None, state_in=None,
            cu_seqlens=None, scale=None, l2_eps=1e-6, norm_eps=1e-6, chunk=64,
            operand_round=None):
    """The prefill by chunks (arguments as the oracle's).  operand_round: see
    chunk_step; when given, the stored output is rounded with it as well."""
    q, k, v, a, b = (np.asarray(x, dtype=np.float64) for x in (q, k, v, a, b))
    T, Hk, Dk = q.shape
    Hv, Dv = v.shape[1:]
    r = Hv // Hk
    scale = Dk ** -0.5 if scale is None else scale
    cu = [0, T] if cu_seqlens is None else [int(x) for x in cu_seqlens]
    N = len(cu) - 1
    o = np.zeros((T, Hv, Dv))
    S_out = np.zeros((N, Hv, Dv, Dk))
    for n in range(N):
        t0, t1 = cu[n], cu[n + 1]
        for h in range(Hv):
            kh = h // r
            H = (np.zeros((Dk, Dv)) if state_in is None
                 else np.asarray(state_in[n, h], dtype=np.float64).T.copy())
            for c0 in range(t0, t1, chunk):
                c1 = min(c0 + chunk, t1)
                Kc = k[c0:c1, kh]
                Qc = q[c0:c1, kh]
                Vc = v[c0:c1, h]
                g = -np.exp(float(A_log[h])) * _softplus(a[c0:c1, h]
                                                         + float(dt_bias[h]))
                beta = _sigmoid(b[c0:c1, h])
                rk = 1.0 / np.sqrt((Kc * Kc).sum(1) + l2_eps)
                rq = scale / np.sqrt((Qc * Qc).sum(1) + l2_eps)
                O, H = chunk_step(Kc, Qc, Vc, g, beta, rk, rq, H,
                                  operand_round)
                o[c0:c1, h] = O
            S_out[n, h] = H.T
    if z is not None:
        z = np.asarray(z, dtype=np.float64)
        w = np.asarray(norm_w, dtype=np.float64)
        rms = 1.0 / np.sqrt((o * o).mean(-1, keepdims=True) + norm_eps)
        o = o * rms * w * (z * _sigmoid(z))
    if operand_round is not None:
        o = operand_round(o)
    return o, S_out
