"""Parity metrics of the GPU tests, in numpy only (no GPU, no oracle call).

A result is compared with the oracle's fp64 value slice by slice: one
(sequence, value head) block of the output, or one (sequence, value head)
state.  Two checks per slice, both against the same bar:

* relative L2 error, ||x - r|| / ||r|| <= bar;
* element by element, |x_i - r_i| <= bar * (|r_i| + rms(r)) for every
  element.  The rms of the slice keeps elements near zero from being held to
  a relative bar their own size cannot carry; an element wrong by more than
  the bar times the slice's scale is counted, and the count must be zero.

The bars are the operator's: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs.

Conditioning (fp32 only).  A one-token slice's output is o = S q^ with S the
state after the token.  When q^ is nearly orthogonal to what S holds, o is
small through cancellation and any fp32 evaluation of the product has a
relative error of about u * kappa, where

    kappa = ||S||_F ||q^|| / ||S q^||   (>= 1)

is the condition number of that matrix-vector product (u = 2^-24).  In a
one-token sequence from a zero state, S = beta v k^T and kappa reduces to
||k^|| ||q^|| / |k^ . q^|.  For such slices the fp32 output bar is 1e-4 * kappa, the
relative error that a relative perturbation of 1e-4 in the product's terms
can produce.  The gated RMSNorm divides each row by its own rms, which keeps
the row's relative error, so the same kappa applies to y.  Slices of more
than one token keep the plain bar (the oracle does not return the per-token
states that kappa would need there), and so do bf16 slices (their 2e-2 bar
is far above the fp32 arithmetic).
"""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(ref))
    num = float(np.linalg.norm(x - ref))
    return num / den if den > 0 else num


def elementwise(x, ref, bar: float):
    """(violations, worst ratio) of |x - r| <= bar * (|r| + rms(r))."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0, 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    bound = bar * (np.abs(ref) + rms)
    err = np.abs(x - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0),
                         np.where(err > 0, np.inf, 0.0))
    # NaN anywhere is a violation, never a pass
    ratio = np.where(np.isnan(ratio), np.inf, ratio)
    return int(np.count_nonzero(ratio > 1.0)), float(ratio.max())


def qhat(q, scale: float, l2_eps: float = 1e-6):
    q = np.asarray(q, dtype=np.float64)
    return scale * q / np.sqrt(np.dot(q, q) + l2_eps)


def one_token_kappa(S, qh) -> float:
    """Condition number ||S||_F ||q^|| / ||S q^|| of o = S q^ (at least 1)."""
    S = np.asarray(S, dtype=np.float64)
    qh = np.asarray(qh, dtype=np.float64)
    num = float(np.linalg.norm(S) * np.linalg.norm(qh))
    den = float(np.linalg.norm(S @ qh))
    if den == 0.0:
        return np.inf if num > 0 else 1.0
    return max(1.0, num / den)


class Tally:
    """Worst figures over the slices of one result."""

    def __init__(self):
        self.rel = 0.0        # largest relative L2 error of a slice
        self.rel_bar = 0.0    # largest (relative L2 error / that slice's bar)
        self.viol = 0         # elements outside their elementwise bound
        self.worst = 0.0      # largest elementwise (error / bound)
        self.kappa = 1.0      # largest bar scale applied
        self.slices = 0

    def add(self, x, ref, bar: float, kappa: float = 1.0):
        r = rel_l2(x, ref)
        b = bar * kappa
        v, w = elementwise(x, ref, b)
        self.rel = max(self.rel, r)
        self.rel_bar = max(self.rel_bar, r / b if np.isfinite(r) else np.inf)
        self.viol += v
        self.worst = max(self.worst, w)
        self.kappa = max(self.kappa, kappa)
        self.slices += 1

    @property
    def ok(self) -> bool:
        return self.rel_bar <= 1.0 and self.viol == 0

    def __repr__(self):
        return ("rel=%.3e rel/bar=%.3f viol=%d worst_elem/bound=%.3f kappa_max=%.3g"
                % (self.rel, self.rel_bar, self.viol, self.worst, self.kappa))


def abs_stats(x, ref) -> dict:
    """max / mean / p99 of |x - ref| over a whole array (the pages' figures)."""
    err = np.abs(np.asarray(x, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    if err.size == 0:
        return dict(max_abs=0.0, mean_abs=0.0, p99_abs=0.0)
    return dict(max_abs=float(err.max()), mean_abs=float(err.mean()),
                p99_abs=float(np.percentile(err, 99)))
