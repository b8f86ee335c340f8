"""Parity metrics of the GPU tests, in numpy only (no GPU, no oracle call).

A result is compared with the oracle's fp64 value slice by slice: one
(sequence, value head) block of the output, or one (sequence, value head)
state.  Two checks per slice, both against the same bar:

* relative L2 error, ||x - r|| / ||r|| <= bar;
* element by element, |x_i - r_i| <= bar * (|r_i| + s_i), with s_i the
  scale an element's rounding errors have:
    - rms(r) of the slice for a state or an output without the gated norm
      (so that elements near zero are not held to a relative bar their own
      size cannot carry);
    - |w_i silu(z_i)| for an output of the gated norm y = o / rms(o) * w *
      silu(z): o's rounding errors are of the size of its row's rms, and
      each element passes them on multiplied by its own gate.  An element
      whose o is near zero under a gate of 4 would otherwise be held to a
      bound four times tighter than its error (seen on bf16 rows).
  For bf16 outputs both scales also take the size of the element's terms.
  o_t[i] is the sum of the products S_t[i,j] q^_t[j]; evaluated from bf16
  operands it carries an error of the order of 2^-9 times the root-sum-
  square of those products (term_rss, returned by the oracle), whatever
  their sum.  When q^_t is nearly orthogonal to what the state holds -- a
  strongly decaying head whose state is dominated by its last few keys,
  read by a query at right angles to them -- the sum is small through
  cancellation and only that absolute accuracy is there to have.  So s_i is
  max(rms(r), term_rss_i) without the norm and |w_i silu(z_i)| *
  max(1, term_rss_i / rms(o_t)) with it.  A randomized bf16 sweep found
  such elements at up to 2.7 times the rms-scaled bound, each within half
  of the term-scaled one; so does the chunk algebra evaluated exactly
  except for the rounding of its operands (tests/test_parity_bound_cpu.py).
  Well-conditioned elements keep the rms scale (term_rss is below it).
  A bf16 final state takes the same reasoning through its own terms: it is
  the decayed carried state plus sums of products k_s[j] w_s[i], and when
  the sizes of those terms separate into a row factor and a column factor,
  element (i, j) has terms of size rms_row(i) * rms_col(j) / rms(slice).
  Its scale is the larger of that envelope and the slice's rms, so an
  element where a large row meets a large column and the sum cancels is held
  to the accuracy its terms allow (one element at 1.04 times the rms-scaled
  bound in 1,200 sweep cases; the same bf16 operand model reproduces it).

The bars are the operator's: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs.

Tail budget.  Elements outside their bound are counted.  fp32 results allow
none.  bf16 results allow a small stated fraction of elements between 1 and
`cap` times their bound (tail rounding: the products take bf16 operands, the
per-element errors are sums of many such roundings), and none beyond `cap`;
a wrong element or row misses its bound by an order of magnitude and fails
the cap.  The SM120 prefill page reports its own comparison the same way,
as a count of localised tail violations over the final-state elements
("feat(qwen35): add SM120 FlashInfer GDN prefill candidate", Correctness).

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
# elements allowed between 1 and CAP times their bound, as a fraction of a
# result's elements (prefill and decode results; the layer's are in
# tests/test_gpu_layer.py)
TAIL = {"f32": 0.0, "bf16": 1e-5}
CAP = {"f32": 1.0, "bf16": 2.0}


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(ref))
    num = float(np.linalg.norm(x - ref))
    return num / den if den > 0 else num


def gate(norm_w, z):
    """|w silu(z)| of each element of a gated-norm output (z [..., D])."""
    z = np.asarray(z, dtype=np.float64)
    return np.abs(np.asarray(norm_w, dtype=np.float64) * (z / (1.0 + np.exp(-z))))


def elementwise(x, ref, bar: float, scale=None):
    """(violations, worst ratio) of |x - r| <= bar * (|r| + s), s = rms(r)
    of the slice or the given per-element scale."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0, 0.0
    s = float(np.sqrt(np.mean(ref * ref))) if scale is None else np.asarray(scale)
    bound = bar * (np.abs(ref) + s)
    err = np.abs(x - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0),
                         np.where(err > 0, np.inf, 0.0))
    # NaN anywhere is a violation, never a pass
    ratio = np.where(np.isnan(ratio), np.inf, ratio)
    return int(np.count_nonzero(ratio > 1.0)), float(ratio.max())


def term_scale(ref, term_rss):
    """Element scale of a bf16 output without the gated norm: the larger of
    the slice's rms and each element's term size."""
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    return np.maximum(rms, np.asarray(term_rss, dtype=np.float64))


def outer_envelope(ref):
    """Element scale of a bf16 state slice [Dv, Dk]: max(rms, rms_row(i) *
    rms_col(j) / rms), the term size of a sum of outer products whose sizes
    separate by row and column."""
    ref = np.asarray(ref, dtype=np.float64)
    sq = ref * ref
    rms = float(np.sqrt(np.mean(sq))) if ref.size else 0.0
    if rms == 0.0:
        return np.zeros_like(ref)
    row = np.sqrt(np.mean(sq, axis=1, keepdims=True))
    col = np.sqrt(np.mean(sq, axis=0, keepdims=True))
    return np.maximum(rms, row * col / rms)


def gated_term_scale(gate_scale, o_raw, term_rss, norm_eps: float = 1e-6):
    """Element scale of a bf16 gated-norm output: the gate |w silu(z)| times
    the element's term size relative to its row's rms (at least 1)."""
    o_raw = np.asarray(o_raw, dtype=np.float64)
    rms = np.sqrt(np.mean(o_raw * o_raw, axis=-1, keepdims=True) + norm_eps)
    return np.asarray(gate_scale) * np.maximum(1.0, np.asarray(term_rss) / rms)


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
    """Worst figures over the slices of one result.  `tail` and `cap`: the
    tail budget (fraction of elements allowed between 1 and cap times their
    bound)."""

    def __init__(self, tail: float = 0.0, cap: float = 1.0):
        self.rel = 0.0        # largest relative L2 error of a slice
        self.rel_bar = 0.0    # largest (relative L2 error / that slice's bar)
        self.viol = 0         # elements outside their elementwise bound
        self.worst = 0.0      # largest elementwise (error / bound)
        self.kappa = 1.0      # largest bar scale applied
        self.slices = 0
        self.elems = 0
        self.tail = tail
        self.cap = max(cap, 1.0)

    @classmethod
    def for_dtype(cls, dtype: str):
        return cls(TAIL[dtype], CAP[dtype])

    def add(self, x, ref, bar: float, kappa: float = 1.0, scale=None):
        r = rel_l2(x, ref)
        b = bar * kappa
        v, w = elementwise(x, ref, b, scale)
        self.rel = max(self.rel, r)
        self.rel_bar = max(self.rel_bar, r / b if np.isfinite(r) else np.inf)
        self.viol += v
        self.worst = max(self.worst, w)
        self.kappa = max(self.kappa, kappa)
        self.slices += 1
        self.elems += int(np.asarray(ref).size)

    @property
    def ok(self) -> bool:
        return (self.rel_bar <= 1.0 and self.worst <= self.cap
                and self.viol <= self.tail * self.elems)

    def __repr__(self):
        return ("rel=%.3e rel/bar=%.3f viol=%d/%d worst_elem/bound=%.3f kappa_max=%.3g"
                % (self.rel, self.rel_bar, self.viol, self.elems, self.worst, self.kappa))


def abs_stats(x, ref) -> dict:
    """max / mean / p99 of |x - ref| over a whole array (the pages' figures)."""
    err = np.abs(np.asarray(x, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    if err.size == 0:
        return dict(max_abs=0.0, mean_abs=0.0, p99_abs=0.0)
    return dict(max_abs=float(err.max()), mean_abs=float(err.mean()),
                p99_abs=float(np.percentile(err, 99)))
