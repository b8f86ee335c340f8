"""Writes tests/golden/delta_rule_tiny.json.

The pages print no worked example for the operator, so this fixture is an
exact-rational one: small dyadic inputs, and outputs from the explicit
product expansion in ``oracle.brute`` (exact ``Fraction`` arithmetic).  Only
``oracle/`` is called.  Run from the repository root:

    python tests/golden/make_golden.py
"""
import json
import os
import sys
from fractions import Fraction as F

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(
    os.path.abspath(__file__)))))
from oracle import brute  # noqa: E402

alpha = [F(1, 2), F(3, 4), F(1), F(7, 8)]
beta = [F(1, 4), F(1, 2), F(1), F(3, 8)]
kn = [[F(1), F(0), F(0)], [F(1, 2), F(1, 2), F(0)], [F(0), F(0), F(1)],
      [F(-1, 4), F(1, 2), F(3, 4)]]
qn = [[F(1), F(1), F(0)], [F(0), F(1, 2), F(-1)], [F(1, 8), F(0), F(1)],
      [F(1), F(-1), F(1, 2)]]
v = [[F(2), F(-1)], [F(1, 2), F(3)], [F(-3, 4), F(1, 4)], [F(1), F(1)]]
S0 = [[F(1, 16), F(0), F(-1, 8)], [F(0), F(1, 4), F(1, 32)]]

o, S = brute.outputs(alpha, beta, kn, qn, v, S0)
fl = lambda m: [[float(x) for x in r] for r in m]
out = {
    "about": "gated delta rule, T=4, Dk=3, Dv=2; exact outputs from the "
             "product expansion S_t = S_0 A_1..A_t + sum_s B_s A_{s+1}..A_t",
    "alpha": [float(x) for x in alpha], "beta": [float(x) for x in beta],
    "kn": fl(kn), "qn": fl(qn), "v": fl(v), "S0": fl(S0),
    "o_exact": [[str(x) for x in r] for r in o],
    "S_exact": [[str(x) for x in r] for r in S],
}
path = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                    "delta_rule_tiny.json")
with open(path, "w") as f:
    json.dump(out, f, indent=1)
print("wrote", path)
