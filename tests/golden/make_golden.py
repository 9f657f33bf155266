"""Write tests/golden/exact_tiny.json from the exact rational oracle.

The pages print no worked numeric example for KDA, so this fixture holds the
exact rational result of the recurrence (oracle/exact.py) on a tiny input whose
entries are dyadic rationals: exactly representable in bf16, fp32 and fp64, with
decays alpha given directly as rationals.  Regenerate with
    python tests/golden/make_golden.py
It imports nothing but oracle/.
"""
import json
import os
import sys
from fractions import Fraction as Fr

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle.exact import brute_force  # noqa: E402


def main():
    T, dk, dv = 6, 4, 3
    # Hand-picked dyadic entries (at most 4 significant bits), mixed signs.
    q = [[0.5, -0.25, 0.75, 0.125], [0.25, 0.5, -0.5, 0.375], [-0.75, 0.25, 0.125, 0.5],
         [0.375, -0.625, 0.25, -0.125], [0.5, 0.5, 0.5, -0.5], [-0.25, 0.875, -0.375, 0.25]]
    k = [[0.5, 0.5, -0.5, 0.5], [0.75, -0.25, 0.25, 0.5], [0.125, 0.625, 0.5, -0.5],
         [-0.5, 0.25, 0.75, 0.25], [0.25, -0.75, 0.375, 0.5], [0.625, 0.125, -0.25, -0.625]]
    v = [[1.0, -0.5, 0.25], [-1.5, 0.75, 2.0], [0.5, 1.25, -0.75], [2.0, -1.0, 0.5],
         [-0.25, 0.5, 1.5], [0.75, -1.75, -0.5]]
    alpha = [[0.875, 0.5, 1.0, 0.75], [0.9375, 0.625, 0.5, 1.0], [0.75, 0.875, 0.9375, 0.5],
             [1.0, 0.75, 0.625, 0.875], [0.5, 0.9375, 0.75, 0.625], [0.625, 1.0, 0.875, 0.9375]]
    beta = [0.5, 0.75, 0.25, 1.0, 0.625, 0.375]
    S0 = [[0.25, -0.5, 0.0], [0.125, 0.25, -0.25], [-0.375, 0.0, 0.5], [0.0, 0.75, 0.125]]
    o, S = brute_force(q, k, v, alpha, beta, S0)
    out = dict(
        source="exact rational brute force of the KDA recurrence (oracle/exact.py); "
               "the pages print no worked example",
        T=T, d_k=dk, d_v=dv, q=q, k=k, v=v, alpha=alpha, beta=beta, S0=S0,
        o=[[str(x) for x in row] for row in o],
        S=[[str(x) for x in row] for row in S],
    )
    with open(os.path.join(HERE, "exact_tiny.json"), "w") as f:
        json.dump(out, f, indent=1)
    print("wrote exact_tiny.json; o[-1] =", [float(Fr(x)) for x in out["o"][-1]])


if __name__ == "__main__":
    main()
