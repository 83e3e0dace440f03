"""Writes the worked-example fixtures in this folder.

Calls only ``oracle.brute`` (exact rational arithmetic on the masked
second-order definition).  Run from the repository root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys
from fractions import Fraction

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import brute  # noqa: E402

CITE = ("Higher-order Linear Attention: masked output q_t^T(S_t C_t - G_t) "
        "(gist.science explainer, Technische Zusammenfassung, Methodik item 1); "
        "mask j <= t (paperlayer.ai summary, sec. 3.1); decay (sec. 4.3); "
        "ridge lambda*I and ratio normalization (sec. 5.1).")

Q = [[1], [2], [-1]]
K = [[1], [1], [2]]
V = [[1], [-1], [3]]


def frac(x):
    return f"{x.numerator}/{x.denominator}"


def main():
    cases = []
    for g, lam in [(Fraction(1), Fraction(0)), (Fraction(1, 2), Fraction(0)),
                   (Fraction(1, 2), Fraction(1, 4)), (Fraction(3, 4), Fraction(1, 2))]:
        num, den = brute.masked_exact(Q, K, V, g, lam)
        cases.append({"gamma": frac(g), "lambda": frac(lam),
                      "num": [[frac(x) for x in row] for row in num],
                      "den": [frac(x) for x in den]})
    doc = {"citation": CITE,
           "note": "d = dv = 1, one head, three tokens; every value is dyadic, "
                   "hence exact in fp32 and fp64.",
           "q": Q, "k": K, "v": V, "cases": cases}
    with open(os.path.join(HERE, "worked_example_d1.json"), "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
