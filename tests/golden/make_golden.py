"""Writes the exact-rational fixtures in this folder.  Calls only oracle/.

Run from the repository root:  python tests/golden/make_golden.py

worked_d2.json: a four-token, two-block, d = 2 example small enough to
check by hand (the derivation is in worked_d2.md).  Visibility follows
the block-causal rule of "Nvidia, MIT ve diğerleri video yapay zeka
devrimini başlattı", section "Sabit Bellekli KV önbelleğe alma
mekanizması": a block's queries see KVsum of the earlier blocks plus the
block's own KV.

exact_random.json: seeded small-integer cases (T <= 12, d <= 4, random
block boundaries) with eps = the float32 value nearest 1e-6, solved in
exact rationals by the quadratic form.
"""

import json
import os
import sys
from fractions import Fraction

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402


def frac_str(x):
    return f"{x.numerator}/{x.denominator}"


def case(q, k, v, blocks, eps):
    out = oracle.quadratic_exact(q, k, v, blocks, eps)
    return {
        "q": q, "k": k, "v": v, "blocks": blocks, "eps": frac_str(Fraction(eps)),
        "out": [[frac_str(x) for x in row] for row in out],
    }


def main():
    worked = case(
        q=[[1, 0], [0, 2], [1, 1], [-1, 3]],
        k=[[1, 1], [2, -1], [0, 1], [3, 0]],
        v=[[1, 0], [0, 1], [2, 2], [-1, 4]],
        blocks=[0, 0, 1, 1],
        eps=Fraction(1, 4),
    )
    hand = [["4/13", "8/13"], ["8/9", "0/1"], ["4/33", "64/33"], ["36/25", "24/25"]]
    assert worked["out"] == hand, worked["out"]
    with open(os.path.join(HERE, "worked_d2.json"), "w") as f:
        json.dump(worked, f, indent=1)

    eps = Fraction(float(np.float32(1e-6)))
    rng = np.random.default_rng(20250924)
    cases = []
    for _ in range(6):
        T = int(rng.integers(3, 13))
        d = int(rng.integers(1, 5))
        cuts = sorted(set(int(c) for c in rng.integers(1, T, size=int(rng.integers(0, 4)))))
        blocks, b = [], 0
        for t in range(T):
            if t in cuts:
                b += 1
            blocks.append(b)
        q, k, v = (rng.integers(-3, 4, size=(T, d)).tolist() for _ in range(3))
        cases.append(case(q, k, v, blocks, eps))
    with open(os.path.join(HERE, "exact_random.json"), "w") as f:
        json.dump(cases, f, indent=1)


if __name__ == "__main__":
    main()
