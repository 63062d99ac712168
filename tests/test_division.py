"""The column solve forms w / s as RN(q0 + RN(w - q0 s) y) with y = RN(1/s) and q0 = RN(w y)
(an FMA correction of the product with the correctly rounded reciprocal).  That this equals
the IEEE quotient RN(w / s), which is how the codes are defined, is Markstein's theorem; this
test checks it with exact rational arithmetic on random and on edge-case operands."""

from fractions import Fraction

import numpy as np


def rn32(x: Fraction) -> np.float32:
    """Round an exact rational to the nearest float32, ties to even."""
    c = np.float32(float(x))
    best = None
    for v in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        key = (abs(Fraction(float(v)) - x), int(np.float32(v).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, np.float32(v))
    return best[1]


def refined_quotient(w: np.float32, s: np.float32) -> np.float32:
    F = lambda v: Fraction(float(v))
    y = rn32(Fraction(1) / F(s))
    q0 = rn32(F(w) * F(y))
    r = rn32(F(w) - F(q0) * F(s))          # exact in an FMA
    return rn32(F(q0) + F(r) * F(y))


def test_refined_quotient_matches_ieee_division():
    rng = np.random.default_rng(2024)
    cases = []
    for _ in range(3000):                   # scales and weights of the magnitudes that occur
        s = np.float32(np.exp(rng.uniform(-12, 2)) * (1 + rng.integers(0, 2 ** 23) / 2 ** 23))
        w = np.float32(rng.uniform(-20, 20) * s * (1 if rng.random() < 0.5 else rng.random()))
        cases.append((w, s))
    for k in list(range(0, 40)) + list(range(2 ** 23 - 40, 2 ** 23)):   # mantissas at the ends
        s = np.float32((1 + k / 2 ** 23) * 2.0 ** int(rng.integers(-8, 3)))
        for m in (0, 1, 2 ** 22, 2 ** 23 - 1, int(rng.integers(0, 2 ** 23))):
            w = np.float32((1 + m / 2 ** 23) * 2.0 ** int(rng.integers(-10, 4)))
            cases += [(w, s), (-w, s)]
    for w, s in cases:
        assert refined_quotient(w, s) == np.float32(w) / np.float32(s), (w, s)
