"""The quotient psi / w of the model residual, formed from y = 1 / w rounded
to nearest with two corrections by fused multiply-adds, is the quotient
rounded to nearest (the assembly forms Z with the division itself, and the
residual on the fly must equal the residual of that Z bit for bit).

The corrections are those of the last step of a Newton-Raphson division
(Markstein's theorem: with y within half an ulp of 1 / w and q faithful,
q + (psi - w q) y rounds to the quotient).  Here each fused multiply-add is
evaluated exactly with rationals and rounded once, as the hardware does, over
the range the kernel takes this path in: |w| in [2^-64, 2^64] and |psi| in
[2^-900, 2^900], with quotients drawn near the midpoints between doubles too.
"""
import random
from fractions import Fraction

import pytest


def fma(a, b, c):
    return float(Fraction(a) * Fraction(b) + Fraction(c))


def by_reciprocal(psi, w):
    y = 1.0 / w
    q = psi * y
    r = fma(-q, w, psi)
    q = fma(r, y, q)
    r = fma(-q, w, psi)
    return fma(r, y, q)


def draw(rng, lo_e, hi_e):
    m = rng.getrandbits(52) | (1 << 52)
    v = m * 2.0 ** (rng.randint(lo_e, hi_e) - 52)
    return -v if rng.random() < 0.5 else v


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_quotient_rounds_like_the_division(seed):
    rng = random.Random(seed)
    for _ in range(2000):
        w = draw(rng, -64, 63)
        psi = draw(rng, -900, 899)
        assert by_reciprocal(psi, w) == psi / w, (psi, w)


def test_quotients_near_midpoints_and_range_ends():
    rng = random.Random(7)
    cases = []
    for _ in range(2000):
        # psi = w (q + ulp(q) / 2), rounded: quotients a hair from a midpoint
        w = draw(rng, -30, 30)
        q = draw(rng, -60, 60)
        psi = float(Fraction(w) * (Fraction(q) + Fraction(abs(q) * 2.0 ** -52) / 2))
        cases.append((psi, w))
    for w in (2.0 ** -64, 2.0 ** 64, -(2.0 ** -64), 1.0 + 2.0 ** -52, 3.0, 0.1, 6.283185307179586e9):
        for psi in (2.0 ** -900, 2.0 ** 900, -(2.0 ** -900) * 1.5, 2.0 ** 899 * 1.9999999999999998, 1.0, -7.0):
            cases.append((psi, w))
    for psi, w in cases:
        assert by_reciprocal(psi, w) == psi / w, (psi, w)
