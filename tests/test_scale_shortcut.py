"""The quantisers' block scale d = fp32(amax / Fmax) without an IEEE
division: d0 = RN(amax * c) with c = RN(1 / Fmax), r = amax - d0 * Fmax
(exact through an FMA), d = RN(d0 + r * c) (one correction step, Markstein's
method).  amax is the maximum of bf16 values, so every possible amax is a
positive finite bf16: this test runs the sequence in exact rational
arithmetic for all 32639 of them, for Fmax = 448 (E4M3) and 57344 (E5M2),
and requires the correctly rounded quotient each time.  (The GPU sweep in
test_gpu_sweeps.py then checks the kernels' codes and scales for every
amax with every |x| <= amax.)"""
import math
from fractions import Fraction as Fr

import numpy as np
import pytest


def rn32(q: Fr) -> float:
    """Nearest float32 (ties to even) of an exact rational, subnormals included."""
    if q == 0:
        return 0.0
    s = -1 if q < 0 else 1
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fr(2) ** e > q:
        e -= 1
    while Fr(2) ** (e + 1) <= q:
        e += 1
    ulp = Fr(2) ** (max(e, -126) - 23)
    n = q / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and fl % 2 == 1):
        fl += 1
    return s * float(fl * ulp)


def test_rn32_matches_numpy_on_random_quotients():
    rng = np.random.default_rng(3)
    for a, b in rng.uniform(1e-3, 1e3, size=(200, 2)):
        a32, b32 = np.float32(a), np.float32(b)
        assert rn32(Fr(float(a32)) / Fr(float(b32))) == float(a32 / b32)


@pytest.mark.parametrize("fmax", [448.0, 57344.0])
def test_corrected_product_is_the_correctly_rounded_quotient(fmax):
    c = float(np.float32(1.0 / fmax))
    cf, ff = Fr(c), Fr(fmax)
    amax = (np.arange(1, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    for a in amax.tolist():
        af = Fr(a)
        d0 = rn32(af * cf)
        r = rn32(af - Fr(d0) * ff)          # exact: a - d0 * Fmax is representable
        assert Fr(r) == af - Fr(d0) * ff
        d = rn32(Fr(r) * cf + Fr(d0))
        assert d == rn32(af / ff), a
