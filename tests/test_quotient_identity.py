"""The quantiser's division-free quotient, checked on the CPU.

The HIP quantiser divides once per 16-element block: y = fl(1/d), q = fl(x*y),
e = fl(x - q*d) (exact, one FMA), r = fl(q + e*y) (one FMA), and relies on r
being the correctly rounded quotient fl(x/d) (Markstein's theorem) for normal
values.  Here every step is emulated exactly in float64 (each product or sum
below fits in 53 bits, except the last sum, which is redone in rational
arithmetic when its float64 value sits on a float32 rounding boundary) and r
is compared with fl(x/d) for bf16-valued x and quotients placed around every
E2M1 rounding tie.
"""
from fractions import Fraction

import numpy as np

F32, F64 = np.float32, np.float64


def _rn32(fr):
    c = np.float32(float(fr))
    cands = [np.nextafter(c, F32(-np.inf)), c, np.nextafter(c, F32(np.inf))]
    return min(cands, key=lambda t: (abs(Fraction(float(t)) - fr), int(np.array(t).view(np.uint32)) & 1))


def test_three_operation_quotient_is_correctly_rounded():
    rng = np.random.default_rng(2024)
    n = 1_000_000
    x = (rng.standard_normal(n) * np.exp2(rng.integers(-60, 60, n))).astype(F32)
    x = (x.view(np.uint32) & 0xFFFF0000).view(F32)                     # bf16 values
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 1.0, 0.1], F64)
    m = rng.choice(ties, n) * (1 + rng.integers(-64, 64, n) * 2.0 ** -24)
    d = (np.abs(x).astype(F64) / m).astype(F32)
    ok = np.isfinite(d) & (d > 2.0 ** -100) & (d < 2.0 ** 100) & (np.abs(x) > 2.0 ** -80)
    x, d = x[ok], d[ok]
    ref = (x.astype(F64) / d.astype(F64)).astype(F32)
    y = (1.0 / d.astype(F64)).astype(F32)
    q = (x.astype(F64) * y.astype(F64)).astype(F32)
    e = (x.astype(F64) - q.astype(F64) * d.astype(F64)).astype(F32)
    s = q.astype(F64) + e.astype(F64) * y.astype(F64)
    r = s.astype(F32)
    up, dn = np.nextafter(r, F32(np.inf)), np.nextafter(r, F32(-np.inf))
    edge = (s == (r.astype(F64) + up.astype(F64)) / 2) | (s == (r.astype(F64) + dn.astype(F64)) / 2)
    for i in np.nonzero(edge)[0]:
        r[i] = _rn32(Fraction(float(q[i])) + Fraction(float(e[i])) * Fraction(float(y[i])))
    assert len(x) > 900_000
    assert np.array_equal(r.view(np.uint32), ref.view(np.uint32))
