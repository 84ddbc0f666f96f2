"""Float64 constants of the device SwiGLU helpers, checked against the
mathematics at 80 decimal digits: the 2^(j/64) table, the exp argument
reduction (64/ln2, and ln2/64 split in a 32-bit head and a tail) and the
Taylor coefficients.  The values are read from the header the kernels compile."""
import math
import os
import re
from decimal import Decimal, getcontext

import pytest

HEADER = os.path.join(os.path.dirname(__file__), "..", "precision_moe_gemm_amd", "csrc", "common.h")
getcontext().prec = 80
LN2 = Decimal(2).ln()


def _nearest(x: Decimal) -> float:
    """The double nearest to x (checked against both neighbours)."""
    f = float(x)
    for nb in (math.nextafter(f, -math.inf), math.nextafter(f, math.inf)):
        if abs(Decimal(nb) - x) < abs(Decimal(f) - x):
            f = nb
    return f


@pytest.fixture(scope="module")
def src():
    return open(HEADER).read()


def _sigmoid_body(src):
    start = src.index("double sigmoid_f64(")
    return src[start:src.index("\n}\n", start)]


def test_exp2_table_is_nearest(src):
    body = src[src.index("kExp2Frac64[64] = {"):]
    body = body[:body.index("};")]
    vals = [float.fromhex(h) for h in re.findall(r"0x[0-9a-f.]+p[+-]\d+", body)]
    assert len(vals) == 64
    for j, v in enumerate(vals):
        assert v == _nearest((Decimal(j) / 64 * LN2).exp()), j


def test_reduction_constants(src):
    lits = list(dict.fromkeys(float.fromhex(h) for h in re.findall(r"0x[0-9a-f.]+p[+-]?\d+", _sigmoid_body(src))))
    inv, shift, head, tail, c5, c4, c3 = lits[:7]   # in order of first use
    assert inv == _nearest(Decimal(64) / LN2)
    assert shift == 1.5 * 2.0 ** 52
    # head: at most 32 significant bits, so k * head is exact for |k| < 2^21
    m, _ = math.frexp(head)
    assert (m * 2 ** 32).is_integer()
    assert abs(tail) < head * 2.0 ** -31
    # |k| < 2^17 over the clamped range [-746, 710]; the reduction's error
    # k (head + tail - ln2/64), an absolute error in r and so a relative one in
    # exp(r), stays far below a float64 ulp
    assert 746 * inv < 2 ** 17
    assert abs(Decimal(head) + Decimal(tail) - LN2 / 64) * 2 ** 17 < Decimal(2) ** -60
    assert (c5, c4, c3) == (_nearest(Decimal(1) / 120), _nearest(Decimal(1) / 24), _nearest(Decimal(1) / 6))


def test_polynomial_truncation_bound():
    """|r| <= ln2/128 after the reduction: the degree-5 Taylor remainder of exp(r)
    is below 2^-54 relative (the claim in the helper's comment)."""
    r = LN2 / 128
    rem = r ** 6 / 720 * r.exp()
    assert rem < Decimal(2) ** -54
