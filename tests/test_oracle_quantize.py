"""Pins of the oracle's NVFP4 row quantiser.

* a hand-derived worked example (tests/golden/quantize_worked_example.txt);
* an independent re-derivation in exact rational arithmetic, with every FP32
  operation rounded explicitly and the codecs found by exhaustive search, on
  random rows and on rows searched so that plausible mistakes (reciprocal
  multiplication, a different order for 6*s, a different divisor) give a
  different answer;
* invariants: on-grid round trip, the block maximum maps to +-6, per-row
  (per-token) independence, zero rows and signed zeros.
"""
import os
from fractions import Fraction

import numpy as np

from oracle import formats as F
from oracle import quantize as Q
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load_worked_example():
    d = {}
    for line in open(os.path.join(GOLD, "quantize_worked_example.txt")):
        if line.startswith("#") or ":" not in line:
            continue
        key, val = line.split(":", 1)
        d[key.strip()] = val.split()
    x = np.array([float(v) for v in d["x"]], np.float32)
    codes = np.array([int(v, 16) for v in d["codes"]], np.uint8)
    bsc = np.array([int(v, 16) for v in d["bscales"]], np.uint8)
    return x, codes, bsc, np.float32(float(d["rscale"][0]))


def test_worked_example():
    x, codes, bsc, rs = _load_worked_example()
    assert np.array_equal(W.bf16_bits_to_f32(W.f32_to_bf16_bits(x)), x), "fixture must be bf16-exact"
    c, b, s = Q.quantize_rows_f32(x[None])
    assert c[0].tolist() == codes.tolist()
    assert b[0].tolist() == bsc.tolist()
    assert s[0] == rs
    # dequantised values equal the inputs wherever t was on the grid
    xd = Q.dequantize(c, b, s)[0]
    on_grid = [0, 1, 9, 10, 11, 12, 13, 14, 16, 24, 25, 26, 27, 28, 29, 30, 31]
    assert np.array_equal(xd[on_grid], x[on_grid].astype(np.float64))


# ---------------------------------------------------------------- exact re-derivation
def _rn32(v: Fraction) -> Fraction:
    """Round a rational to the nearest float32 (ties to even), subnormals included."""
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    return (1 if v > 0 else -1) * round(a / ulp) * ulp


_E4M3 = [Fraction(float(v)) for v in F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))]
_E2M1 = [Fraction(v).limit_denominator() for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]


def _nearest_even(table, v):
    d = [abs(v - t) for t in table]
    best = min(d)
    c = [i for i, x in enumerate(d) if x == best]
    return c[0] if len(c) == 1 else [i for i in c if i % 2 == 0][0]


def _quantize_row_exact(x, variant="spec"):
    """x: list of float (bf16-exact).  Returns (codes list, bscales list, rscale Fraction)."""
    xs = [Fraction(float(v)) for v in x]
    neg = [bool(np.signbit(v)) for v in x]
    a = max(abs(v) for v in xs)
    if variant == "div448":
        s = _rn32(a / 448)
    elif variant == "recip2688":
        s = _rn32(a * _rn32(Fraction(1, 2688)))
    else:
        s = _rn32(a / 2688)
    codes, bs = [], []
    for j in range(0, len(xs), 16):
        blk = xs[j:j + 16]
        aj = max(abs(v) for v in blk)
        if s == 0:
            b = 0
        else:
            if variant == "div6_then_s":
                v = _rn32(_rn32(aj / 6) / s)
            else:
                v = _rn32(aj / _rn32(6 * s))
            b = 0x7E if v >= 448 else _nearest_even(_E4M3, v)
        bs.append(b)
        d = _rn32(_E4M3[b] * s)
        for i, xv in enumerate(blk):
            if d == 0:
                idx = 0
            else:
                r = _rn32(xv * _rn32(1 / d)) if variant == "recip" else _rn32(xv / d)
                idx = 7 if abs(r) >= 6 else _nearest_even(_E2M1, abs(r))
            codes.append(idx | (8 if neg[j + i] else 0))
    return codes, bs, s


def _oracle_row(x):
    c, b, s = Q.quantize_rows_f32(np.array(x, np.float32)[None])
    return F.unpack_nibbles(c)[0].tolist(), b[0].tolist(), Fraction(float(s[0]))


def test_exact_rederivation_random_rows():
    rng = np.random.default_rng(11)
    for i in range(40):
        K = 32 if i % 2 else 48
        scale = float(np.exp2(rng.uniform(-40, 20)))
        x = rng.standard_normal(K) * scale
        if i % 5 == 0:
            x[rng.integers(0, K, 3)] *= 20
        x = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x.astype(np.float32)))
        assert _oracle_row(x) == _quantize_row_exact(x), i


def _discriminating_rows(variant, want=3, tries=3000, seed=0):
    """Search bf16 rows on which `variant` and the specification disagree.

    Block 0 holds the row maximum (its scale is 448); block 1 is steered onto
    E2M1 rounding midpoints relative to a random E4M3 block scale b.
    """
    rng = np.random.default_rng(seed)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    found = []
    for _ in range(tries):
        amax = float(np.exp2(rng.integers(-6, 6))) * float(rng.choice([1, 1.5, 1.25, 1.75]))
        s = amax / 2688.0
        b = float(F.e4m3_decode(np.array([rng.integers(0x30, 0x7E)], np.uint8))[0])
        x = np.zeros(32)
        x[:16] = rng.standard_normal(16) * amax / 4
        x[0] = amax
        x[16:] = rng.choice(mids, 16) * b * s * rng.choice([-1, 1], 16)
        x[16] = 6 * b * s
        x = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x.astype(np.float32)))
        if _quantize_row_exact(x, variant) != _quantize_row_exact(x):
            found.append(x)
            if len(found) >= want:
                break
    return found


def test_exact_rederivation_catches_plausible_mistakes():
    x, _, _, _ = _load_worked_example()
    assert _quantize_row_exact(x, "recip") != _quantize_row_exact(x)
    assert _oracle_row(x) == _quantize_row_exact(x)
    for seed, variant in enumerate(("recip", "div448", "div6_then_s", "recip2688")):
        rows = _discriminating_rows(variant, seed=seed)
        if variant in ("recip", "div448"):
            assert rows, f"search must find rows that tell {variant} apart"
        for x in rows:
            assert _oracle_row(x) == _quantize_row_exact(x), variant


# ---------------------------------------------------------------- invariants
def test_on_grid_round_trip():
    rng = np.random.default_rng(5)
    rows, K = 64, 64
    s = np.exp2(rng.integers(-20, 4, rows)).astype(np.float64)
    b = F.e4m3_decode(rng.integers(0x20, 0x7E, (rows, K // 16)).astype(np.uint8))
    b[:, 0] = 448.0                                     # the row max block has b = 448
    q = F.E2M1_GRID[rng.integers(0, 8, (rows, K))] * rng.choice([-1, 1], (rows, K))
    q[:, ::16] = 6.0                                    # every block reaches +-6
    x = q * np.repeat(b, 16, axis=1) * s[:, None]
    x32 = x.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), x)
    c, bb, ss = Q.quantize_rows_f32(x32)
    assert np.array_equal(ss.astype(np.float64), s)
    assert np.array_equal(F.e4m3_decode(bb), b)
    assert np.array_equal(Q.dequantize(c, bb, ss), x)


def test_block_max_maps_to_six_when_scale_is_normal():
    x = W.activations(256, 2048, config=2)
    c, b, s = Q.quantize_rows_bf16(x)
    xf = np.abs(W.bf16_bits_to_f32(x)).reshape(256, 128, 16)
    q = F.unpack_nibbles(c).reshape(256, 128, 16) & 7
    arg = xf.argmax(axis=2)
    qmax = np.take_along_axis(q, arg[..., None], axis=2)[..., 0]
    normal = F.e4m3_decode(b) >= 2.0 ** -6
    assert normal.mean() > 0.99
    assert np.all(qmax[normal] == 7)
    # the row-max block carries the largest scale
    rowmax_blk = xf.max(axis=2).argmax(axis=1)
    assert np.all(b[np.arange(256), rowmax_blk] == 0x7E)


def test_per_token_independence():
    x = W.activations(64, 512, config=2, tensor=7)
    c, b, s = Q.quantize_rows_bf16(x)
    for t in (0, 17, 63):
        c1, b1, s1 = Q.quantize_rows_bf16(x[t:t + 1])
        assert np.array_equal(c1[0], c[t]) and np.array_equal(b1[0], b[t]) and s1[0] == s[t]
    # a neighbour with a huge outlier does not change this row
    x2 = x.copy()
    x2[1] = W.f32_to_bf16_bits(np.full(512, 1e4, np.float32))
    c2, b2, s2 = Q.quantize_rows_bf16(x2)
    assert np.array_equal(c2[0], c[0]) and np.array_equal(b2[0], b[0])


def test_zero_rows_and_signed_zero():
    x = np.zeros((2, 32), np.float32)
    x[1, ::2] = -0.0
    c, b, s = Q.quantize_rows_f32(x)
    assert np.all(s == 0) and np.all(b == 0)
    q = F.unpack_nibbles(c)
    assert np.all(q[0] == 0)
    assert np.all(q[1, ::2] == 8) and np.all(q[1, 1::2] == 0)


def test_tiny_rows_subnormal_scales():
    # block 1 gets an E4M3-subnormal scale, block 2 a zero scale (codes keep the sign)
    x = np.zeros((1, 48), np.float32)
    x[0, 0] = 1e-30
    x[0, 16:32] = np.float32(1.1e-35)
    x[0, 32:] = np.float32(-1e-38)
    x = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x))
    assert _oracle_row(x[0]) == _quantize_row_exact(x[0])
    c, b, s = Q.quantize_rows_f32(x)
    assert b[0, 0] == 0x7E and 1 <= b[0, 1] < 0x08 and b[0, 2] == 0
    q = F.unpack_nibbles(c)[0]
    assert np.all(q[32:] == 8)
