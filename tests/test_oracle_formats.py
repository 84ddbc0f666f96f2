"""Pins of the oracle's codecs against the format definitions, brute force and torch.

The NVFP4 element grid and the E4M3 scale type are checked against hand-derived
fixtures (tests/golden), exhaustive nearest-value searches written here
independently of the oracle, and torch's float8_e4m3fn / bfloat16 conversions
(library special cases).
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_pairs(name):
    out = []
    for line in open(os.path.join(GOLD, name)):
        line = line.split("#")[0].strip()
        if line:
            a, b = line.split()[:2]
            out.append((a, b))
    return out


# ------------------------------------------------------------------ E2M1
def test_e2m1_grid_is_the_nvfp4_grid():
    assert F.e2m1_decode(np.arange(8)).tolist() == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    neg = F.e2m1_decode(np.arange(8, 16))
    assert neg.tolist() == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    assert np.signbit(neg[0])


def test_e2m1_golden_ties():
    for v, c in _read_pairs("e2m1_ties.txt"):
        got = int(F.e2m1_encode(np.array([float(v)], np.float32))[0])
        assert got == int(c, 16), (v, c, got)


def _e2m1_brute(v: float) -> int:
    """Nearest magnitude by exhaustive search; ties to the even index; saturate."""
    m = Fraction(abs(v))
    grid = [Fraction(g).limit_denominator() for g in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    if m >= 6:
        idx = 7
    else:
        d = [abs(m - g) for g in grid]
        best = min(d)
        cands = [i for i, x in enumerate(d) if x == best]
        idx = cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]
    return idx | (8 if np.signbit(v) else 0)


def test_e2m1_encode_brute_force():
    rng = np.random.default_rng(0)
    vals = [np.float32(x) for x in np.arange(-8, 8.0001, 1 / 64)]
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]
    for m in mids:
        for s in (1, -1):
            c = np.float32(s * m)
            vals += [c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(-np.inf))]
    vals += list(rng.standard_normal(3000).astype(np.float32) * 3)
    vals += [np.float32(1e-40), np.float32(-1e-40), np.float32(3e38), np.float32(-0.0)]
    v = np.array(vals, np.float32)
    got = F.e2m1_encode(v)
    exp = np.array([_e2m1_brute(float(x)) if not np.signbit(x) or x != 0 else 8 for x in v])
    assert np.array_equal(got, exp)


def test_nibble_packing_order():
    c = np.array([[1, 2, 3, 4]], np.uint8)
    p = F.pack_nibbles(c)
    assert p.tolist() == [[0x21, 0x43]]          # even element in the low nibble
    assert np.array_equal(F.unpack_nibbles(p), c)


# ------------------------------------------------------------------ E4M3
def test_e4m3_golden_anchors():
    for c, v in _read_pairs("e4m3_anchors.txt"):
        got = F.e4m3_decode(np.array([int(c, 16)], np.uint8))[0]
        if v == "nan":
            assert np.isnan(got)
        else:
            assert got == float(v) and np.signbit(got) == v.startswith("-"), (c, v, got)


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_decode(codes)
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(t)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], t[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(t[~nan]))


def _e4m3_brute(v: float) -> int:
    table = [Fraction(float(x)) for x in F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))]
    fv = Fraction(v)
    if fv >= 448:
        return 0x7E
    d = [abs(fv - t) for t in table]
    best = min(d)
    cands = [i for i, x in enumerate(d) if x == best]
    return cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]


def test_e4m3_encode_brute_force_and_torch():
    rng = np.random.default_rng(1)
    table = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (table[:-1] + table[1:]) / 2                       # exact rounding midpoints
    vals = list(table) + list(mids)
    for m in mids:
        m32 = np.float32(m)
        vals += [np.nextafter(m32, np.float32(np.inf)), np.nextafter(m32, np.float32(0))]
    vals += list(np.exp2(rng.uniform(-14, 9.5, 4000)).astype(np.float32))
    vals += [0.0, 1e-30, 447.9, 448.0, 455.9, 464.0, 500.0, 1e9]
    v = np.array(vals, np.float32)
    got = F.e4m3_encode_nonneg(v)
    brute = np.array([_e4m3_brute(float(x)) for x in v], np.uint8)
    assert np.array_equal(got, brute)
    # torch rounds to nearest-even too; it returns NaN instead of saturating above 464
    ok = v < 464
    t = torch.from_numpy(v[ok]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got[ok], t)


# ------------------------------------------------------------------ bf16
def test_round_to_bf16_matches_torch_from_float32():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10,
                        np.exp2(rng.uniform(-130, 120, 5000)).astype(np.float32),
                        np.array([0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1e-39], np.float32)])
    ours = F.round_to_bf16(x)
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, t)


def _rn_bf16_fraction(v: Fraction) -> Fraction:
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 7)
    return (1 if v > 0 else -1) * round(a / ulp) * ulp


def test_round_to_bf16_from_float64_rounds_once():
    # float64 values just above a bf16 midpoint: rounding through float32 first
    # would land exactly on the midpoint and then go to even (down).
    base = np.array([1.0, 3.0, 1.5, 100.0, 2 ** -120])
    ulp = base * 2.0 ** -7
    x = base + ulp / 2 + base * 2.0 ** -40
    rng = np.random.default_rng(3)
    x = np.concatenate([x, -x, rng.standard_normal(2000) * 50])
    got = F.bf16_to_f32(F.round_to_bf16(x)).astype(np.float64)
    exp = np.array([float(_rn_bf16_fraction(Fraction(float(v)))) for v in x])
    assert np.array_equal(got, exp)
