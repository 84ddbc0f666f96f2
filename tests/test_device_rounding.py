"""The float64 -> bf16 rounding of the SwiGLU backward kernel, replayed on the
CPU: its steps (clamp the binade, add and subtract C = 2^(e+45) in float64,
narrow to float32, take the top 16 bits with d's sign) in numpy, which rounds
float64 additions the same way, against the oracle's round_to_bf16 on every
bf16 rounding midpoint and its float64 neighbours, the subnormal range, the
overflow edge, zeros and random doubles.  The clamp bounds and the binade
offset are read from the header the kernels compile."""
import os
import re

import numpy as np
import pytest

from oracle import formats as of

HEADER = os.path.join(os.path.dirname(__file__), "..", "precision_moe_gemm_amd", "csrc", "common.h")


@pytest.fixture(scope="module")
def consts():
    src = open(HEADER).read()
    body = src[src.index("uint32_t f64_to_bf16_rne(double d)"):]
    body = body[:body.index("\n}\n")]
    lo, hi = map(int, re.search(r"max\(\(hi >> 20\) & 0x7FFu, (\d+)u\), (\d+)u\)", body).groups())
    off = int(re.search(r"\(be \+ (\d+)u\) << 20", body).group(1))
    return lo, hi, off


def device_rne(d: np.ndarray, lo: int, hi: int, off: int) -> np.ndarray:
    d = np.asarray(d, np.float64)
    bits = d.view(np.uint64)
    top = (bits >> np.uint64(32)).astype(np.uint32)
    be = np.clip((top >> np.uint32(20)) & np.uint32(0x7FF), lo, hi).astype(np.uint64)
    C = (((be + np.uint64(off)) << np.uint64(20)) << np.uint64(32)).view(np.float64)
    with np.errstate(over="ignore"):
        r = (np.abs(d) + C) - C
        f = r.astype(np.float32)
    return ((f.view(np.uint32) | (top & np.uint32(0x80000000))) >> np.uint32(16)).astype(np.uint16)


def _check(d, consts):
    got = device_rne(d, *consts)
    with np.errstate(over="ignore"):
        ref = of.round_to_bf16(d)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, [(float(d[i]).hex(), int(got[i]), int(ref[i])) for i in bad[:5]]


def test_constants_cover_the_bf16_range(consts):
    lo, hi, off = consts
    # the lowest binade is the bf16 subnormal step's: C = 2^(lo - 1023 + off) has ulp 2^-133
    assert lo - 1023 + off - 52 == -133
    # C stays finite: its biased exponent is at most 2046
    assert hi + off == 2046


def test_every_midpoint_and_its_neighbours(consts):
    b = np.arange(0, 0x7F80, dtype=np.uint32)                  # every finite non-negative bf16 value
    lo_v = (b << 16).view(np.float32).astype(np.float64)
    hi_v = ((b + 1) << 16).view(np.float32).astype(np.float64)  # the next one (0x7F80: inf above the top)
    mid = np.where(np.isinf(hi_v), lo_v + (lo_v - ((b - 1) << 16).view(np.float32).astype(np.float64)) / 2,
                   (lo_v + hi_v) / 2)
    d = np.concatenate([mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf), lo_v])
    _check(np.concatenate([d, -d]), consts)


def test_subnormal_overflow_zero_and_random(consts):
    rng = np.random.default_rng(7)
    sub = np.ldexp(rng.random(1 << 20), rng.integers(-150, -120, 1 << 20))
    big = np.ldexp(1.0 + rng.random(1 << 18), rng.integers(126, 1024, 1 << 18))
    anyd = rng.integers(0, 1 << 63, 1 << 21, dtype=np.uint64).view(np.float64)
    anyd = anyd[np.isfinite(anyd)]
    edge = np.array([0.0, 2.0 ** -133, 2.0 ** -134, 1.5 * 2.0 ** -134, 2.0 ** -135, 2.0 ** -126,
                     float.fromhex("0x1.fefp127"), float.fromhex("0x1.ffp127"), np.finfo(np.float64).max,
                     np.finfo(np.float64).tiny, 5e-324])
    d = np.concatenate([sub, big, anyd, edge])
    _check(np.concatenate([d, -d]), consts)
    assert device_rne(np.array([-0.0]), *consts)[0] == 0x8000
