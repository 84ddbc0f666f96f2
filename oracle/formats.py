"""Element and scale codecs of NVFP4, written from the format definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

NVFP4 (the 4-bit format the miniTE pages train in natively; news.hamidun.com,
§Paramètres clés) stores
  * elements as E2M1: sign bit (bit 3) and a 3-bit magnitude index into the
    grid {0, 0.5, 1, 1.5, 2, 3, 4, 6};
  * one scale per 16 consecutive elements as E4M3 "fn" (bias 7, no infinities,
    0x7F/0xFF are NaN, largest finite 448, subnormals M * 2^-9).
Rounding is to nearest with ties to even; values beyond the largest finite
value saturate to it (reading: the pages do not say; saturation is the usual
NVFP4 conversion and the only choice that keeps every code finite).

All functions work on numpy arrays and use float64 internally; every value the
codecs handle is exactly representable in float64, so no step here rounds
except the explicit ``np.rint`` (half to even).
"""
from __future__ import annotations

import numpy as np

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0
E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUBNORMAL_STEP = 2.0 ** -9


# ----------------------------------------------------------------------------- bf16
def bf16_to_f32(bits) -> np.ndarray:
    """bf16 storage (uint16 bits) to float32: bf16 is the top half of a float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x) -> np.ndarray:
    """Round float64/float32 values to the nearest bf16 (8 significant bits), ties to even.

    Returns uint16 bits.  Works from the value (exponent and a rint of the
    scaled significand), so a float64 input is rounded once, never through
    float32.  Finite inputs only; results beyond the bf16 range become inf.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)                      # a = m * 2**e, m in [0.5, 1)
    e = np.maximum(e, -125)                 # below 2**-126 the bf16 step is fixed: 2**-133
    step = np.ldexp(1.0, e - 8)             # 8 significant bits
    r = np.rint(a / step) * step
    r = np.where(a == 0, 0.0, r)
    out = np.copysign(r, x).astype(np.float32)   # exact: r has <= 8 significant bits
    return (out.view(np.uint32) >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------- E4M3
def e4m3_decode(codes) -> np.ndarray:
    """E4M3fn byte -> float64.  E>0: 2^(E-7)(1+M/8); E=0: M*2^-9; 0x7F/0xFF -> NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    M = c & 7
    mag = np.where(E == 0, M * E4M3_SUBNORMAL_STEP, np.ldexp(1.0 + M / 8.0, E - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


# ascending table of the 127 finite non-negative E4M3 values; index == code
_E4M3_POS = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode_nonneg(v) -> np.ndarray:
    """Non-negative finite value -> nearest E4M3fn code (ties to even mantissa), saturating at 448.

    Step of the grid: 2^(floor(log2 v) - 3) for normal values (3 mantissa bits),
    2^-9 below 2^-6.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or not np.all(np.isfinite(v)):
        raise ValueError("e4m3_encode_nonneg expects finite non-negative values")
    _, e = np.frexp(v)                                  # v = m 2^e, m in [0.5,1): floor(log2 v) = e-1
    step = np.where(v >= E4M3_MIN_NORMAL, np.ldexp(1.0, e - 1 - 3), E4M3_SUBNORMAL_STEP)
    r = np.rint(v / step) * step                        # v/step only rescales by a power of two
    r = np.minimum(r, E4M3_MAX)
    code = np.searchsorted(_E4M3_POS, r)
    assert np.array_equal(_E4M3_POS[code], r), "rounded value must lie on the E4M3 grid"
    return code.astype(np.uint8)


# ----------------------------------------------------------------------------- E2M1
def e2m1_decode(codes) -> np.ndarray:
    """4-bit E2M1 code (low nibble of the argument) -> float64; bit 3 is the sign."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    mag = E2M1_GRID[c & 7]
    return np.where(c & 8, -mag, mag)


def e2m1_encode(v) -> np.ndarray:
    """Value -> nearest E2M1 code, ties to the even magnitude index, |v| >= 6 -> 6.

    The grid spacing is 0.5 below 2, 1 in [2, 4) and 2 in [4, 6]; rounding to a
    multiple of the spacing with ties to even is the same as ties to the even
    grid index.  The sign bit copies the sign of v (so -0.1 and -0.0 give 0x8).
    """
    v = np.asarray(v, dtype=np.float64)
    m = np.abs(v)
    step = np.where(m < 2.0, 0.5, np.where(m < 4.0, 1.0, 2.0))
    r = np.minimum(np.rint(m / step) * step, E2M1_MAX)
    idx = np.searchsorted(E2M1_GRID, r)
    assert np.array_equal(E2M1_GRID[idx], r)
    return (idx | (np.signbit(v).astype(np.int64) << 3)).astype(np.uint8)


def pack_nibbles(codes) -> np.ndarray:
    """[..., K] 4-bit codes -> [..., K/2] bytes; element 2i in the low nibble of byte i."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_nibbles(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out
