"""NVFP4 quantisation of rows with a per-row FP32 second-level scale.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Per-token scaling: the blog page "miniTE NVFP4" (yuxiaoba.github.io),
§Follow the numerical execution path, explains that a tensor-wide activation
maximum lets a token's scale depend on its neighbours and that per-token
scaling removes that dependency.  So every row (a token, or a weight output
row) is quantised on its own:

  1. a   = max_i |x_i|                                  (exact)
  2. s   = a / 2688            FP32 division;  2688 = 6 * 448, so the row's
                               largest block gets the largest E4M3 scale and its
                               largest element the largest E2M1 value
  3. per block j of 16 elements: a_j = max |x_i|;
        b_j = 0 if s == 0, else E4M3( a_j / (6 * s) )   (6*s and / in FP32)
  4. d_j = float(b_j) * s      FP32 multiplication
  5. q_i = E2M1( x_i / d_j )   FP32 division; if d_j == 0, q_i is a zero of
                               x_i's sign
  6. codes packed two per byte (even element in the low nibble),
     block scales as E4M3 bytes, row scale as float32.

Readings (the pages give none of these): the factor 2688 and the order of the
FP32 operations above (a correctly rounded division, no fused multiply-add);
rows whose maximum is zero get s = 0 and all-zero scales.  Every operation is
an IEEE float32 operation with round-to-nearest-even, done here by numpy on
float32 arrays, so the result is fully determined.
"""
from __future__ import annotations

import numpy as np

from .formats import (bf16_to_f32, e2m1_decode, e2m1_encode, e4m3_decode,
                      e4m3_encode_nonneg, pack_nibbles, unpack_nibbles)

BLOCK = 16
SECOND_LEVEL_DIVISOR = np.float32(6.0 * 448.0)   # 2688


def quantize_rows_f32(x) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Quantise float32 rows [rows, K] (K % 16 == 0).

    Returns (codes uint8 [rows, K/2], bscales uint8 [rows, K/16], rscales float32 [rows]).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, K = x.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 16")
    ax = np.abs(x)
    a = ax.max(axis=1) if K else np.zeros(rows, np.float32)                 # step 1
    s = (a / SECOND_LEVEL_DIVISOR).astype(np.float32)                        # step 2
    a_blk = ax.reshape(rows, K // BLOCK, BLOCK).max(axis=2)                  # step 3
    six_s = (np.float32(6.0) * s).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (a_blk / six_s[:, None]).astype(np.float32)
    v = np.where(s[:, None] == 0, np.float32(0), v)
    b = e4m3_encode_nonneg(v)
    d = (e4m3_decode(b).astype(np.float32) * s[:, None]).astype(np.float32)   # step 4
    d_el = np.repeat(d, BLOCK, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (x / d_el).astype(np.float32)                                # step 5
    ratio = np.where(d_el == 0, x * np.float32(0), ratio)                    # signed zero
    q = e2m1_encode(ratio)
    return pack_nibbles(q), b, s                                             # step 6


def quantize_rows_bf16(bits):
    """Quantise bf16 rows given as uint16 bits [rows, K]."""
    return quantize_rows_f32(bf16_to_f32(bits))


def dequantize_qb(codes, bscales) -> np.ndarray:
    """Element value without the row scale: e2m1(q) * e4m3(b), exact in float64. [rows, K]."""
    q = e2m1_decode(unpack_nibbles(codes))
    b = e4m3_decode(bscales)
    return q * np.repeat(b, BLOCK, axis=-1)


def dequantize(codes, bscales, rscales) -> np.ndarray:
    """Full dequantisation q * b * s in float64 (exact: at most 6 + 24 significant bits)."""
    return dequantize_qb(codes, bscales) * np.asarray(rscales, np.float64)[..., None]
