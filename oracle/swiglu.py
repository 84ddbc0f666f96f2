"""Weighted SwiGLU with NVFP4 quantisation of its output, and the SwiGLU backward.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The blog page "miniTE NVFP4" (yuxiaoba.github.io), §Two complementary
interventions, says the amax needed for quantisation is taken during the
weighted SwiGLU rather than by another scan; the result feeds the down
projection in NVFP4.  Backward precision is an independent choice (same
section); the forward runs NVFP4 and the backward here is BF16 (the timed
learner paths of §Respect the timing boundaries use BF16 backward).

Forward, per routed row r with router weight w (reading: the pages give no
formula; gate = columns [0, I) and up = columns [I, 2I) of the gate_up output,
the router weight is applied here and only here):
    e   = exp(-g)              float64
    h64 = ((g / (1 + e)) * u) * w     each operation in float64
    h   = float32(h64)         one rounding to nearest
then ``quantize_rows_f32(h)``.  The GPU computes the same float64 sequence;
its ``exp`` may differ from numpy's in the last float64 bit, which can flip
the float32 rounding only when h64 lies within a few float64 ulps of a float32
rounding midpoint.  ``rn32_ambiguous`` marks those elements so the tests can
leave their rows out of the bit-exact comparison.

Backward of h = w * silu(g) * u with respect to g and u, given dH:
    sig = 1 / (1 + exp(-g)),  silu = g / (1 + exp(-g))
    t   = dH * w
    du  = t * silu
    dg  = (t * u) * (sig * (1 + g * (1 - sig)))
in float64, each rounded once to bf16 (the operand type of the BF16 dgrad
GEMM that follows).
"""
from __future__ import annotations

import numpy as np

from .formats import round_to_bf16
from .quantize import quantize_rows_f32


def row_weights(topk_w, row_to_tk):
    """Router weight of each routed row: topk_w flattened in (token, slot) order, gathered by row_to_tk."""
    return np.asarray(topk_w, np.float32).reshape(-1)[np.asarray(row_to_tk, np.int64)]


def swiglu_h64(gu, w_rows=None) -> np.ndarray:
    gu = np.asarray(gu, np.float32)
    I = gu.shape[1] // 2
    g = gu[:, :I].astype(np.float64)
    u = gu[:, I:].astype(np.float64)
    with np.errstate(over="ignore"):
        e = np.exp(-g)
    h = (g / (1.0 + e)) * u
    if w_rows is not None:
        h = h * np.asarray(w_rows, np.float64)[:, None]
    return h


def swiglu_quantize_ref(gu, w_rows=None):
    """Returns (codes, bscales, rscales, h float32, ambiguous-element mask)."""
    h64 = swiglu_h64(gu, w_rows)
    h = h64.astype(np.float32)
    codes, bsc, rsc = quantize_rows_f32(h)
    return codes, bsc, rsc, h, rn32_ambiguous(h64)


def rn32_ambiguous(x64, rel_margin: float = 2.0 ** -45) -> np.ndarray:
    """True where float64 x lies within rel_margin*|x| of a float32 rounding midpoint."""
    x64 = np.asarray(x64, np.float64)
    x32 = x64.astype(np.float32)
    up = np.nextafter(x32, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(x32, np.float32(-np.inf)).astype(np.float64)
    c = x32.astype(np.float64)
    dist = np.minimum(np.abs(x64 - (c + up) / 2), np.abs(x64 - (c + dn) / 2))
    return dist <= rel_margin * np.maximum(np.abs(x64), 2.0 ** -126)


def swiglu_backward_ref(gu, dH, w_rows=None):
    """Returns (dGU bf16 bits [R, 2I], dGU float64 before rounding)."""
    gu = np.asarray(gu, np.float32)
    I = gu.shape[1] // 2
    g = gu[:, :I].astype(np.float64)
    u = gu[:, I:].astype(np.float64)
    t = np.asarray(dH, np.float64)
    if w_rows is not None:
        t = t * np.asarray(w_rows, np.float64)[:, None]
    with np.errstate(over="ignore"):
        den = 1.0 + np.exp(-g)
    sig = 1.0 / den
    silu = g / den
    du = t * silu
    dg = (t * u) * (sig * (1.0 + g * (1.0 - sig)))
    d64 = np.concatenate([dg, du], axis=1)
    return round_to_bf16(d64), d64
