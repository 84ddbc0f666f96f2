"""NVFP4 weight gradient of the expert GEMMs, quantised along tokens.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The blog page "miniTE NVFP4" (yuxiaoba.github.io), §Two complementary
interventions, keeps the backward's precision a free choice, independent of
the forward's, and notes that a lower-bit backward is not automatically
faster.  The weight gradient of an expert GEMM C = A W^T contracts over the
tokens routed to that expert:
    dW_e[n][c] = sum over rows r of expert e of  G[r][n] * X[r][c]
(G the gradient of the GEMM's output, X its input).  In NVFP4 both operands
are quantised along that contraction, i.e. along tokens.

Reading (the pages give no recipe): for each expert e the operands are the
transposed slabs G_e^T [N][K_e] and X_e^T [C][K_e], where K_e is the number of
the expert's rows rounded up to a multiple of 64 (at least 64), the extra
columns zero; each row of a slab (one output channel of one expert) is
quantised on its own by ``quantize.quantize_rows_f32`` - an FP32 scale per
(expert, channel), an E4M3 scale per 16 consecutive tokens, E2M1 codes.  Then
dW_e = dequant(G_e^T) dequant(X_e^T)^T exactly in float64 (``gemm``).
"""
from __future__ import annotations

import numpy as np

from .gemm import grouped_gemm_ref
from .quantize import quantize_rows_f32


def token_blocks(offsets) -> np.ndarray:
    """kofs [E+1]: the first 64-token step of each expert's padded slab."""
    counts = np.diff(np.asarray(offsets, np.int64))
    steps = np.maximum(1, (counts + 63) // 64)
    return np.concatenate([[0], np.cumsum(steps)]).astype(np.int32)


def expert_slab(rows_f32, offsets, e: int, kofs) -> np.ndarray:
    """X_e^T [C][K_e] float32: the expert's rows transposed, zero-padded to K_e."""
    o0, o1 = int(offsets[e]), int(offsets[e + 1])
    K_e = 64 * int(kofs[e + 1] - kofs[e])
    xs = np.zeros((rows_f32.shape[1], K_e), np.float32)
    xs[:, : o1 - o0] = np.asarray(rows_f32[o0:o1], np.float32).T
    return xs


def quantize_expert_ref(rows_f32, offsets, e: int, kofs):
    """The NVFP4 of X_e^T quantised along tokens: (codes [C][K_e/2], bscales [C][K_e/16], rscales [C])."""
    return quantize_rows_f32(expert_slab(rows_f32, offsets, e, kofs))


def quantize_tokens_ref(rows_f32, offsets):
    """Per expert, the NVFP4 of X_e^T quantised along tokens: a list of
    ``quantize_expert_ref`` results, and kofs."""
    kofs = token_blocks(offsets)
    E = len(offsets) - 1
    return [quantize_expert_ref(rows_f32, offsets, e, kofs) for e in range(E)], kofs


def wgrad_ref(g_q, x_q):
    """dW_e = dequant(G_e^T) dequant(X_e^T)^T per expert, float64.

    g_q / x_q: per-expert lists from ``quantize_tokens_ref``.
    Returns (dW [E][N][C], bound [E][N][C]) with the 2e-5 * sum |a w| bound."""
    out, bnd = [], []
    for (gc, gb, gs), (xc, xb, xs) in zip(g_q, x_q):
        n = gc.shape[0]
        c, b = grouped_gemm_ref(gc, gb, gs, np.array([0, n]), xc[None], xb[None], xs[None])
        out.append(c)
        bnd.append(b)
    return np.stack(out), np.stack(bnd)
