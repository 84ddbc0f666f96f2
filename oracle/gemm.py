"""Grouped NVFP4 GEMM by exact dequantisation, and a dense bf16 GEMM, both in FP64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The grouped expert GEMMs are the kernels the pages single out for MoE
(news.hamidun.com, §Diagnostic, alignement et noyaux rapides; W4A4 GEMM in
zicq.com, §Technical Mechanism Analysis).  Rows of the expert-grouped buffer
[offsets[e], offsets[e+1]) are multiplied by expert e's weight W[e] (stored
[N][K], C = A W^T).

Plain definition used here: C[r, n] = sum_k xA[r, k] * xW[e, n, k] with
x = e2m1(q) * e4m3(b) * s.  It is evaluated as
    P = (q_A b_A) @ (q_W b_W)^T     (float64 matmul)
    C = P * s_A[r] * s_W[n]         (float64)
Each q*b has at most 6 significant bits, so each product has at most 12; for
the value ranges of these workloads every partial sum of P is exact in
float64, whatever order the matmul uses.  The tolerance bound of an element is
``2e-5 * sum_k |xA xW|``, also returned.
"""
from __future__ import annotations

import numpy as np

from .quantize import dequantize_qb

GEMM_REL_TOL = 2e-5


def grouped_gemm_ref(a_codes, a_bscales, a_rscales, offsets,
                     w_codes, w_bscales, w_rscales, rows=None):
    """Returns (C float64 [R or len(rows), N], bound float64 same shape).

    a_* are the expert-grouped NVFP4 rows [R, K/2], [R, K/16], [R];
    w_* are [E, N, K/2], [E, N, K/16], [E, N]; offsets [E+1].
    ``rows`` (optional, sorted int array) restricts the output to those rows.
    """
    offsets = np.asarray(offsets, np.int64)
    E = offsets.size - 1
    N = w_codes.shape[1]
    R = int(offsets[-1])
    rows = np.arange(R) if rows is None else np.asarray(rows, np.int64)
    C = np.zeros((rows.size, N), np.float64)
    B = np.zeros((rows.size, N), np.float64)
    expert_of = np.searchsorted(offsets, rows, side="right") - 1
    for e in range(E):
        sel = np.nonzero(expert_of == e)[0]
        if sel.size == 0:
            continue
        r = rows[sel]
        xa = dequantize_qb(a_codes[r], a_bscales[r])
        xw = dequantize_qb(w_codes[e], w_bscales[e])
        sa = np.asarray(a_rscales, np.float64)[r][:, None]
        sw = np.asarray(w_rscales[e], np.float64)[None, :]
        C[sel] = (xa @ xw.T) * sa * sw
        B[sel] = (np.abs(xa) @ np.abs(xw).T) * np.abs(sa) * np.abs(sw)
    return C, GEMM_REL_TOL * B


def bf16_grouped_gemm_ref(a, offsets, w, trans_w: bool, rows=None):
    """bf16 operands given as float arrays.  a [R, K]; w [E, K, N] (trans_w False) or [E, N, K] (True).

    C[r] = a[r] @ w[e]  (or a[r] @ w[e]^T), float64.  Returns (C, 2e-5 * sum|a w|).
    """
    offsets = np.asarray(offsets, np.int64)
    E = offsets.size - 1
    R = int(offsets[-1])
    rows = np.arange(R) if rows is None else np.asarray(rows, np.int64)
    N = w.shape[1] if trans_w else w.shape[2]
    C = np.zeros((rows.size, N), np.float64)
    B = np.zeros((rows.size, N), np.float64)
    expert_of = np.searchsorted(offsets, rows, side="right") - 1
    for e in range(E):
        sel = np.nonzero(expert_of == e)[0]
        if sel.size == 0:
            continue
        xa = np.asarray(a[rows[sel]], np.float64)
        we = np.asarray(w[e], np.float64)
        if trans_w:
            we = we.T
        C[sel] = xa @ we
        B[sel] = np.abs(xa) @ np.abs(we)
    return C, GEMM_REL_TOL * B
