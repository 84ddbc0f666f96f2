"""The chained MoE layer: NVFP4 forward and BF16 dgrad backward, plus the dense W4A4 QKV projection.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Order of the steps (each defined in its own module):
  forward  : permute + quantize (per-token scale, replicated to the token's k
             rows) -> grouped gate_up GEMM -> weighted SwiGLU + quantize ->
             grouped down GEMM -> un-permute + sum over slots
  backward : gather dY to routed rows -> BF16 grouped GEMM with W_d ->
             SwiGLU backward -> BF16 grouped GEMM with W_gu -> un-permute + sum
  QKV      : per-row quantize of x -> one-group NVFP4 GEMM
Forward NVFP4 with BF16 backward is the pairing the timed learner runs use
(blog page "miniTE NVFP4", §Respect the timing boundaries; §Two complementary
interventions: forward and backward precision are independent choices).
The backward treats every quantiser as the identity (straight-through) and
uses the bf16 master weights that were quantised for the forward.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .combine import permute_gather_ref, unpermute_combine_ref
from .formats import bf16_to_f32
from .gemm import bf16_grouped_gemm_ref, grouped_gemm_ref
from .permute import permute
from .quantize import quantize_rows_bf16
from .swiglu import row_weights, swiglu_backward_ref, swiglu_quantize_ref


@dataclass
class ForwardResult:
    offsets: np.ndarray
    row_to_tk: np.ndarray
    tk_to_row: np.ndarray
    a: tuple            # (codes, bscales, rscales) of the routed rows
    gu: np.ndarray      # float32 gate_up output
    a2: tuple           # NVFP4 of the weighted SwiGLU output
    h: np.ndarray       # float32 weighted SwiGLU output
    d: np.ndarray       # float32 down output
    y: np.ndarray       # bf16 bits [T, H]


def quantize_permute_ref(x_bits, ids, E: int):
    """Per-token quantisation, replicated into the token's k expert-grouped rows."""
    k = ids.shape[1]
    offsets, row_to_tk, tk_to_row, _ = permute(ids, E)
    codes, bsc, rsc = quantize_rows_bf16(x_bits)
    tok = row_to_tk.astype(np.int64) // k
    return (offsets, row_to_tk, tk_to_row), (codes[tok], bsc[tok], rsc[tok])


def moe_forward_ref(x_bits, ids, topk_w, w_gu_q, w_d_q, E: int) -> ForwardResult:
    """w_gu_q / w_d_q: (codes, bscales, rscales) of the NVFP4 expert weights."""
    k = ids.shape[1]
    (offsets, row_to_tk, tk_to_row), a = quantize_permute_ref(x_bits, ids, E)
    gu, _ = grouped_gemm_ref(*a, offsets, *w_gu_q)
    gu32 = gu.astype(np.float32)
    c2, b2, s2, h, _ = swiglu_quantize_ref(gu32, row_weights(topk_w, row_to_tk))
    d, _ = grouped_gemm_ref(c2, b2, s2, offsets, *w_d_q)
    d32 = d.astype(np.float32)
    y, _ = unpermute_combine_ref(d32, tk_to_row, k)
    return ForwardResult(offsets, row_to_tk, tk_to_row, a, gu32, (c2, b2, s2), h, d32, y)


def moe_dgrad_ref(dy_bits, fwd: ForwardResult, topk_w, w_gu_bits, w_d_bits, k: int):
    """Returns dict of float64/bf16 intermediates and dX (bf16 bits [T, H])."""
    dy_perm = permute_gather_ref(dy_bits, fwd.row_to_tk, k)
    w_d = bf16_to_f32(w_d_bits)            # [E, H, I]  (forward computes A W_d^T)
    w_gu = bf16_to_f32(w_gu_bits)          # [E, 2I, H]
    dH, _ = bf16_grouped_gemm_ref(bf16_to_f32(dy_perm), fwd.offsets, w_d, trans_w=False)
    dgu_bits, _ = swiglu_backward_ref(fwd.gu, dH.astype(np.float32), row_weights(topk_w, fwd.row_to_tk))
    dxp, _ = bf16_grouped_gemm_ref(bf16_to_f32(dgu_bits), fwd.offsets, w_gu, trans_w=False)
    dx, _ = unpermute_combine_ref(dxp.astype(np.float32), fwd.tk_to_row, k)
    return {"dy_perm": dy_perm, "dH": dH, "dgu": dgu_bits, "dx_perm": dxp, "dx": dx}


def qkv_ref(x_bits, w_qkv_q):
    a = quantize_rows_bf16(x_bits)
    T = a[0].shape[0]
    offsets = np.array([0, T], np.int32)
    w = tuple(np.asarray(t)[None] for t in w_qkv_q)
    c, _ = grouped_gemm_ref(*a, offsets, *w)
    return a, c
