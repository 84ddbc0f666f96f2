"""Un-permutation with the top-k combine, and the gather used by the backward.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

After the down projection each token's k expert outputs sit in the rows the
permutation gave its (token, slot) pairs (identity maps as in
``oracle.permute``; the blog page "miniTE NVFP4", §Follow the numerical
execution path, stresses comparing through those identities).  The combine
sums them back per token.

Definition (reading: the pages give no formula): in float32, in slot order,
    acc = c_0 * D[row(t,0)];  acc = acc + c_s * D[row(t,s)]  for s = 1..k-1
with c_s = 1 when no combine weights are given (the router weight was already
applied in the weighted SwiGLU), each product and sum rounded separately (no
fused multiply-add), then y = bf16(acc) to nearest, ties to even.  Pairs with
no row (invalid expert id) contribute nothing.
"""
from __future__ import annotations

import numpy as np

from .formats import round_to_bf16


def unpermute_combine_ref(D, tk_to_row, k: int, topk_w=None):
    """D float32 [R, H]; tk_to_row [T*k].  Returns (y bf16 bits [T, H], acc float32 [T, H])."""
    D = np.asarray(D, np.float32)
    rows = np.asarray(tk_to_row, np.int64).reshape(-1, k)
    T, H = rows.shape[0], D.shape[1]
    w = None if topk_w is None else np.asarray(topk_w, np.float32).reshape(T, k)
    acc = np.zeros((T, H), np.float32)
    started = np.zeros((T, 1), bool)
    for s in range(k):
        r = rows[:, s]
        ok = (r >= 0)[:, None]
        term = D[np.maximum(r, 0)] if D.shape[0] else np.zeros((T, H), np.float32)
        if w is not None:
            term = (w[:, s:s + 1] * term).astype(np.float32)
        acc = np.where(ok, np.where(started, (acc + term).astype(np.float32), term), acc)
        started |= ok
    return round_to_bf16(acc), acc


def permute_gather_ref(x_bits, row_to_tk, k: int):
    """Row r of the result is token row_to_tk[r] // k of x (bf16 bits copied)."""
    return np.asarray(x_bits)[np.asarray(row_to_tk, np.int64) // k]
