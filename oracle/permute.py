"""Expert-major permutation of routed (token, slot) pairs.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The blog page "miniTE NVFP4" (yuxiaoba.github.io), §Two complementary
interventions, describes contiguous buffers with device-side metadata in place
of splitting and repacking per-expert tensors; §Follow the numerical execution
path says comparisons are made after aligning token and expert identities.
The permutation below gives every routed pair (t, slot) one row of a buffer
grouped by expert, and keeps both identity maps.

Definition (reading: the pages do not fix the order inside an expert):
  * flatten the routing list in (token, slot) order: i = t * k + slot;
  * counts[e] = number of i with ids[i] == e; offsets = exclusive prefix sum
    (length E + 1);
  * row(i) = offsets[ids[i]] + number of earlier i' < i with the same expert
    (a stable counting sort by expert id);
  * row_to_tk[row(i)] = i and tk_to_row[i] = row(i).
Entries whose expert id lies outside [0, E) take no row: tk_to_row = -1 and
they are left out of the counts.
"""
from __future__ import annotations

import numpy as np


def permute(ids, E: int):
    """ids int [T, k] -> (offsets int32 [E+1], row_to_tk int32 [R], tk_to_row int32 [T*k], bad int)."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    valid = (flat >= 0) & (flat < E)
    counts = np.zeros(E, dtype=np.int64)
    for e in flat[valid]:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    R = int(offsets[-1])
    fill = offsets[:-1].copy()
    tk_to_row = np.full(flat.size, -1, dtype=np.int64)
    row_to_tk = np.full(R, -1, dtype=np.int64)
    for i, e in enumerate(flat.tolist()):        # pure-Python walk in (token, slot) order
        if 0 <= e < E:
            r = fill[e]
            fill[e] += 1
            tk_to_row[i] = r
            row_to_tk[r] = i
    return (offsets.astype(np.int32), row_to_tk.astype(np.int32),
            tk_to_row.astype(np.int32), int((~valid).sum()))
