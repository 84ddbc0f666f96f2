"""Pins of the oracle's weight gradient quantised along tokens (oracle/wgrad.py).

* token_blocks against a brute-force count;
* quantisation along tokens of columns built on the NVFP4 grid (a power-of-two
  row scale, block scales 448 * 2^-m, a +-6 in every non-empty block): the
  codes, block scales and row scales decode back to every value exactly,
  including partial blocks, the zero padding and empty experts;
* the weight gradient of such data equals, exactly, the float64 product of the
  raw rows over each expert's range (so a transposed operand, a shifted
  expert range or a wrong padding would fail);
* an expert's bytes do not depend on the other experts' rows.
"""
import numpy as np

from oracle import quantize as oq, wgrad as ow


def _on_grid_columns(rng, counts, C):
    """Rows [sum(counts)][C] float32 whose columns, per expert, lie on the NVFP4 grid."""
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    R = int(sum(counts))
    x = np.zeros((R, C), np.float64)
    o = 0
    for n in counts:
        for c in range(C):
            s = 2.0 ** int(rng.integers(-8, 1))
            nblk = -(-n // 16)
            for j in range(nblk):
                lo, hi = o + 16 * j, min(o + 16 * j + 16, o + n)
                b = 448.0 if j == 0 else 448.0 * 2.0 ** -int(rng.integers(0, 6))
                q = rng.choice(grid, hi - lo) * rng.choice([-1.0, 1.0], hi - lo)
                q[int(rng.integers(0, hi - lo))] = 6.0 * rng.choice([-1.0, 1.0])   # the block's maximum
                x[lo:hi, c] = q * b * s
        o += n
    return x.astype(np.float32)


def test_token_blocks_brute_force():
    counts = [0, 1, 63, 64, 65, 200, 0]
    off = np.concatenate([[0], np.cumsum(counts)])
    kofs = ow.token_blocks(off)
    want = [0]
    for n in counts:
        want.append(want[-1] + max(1, -(-n // 64)))
    assert kofs.tolist() == want


def test_quantize_along_tokens_recovers_on_grid_columns():
    rng = np.random.default_rng(0)
    counts = [0, 1, 17, 64, 70]
    C = 24
    x = _on_grid_columns(rng, counts, C)
    off = np.concatenate([[0], np.cumsum(counts)])
    q, kofs = ow.quantize_tokens_ref(x, off)
    for e, (codes, bsc, rsc) in enumerate(q):
        K_e = 64 * int(kofs[e + 1] - kofs[e])
        assert codes.shape == (C, K_e // 2) and bsc.shape == (C, K_e // 16) and rsc.shape == (C,)
        back = oq.dequantize(codes, bsc, rsc)                  # [C][K_e] float64
        want = np.zeros((C, K_e))
        want[:, : counts[e]] = x[off[e]:off[e + 1]].T
        assert np.array_equal(back, want), f"expert {e}"
        assert np.all(bsc[:, -(-counts[e] // 16):] == 0)      # blocks of padding only
        if counts[e] == 0:
            assert np.all(rsc == 0) and np.all(codes == 0)


def test_wgrad_exact_on_grid_data():
    rng = np.random.default_rng(1)
    counts = [5, 0, 33, 64, 81]
    N, C = 12, 20
    g = _on_grid_columns(rng, counts, N)
    x = _on_grid_columns(rng, counts, C)
    off = np.concatenate([[0], np.cumsum(counts)])
    gq, _ = ow.quantize_tokens_ref(g, off)
    xq, _ = ow.quantize_tokens_ref(x, off)
    dw, bound = ow.wgrad_ref(gq, xq)
    assert dw.shape == (len(counts), N, C)
    for e in range(len(counts)):
        ge = g[off[e]:off[e + 1]].astype(np.float64)
        xe = x[off[e]:off[e + 1]].astype(np.float64)
        assert np.array_equal(dw[e], ge.T @ xe), f"expert {e}"
        assert np.all(bound[e] >= 0)


def test_experts_are_independent():
    rng = np.random.default_rng(2)
    counts = [40, 30, 50]
    off = np.concatenate([[0], np.cumsum(counts)])
    x = rng.standard_normal((120, 16)).astype(np.float32)
    q1, _ = ow.quantize_tokens_ref(x, off)
    y = x.copy()
    y[off[1]:off[2]] *= 7.0                                    # change expert 1 only
    q2, _ = ow.quantize_tokens_ref(y, off)
    for e in (0, 2):
        assert all(np.array_equal(a, b) for a, b in zip(q1[e], q2[e]))
    assert not np.array_equal(q1[1][2], q2[1][2])
