"""Pins of the oracle's permutation and GEMMs.

Permutation: brute force from the definition on tiny cases, numpy's stable
argsort (a library special case), inverse maps, counts, invalid ids.
GEMM: exact rational brute force on tiny shapes, single expert == dense,
the exactness claim on workload-like data, and the bf16 GEMM in both layouts.
"""
from fractions import Fraction
import itertools

import numpy as np

from oracle import formats as F, gemm as G, permute as P, quantize as Q
import workloads as W


# ---------------------------------------------------------------- permutation
def _brute_rows(ids, E):
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    rows = []
    for i, e in enumerate(flat):
        if not 0 <= e < E:
            rows.append(-1)
            continue
        before = sum(1 for e2 in flat if 0 <= e2 < E and e2 < e)
        same_earlier = sum(1 for e2 in flat[:i] if e2 == e)
        rows.append(before + same_earlier)
    return rows


def test_permute_brute_force_tiny():
    rng = np.random.default_rng(0)
    for T, E, k in [(5, 4, 2), (1, 1, 1), (3, 8, 3), (7, 3, 2), (6, 5, 5)]:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        off, r2t, t2r, bad = P.permute(ids, E)
        assert bad == 0
        assert t2r.tolist() == _brute_rows(ids, E)
        assert np.array_equal(r2t[t2r], np.arange(T * k))
        assert np.array_equal(np.diff(off), np.bincount(ids.reshape(-1), minlength=E))


def test_permute_equals_stable_argsort():
    ids, _ = W.make_routing("softmax", 4096, 128, 8, 2)
    off, r2t, t2r, _ = P.permute(ids, 128)
    assert np.array_equal(r2t, np.argsort(ids.reshape(-1), kind="stable"))
    assert off[-1] == 4096 * 8


def test_permute_invalid_ids_take_no_row():
    ids = np.array([[0, 5], [-1, 1], [1, 0]], np.int32)
    off, r2t, t2r, bad = P.permute(ids, 2)
    assert bad == 2
    assert t2r.tolist() == [0, -1, -1, 2, 3, 1]
    assert off.tolist() == [0, 2, 4]
    assert r2t.tolist() == [0, 5, 3, 4]


def test_permute_empty_experts():
    ids = np.array([[3, 0]] * 4, np.int32)
    off, _, t2r, _ = P.permute(ids, 6)
    assert off.tolist() == [0, 4, 4, 4, 8, 8, 8]


# ---------------------------------------------------------------- NVFP4 GEMM
def _nvfp4(rows, K, seed, scale=1.0):
    x = W.f32_to_bf16_bits((np.random.default_rng(seed).standard_normal((rows, K)) * scale).astype(np.float32))
    return Q.quantize_rows_bf16(x)


def _exact_value(codes, bsc, rs, r, k):
    q = Fraction(float(F.e2m1_decode(F.unpack_nibbles(codes[r:r + 1])[0, k])))
    b = Fraction(float(F.e4m3_decode(bsc[r, k // 16])))
    return q * b * Fraction(float(rs[r]))


def test_grouped_gemm_rational_brute_force():
    K, N = 32, 3
    a = _nvfp4(7, K, 1)
    w = [_nvfp4(N, K, 10 + e, 0.02) for e in range(3)]
    wc = np.stack([t[0] for t in w]); wb = np.stack([t[1] for t in w]); ws = np.stack([t[2] for t in w])
    offsets = np.array([0, 3, 3, 7], np.int32)            # expert 1 empty
    C, B = G.grouped_gemm_ref(*a, offsets, wc, wb, ws)
    for r, n in itertools.product(range(7), range(N)):
        e = 0 if r < 3 else 2
        exact = sum(_exact_value(*a, r, kk) * _exact_value(wc[e], wb[e], ws[e], n, kk) for kk in range(K))
        absum = sum(abs(_exact_value(*a, r, kk) * _exact_value(wc[e], wb[e], ws[e], n, kk)) for kk in range(K))
        assert abs(Fraction(C[r, n]) - exact) <= abs(exact) * Fraction(2) ** -52
        assert abs(Fraction(B[r, n]) - Fraction(2e-5) * absum) <= absum * Fraction(2) ** -40


def test_grouped_gemm_single_expert_is_dense_and_rows_subset():
    a = _nvfp4(64, 256, 2)
    w = _nvfp4(128, 256, 3, 0.02)
    C, B = G.grouped_gemm_ref(*a, np.array([0, 64]), *(t[None] for t in w))
    dense = Q.dequantize(*a) @ Q.dequantize(*w).T
    assert np.all(np.abs(C - dense) <= 1e-12 * B / G.GEMM_REL_TOL)
    Cs, _ = G.grouped_gemm_ref(*a, np.array([0, 64]), *(t[None] for t in w), rows=np.array([5, 63]))
    assert np.array_equal(Cs, C[[5, 63]])


def test_qb_products_sum_exactly_on_workload_data():
    """The FP64 matmul of q*b values equals the exact rational sum (no rounding anywhere)."""
    x = W.activations(4, 2048, config=2)
    a = Q.quantize_rows_bf16(x)
    w = _nvfp4(3, 2048, 5, 0.02)
    xa = Q.dequantize_qb(a[0], a[1])
    xw = Q.dequantize_qb(w[0], w[1])
    P64 = xa @ xw.T
    for r in range(4):
        for n in range(3):
            exact = sum(Fraction(float(p)) * Fraction(float(q)) for p, q in zip(xa[r], xw[n]))
            assert Fraction(P64[r, n]) == exact


def test_bf16_grouped_gemm_layouts():
    rng = np.random.default_rng(4)
    a = W.bf16_bits_to_f32(W.f32_to_bf16_bits(rng.standard_normal((6, 16)).astype(np.float32)))
    w = W.bf16_bits_to_f32(W.f32_to_bf16_bits(rng.standard_normal((2, 16, 5)).astype(np.float32)))
    off = np.array([0, 2, 6])
    C, B = G.bf16_grouped_gemm_ref(a, off, w, trans_w=False)
    Ct, _ = G.bf16_grouped_gemm_ref(a, off, np.ascontiguousarray(w.transpose(0, 2, 1)), trans_w=True)
    assert np.array_equal(C, Ct)
    for r in range(6):
        e = 0 if r < 2 else 1
        for n in range(5):
            exact = sum(Fraction(float(a[r, kk])) * Fraction(float(w[e, kk, n])) for kk in range(16))
            assert abs(Fraction(C[r, n]) - exact) <= abs(exact) * Fraction(2) ** -50 + Fraction(2) ** -60
