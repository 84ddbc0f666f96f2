"""GPU parity: weighted SwiGLU + quantise, combine, gather, SwiGLU backward, BF16 grouped GEMM.

SwiGLU forward/backward: the GPU evaluates in float64 like the oracle, with
its own exp (table and polynomial) and a refined reciprocal, multiplying where
the oracle divides, so its float64 values may differ from the oracle's by a
few ulps.  That can
change a float32 (bf16) rounding only when the oracle's float64 value lies
within a few float64 ulps of a rounding midpoint.  Those elements (found by
the oracle alone) are listed; every other element must match bit for bit.
The NVFP4 bytes of every row must equal the oracle's quantiser applied to the
GPU's own h (so rows holding such an element are checked too), and those of
rows without one must also equal the oracle's from its own h.
Combine and gather: bit-exact.  BF16 GEMM: 2e-5 * sum |a w|.
"""
import numpy as np
import pytest
import torch

import precision_moe_gemm_amd as pmg
import workloads as W
from oracle import combine as oc, formats as of, gemm as og, permute as op, quantize as oq, swiglu as osw
from helpers import (assert_within, bf16_dev, bf16_host, bf16_midpoint_adjacent as _bf16_midpoint_adjacent,
                     dev, host, gpu_ready, sample_rows)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs a GPU")]


def _routing(T, E, k, kind, seed):
    ids, w = W.make_routing(kind, T, E, k, seed)
    off, r2t, t2r, _ = op.permute(ids, E)
    return ids, w, off, r2t, t2r


def _gu(R, I, seed, scale=2.0):
    return (W.rng(seed, 30).standard_normal((R, 2 * I)) * scale).astype(np.float32)


@pytest.mark.parametrize("T,E,k,I,weighted", [(4096, 128, 8, 768, True), (100, 8, 2, 768, False),
                                               (50, 4, 2, 48, True), (64, 2, 1, 4096, True),
                                               # rows of one chunk without the split tail (several
                                               # rows per wavefront), of two chunks without it
                                               # (lanes past the row end; a whole last chunk)
                                               (2048, 16, 4, 384, True), (300, 8, 4, 1008, False),
                                               (512, 8, 2, 1024, True),
                                               (64, 4, 2, 8192, True)])   # the longest row
def test_swiglu_quantize(T, E, k, I, weighted):
    print(f"[swiglu_quantize] T={T} E={E} k={k} I={I} weighted={weighted}", flush=True)
    ids, tw, off, r2t, t2r = _routing(T, E, k, "uniform", 50)
    R = T * k
    gu = _gu(R, I, 51)
    codes, bsc, rsc, h = pmg.swiglu_quantize(dev(gu), dev(off), dev(tw.reshape(-1)) if weighted else None,
                                             dev(r2t) if weighted else None, h_out=True)
    torch.cuda.synchronize()
    w_rows = osw.row_weights(tw, r2t) if weighted else None
    rc, rb, rs, rh, amb = osw.swiglu_quantize_ref(gu, w_rows)
    gh = host(h)
    same = gh.view(np.uint32) == rh.view(np.uint32)
    assert np.all(same | amb), f"h differs off the midpoints at {np.argwhere(~(same | amb))[:5].tolist()}"
    # every row: the GPU's bytes are the oracle's quantiser of the GPU's own h
    oc_, ob_, os_ = oq.quantize_rows_f32(gh)
    R_ = int(off[-1])
    assert np.array_equal(host(codes)[:R_], oc_[:R_])
    assert np.array_equal(host(bsc)[:R_], ob_[:R_])
    assert np.array_equal(host(rsc)[:R_].view(np.uint32), os_[:R_].view(np.uint32))
    clean = ~amb.any(axis=1)
    print(f"  midpoint-adjacent elements: {int(amb.sum())} in {int((~clean).sum())} rows")
    assert np.array_equal(host(codes)[clean], rc[clean])
    assert np.array_equal(host(bsc)[clean], rb[clean])
    assert np.array_equal(host(rsc)[clean].view(np.uint32), rs[clean].view(np.uint32))


def test_swiglu_quantize_skips_rows_past_offsets():
    """Rows at or beyond expert_offsets[E] are not written (poisoned buffers stay poisoned)."""
    off = np.array([0, 1, 2, 2], np.int32)                      # 2 routed rows, capacity 4
    gu = _gu(4, 64, 52)
    codes = torch.full((4, 32), 0xAB, dtype=torch.uint8, device="cuda:0")
    bsc = torch.full((4, 4), 0xCD, dtype=torch.uint8, device="cuda:0")
    rsc = torch.full((4,), -7.0, dtype=torch.float32, device="cuda:0")
    pmg.swiglu_quantize(dev(gu), dev(off), out={"codes": codes, "bscales": bsc, "rscales": rsc})
    torch.cuda.synchronize()
    assert np.all(host(codes)[2:] == 0xAB) and np.all(host(bsc)[2:] == 0xCD) and np.all(host(rsc)[2:] == -7.0)
    rc, rb, rs, _, _ = osw.swiglu_quantize_ref(gu[:2])
    assert np.array_equal(host(codes)[:2], rc)


@pytest.mark.parametrize("T,E,k,H,weighted,bad", [(4096, 128, 8, 2048, False, False),
                                                   (64, 8, 7, 2048, True, True),    # slot pairs, odd k
                                                   (300, 32, 5, 1024, True, True),  # groups of 4 slots
                                                   (100, 16, 3, 4096, True, False), # one slot at a time
                                                   (37, 16, 4, 264, True, False),   # other H: column loop
                                                   (20, 8, 3, 64, True, True),
                                                   (64, 64, 32, 2048, True, True),  # top-32, the most slots
                                                   (16, 64, 32, 8200, True, False)])  # long rows, column loop
def test_unpermute_combine(T, E, k, H, weighted, bad):
    print(f"[combine] T={T} k={k} H={H} weighted={weighted} invalid={bad}", flush=True)
    ids, tw, _, _, _ = _routing(T, E, k, "uniform", 60)
    if bad:
        ids[2, 1] = E
        ids[5, 0] = -1
    off, r2t, t2r, _ = op.permute(ids, E)
    R = int(off[-1])
    d = (W.rng(60, 31).standard_normal((T * k, H)) * 3).astype(np.float32)
    y = pmg.unpermute_combine(dev(d), dev(t2r), k, dev(tw.reshape(-1)) if weighted else None)
    torch.cuda.synchronize()
    ry, _ = oc.unpermute_combine_ref(d, t2r, k, tw if weighted else None)
    assert np.array_equal(bf16_host(y), ry)


@pytest.mark.parametrize("T,E,k,H,kind", [(4096, 128, 8, 2048, "softmax"),
                                          (64, 64, 32, 264, "zipf"),      # top-32, short odd-width rows
                                          (50, 16, 3, 8192, "uniform")])  # the longest rows
def test_permute_gather(T, E, k, H, kind):
    print(f"[gather] T={T} E={E} k={k} H={H}", flush=True)
    ids, tw, off, r2t, t2r = _routing(T, E, k, kind, 61)
    x = W.gaussian_bf16((T, H), 1.0, 61, 32)
    out = pmg.permute_gather_bf16(bf16_dev(x), dev(off), dev(r2t), k)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_host(out), oc.permute_gather_ref(x, r2t, k))


@pytest.mark.parametrize("T,E,k,I,weighted", [(4096, 128, 8, 768, True), (40, 4, 2, 24, False),
                                               (64, 4, 2, 8192, True)])   # the longest row
def test_swiglu_backward(T, E, k, I, weighted):
    print(f"[swiglu_backward] T={T} I={I}", flush=True)
    ids, tw, off, r2t, t2r = _routing(T, E, k, "uniform", 62)
    R = T * k
    gu = _gu(R, I, 62)
    dh = (W.rng(62, 33).standard_normal((R, I)) * 0.1).astype(np.float32)
    dgu = pmg.swiglu_backward(dev(gu), dev(dh), dev(off), dev(tw.reshape(-1)) if weighted else None,
                              dev(r2t) if weighted else None)
    torch.cuda.synchronize()
    w_rows = osw.row_weights(tw, r2t) if weighted else None
    ref_bits, d64 = osw.swiglu_backward_ref(gu, dh, w_rows)
    got = bf16_host(dgu)
    amb = _bf16_midpoint_adjacent(d64)
    diff = got != ref_bits
    assert not np.any(diff & ~amb), f"{int((diff & ~amb).sum())} bf16 values differ"


# g values at the edges of the float64 exp: zeros, tiny values, both sides of
# exp(-g) overflowing (g near -709.78) and of it underflowing to 0 (g near
# 745.13), far beyond both, and the float32 extremes
_G_SPECIAL = np.array([0.0, -0.0, 1e-30, -1e-30, 0.5, -0.5, 20.0, -20.0, 40.0, -40.0, 87.5, -87.5,
                       88.75, -88.75, 103.9, -103.9, 500.0, -500.0, 709.75, -709.75, 709.7826, -709.7826,
                       709.7828, -709.7828, 710.0, -710.0, 745.0, -745.0, 745.2, -745.2, 746.0, -746.0,
                       800.0, -800.0, 1e10, -1e10, 3e38, -3e38], np.float32)


def _gu_special(R, I, seed):
    """Rows whose first gate values are _G_SPECIAL (rotated per row), the rest
    Gaussian; up values of several magnitudes, capped so |g u| stays finite."""
    gu = _gu(R, I, seed)
    n = len(_G_SPECIAL)
    for r in range(R):
        gu[r, :n] = np.roll(_G_SPECIAL, r)
    u_mag = np.array([1.0, -1.0, 1e-20, 1e-39, 0.0, -0.0, 1e20, 3.0], np.float32)
    gu[:, I:I + n] = u_mag[np.arange(R) % len(u_mag)][:, None]
    big = np.abs(gu[:, :I].astype(np.float64) * gu[:, I:].astype(np.float64)) > 1e37
    gu[:, I:][big] = np.float32(0.25)
    return gu


def test_swiglu_quantize_special_values():
    """h at the edges of exp's range (see _G_SPECIAL), bit for bit off float32 midpoints."""
    R, I = 16, 512
    gu = _gu_special(R, I, 64)
    off = np.array([0, 7, R], np.int32)
    w_rows = np.linspace(0.05, 1.0, R).astype(np.float32)
    r2t = np.arange(R, dtype=np.int32)
    codes, bsc, rsc, h = pmg.swiglu_quantize(dev(gu), dev(off), dev(w_rows), dev(r2t), h_out=True)
    torch.cuda.synchronize()
    rc, rb, rs, rh, amb = osw.swiglu_quantize_ref(gu, w_rows)
    gh = host(h)
    assert np.all(np.isfinite(rh))
    same = gh.view(np.uint32) == rh.view(np.uint32)
    assert np.all(same | amb), f"h differs at {np.argwhere(~(same | amb))[:5].tolist()}"
    oc_, ob_, os_ = oq.quantize_rows_f32(gh)
    assert np.array_equal(host(codes), oc_) and np.array_equal(host(bsc), ob_)
    assert np.array_equal(host(rsc).view(np.uint32), os_.view(np.uint32))


def test_swiglu_backward_special_values():
    """dG and dU at the edges of exp's range, and output gradients whose results
    round into bf16 subnormals or past the bf16 range, bit for bit off bf16
    midpoints (NaN where the oracle has NaN, from g = +-inf)."""
    R, I = 16, 512
    gu = _gu_special(R, I, 65)
    gu[0, 100], gu[1, 101] = np.inf, -np.inf
    dh = (W.rng(65, 33).standard_normal((R, I)) * 0.1).astype(np.float32)
    dh[:, 40:48] = np.array([1e-40, -1e-40, 3e-39, 1e-38, 1e38, -1e38, 3e38, 1e-45], np.float32)
    off = np.array([0, 5, R], np.int32)
    w_rows = np.linspace(0.05, 1.0, R).astype(np.float32)
    r2t = np.arange(R, dtype=np.int32)
    dgu = pmg.swiglu_backward(dev(gu), dev(dh), dev(off), dev(w_rows), dev(r2t))
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore", over="ignore"):
        ref_bits, d64 = osw.swiglu_backward_ref(gu, dh, w_rows)
        amb = _bf16_midpoint_adjacent(d64)
    got = bf16_host(dgu)
    nan_ref = np.isnan(d64)
    assert nan_ref.any()
    nan_got = (got & 0x7F80) == 0x7F80
    nan_got &= (got & 0x7F) != 0
    assert np.array_equal(nan_got, nan_ref)
    sub = (np.abs(d64) < 2.0 ** -126) & (d64 != 0)
    assert sub.any() and (np.abs(d64[~nan_ref]) >= 2.0 ** 128).any()
    diff = (got != ref_bits) & ~nan_ref
    assert not np.any(diff & ~amb), f"{int((diff & ~amb).sum())} bf16 values differ"


def _g_sweep(I):
    """Every 257th float32 bit pattern that is finite, both signs: ~16.7M gate
    values over the whole float32 range, in rows of 2I (up values 1)."""
    bits = np.arange(0, 1 << 32, 257, dtype=np.uint64).astype(np.uint32)
    g = bits.view(np.float32)
    g = g[np.isfinite(g)]
    R = -(-g.size // I)
    gu = np.ones((R, 2 * I), np.float32)
    gu[:, :I].reshape(-1)[:g.size] = g
    gu[:, :I].reshape(-1)[g.size:] = 0.0
    return gu


def test_swiglu_quantize_gate_sweep():
    """The float64 SwiGLU over the whole float32 range of g (its own exp and
    reciprocal against numpy's exp and division): h bit for bit off float32
    midpoints, and every row's bytes equal the oracle's quantiser of the GPU's h."""
    I = 4096
    gu = _g_sweep(I)
    R = gu.shape[0]
    off = np.array([0, R], np.int32)
    codes, bsc, rsc, h = pmg.swiglu_quantize(dev(gu), dev(off), h_out=True)
    torch.cuda.synchronize()
    with np.errstate(over="ignore"):
        h64 = osw.swiglu_h64(gu)
    rh = h64.astype(np.float32)
    amb = osw.rn32_ambiguous(h64)
    gh = host(h)
    same = gh.view(np.uint32) == rh.view(np.uint32)
    print(f"  {R * I} gate values, midpoint-adjacent: {int(amb.sum())}")
    assert np.all(same | amb), f"h differs at {np.argwhere(~(same | amb))[:5].tolist()}"
    oc_, ob_, os_ = oq.quantize_rows_f32(gh)
    assert np.array_equal(host(codes), oc_) and np.array_equal(host(bsc), ob_)
    assert np.array_equal(host(rsc).view(np.uint32), os_.view(np.uint32))


def test_swiglu_backward_gate_sweep():
    """dG and dU over the whole float32 range of g (dh = 1): bit for bit off bf16 midpoints."""
    I = 4096
    gu = _g_sweep(I)
    R = gu.shape[0]
    off = np.array([0, R], np.int32)
    dh = np.ones((R, I), np.float32)
    dgu = pmg.swiglu_backward(dev(gu), dev(dh), dev(off))
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore", over="ignore"):
        ref_bits, d64 = osw.swiglu_backward_ref(gu, dh)
        amb = _bf16_midpoint_adjacent(d64)
    got = bf16_host(dgu)
    nan_ref = np.isnan(d64)
    print(f"  {R * I} gate values, midpoint-adjacent: {int(amb.sum())}, NaN: {int(nan_ref.sum())}")
    diff = (got != ref_bits) & ~nan_ref
    assert not np.any(diff & ~amb), f"{int((diff & ~amb).sum())} bf16 values differ"


@pytest.mark.parametrize("layout", [pmg.W_KN, pmg.W_NK])
@pytest.mark.parametrize("T,E,k,K,N,kind", [(256, 8, 4, 256, 192, "uniform"),
                                             (40, 16, 2, 96, 64, "zipf"),
                                             (64, 4, 2, 32, 64, "uniform"),   # K = 32: one K-step
                                             (256, 1024, 8, 64, 48, "zipf")])  # the most experts
def test_bf16_grouped_gemm_small(layout, T, E, k, K, N, kind):
    print(f"[bf16 gemm] layout={layout} T={T} E={E} K={K} N={N}", flush=True)
    ids, tw, off, r2t, t2r = _routing(T, E, k, kind, 63)
    R = T * k
    a = W.gaussian_bf16((R, K), 1.0, 63, 34)
    w = W.gaussian_bf16((E, K, N), 0.02, 63, 35)
    wl = w if layout == pmg.W_KN else np.ascontiguousarray(w.transpose(0, 2, 1))
    c = host(pmg.bf16_grouped_gemm(bf16_dev(a), dev(off), bf16_dev(wl), layout))
    ref, bound = og.bf16_grouped_gemm_ref(of.bf16_to_f32(a), off, of.bf16_to_f32(w), trans_w=False)
    Rv = int(off[-1])
    print("  err/bound", assert_within(c[:Rv], ref, bound, "bf16 gemm"))


@pytest.mark.parametrize("kind", ["softmax", "zipf"])
@pytest.mark.parametrize("K,N", [(2048, 768), (1536, 2048)])
def test_bf16_dgrad_shapes_sampled(K, N, kind):
    """The two dgrad GEMMs: dY_perm [32768x2048] W_d[e] [2048x768]; dGU [32768x1536] W_gu[e] [1536x2048].

    The kernel picks its tile height from the routing: near-uniform routing
    gives one tile per expert and weight slab, Zipf routing (experts of up to
    thousands of rows) shorter tiles and many per expert."""
    print(f"[bf16 gemm] dgrad K={K} N={N} routing={kind}", flush=True)
    T, E, k = 4096, 128, 8
    ids, tw, off, r2t, t2r = _routing(T, E, k, kind, 64)
    a = W.gaussian_bf16((T * k, K), 1.0, 64, 36)
    w = W.gaussian_bf16((E, K, N), 0.02, 64, 37)
    c = host(pmg.bf16_grouped_gemm(bf16_dev(a), dev(off), bf16_dev(w), pmg.W_KN))
    rows, _ = sample_rows(off, [0, 64, 127], extra=5, seed=4)
    ref, bound = og.bf16_grouped_gemm_ref(of.bf16_to_f32(a), off, of.bf16_to_f32(w), trans_w=False, rows=rows)
    print("  err/bound", assert_within(c[rows], ref, bound, "dgrad"))


@pytest.mark.parametrize("T,E,k,K,N,kind", [(4096, 128, 8, 2048, 768, "softmax"),
                                             (40, 16, 2, 96, 64, "zipf"),
                                             (64, 64, 32, 128, 96, "uniform")])   # top-32: row r / 32
def test_bf16_grouped_gemm_gather(T, E, k, K, N, kind):
    """The gathered-operand GEMM equals the GEMM of the gathered rows bit for bit, and the oracle."""
    print(f"[bf16 gemm gather] T={T} E={E} k={k} K={K} N={N} {kind}", flush=True)
    ids, tw, off, r2t, t2r = _routing(T, E, k, kind, 65)
    x = W.gaussian_bf16((T, K), 1.0, 65, 38)
    w = W.gaussian_bf16((E, K, N), 0.02, 65, 39)
    xd, wd, offd, r2td = bf16_dev(x), bf16_dev(w), dev(off), dev(r2t)
    c = host(pmg.bf16_grouped_gemm_gather(xd, r2td, k, offd, wd))
    c2 = host(pmg.bf16_grouped_gemm(pmg.permute_gather_bf16(xd, offd, r2td, k), offd, wd))
    Rv = int(off[-1])
    assert np.array_equal(c[:Rv].view(np.uint32), c2[:Rv].view(np.uint32))
    a_perm = of.bf16_to_f32(x)[r2t[:Rv] // k]
    if T * k > 1000:
        rows, _ = sample_rows(off, [0, E - 1], extra=3, seed=5)
    else:
        rows = np.arange(Rv)
    ref, bound = og.bf16_grouped_gemm_ref(a_perm, off, of.bf16_to_f32(w), trans_w=False, rows=rows)
    print("  err/bound", assert_within(c[rows], ref, bound, "gather gemm"))


@pytest.mark.parametrize("N", [16, 272])
def test_bf16_grouped_gemm_narrow_and_ragged_columns(N):
    """N = 16 (one 16-column group) and N = 272 (a ragged last 256-column tile)."""
    print(f"[bf16 gemm] N={N}", flush=True)
    T, E, k, K = 300, 8, 2, 64
    ids, tw, off, r2t, t2r = _routing(T, E, k, "zipf", 66)
    a = W.gaussian_bf16((T * k, K), 1.0, 66, 40)
    w = W.gaussian_bf16((E, K, N), 0.02, 66, 41)
    c = host(pmg.bf16_grouped_gemm(bf16_dev(a), dev(off), bf16_dev(w), pmg.W_KN))
    ref, bound = og.bf16_grouped_gemm_ref(of.bf16_to_f32(a), off, of.bf16_to_f32(w), trans_w=False)
    Rv = int(off[-1])
    print("  err/bound", assert_within(c[:Rv], ref, bound, "bf16 gemm"))


def test_bf16_grouped_gemm_gather_clamps_bad_map_entries():
    """Map entries outside [0, T k) read a row clamped into [0, T): a wrong row, never outside a."""
    print("[bf16 gemm gather] bad map entries", flush=True)
    T, E, k, K, N = 64, 4, 2, 64, 48
    ids, tw, off, r2t, t2r = _routing(T, E, k, "uniform", 67)
    bad = r2t.copy()
    bad[3], bad[10], bad[20] = 10 ** 9, -5, T * k + 7
    x = W.gaussian_bf16((T, K), 1.0, 67, 42)
    w = W.gaussian_bf16((E, K, N), 0.02, 67, 43)
    c = host(pmg.bf16_grouped_gemm_gather(bf16_dev(x), dev(bad), k, dev(off), bf16_dev(w)))
    Rv = int(off[-1])
    tok = np.minimum(np.maximum(bad[:Rv].astype(np.int64), 0) // k, T - 1)
    ref, bound = og.bf16_grouped_gemm_ref(of.bf16_to_f32(x)[tok], off, of.bf16_to_f32(w), trans_w=False)
    print("  err/bound", assert_within(c[:Rv], ref, bound, "gather gemm (clamped)"))
