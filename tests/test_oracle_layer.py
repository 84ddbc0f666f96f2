"""Pins of the oracle's chained layer (oracle/layer.py) against references that
do not use its row maps or its GEMM routine.

* quantize_permute_ref: every (token, slot) entry's row is found by brute
  force (experts with a smaller id, then earlier entries of the same expert),
  and that row must hold the quantisation of the token's row on its own;
* moe_forward_ref: each token is rebuilt by explicit loops over its slots -
  exact rational products for both GEMMs, the weighted SwiGLU written out with
  the slot's router weight, the per-row quantiser, and the combine in slot
  order - and every intermediate row is compared with the oracle's;
* moe_dgrad_ref: torch float64 autograd through the dequantised forward, with
  every quantiser straight-through (the SwiGLU evaluated at the forward's
  gate_up values, the GEMMs on the bf16 master weights);
* qkv_ref: exact rational dense product.

Plausible wiring mistakes - a token index taken as row_to_tk % k, the router
weight applied twice or not at all, a weight used untransposed, slots summed in
another order - change at least one compared value by far more than the
tolerances used.  The pages fix the chain only in words (blog "miniTE NVFP4",
sections "Follow the numerical execution path" and "Two complementary
interventions"); these tests pin the oracle's composition of its own, already
pinned, primitives.
"""
from fractions import Fraction

import numpy as np
import torch

from oracle import formats as F, layer as L, quantize as Q
import workloads as W

SHAPE = W.LayerShape(T=8, H=64, E=4, k=2, I=48, qkv_n=24)   # 2I = 96 != H, so a transpose mistake shows


def _brute_row(ids, E, t, s):
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    i = t * ids.shape[1] + s
    e = flat[i]
    return sum(1 for v in flat if v < e) + sum(1 for v in flat[:i] if v == e)


def _exact_rows(codes, bsc, rsc):
    """Exact rational value of every element of NVFP4 rows: list of lists of Fraction."""
    q = F.e2m1_decode(F.unpack_nibbles(codes))
    b = F.e4m3_decode(bsc)
    out = []
    for r in range(codes.shape[0]):
        s = Fraction(float(rsc[r]))
        out.append([Fraction(float(q[r, j])) * Fraction(float(b[r, j // 16])) * s for j in range(q.shape[1])])
    return out


def _dot(xs, ys):
    return sum((a * b for a, b in zip(xs, ys)), Fraction(0))


def _setup(seed_cfg=5):
    S = SHAPE
    x = W.activations(S.T, S.H, config=seed_cfg)
    ids, tw = W.make_routing("softmax", S.T, S.E, S.k, seed_cfg)
    wgu, wd = W.moe_weights_bf16(S, seed_cfg)
    wgu_q = tuple(t.reshape((S.E, 2 * S.I) + t.shape[1:]) for t in Q.quantize_rows_bf16(wgu.reshape(-1, S.H)))
    wd_q = tuple(t.reshape((S.E, S.H) + t.shape[1:]) for t in Q.quantize_rows_bf16(wd.reshape(-1, S.I)))
    return x, ids, tw, wgu, wd, wgu_q, wd_q


def _close_f32(got, exact, what):
    """got (float32) must be the exact value within one float32 ulp (the oracle rounds
    the exact sum a few times: by the two row scales in float64, then to float32)."""
    for j, (g, ex) in enumerate(zip(got, exact)):
        err = abs(Fraction(float(g)) - ex)
        assert err <= abs(ex) * Fraction(2) ** -23 + Fraction(2) ** -149, f"{what}[{j}]: {float(g)} vs {float(ex)}"


def test_quantize_permute_ref_rows_by_brute_force():
    S = W.LayerShape(T=12, H=32, E=5, k=3)
    x = W.activations(S.T, S.H, config=7)
    ids, _ = W.make_routing("uniform", S.T, S.E, S.k, 7)
    (off, r2t, t2r), (codes, bsc, rsc) = L.quantize_permute_ref(x, ids, S.E)
    assert np.array_equal(np.diff(off), np.bincount(ids.reshape(-1), minlength=S.E))
    for t in range(S.T):
        own = Q.quantize_rows_bf16(x[t:t + 1])     # the token quantised on its own
        for s in range(S.k):
            r = _brute_row(ids, S.E, t, s)
            assert t2r[t * S.k + s] == r and r2t[r] == t * S.k + s
            assert np.array_equal(codes[r], own[0][0]) and np.array_equal(bsc[r], own[1][0])
            assert rsc[r] == own[2][0]
    # the k rows of a token hold the same bytes, and different tokens differ
    assert not np.array_equal(codes[t2r[0]], codes[t2r[S.k]])


def test_moe_forward_ref_by_token_slot_loops():
    S = SHAPE
    x, ids, tw, _, _, wgu_q, wd_q = _setup()
    fwd = L.moe_forward_ref(x, ids, tw, wgu_q, wd_q, S.E)
    wgu_ex = [_exact_rows(*(t[e] for t in wgu_q)) for e in range(S.E)]
    wd_ex = [_exact_rows(*(t[e] for t in wd_q)) for e in range(S.E)]
    for t in range(S.T):
        a_ex = _exact_rows(*Q.quantize_rows_bf16(x[t:t + 1]))[0]
        acc = None
        for s in range(S.k):
            e, r = int(ids[t, s]), _brute_row(ids, S.E, t, s)
            assert fwd.tk_to_row[t * S.k + s] == r
            # gate_up: row of the token times expert e's weight rows (W stored [2I][H], C = A W^T)
            _close_f32(fwd.gu[r], [_dot(a_ex, wgu_ex[e][n]) for n in range(2 * S.I)], f"gu t{t} s{s}")
            # weighted SwiGLU with this slot's router weight, once
            g = fwd.gu[r, :S.I].astype(np.float64)
            u = fwd.gu[r, S.I:].astype(np.float64)
            h = (((g / (1.0 + np.exp(-g))) * u) * np.float64(tw[t, s])).astype(np.float32)
            assert np.array_equal(h, fwd.h[r]), f"h t{t} s{s}"
            q2 = Q.quantize_rows_f32(h[None])
            for got, want in zip(fwd.a2, q2):
                assert np.array_equal(got[r], want[0])
            # down: W_d stored [H][I]
            h_ex = _exact_rows(*q2)[0]
            _close_f32(fwd.d[r], [_dot(h_ex, wd_ex[e][n]) for n in range(S.H)], f"d t{t} s{s}")
            # combine: float32, slot order, no weights (applied in the SwiGLU)
            acc = fwd.d[r].copy() if acc is None else (acc + fwd.d[r]).astype(np.float32)
        assert np.array_equal(fwd.y[t], F.round_to_bf16(acc)), f"y t{t}"


def test_moe_dgrad_ref_against_autograd():
    S = SHAPE
    x, ids, tw, wgu, wd, wgu_q, wd_q = _setup(6)
    fwd = L.moe_forward_ref(x, ids, tw, wgu_q, wd_q, S.E)
    dy = W.grad_output_bf16(S, 6)
    bwd = L.moe_dgrad_ref(dy, fwd, tw, wgu, wd, S.k)
    f64 = lambda a: torch.tensor(np.asarray(a, np.float64))
    Wgu = f64(W.bf16_bits_to_f32(wgu))          # [E, 2I, H]
    Wd = f64(W.bf16_bits_to_f32(wd))            # [E, H, I]
    xt = f64(W.bf16_bits_to_f32(x)).requires_grad_(True)
    dyt = f64(W.bf16_bits_to_f32(dy))
    loss = torch.zeros((), dtype=torch.float64)
    dgu_abs = torch.zeros(S.T, S.H, dtype=torch.float64)      # sum_s |dgu_ts| |W_gu[e]|, for the bound
    for t in range(S.T):
        for s in range(S.k):
            e, r = int(ids[t, s]), _brute_row(ids, S.E, t, s)
            gu_lin = xt[t] @ Wgu[e].T                                 # straight-through quantisers:
            gu = gu_lin + (f64(fwd.gu[r]) - gu_lin).detach()          # the forward's values, identity gradient
            g, u = gu[:S.I], gu[S.I:]
            h = torch.nn.functional.silu(g) * u * float(tw[t, s])
            loss = loss + (dyt[t] * (h @ Wd[e].T)).sum()
            dgu_abs[t] += torch.tensor(np.abs(W.bf16_bits_to_f32(bwd["dgu"][r]).astype(np.float64))) @ Wgu[e].abs()
    loss.backward()
    ref = xt.grad.numpy()
    got = W.bf16_bits_to_f32(bwd["dx"]).astype(np.float64)
    # the oracle rounds the SwiGLU gradient to bf16 (2^-9 relative) before the second GEMM and the
    # result to bf16 at the end; float32 steps are far smaller
    bound = 2.0 ** -8 * dgu_abs.numpy() + 2.0 ** -8 * np.abs(ref) + 1e-30
    assert np.all(np.abs(got - ref) <= bound), float((np.abs(got - ref) / bound).max())
    # the first stage on its own: dH of row r = dY[token] W_d[e] in float64
    for t in range(S.T):
        for s in range(S.k):
            e, r = int(ids[t, s]), _brute_row(ids, S.E, t, s)
            np.testing.assert_allclose(bwd["dH"][r], (dyt[t] @ Wd[e]).numpy(), rtol=1e-12, atol=1e-13)
            assert np.array_equal(bwd["dy_perm"][r], dy[t])


def test_qkv_ref_exact_rational():
    T, H, N = 3, 32, 5
    x = W.activations(T, H, config=8)
    w = W.gaussian_bf16((N, H), 0.02, 8, 12)
    a, c = L.qkv_ref(x, Q.quantize_rows_bf16(w))
    for t in range(T):
        own = Q.quantize_rows_bf16(x[t:t + 1])
        assert all(np.array_equal(p[t], q[0]) for p, q in zip(a, own))
    a_ex = _exact_rows(*a)
    w_ex = _exact_rows(*Q.quantize_rows_bf16(w))
    for t in range(T):
        for n in range(N):
            ex = _dot(a_ex[t], w_ex[n])
            assert abs(Fraction(float(c[t, n])) - ex) <= abs(ex) * Fraction(2) ** -50
