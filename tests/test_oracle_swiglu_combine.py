"""Pins of the oracle's weighted SwiGLU (forward + backward), combine, gather and layer chain.

* SwiGLU forward against scipy's logistic function (a library routine) and at
  closed-form points; the backward against torch autograd in float64 and
  against central finite differences;
* the midpoint detector on constructed midpoints;
* combine on identity experts and on power-of-two data where every FP32 sum is
  exact, and its slot order on data where the order changes the result.
The chained layer (oracle/layer.py) is pinned in test_oracle_layer.py.
"""
import numpy as np
import scipy.special
import torch

from oracle import combine as C, formats as F, quantize as Q, swiglu as S
import workloads as W


def test_swiglu_forward_against_expit():
    rng = np.random.default_rng(0)
    gu = (rng.standard_normal((16, 64)) * 3).astype(np.float32)
    w = rng.random(16).astype(np.float32)
    h = S.swiglu_h64(gu, w)
    g, u = gu[:, :32].astype(np.float64), gu[:, 32:].astype(np.float64)
    ref = g * scipy.special.expit(g) * u * w[:, None].astype(np.float64)
    np.testing.assert_allclose(h, ref, rtol=1e-14, atol=1e-300)


def test_swiglu_closed_form_points():
    gu = np.array([[0.0, 50.0, -50.0, 2.0, 1.0, 1.0, 1.0, 0.0]], np.float32)
    h = S.swiglu_h64(gu)
    assert h[0, 0] == 0.0                              # silu(0) = 0
    assert abs(h[0, 1] - 50.0) < 1e-15 * 50            # silu(g) -> g for large g
    assert abs(h[0, 2]) < 1e-18                        # silu(g) -> 0 for very negative g
    assert h[0, 3] == 0.0                              # u = 0


def test_swiglu_quantize_is_quantize_of_h():
    rng = np.random.default_rng(1)
    gu = rng.standard_normal((8, 1536)).astype(np.float32)
    w = rng.random(8).astype(np.float32)
    codes, b, s, h, amb = S.swiglu_quantize_ref(gu, w)
    c2, b2, s2 = Q.quantize_rows_f32(h)
    assert np.array_equal(codes, c2) and np.array_equal(b, b2) and np.array_equal(s, s2)
    assert h.dtype == np.float32 and amb.shape == h.shape


def test_rn32_midpoint_detector():
    c = np.float32(1.5)
    up = np.nextafter(c, np.float32(2))
    mid = (np.float64(c) + np.float64(up)) / 2
    x = np.array([mid, mid * (1 + 2.0 ** -50), 1.5, 1.5 + 2.0 ** -30])
    assert S.rn32_ambiguous(x).tolist() == [True, True, False, False]


def test_swiglu_backward_against_autograd_and_fd():
    rng = np.random.default_rng(2)
    R, I = 8, 16
    # values on a 2^-8 grid so that +-2^-14 perturbations are exact in float32
    gu = (np.round(rng.standard_normal((R, 2 * I)) * 2 * 256) / 256).astype(np.float32)
    dH = rng.standard_normal((R, I)).astype(np.float32)
    w = rng.random(R).astype(np.float32)
    _, d64 = S.swiglu_backward_ref(gu, dH, w)
    g = torch.tensor(gu[:, :I], dtype=torch.float64, requires_grad=True)
    u = torch.tensor(gu[:, I:], dtype=torch.float64, requires_grad=True)
    h = torch.nn.functional.silu(g) * u * torch.tensor(w, dtype=torch.float64)[:, None]
    h.backward(torch.tensor(dH, dtype=torch.float64))
    ref = np.concatenate([g.grad.numpy(), u.grad.numpy()], axis=1)
    np.testing.assert_allclose(d64, ref, rtol=1e-12, atol=1e-14)
    # central differences of the oracle's own forward
    eps = 2.0 ** -14
    for (r, j) in [(0, 0), (3, 5), (7, I + 2), (5, 2 * I - 1)]:
        p = gu.copy(); m = gu.copy()
        p[r, j] += eps; m[r, j] -= eps
        fd = ((S.swiglu_h64(p, w) - S.swiglu_h64(m, w)) / (2 * eps) * dH.astype(np.float64)).sum()
        assert abs(fd - d64[r, j]) < 1e-6 * max(1.0, abs(fd))


def test_swiglu_backward_rounds_once_to_bf16():
    rng = np.random.default_rng(3)
    gu = rng.standard_normal((4, 64)).astype(np.float32)
    dH = rng.standard_normal((4, 32)).astype(np.float32)
    bits, d64 = S.swiglu_backward_ref(gu, dH)
    assert np.array_equal(bits, F.round_to_bf16(d64))


def test_combine_identity_experts_and_exact_sums():
    T, k, H = 6, 4, 32
    rng = np.random.default_rng(4)
    ids = np.stack([rng.permutation(8)[:k] for _ in range(T)]).astype(np.int32)
    from oracle.permute import permute
    _, r2t, t2r, _ = permute(ids, 8)
    # rows hold powers of two: every FP32 sum exact, result = sum over slots
    vals = np.exp2(rng.integers(-3, 3, (T * k, H))).astype(np.float32)
    D = vals[r2t]
    y, acc = C.unpermute_combine_ref(D, t2r, k)
    assert np.array_equal(acc, vals.reshape(T, k, H).sum(axis=1))
    # identity experts with normalised weights give back the token
    x = W.bf16_bits_to_f32(W.gaussian_bf16((T, H), 1.0, 9, 0))
    w = np.full((T, k), 0.25, np.float32)
    Dx = x[r2t // k]
    y2, acc2 = C.unpermute_combine_ref(Dx, t2r, k, w)
    assert np.array_equal(acc2, x)


def test_combine_slot_order_is_left_to_right():
    # (1 + 2^-24) + 2^-24 ... ordering changes the float32 result
    D = np.array([[1.0], [2.0 ** -24], [2.0 ** -24], [2.0 ** -24]], np.float32)
    t2r = np.array([0, 1, 2, 3])
    _, acc = C.unpermute_combine_ref(D, t2r, 4)
    assert acc[0, 0] == np.float32(1.0)                # each 2^-24 is lost against 1.0
    t2r2 = np.array([1, 2, 3, 0])
    _, acc2 = C.unpermute_combine_ref(D, t2r2, 4)
    assert acc2[0, 0] == np.float32(1.0) + np.float32(2.0 ** -22)


def test_gather_inverts_combine_rows():
    ids = np.array([[1, 0], [0, 2], [2, 1]], np.int32)
    from oracle.permute import permute
    _, r2t, t2r, _ = permute(ids, 3)
    x = np.arange(3 * 4, dtype=np.uint16).reshape(3, 4)
    g = C.permute_gather_ref(x, r2t, 2)
    assert np.array_equal(g[t2r.reshape(3, 2)[:, 0]], x)
    assert np.array_equal(g[t2r.reshape(3, 2)[:, 1]], x)
