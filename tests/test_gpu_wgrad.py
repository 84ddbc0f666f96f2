"""GPU parity: the expert weight gradient in NVFP4, quantised along tokens.

dW_d[e] = dY_e^T h_e (down projection: output gradient gathered from token
order by the routing map, SwiGLU output in the expert-grouped order) and
dW_gu[e] = dGU_e^T x_e (gate_up projection: SwiGLU gradient in the
expert-grouped order, input gathered from token order).  Quantiser bytes
(codes, block scales, per-(expert, channel) scales) bit-exact against the
oracle's per-expert slabs; the K-grouped GEMM within 2e-5 * sum |a w| per
element against the oracle's exact product.  Small cases compare every
expert; the full layer (4096 tokens, 128 experts) compares sampled experts.
"""
import numpy as np
import pytest
import torch

import precision_moe_gemm_amd as pmg
import workloads as W
from oracle import formats as of, permute as op, wgrad as ow
from helpers import assert_within, bf16_dev, dev, gpu_ready, host, ktile

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs a GPU")]


def _check_quantized(got_rm, got_kt, ref, kofs, experts, tag):
    """got_rm: row-major (codes [C][Kp/2], bscales [C][Kp/16], rscales [E][C]) or None;
    got_kt: K-tiled ([Kp/64][C][32], [Kp/64][C][4], [E][C]) or None."""
    for e in experts:
        rc, rb, rs = ref[e]
        k0, k1 = int(kofs[e]), int(kofs[e + 1])
        if got_rm is not None:
            c, b, s = got_rm
            assert np.array_equal(c[:, 32 * k0:32 * k1], rc), f"{tag} codes e{e}"
            assert np.array_equal(b[:, 4 * k0:4 * k1], rb), f"{tag} bscales e{e}"
            assert np.array_equal(s[e].view(np.uint32), rs.view(np.uint32)), f"{tag} rscales e{e}"
        if got_kt is not None:
            c, b, s = got_kt
            assert np.array_equal(c[k0:k1].transpose(1, 0, 2).reshape(rc.shape), rc), f"{tag} K-tiled codes e{e}"
            assert np.array_equal(b[k0:k1].transpose(1, 0, 2).reshape(rb.shape), rb), f"{tag} K-tiled bscales e{e}"
            assert np.array_equal(s[e].view(np.uint32), rs.view(np.uint32))


def _run(g_rows, x_rows, T, E, k, kind, seed, sample=None):
    """g_rows / x_rows: ('token', bf16 bits [T][C]) or ('grouped', float32 or bf16 bits [R][C])."""
    ids, _ = W.make_routing(kind, T, E, k, seed)
    off, r2t, _, _ = op.permute(ids, E)
    R = int(off[-1])
    off_d, r2t_d = dev(off), dev(r2t)
    kofs_d = pmg.token_blocks(off_d)
    kofs = host(kofs_d)
    assert np.array_equal(kofs, ow.token_blocks(off))
    Kp = pmg.token_capacity(R, E)

    def side(spec, layout):
        how, arr = spec
        if arr.dtype == np.uint16:
            t = bf16_dev(arr)
            f32 = of.bf16_to_f32(arr)
        else:
            t = dev(arr)
            f32 = arr
        if how == "token":
            q = pmg.nvfp4_quantize_tokens(t, off_d, kofs_d, Kp, layout, row_to_tk=r2t_d, k=k)
            grouped = f32[r2t.astype(np.int64) // k]
        else:
            q = pmg.nvfp4_quantize_tokens(t, off_d, kofs_d, Kp, layout)
            grouped = f32
        return q, grouped

    gq, g_grp = side(g_rows, pmg.W_ROWMAJOR)
    xq, x_grp = side(x_rows, pmg.W_KTILED)
    dw = pmg.nvfp4_grouped_gemm_wgrad(gq, xq, kofs_d)
    dwb = pmg.nvfp4_grouped_gemm_wgrad(gq, xq, kofs_d, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    # BF16 output: the FP32 result rounded to nearest even, bit for bit (every expert's first
    # 64 rows; all of them for the small cases)
    rows = slice(None) if sample is None else slice(0, 64)
    assert np.array_equal(dwb[:, rows].contiguous().view(torch.int16).cpu().numpy().view(np.uint16),
                          W.f32_to_bf16_bits(host(dw[:, rows].contiguous())))
    del dwb
    experts = list(range(E)) if sample is None else sample(np.diff(off))
    g_ref = {e: ow.quantize_expert_ref(g_grp, off, e, kofs) for e in experts}
    x_ref = {e: ow.quantize_expert_ref(x_grp, off, e, kofs) for e in experts}
    _check_quantized(tuple(host(t) for t in gq), None, g_ref, kofs, experts, "G")
    _check_quantized(None, tuple(host(t) for t in xq), x_ref, kofs, experts, "X")
    if sample is None:   # small case: the K-tiled bytes against the row-major oracle moved by the index functions
        M_x = x_grp.shape[1]
        full_c = np.zeros((M_x, Kp // 2), np.uint8)
        full_b = np.zeros((M_x, Kp // 16), np.uint8)
        for e in experts:
            full_c[:, 32 * kofs[e]:32 * kofs[e + 1]] = x_ref[e][0]
            full_b[:, 4 * kofs[e]:4 * kofs[e + 1]] = x_ref[e][1]
        tc, tb = ktile(full_c[None], full_b[None])
        n_steps = int(kofs[-1])
        assert np.array_equal(host(xq[0])[:n_steps], tc[0][:n_steps])
        assert np.array_equal(host(xq[1])[:n_steps], tb[0][:n_steps])
    ref, bound = ow.wgrad_ref([g_ref[e] for e in experts], [x_ref[e] for e in experts])
    got = host(dw[torch.tensor(experts, device=dw.device)])
    print(f"  experts {len(experts)}, err/bound", assert_within(got, ref, bound, "wgrad"), flush=True)


@pytest.mark.parametrize("T,E,k,C_g,C_x,kind", [(300, 16, 4, 256, 512, "uniform"),
                                                 (40, 8, 2, 768, 256, "zipf")])   # empty experts
def test_wgrad_small_all_experts(T, E, k, C_g, C_x, kind):
    print(f"[wgrad] T={T} E={E} k={k} C_g={C_g} C_x={C_x} {kind}", flush=True)
    dy = W.gaussian_bf16((T, C_g), 1.0, 60, 1)                                # token order
    h = (W.rng(60, 2).standard_normal((T * k, C_x)) * 0.5).astype(np.float32)  # expert-grouped rows
    _run(("token", dy), ("grouped", h), T, E, k, kind, 60)


def _sample(counts):
    rng = np.random.default_rng(9)
    return sorted(set([int(np.argmax(counts)), int(np.argmin(counts))] + [int(e) for e in rng.choice(counts.size, 3)]))


def test_wgrad_most_experts():
    """1024 experts (the library's limit), 1024 routed rows: most experts hold 0-2 tokens in their
    64-token slab; a sample of experts (with the largest and an empty one) against the oracle."""
    print("[wgrad] E=1024", flush=True)
    T, E, k = 128, 1024, 8
    dy = W.gaussian_bf16((T, 256), 1.0, 61, 1)
    h = (W.rng(61, 2).standard_normal((T * k, 256)) * 0.5).astype(np.float32)

    def sample(rows):
        picks = set(range(0, E, 37)) | {int(np.argmax(rows))}
        empty = np.flatnonzero(rows == 0)
        if empty.size:
            picks.add(int(empty[0]))
        return sorted(picks)
    _run(("token", dy), ("grouped", h), T, E, k, "uniform", 61, sample=sample)


@pytest.mark.parametrize("which", ["down", "gate_up"])
def test_wgrad_layer_sampled(which):
    S = W.LayerShape()
    print(f"[wgrad] layer {which}", flush=True)
    if which == "down":      # dW_d = dY^T h: dY token order [T][H], h grouped [R][I] float32
        g = ("token", W.grad_output_bf16(S, W.CFG_LAYER))
        x = ("grouped", (W.rng(W.CFG_LAYER, 40).standard_normal((S.R, S.I)) * 0.3).astype(np.float32))
    else:                    # dW_gu = dGU^T x: dGU grouped [R][2I] bf16, x token order [T][H]
        g = ("grouped", W.gaussian_bf16((S.R, 2 * S.I), 0.01, W.CFG_LAYER, 41))
        x = ("token", W.activations(S.T, S.H, config=W.CFG_LAYER))
    _run(g, x, S.T, S.E, S.k, "softmax", W.CFG_LAYER, sample=_sample)
