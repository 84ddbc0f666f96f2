"""GPU parity: the other precisions around the layer step.

* bf16_transpose: bit-exact against numpy's transpose (a move of bytes).
* BF16 forward grouped GEMMs (the forward at the precision NVFP4 replaces):
  bf16_grouped_gemm_gather with [E][N][K] weights reads token rows in expert
  order; against the FP64 oracle, and bit for bit against the GEMM of the
  gathered rows.
* NVFP4 input gradient (a lower-precision backward): the output gradient is
  quantised and permuted like the forward's activations, the forward weight
  is transposed and quantised along its output dimension, and the grouped
  NVFP4 GEMM contracts the two; against the oracle's quantiser and its
  exact-dequantisation GEMM, with the GEMM bar |err| <= 2e-5 * sum |a w|.
"""
import numpy as np
import pytest
import torch

import precision_moe_gemm_amd as pmg
import workloads as W
from oracle import formats as of, gemm as og, layer as ol, permute as op, quantize as oq
from helpers import (assert_within, bf16_dev, bf16_host, dev, gpu_ready, host, ktile,
                     quantize_weights_oracle, sample_rows)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs a GPU")]


@pytest.mark.parametrize("B,rows,cols", [(1, 8, 8), (3, 72, 136), (2, 64, 64), (4, 2048, 768),
                                         (2, 1536, 2048)])
def test_bf16_transpose_bit_exact(B, rows, cols):
    print(f"[transpose] B={B} rows={rows} cols={cols}", flush=True)
    x = W.gaussian_bf16((B, rows, cols), 1.0, 71, rows + cols)
    got = bf16_host(pmg.bf16_transpose(bf16_dev(x)))
    torch.cuda.synchronize()
    assert np.array_equal(got, x.transpose(0, 2, 1))


class _F32View:
    """bf16 bits [E, ...] seen as float32 one expert at a time (the oracle reads w[e])."""

    def __init__(self, bits):
        self.bits, self.shape = bits, bits.shape

    def __getitem__(self, e):
        return of.bf16_to_f32(self.bits[e])


def _routing(T, E, k, kind, seed):
    ids, _ = W.make_routing(kind, T, E, k, seed)
    off, r2t, t2r, _ = op.permute(ids, E)
    return ids, off, r2t, t2r


@pytest.mark.parametrize("T,E,k,H,N,kind", [(256, 8, 4, 256, 192, "uniform"),
                                             (40, 16, 2, 96, 64, "zipf"),
                                             (4096, 128, 8, 2048, 1536, "softmax")])
def test_bf16_forward_gemm_gather_nk(T, E, k, H, N, kind):
    """c[r] = x[t(r)] W_e^T with W [E][N][K]: the BF16 forward gate_up."""
    print(f"[bf16 forward] T={T} E={E} k={k} H={H} N={N} {kind}", flush=True)
    ids, off, r2t, t2r = _routing(T, E, k, kind, 72)
    x = W.gaussian_bf16((T, H), 1.0, 72, 40)
    w = W.gaussian_bf16((E, N, H), 0.02, 72, 41)
    xd, wd, offd, r2td = bf16_dev(x), bf16_dev(w), dev(off), dev(r2t)
    c = host(pmg.bf16_grouped_gemm_gather(xd, r2td, k, offd, wd, pmg.W_NK))
    c2 = host(pmg.bf16_grouped_gemm(pmg.permute_gather_bf16(xd, offd, r2td, k), offd, wd, pmg.W_NK))
    Rv = int(off[-1])
    assert np.array_equal(c[:Rv].view(np.uint32), c2[:Rv].view(np.uint32))
    rows = sample_rows(off, [0, E - 1], extra=3, seed=6)[0] if T * k > 1000 else np.arange(Rv)
    a_perm = of.bf16_to_f32(x)[r2t[:Rv] // k]
    ref, bound = og.bf16_grouped_gemm_ref(a_perm, off, _F32View(w), trans_w=True, rows=rows)
    print("  err/bound", assert_within(c[rows], ref, bound, "bf16 forward"))


def _transposed_weights_gpu(w_bits):
    """[E, out, in] bf16 -> the transpose [E, in, out] on the device, quantised
    along `out` into the K-tiled layout (codes, bscales, rscales [E, in])."""
    E, n_out, n_in = w_bits.shape
    wt = pmg.bf16_transpose(bf16_dev(w_bits))
    c, b, s = pmg.nvfp4_quantize_rows_tiled(wt.view(E * n_in, n_out), n_in)
    return c, b, s.view(E, n_in)


def _check_tiled_weights(w_bits, got):
    """The device's transposed K-tiled weights are the oracle's quantisation of
    the transpose, bytes moved into the K-tiled layout."""
    E, n_out, n_in = w_bits.shape
    rc, rb, rs = oq.quantize_rows_bf16(np.ascontiguousarray(w_bits.transpose(0, 2, 1)).reshape(E * n_in, n_out))
    tc, tb = ktile(rc.reshape(E, n_in, n_out // 2), rb.reshape(E, n_in, n_out // 16))
    assert np.array_equal(host(got[0]), tc)
    assert np.array_equal(host(got[1]), tb)
    assert np.array_equal(host(got[2]).reshape(-1).view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("T,E,k,H,I,kind", [(256, 8, 4, 256, 128, "uniform"),
                                             (60, 16, 2, 128, 64, "zipf"),
                                             (4096, 128, 8, 2048, 768, "softmax")])
def test_nvfp4_input_gradient(T, E, k, H, I, kind):
    """Both input-gradient GEMMs of the MoE layer in NVFP4:
    dH = Q(dY_perm) Q(W_d^T)^T  ([R x H] x [E][I][H]),
    dX_perm = Q(dGU) Q(W_gu^T)^T  ([R x 2I] x [E][H][2I])."""
    print(f"[nvfp4 dgrad] T={T} E={E} k={k} H={H} I={I} {kind}", flush=True)
    ids, off, r2t, t2r = _routing(T, E, k, kind, 73)
    dy = W.gaussian_bf16((T, H), 1.0, 73, 42)
    w_d = W.gaussian_bf16((E, H, I), 0.02, 73, 43)        # forward down weight [E][out=H][in=I]
    w_gu = W.gaussian_bf16((E, 2 * I, H), 0.02, 73, 44)   # forward gate_up weight [E][out=2I][in=H]
    dgu = W.gaussian_bf16((T * k, 2 * I), 1.0, 73, 45)
    Rv = int(off[-1])
    if T * k > 1000:
        rows, experts = sample_rows(off, [0, E - 1], extra=3, seed=7)
    else:
        rows, experts = np.arange(Rv), None
    wq_d, wq_gu = _transposed_weights_gpu(w_d), _transposed_weights_gpu(w_gu)
    # down's input gradient: the output gradient quantised and permuted like the forward input
    q = pmg.nvfp4_quantize_permute(bf16_dev(dy), dev(ids), E)
    assert np.array_equal(host(q["expert_offsets"]), off)
    dh = host(pmg.nvfp4_grouped_gemm(q["codes"], q["bscales"], q["rscales"], q["expert_offsets"], *wq_d))
    (_, _, _), a_ref = ol.quantize_permute_ref(dy, ids, E)
    w_dt = np.ascontiguousarray(w_d.transpose(0, 2, 1))
    ref, bound = og.grouped_gemm_ref(*a_ref, off, *quantize_weights_oracle(w_dt, experts), rows=rows)
    print("  dH err/bound", assert_within(dh[rows], ref, bound, "nvfp4 dgrad down"))
    # gate_up's input gradient: the SwiGLU gradient rows quantised in place
    g = pmg.nvfp4_quantize_rows(bf16_dev(dgu))
    dxp = host(pmg.nvfp4_grouped_gemm(*g, q["expert_offsets"], *wq_gu))
    # the oracle quantises only the compared rows (the others stay zero and are not read)
    qc = np.zeros((T * k, I), np.uint8); qb = np.zeros((T * k, I // 8), np.uint8)
    qs = np.zeros(T * k, np.float32)
    qc[rows], qb[rows], qs[rows] = oq.quantize_rows_bf16(dgu[rows])
    w_gut = np.ascontiguousarray(w_gu.transpose(0, 2, 1))
    ref, bound = og.grouped_gemm_ref(qc, qb, qs, off, *quantize_weights_oracle(w_gut, experts), rows=rows)
    print("  dX_perm err/bound", assert_within(dxp[rows], ref, bound, "nvfp4 dgrad gate_up"))
    if T * k <= 2048:
        _check_tiled_weights(w_d, wq_d)
