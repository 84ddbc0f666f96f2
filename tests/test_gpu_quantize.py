"""GPU parity: NVFP4 row quantisation and the route + permute + quantise pass.

Bit-exact against the oracle: codes, block scales, row scales, expert offsets
and both identity maps.
"""
import numpy as np
import pytest
import torch

import precision_moe_gemm_amd as pmg
import workloads as W
from oracle import layer as ol, permute as op, quantize as oq
from helpers import bf16_dev, dev, host, gpu_ready, ktile

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs a GPU")]


def _check_rows(bits, tag):
    print(f"[quantize_rows] {tag} shape={bits.shape}", flush=True)
    got = pmg.nvfp4_quantize_rows(bf16_dev(bits))
    torch.cuda.synchronize()
    ref = oq.quantize_rows_bf16(bits)
    for g, r, name in zip(got, ref, ("codes", "bscales", "rscales")):
        g = host(g)
        if name == "rscales":
            assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), f"{tag}: {name}"
        else:
            bad = np.argwhere(g != r)
            assert bad.size == 0, f"{tag}: {name} differs at {bad[:5].tolist()}"


def test_quantize_rows_tiny_config():
    _check_rows(W.gaussian_bf16((64, 256), 1.0, W.CFG_TINY, 0), "A 64x256")
    _check_rows(W.gaussian_bf16((128, 256), 1.0, W.CFG_TINY, 1), "W 128x256")


@pytest.mark.parametrize("K", [16, 48, 256, 512, 528, 768, 1024, 1040, 2048, 4096, 8192])
def test_quantize_rows_lengths(K):
    _check_rows(W.activations(37, K, config=2, tensor=K), f"K={K}")


@pytest.mark.parametrize("rows,K,G", [(12, 64, 12), (256, 2048, 128), (6, 8192, 2), (40, 768, 8)])
def test_quantize_rows_tiled_is_the_oracle_in_the_tiled_layout(rows, K, G):
    """K-tiled output = the oracle's row-major codes and scales, bytes moved."""
    print(f"[quantize_rows_tiled] rows={rows} K={K} G={G}", flush=True)
    bits = W.activations(rows, K, config=3, tensor=K + G)
    c, b, s = pmg.nvfp4_quantize_rows_tiled(bf16_dev(bits), G)
    torch.cuda.synchronize()
    rc, rb, rs = oq.quantize_rows_bf16(bits)
    tc, tb = ktile(rc.reshape(rows // G, G, K // 2), rb.reshape(rows // G, G, K // 16))
    assert np.array_equal(host(c), tc)
    assert np.array_equal(host(b), tb)
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))


def test_quantize_rows_edge_values():
    rng = np.random.default_rng(7)
    rows = []
    rows.append(np.zeros(64, np.float32))                                   # zero row
    z = np.zeros(64, np.float32); z[::3] = -0.0; rows.append(z)             # signed zeros
    t = np.zeros(64, np.float32); t[0] = 1e-30; t[16:32] = 1.1e-35; t[32:] = -1e-38
    rows.append(t)                                                          # subnormal / zero block scales
    rows.append(np.full(64, 3.3e38, np.float32))                            # near bf16 max
    rows.append(np.full(64, -1e-39, np.float32))                            # bf16 subnormals
    r = rng.standard_normal(64).astype(np.float32); r[5] = 1e6; rows.append(r)
    ties = (np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 8) * 1.875 * 2.0 ** -8).astype(np.float32)
    ties[::16] = 11.25 * 2.0 ** -8
    ties[0] = 10.5
    rows.append(ties)                                                       # E2M1 midpoints
    x = np.stack(rows)
    _check_rows(W.f32_to_bf16_bits(x), "edge values")
    worked = np.array([10.5, -10.5, 0.4375, -1.3125, 2.1875, 3.0625, 4.375, 6.125, 8.75, 0.0,
                       -0.0, 1.75, 5.25, 0.875, 7.0, 0.5] +
                      [t * 1.875 * 2.0 ** -8 for t in (6, 1.25, -2.5, 5, 0.25, 0.75, 3.5, 1.75, 1,
                                                        2, 3, 4, 0.5, 1.5, -6, 0)], np.float32)
    _check_rows(W.f32_to_bf16_bits(worked[None]), "worked example")


def _check_rows_f32(x, tag):
    print(f"[quantize_rows_f32] {tag} shape={x.shape}", flush=True)
    got = pmg.nvfp4_quantize_rows_f32(dev(x))
    torch.cuda.synchronize()
    for g, r, name in zip(got, oq.quantize_rows_f32(x), ("codes", "bscales", "rscales")):
        g = host(g)
        if name == "rscales":
            assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), f"{tag}: {name}"
        else:
            bad = np.argwhere(g != r)
            assert bad.size == 0, f"{tag}: {name} differs at {bad[:5].tolist()}"


@pytest.mark.parametrize("K", [16, 48, 256, 528, 768, 1024, 2048, 4096, 8192])
def test_quantize_rows_f32_lengths(K):
    """FP32 rows with full 24-bit significands (the fused SwiGLU path's h) of every row kernel's length."""
    x = (W.rng(4, K).standard_normal((37, K)) * 3.0).astype(np.float32)
    x[::5, K // 3] *= 50.0                                                  # outliers
    _check_rows_f32(x, f"K={K}")


def test_quantize_rows_f32_edge_values():
    rng = np.random.default_rng(8)
    rows = [np.zeros(64, np.float32)]                                       # zero row
    z = np.zeros(64, np.float32); z[::3] = -0.0; rows.append(z)             # signed zeros
    t = np.zeros(64, np.float32); t[0] = 1e-30; t[16:32] = 1.1e-35; t[32:] = -1e-38
    rows.append(t)                                                          # tiny and zero block scales
    rows.append(np.full(64, 3.4e38, np.float32))                            # near the float32 maximum
    rows.append(np.full(64, -1.4e-45, np.float32))                          # the least float32 subnormal
    sub = (rng.standard_normal(64) * 1e-40).astype(np.float32); rows.append(sub)   # float32 subnormals
    one = np.zeros(64, np.float32); one[37] = np.float32(0.1); rows.append(one)    # a single nonzero
    r = rng.standard_normal(64).astype(np.float32); r[5] = 1e6; rows.append(r)
    ties = (np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 8) * 1.875 * 2.0 ** -8).astype(np.float32)
    ties[::16] = 11.25 * 2.0 ** -8
    ties[0] = 10.5
    rows.append(ties)                                                       # E2M1 midpoints
    near = ties.copy()
    near[1::2] = np.nextafter(near[1::2], np.float32(np.inf))               # one float32 ulp above them
    rows.append(near)
    _check_rows_f32(np.stack(rows), "edge values")


def test_quantize_rows_f32_routed_rows_only():
    """With expert offsets, rows from offsets[E] on are not written."""
    x = (W.rng(5, 1).standard_normal((40, 768)) * 2.0).astype(np.float32)
    off = np.array([0, 10, 10, 29], np.int32)
    codes = torch.full((40, 384), 0xAB, dtype=torch.uint8, device="cuda:0")
    bsc = torch.full((40, 48), 0xCD, dtype=torch.uint8, device="cuda:0")
    rsc = torch.full((40,), -7.0, dtype=torch.float32, device="cuda:0")
    pmg.nvfp4_quantize_rows_f32(dev(x), dev(off), codes, bsc, rsc)
    torch.cuda.synchronize()
    rc, rb, rs = oq.quantize_rows_f32(x[:29])
    assert np.array_equal(host(codes)[:29], rc) and np.array_equal(host(bsc)[:29], rb)
    assert np.array_equal(host(rsc)[:29].view(np.uint32), rs.view(np.uint32))
    assert np.all(host(codes)[29:] == 0xAB) and np.all(host(bsc)[29:] == 0xCD) and np.all(host(rsc)[29:] == -7.0)


def test_quantize_rows_e2m1_encode_sweep():
    """Every bf16 value of magnitude up to 6, both signs, as an exact quotient
    x / d: the row amax 2688 makes s = 1, and every other block holds a +-6, so
    its scale is E4M3(1) and d = 1.  The codes then are the E2M1 encoding of
    each bf16 value itself (every tie, and every bf16 neighbour of a tie)."""
    bits = np.arange(0, 0x8000, dtype=np.uint32)
    vals = W.bf16_bits_to_f32(bits.astype(np.uint16))
    mags = vals[np.isfinite(vals) & (vals <= 6.0)]
    sweep = np.concatenate([mags, -mags]).astype(np.float32)
    per_row = 127 * 15                                   # 127 blocks of 15 sweep values after the 2688 block
    n_rows = -(-sweep.size // per_row)
    sweep = np.concatenate([sweep, np.zeros(n_rows * per_row - sweep.size, np.float32)])
    rows = np.zeros((n_rows, 2048), np.float32)
    rows[:, 0] = 2688.0
    blocks = rows[:, 16:].reshape(n_rows, 127, 16)
    blocks[:, :, 0] = np.where(np.arange(127) % 2 == 0, 6.0, -6.0)
    blocks[:, :, 1:] = sweep.reshape(n_rows, 127, 15)
    x = W.f32_to_bf16_bits(rows)
    assert np.array_equal(W.bf16_bits_to_f32(x), rows)  # every value is a bf16 value
    _check_rows(x, "E2M1 encode sweep")
    c, b, s = oq.quantize_rows_bf16(x)
    assert np.all(s == 1.0) and np.all(b[:, 1:] == 0x38)  # d = 1 in every sweep block


def _check_permute(x_bits, ids, E, tag, dev_err_expected=0):
    print(f"[quantize_permute] {tag} T={x_bits.shape[0]} H={x_bits.shape[1]} k={ids.shape[1]} E={E}", flush=True)
    err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    res = pmg.nvfp4_quantize_permute(bf16_dev(x_bits), dev(ids.astype(np.int32)), E, dev_err=err)
    torch.cuda.synchronize()
    off, r2t, t2r, nbad = op.permute(ids, E)
    assert int(host(err)[0]) == dev_err_expected, tag
    assert np.array_equal(host(res["expert_offsets"]), off), tag
    assert np.array_equal(host(res["tk_to_row"]), t2r), tag
    R = int(off[-1])
    assert np.array_equal(host(res["row_to_tk"])[:R], r2t), tag
    codes, bsc, rsc = oq.quantize_rows_bf16(x_bits)
    tok = r2t.astype(np.int64) // ids.shape[1]
    assert np.array_equal(host(res["codes"])[:R], codes[tok]), tag
    assert np.array_equal(host(res["bscales"])[:R], bsc[tok]), tag
    assert np.array_equal(host(res["rscales"])[:R].view(np.uint32), rsc[tok].view(np.uint32)), tag
    return res


def test_quantize_permute_full_config():
    """4096 tokens x 2048, softmax top-8 of 128 experts, 1% x20 outliers."""
    x = W.activations(4096, 2048, config=W.CFG_QPERM)
    ids, _ = W.make_routing("softmax", 4096, 128, 8, W.CFG_QPERM)
    res = _check_permute(x, ids, 128, "config 4096x2048 top8/128")
    # same bytes in all k rows of a token (per-token scaling)
    t2r = host(res["tk_to_row"]).reshape(4096, 8)
    c = host(res["codes"])
    assert np.all(c[t2r[:, 0]] == c[t2r[:, 7]])


@pytest.mark.parametrize("T,E,k,kind", [(5, 4, 2, "uniform"), (1, 1, 1, "uniform"), (1, 128, 8, "uniform"),
                                          (1000, 128, 8, "zipf"), (777, 16, 3, "uniform"),
                                          (2049, 64, 8, "softmax"), (300, 1, 1, "uniform"),
                                          (128, 1024, 32, "uniform"),   # E > 512
                                          (2000, 32, 3, "zipf"),        # groups of 24 entries straddle 2048-entry chunks
                                          (1700, 64, 5, "softmax"),     # ditto, 5 chunks
                                          (600, 1024, 8, "uniform"),    # 3 chunks x 1024 experts in the count table
                                          (10000, 128, 8, "zipf"),      # 20 chunks of 4096 (40 of 2048 would not fit the table)
                                          (3000, 512, 7, "zipf"),       # 6 chunks of 4096 x 512 experts, groups of 56 straddle them
                                          (40000, 128, 8, "zipf"),      # 79 chunks: first rows by one workgroup, 8 threads per expert
                                          (60000, 100, 6, "zipf"),      # 88 chunks, 10 scan threads per expert (1000 of 1024)
                                          (3000, 1024, 32, "uniform")]) # 24 chunks x 1024 experts: one scan thread per expert
def test_quantize_permute_ragged(T, E, k, kind):
    x = W.activations(T, 64 if T > 10000 else 256, config=9, tensor=T)
    ids, _ = W.make_routing(kind, T, E, k, config=9)
    _check_permute(x, ids, E, f"{kind}")


@pytest.mark.parametrize("H", [1024, 3072, 4096])
def test_quantize_permute_row_lengths(H):
    """Rows of 1024/2048/4096 elements take the contiguous-lane quantiser, others the strided one."""
    x = W.activations(300, H, config=9, tensor=H)
    ids, _ = W.make_routing("zipf", 300, 32, 4, config=9)
    _check_permute(x, ids, 32, f"H={H}")


def test_quantize_permute_long_rows():
    """H > 4096 takes the first-row scan and the independent-wavefront pass (16 chunks of 512 per lane)."""
    x = W.activations(50, 8192, config=9, tensor=3)
    ids, _ = W.make_routing("uniform", 50, 16, 4, config=9)
    _check_permute(x, ids, 16, "H=8192")


def test_quantize_permute_empty_experts_and_zero_tokens():
    x = W.activations(64, 512, config=9, tensor=1)
    ids = np.tile(np.array([[3, 0]], np.int32), (64, 1))
    _check_permute(x, ids, 6, "empty experts")
    res = pmg.nvfp4_quantize_permute(bf16_dev(np.zeros((0, 512), np.uint16)),
                                     dev(np.zeros((0, 2), np.int32)), 6)
    torch.cuda.synchronize()
    assert host(res["expert_offsets"]).tolist() == [0] * 7


def test_quantize_permute_invalid_ids_flagged():
    x = W.activations(40, 256, config=9, tensor=2)
    ids, _ = W.make_routing("uniform", 40, 8, 2, config=9)
    ids[3, 1] = 8
    ids[17, 0] = -5
    _check_permute(x, ids, 8, "invalid ids", dev_err_expected=1)


def test_quantize_permute_deterministic():
    x = bf16_dev(W.activations(2048, 2048, config=2))
    ids = dev(W.make_routing("zipf", 2048, 128, 8, 2)[0])
    a = pmg.nvfp4_quantize_permute(x, ids, 128)
    b = pmg.nvfp4_quantize_permute(x, ids, 128)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key


def test_dense_projection_path_k1_e1():
    """k = 1, E = 1 with all ids 0 is plain per-token quantisation in token order."""
    x = W.activations(300, 2048, config=5)
    ids = np.zeros((300, 1), np.int32)
    res = _check_permute(x, ids, 1, "k=1 E=1")
    assert np.array_equal(host(res["row_to_tk"]), np.arange(300))
