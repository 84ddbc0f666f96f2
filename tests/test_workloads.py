"""The seeded input generators: determinism, shapes and the routing statistics they promise."""
import numpy as np

import workloads as W


def test_seeded_and_deterministic():
    a = W.activations(8, 64, config=2)
    b = W.activations(8, 64, config=2)
    c = W.activations(8, 64, config=3)
    assert a.dtype == np.uint16 and np.array_equal(a, b) and not np.array_equal(a, c)


def test_outliers_are_about_one_percent():
    x = W.bf16_bits_to_f32(W.activations(512, 2048, config=2))
    frac = (np.abs(x) > 6).mean()          # N(0,1) almost never exceeds 6; x20 outliers often do
    assert 0.005 < frac < 0.012


def test_softmax_topk_routing():
    ids, w = W.make_routing("softmax", 4096, 128, 8, 2)
    assert ids.shape == (4096, 8) and ids.dtype == np.int32
    assert all(len(set(r)) == 8 for r in ids[:256].tolist())
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)          # ordered by logit, so by weight


def test_zipf_is_skewed_and_uniform_is_flat():
    ids, _ = W.make_routing("zipf", 4096, 128, 8, 3)
    cnt = np.bincount(ids.reshape(-1), minlength=128)
    assert cnt.sum() == 32768 and cnt[0] > 3000 and cnt.min() > 0
    assert all(len(set(r)) == 8 for r in ids[:256].tolist())
    ids, _ = W.make_routing("uniform", 4096, 128, 8, 3)
    cnt = np.bincount(ids.reshape(-1), minlength=128)
    assert 180 < cnt.min() and cnt.max() < 340
