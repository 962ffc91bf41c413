"""Checks of the seeded workload generators (their Zipf notion itself is a
reading of the workload description and has no external pin)."""

import numpy as np
import pytest

from synth import CONFIGS, algorithmic_bytes, make_workload, zipf_probs


@pytest.mark.parametrize("name", list(CONFIGS))
def test_shapes_ranges_and_weights(name):
    cfg = CONFIGS[name]
    T = min(cfg.T, 1024)
    wl = make_workload(name, T=T)
    assert wl.topk_idx.shape == (T, cfg.k) and wl.topk_idx.dtype == np.int32
    assert wl.topk_idx.min() >= 0 and wl.topk_idx.max() < cfg.E
    for row in wl.topk_idx:
        assert len(set(row.tolist())) == cfg.k
    assert wl.topk_w.dtype == np.float32
    assert np.all(wl.topk_w > 0)
    np.testing.assert_allclose(wl.topk_w.sum(axis=1), 1.0, atol=1e-6)
    if cfg.ops == "combine":
        assert wl.x is None and wl.y.shape == (T * cfg.k, cfg.H)
    else:
        assert wl.x.shape == (T, cfg.H) and wl.x.dtype == np.uint16
    if cfg.expert == "scale":
        assert wl.scales.shape == (cfg.E,) and wl.scales.min() >= 0.5 and wl.scales.max() <= 1.5


def test_seeds_reproduce_and_differ():
    a = make_workload("tiny")
    b = make_workload("tiny")
    c = make_workload("tiny", seed=99)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.topk_idx, b.topk_idx)
    assert np.array_equal(a.topk_w, b.topk_w)
    assert not np.array_equal(a.topk_idx, c.topk_idx)


def test_x_is_standard_normal_bf16():
    wl = make_workload("tiny")
    xf = (wl.x.astype(np.uint32) << 16).view(np.float32)
    assert abs(xf.mean()) < 0.02 and abs(xf.std() - 1.0) < 0.02


def test_zipf_popularity_decreases():
    p = zipf_probs(64, 1.0)
    assert np.all(np.diff(p) < 0) and abs(p.sum() - 1) < 1e-12
    wl = make_workload("prefill", T=4096)
    counts = np.bincount(wl.topk_idx.ravel(), minlength=64)
    # on average popularity falls with the expert index
    assert counts[:8].mean() > counts[8:32].mean() > counts[32:].mean()
    assert counts[0] == counts.max()


def test_uniform_routing_is_roughly_flat():
    wl = make_workload("train", T=4096)
    counts = np.bincount(wl.topk_idx.ravel(), minlength=256)
    assert counts.min() > 0.6 * counts.mean() and counts.max() < 1.4 * counts.mean()


def test_algorithmic_bytes_closed_forms():
    # dispatch = T*2H + T*k*2H + 4Tk ; combine = T*k*2H + T*2H + 8Tk
    assert algorithmic_bytes(128, 1024, 2, 8)["dispatch"] == 787_456
    assert algorithmic_bytes(128, 1024, 2, 8)["combine"] == 788_480
    assert algorithmic_bytes(4096, 7168, 8, 256)["dispatch"] == 528_613_376
    assert algorithmic_bytes(4096, 7168, 8, 256)["combine"] == 528_744_448
    assert algorithmic_bytes(16384, 7168, 6, 64)["dispatch"] == 1_644_560_384
    assert algorithmic_bytes(8192, 4096, 8, 256)["combine"] == 604_504_064
    assert algorithmic_bytes(4096, 7168, 8, 256)["layout"] == 12 * 32768 + 8 * 256 + 4
