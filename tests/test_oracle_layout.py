"""Pins for the oracle's layout: a stable sort from numpy, brute force on tiny
inputs, and the invariants any expert-grouped layout must satisfy."""

import itertools

import numpy as np
import pytest

from oracle import STATUS_DUPLICATE_EXPERT, STATUS_EXPERT_OUT_OF_RANGE, layout
from synth import CONFIGS, make_workload


def check_invariants(idx, E, lay):
    T, k = idx.shape
    R = T * k
    counts, offsets = lay["counts"], lay["offsets"]
    dest, src = lay["dest_row"], lay["src_token"]
    assert counts.sum() == R
    assert offsets[0] == 0 and offsets[E] == R
    assert np.all(np.diff(offsets) == counts)
    # dest_row is a bijection onto [0, R)
    assert np.array_equal(np.sort(dest.ravel()), np.arange(R))
    for t in range(T):
        for j in range(k):
            r = dest[t, j]
            assert src[r] == t
            e = idx[t, j]
            assert offsets[e] <= r < offsets[e + 1]
    # tokens ascend strictly inside each segment (distinct experts per token)
    for e in range(E):
        seg = src[offsets[e] : offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)
        for r in range(offsets[e], offsets[e + 1]):
            assert e in idx[src[r]]


def argsort_layout(idx, E):
    """Same layout from a library stable sort (independent of the oracle's loops)."""
    T, k = idx.shape
    flat = idx.ravel()
    order = np.argsort(flat, kind="stable")
    dest = np.empty(T * k, dtype=np.int64)
    dest[order] = np.arange(T * k)
    counts = np.bincount(flat, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    return counts, offsets, dest.reshape(T, k), order // k


@pytest.mark.parametrize("name", list(CONFIGS))
def test_matches_stable_argsort_on_configs(name):
    cfg = CONFIGS[name]
    T = min(cfg.T, 4096)
    wl = make_workload(name, T=T)
    lay = layout(wl.topk_idx, cfg.E)
    counts, offsets, dest, src = argsort_layout(wl.topk_idx, cfg.E)
    np.testing.assert_array_equal(lay["counts"], counts)
    np.testing.assert_array_equal(lay["offsets"], offsets)
    np.testing.assert_array_equal(lay["dest_row"], dest)
    np.testing.assert_array_equal(lay["src_token"], src)
    assert lay["status"] == 0


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_invariants_full_size(name):
    cfg = CONFIGS[name]
    wl = make_workload(name)
    check_invariants(wl.topk_idx, cfg.E, layout(wl.topk_idx, cfg.E))


def brute_force(idx, E):
    """Per-expert token lists built by scanning experts, then tokens."""
    T, k = idx.shape
    rows = []  # (expert, token, slot) in receive order
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if idx[t, j] == e:
                    rows.append((e, t, j))
    dest = np.full((T, k), -1)
    for r, (e, t, j) in enumerate(rows):
        dest[t, j] = r
    counts = [sum(1 for row in rows if row[0] == e) for e in range(E)]
    return counts, dest, [t for (_, t, _) in rows]


def test_brute_force_tiny_seed_sweep():
    for seed in range(60):
        rng = np.random.default_rng(seed)
        E = int(rng.integers(1, 7))
        k = int(rng.integers(1, min(3, E) + 1))
        T = int(rng.integers(0, 17))
        idx = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32).reshape(T, k)
        lay = layout(idx, E)
        counts, dest, src = brute_force(idx, E)
        np.testing.assert_array_equal(lay["counts"], counts)
        np.testing.assert_array_equal(lay["dest_row"], dest)
        np.testing.assert_array_equal(lay["src_token"][: T * k], src)
        if T:
            check_invariants(idx, E, lay)


def test_exhaustive_small():
    # every routing of T=3 tokens, k=2 distinct experts among E=3
    pairs = [p for p in itertools.permutations(range(3), 2)]
    for rows in itertools.product(pairs, repeat=3):
        idx = np.array(rows, dtype=np.int32)
        lay = layout(idx, 3)
        counts, dest, src = brute_force(idx, 3)
        np.testing.assert_array_equal(lay["dest_row"], dest)
        np.testing.assert_array_equal(lay["src_token"], src)


def test_empty_and_single():
    lay = layout(np.zeros((0, 4), dtype=np.int32), 16)
    assert lay["counts"].sum() == 0 and np.all(lay["offsets"] == 0)
    lay = layout(np.array([[3]], dtype=np.int32), 4)
    assert list(lay["offsets"]) == [0, 0, 0, 0, 1]
    assert lay["dest_row"][0, 0] == 0 and lay["src_token"][0] == 0


def test_out_of_range_entries_are_flagged_and_skipped():
    idx = np.array([[0, 5], [-1, 1], [1, 0]], dtype=np.int32)
    lay = layout(idx, 4)
    assert lay["status"] == STATUS_EXPERT_OUT_OF_RANGE
    assert lay["dest_row"][0, 1] == -1 and lay["dest_row"][1, 0] == -1
    assert list(lay["counts"]) == [2, 2, 0, 0]
    assert list(lay["offsets"]) == [0, 2, 4, 4, 4]
    # valid entries keep stable order: expert 0 <- tokens 0, 2 ; expert 1 <- 1, 2
    assert lay["dest_row"][0, 0] == 0 and lay["dest_row"][2, 1] == 1
    assert lay["dest_row"][1, 1] == 2 and lay["dest_row"][2, 0] == 3
    assert list(lay["src_token"][:4]) == [0, 2, 1, 2]


def test_duplicates_are_flagged_but_placed():
    idx = np.array([[2, 2], [2, 0]], dtype=np.int32)
    lay = layout(idx, 3)
    assert lay["status"] == STATUS_DUPLICATE_EXPERT
    assert lay["dest_row"].tolist() == [[1, 2], [3, 0]]
    assert list(lay["src_token"]) == [1, 0, 0, 1]


def test_zipf_imbalance_shape():
    # decode: many empty experts and one hot one (a property of the workload,
    # which the layout must handle; counts come from the oracle)
    wl = make_workload("decode")
    lay = layout(wl.topk_idx, 256)
    assert (lay["counts"] == 0).sum() > 40
    assert lay["counts"].max() > 64
