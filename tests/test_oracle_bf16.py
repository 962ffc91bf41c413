"""Pins for the oracle's bf16 conversions: hand-derived IEEE cases and the
conversions of an independent library (torch's CPU bfloat16)."""

import os

import numpy as np
import torch

from oracle import bf16_to_f32, f32_to_bf16_rne

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bf16_rne_cases.txt")


def _golden_cases():
    cases = []
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            f_hex, b_hex = line.split()[:2]
            cases.append((int(f_hex, 16), int(b_hex, 16)))
    return cases


def test_golden_rne_cases():
    cases = _golden_cases()
    assert len(cases) >= 15
    f = np.array([c[0] for c in cases], dtype=np.uint32).view(np.float32)
    got = f32_to_bf16_rne(f)
    want = np.array([c[1] for c in cases], dtype=np.uint16)
    np.testing.assert_array_equal(got, want)


def test_nan_stays_nan():
    pats = np.array([0x7FC00000, 0x7F800001, 0xFFFFFFFF, 0x7FFFFFFF, 0xFF800001], dtype=np.uint32)
    out = f32_to_bf16_rne(pats.view(np.float32))
    assert np.all(np.isnan(bf16_to_f32(out)))
    # signalling NaN with only low payload bits must not collapse to inf
    assert out[1] != 0x7F80 and out[4] != 0xFF80


def test_widen_matches_torch_all_patterns():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = bf16_to_f32(h)
    ref = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_round_matches_torch_random_and_special():
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 2**32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    # force many exact ties and near-ties
    bits[: 1 << 16] = (bits[: 1 << 16] & 0xFFFF0000) | 0x8000
    bits[1 << 16 : 1 << 17] = (bits[1 << 16 : 1 << 17] & 0xFFFF0000) | 0x7FFF
    f = bits.view(np.float32)
    ours = f32_to_bf16_rne(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours_nan = np.isnan(bf16_to_f32(ours))
    ref_nan = np.isnan(bf16_to_f32(ref))
    np.testing.assert_array_equal(ours_nan, ref_nan)
    np.testing.assert_array_equal(ours[~ours_nan], ref[~ref_nan])


def test_round_trip_is_identity():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    back = f32_to_bf16_rne(bf16_to_f32(h))
    nan = np.isnan(bf16_to_f32(h))
    np.testing.assert_array_equal(back[~nan], h[~nan])
