"""Pins for the oracle's dispatch and combine: the invariants of a copy with
duplication k, brute force, the identity-expert round trip, the scale-expert
closed form, exact rational sums with a rounding-error bound, and a
hand-derived case that fixes the summation order and the final rounding."""

from fractions import Fraction

import numpy as np
import pytest

from golden_io import read_unfused_cases
from oracle import bf16_to_f32, combine, dispatch, expert_identity, expert_scale, f32_to_bf16_rne, layout
from synth import make_workload


def _layout_and_recv(wl):
    cfg = wl.config
    lay = layout(wl.topk_idx, cfg.E)
    recv = dispatch(wl.x, lay["dest_row"], cfg.T * cfg.k)
    return lay, recv


@pytest.mark.parametrize("name,T", [("tiny", 128), ("decode", 128), ("prefill", 512), ("train", 128)])
def test_dispatch_invariants(name, T):
    wl = make_workload(name, T=T)
    cfg = wl.config
    lay, recv = _layout_and_recv(wl)
    src = lay["src_token"]
    # every receive row is a bit copy of its source token
    np.testing.assert_array_equal(recv, wl.x[src])
    # each token appears exactly k times
    assert np.all(np.bincount(src, minlength=cfg.T) == cfg.k)
    for t in range(cfg.T):
        for j in range(cfg.k):
            assert np.array_equal(recv[lay["dest_row"][t, j]], wl.x[t])
    # segment e holds exactly the tokens routed to e, ascending
    for e in range(cfg.E):
        seg = src[lay["offsets"][e] : lay["offsets"][e + 1]]
        want = [t for t in range(cfg.T) if e in wl.topk_idx[t]]
        assert list(seg) == want


def test_dispatch_brute_force_tiny():
    for seed in range(20):
        rng = np.random.default_rng(seed)
        E, k, T, H = 5, 2, int(rng.integers(1, 12)), 8
        idx = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32)
        x = rng.integers(0, 2**16, size=(T, H), dtype=np.uint32).astype(np.uint16)
        lay = layout(idx, E)
        recv = dispatch(x, lay["dest_row"], T * k)
        rows = []
        for e in range(E):
            for t in range(T):
                if e in idx[t]:
                    rows.append(list(x[t]))
        assert recv.tolist() == rows


def test_dispatch_skips_out_of_range_destinations():
    x = np.arange(12, dtype=np.uint16).reshape(3, 4)
    recv = dispatch(x, np.array([[1], [-1], [7]]), 2)
    assert recv.tolist() == [[0, 0, 0, 0], [0, 1, 2, 3]]


@pytest.mark.parametrize("name,T", [("tiny", 128), ("decode", 128), ("prefill", 512)])
def test_identity_round_trip_is_exact(name, T):
    wl = make_workload(name, T=T)
    lay, recv = _layout_and_recv(wl)
    out = combine(expert_identity(recv), lay["dest_row"], wl.topk_w)
    # +-0 compare equal: compare as float values, and bits elsewhere
    a, b = bf16_to_f32(out), bf16_to_f32(wl.x)
    assert np.array_equal(a, b)
    nz = b != 0
    np.testing.assert_array_equal(out[nz], wl.x[nz])


def test_scale_expert_closed_form():
    wl = make_workload("train", T=96)
    cfg = wl.config
    lay, recv = _layout_and_recv(wl)
    y = expert_scale(recv, lay["offsets"], wl.scales)
    out = bf16_to_f32(combine(y, lay["dest_row"], wl.topk_w)).astype(np.float64)
    x = bf16_to_f32(wl.x).astype(np.float64)
    factor = (wl.topk_w.astype(np.float64) * wl.scales[wl.topk_idx].astype(np.float64)).sum(axis=1)
    want = x * factor[:, None]
    tol = (2.0**-7 + 1e-5) * np.abs(want)
    assert np.all(np.abs(out - want) <= tol)
    # a transposed weight matrix or a wrong expert scale would break it
    assert cfg.k != cfg.T


def test_expert_scale_uses_row_segment():
    recv = np.array([[0x3F80], [0x3F80], [0x4000]], dtype=np.uint16)  # 1, 1, 2
    y = expert_scale(recv, np.array([0, 1, 3]), np.array([0.5, 3.0], dtype=np.float32))
    assert bf16_to_f32(y).ravel().tolist() == [0.5, 3.0, 6.0]


def _gamma(n):
    u = Fraction(1, 2**24)
    return n * u / (1 - n * u)


def test_combine_exact_rational_bound():
    """fp32 accumulation stays within Higham's recursive-summation bound of
    the exact rational sum, and the final bf16 rounding adds at most a
    relative 2^-8 (plus half the smallest bf16 denormal)."""
    tiny = Fraction(1, 2**133) + Fraction(1, 2**140)
    for seed in range(30):
        rng = np.random.default_rng(1000 + seed)
        T, k, H = int(rng.integers(1, 6)), int(rng.integers(1, 9)), 8
        R = T * k
        y = rng.integers(0, 2**16, size=(R, H), dtype=np.uint32).astype(np.uint16)
        bad = ~np.isfinite(bf16_to_f32(y)) | (np.abs(bf16_to_f32(y)) > 1e30)
        y[bad] = 0x3F80
        w = rng.standard_normal((T, k)).astype(np.float32)
        dest = rng.permutation(R).reshape(T, k).astype(np.int32)
        out = combine(y, dest, w)
        yf = bf16_to_f32(y)
        for t in range(T):
            for h in range(H):
                terms = [Fraction(float(w[t, j])) * Fraction(float(yf[dest[t, j], h])) for j in range(k)]
                exact = sum(terms, Fraction(0))
                acc_err = _gamma(k) * sum(abs(x) for x in terms) + k * Fraction(1, 2**149)
                got = Fraction(float(bf16_to_f32(out[t, h])))
                round_err = Fraction(1, 2**8) * (abs(exact) + acc_err) + tiny
                assert abs(got - exact) <= acc_err + round_err, (seed, t, h)


def test_combine_order_and_tie_rounding():
    """Hand-derived: slot 0 contributes 1 + 2^-8 (exactly halfway between the
    bf16 neighbours 1 and 1 + 2^-7), slots 1..3 contribute 2^-25 each.

    In slot order the fp32 accumulator holds 1 + 2^-8, and every 2^-25 is a
    quarter of an fp32 ulp at 1, so each add rounds back down: the sum stays
    1 + 2^-8, a bf16 tie, which rounds to the even neighbour 1.0 (0x3F80).
    Summed in reverse, the three small terms first make 3 * 2^-25, then the
    add gives 1 + 2^-8 + 1.5 * 2^-24 -> 1 + 2^-8 + 2^-23 in fp32, which is
    above the tie and would round up to 0x3F81.  A fused multiply-add changes
    nothing here (all products are exact)."""
    y = np.array([[0x3F80], [0x3F80], [0x3F80], [0x3F80]], dtype=np.uint16)  # 1.0
    w = np.array([[1 + 2.0**-8, 2.0**-25, 2.0**-25, 2.0**-25]], dtype=np.float32)
    dest = np.array([[0, 1, 2, 3]], dtype=np.int32)
    out = combine(y, dest, w)
    assert out[0, 0] == 0x3F80
    # the same four terms summed small-first land above the tie
    out_rev = combine(y, dest[:, ::-1].copy(), w[:, ::-1].copy())
    assert out_rev[0, 0] == 0x3F81


def test_combine_products_rounded_separately():
    """Pins the no-fused-multiply-add reading with the hand-derived cases of
    tests/golden/combine_unfused_cases.txt.  The oracle must give the
    separately rounded value; the fused evaluation of the same terms (each
    product exact, one binary32 rounding per slot) is computed here as well
    and must give the other value, so a contracted oracle fails this test."""
    cases = read_unfused_cases()
    assert len(cases) >= 2
    for c in cases:
        y = np.array([[c["y"][0]], [c["y"][1]]], dtype=np.uint16)
        w = c["w"].reshape(1, 2)
        dest = np.array([[0, 1]], dtype=np.int32)
        assert combine(y, dest, w)[0, 0] == c["unfused"], c["name"]
        # fused: float64 holds each product (24 + 8 significant bits) and its
        # sum with the binary32 accumulator exactly; then one rounding
        yf = bf16_to_f32(y[:, 0])
        acc = np.float32(0.0)
        for j in range(2):
            s64 = np.float64(acc) + np.float64(w[0, j]) * np.float64(yf[j])
            assert Fraction(float(s64)) == Fraction(float(acc)) + Fraction(float(w[0, j])) * Fraction(float(yf[j]))
            acc = np.float32(s64)
        assert f32_to_bf16_rne(np.array([acc], dtype=np.float32))[0] == c["fused"], c["name"]
        assert c["fused"] != c["unfused"]


def test_combine_signed_zero_and_skip():
    y = np.array([[0x8000], [0x3F80]], dtype=np.uint16)  # -0.0, 1.0
    w = np.array([[0.5, 0.25]], dtype=np.float32)
    out = combine(y, np.array([[0, -1]], dtype=np.int32), w)
    assert out[0, 0] == 0x0000  # +0 + (-0) = +0; slot 1 skipped
    out = combine(y, np.array([[0, 1]], dtype=np.int32), w)
    assert out[0, 0] == 0x3E80  # 0.25


def test_combine_weights_used_as_given():
    y = np.array([[0x3F80, 0x4000]], dtype=np.uint16)  # [1, 2]
    out = combine(y, np.array([[0, 0]], dtype=np.int32), np.array([[2.0, 1.0]], dtype=np.float32))
    assert bf16_to_f32(out).tolist() == [[3.0, 6.0]]
