"""GPU parity of the reduce-on-store combine (ep_combine_reduce) through the C ABI.

The k atomic additions into an accumulator element happen in no fixed order,
so the result is not compared bit for bit with the oracle's slot-order sum.
Instead every output element is checked against

  * the combine gate: abs(g - r) <= 1e-2 * abs(r) + 1e-3 against the oracle;
  * a rigorous, order-independent bound: with s the exact sum of the k
    products (fp64, exact for bf16 x fp32 terms up to 2^-53) and A the sum
    of their magnitudes, any fp32 evaluation S (each product rounded, then
    k - 1 additions in any order) satisfies abs(S - s) <= gamma_k * A, with
    gamma_n = n u / (1 - n u) and u = 2^-24 (Higham, "Accuracy and Stability
    of Numerical Algorithms", ch. 4, recursive summation); the final bf16
    round-to-nearest-even adds at most 2^-8 abs(S);
  * where the expert is the identity and each token's weights sum to 1, the
    closed form combine(dispatch(x)) == x exactly (S = x (1 + theta) with
    abs(theta) far below half a bf16 ulp, whatever the order).
"""

import numpy as np
import pytest
import torch

import bulk_async_tensor_amd as ep
import oracle
from synth import CONFIGS, make_workload

from gpu_helpers import (
    DEV,
    assert_combine_close,
    expert_outputs,
    from_dev_bf16,
    oracle_layout,
    oracle_out,
    to_dev,
    to_dev_bf16,
    workload,
)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _reset_settings():
    ep.ep_set_num_cus(0)
    ep.ep_set_variant("auto")
    yield
    ep.ep_set_num_cus(0)


def run_reduce(y_u16, src_token, dest_row, w, T, H, workspace=None):
    out = torch.full((T, H), 0x7E57, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    ep.ep_combine_reduce(to_dev_bf16(y_u16.reshape(-1, H)), to_dev(src_token.astype(np.int32)),
                         to_dev(dest_row.astype(np.int32)), to_dev(w.astype(np.float32)), out, workspace=workspace)
    torch.cuda.synchronize()
    return from_dev_bf16(out)


def assert_within_sum_bound(got_u16, y_u16, dest_row, w):
    """abs(g - s) <= 2^-8 (abs(s) + gamma_k A) + gamma_k A for every element."""
    T, k = dest_row.shape
    R = y_u16.shape[0]
    yf = oracle.bf16_to_f32(y_u16).astype(np.float64)
    s = np.zeros((T, y_u16.shape[1]), dtype=np.float64)
    a = np.zeros_like(s)
    for j in range(k):
        d = dest_row[:, j].astype(np.int64)
        ok = (d >= 0) & (d < R)
        term = np.where(ok[:, None], w[:, j].astype(np.float64)[:, None] * yf[np.where(ok, d, 0)], 0.0)
        s += term
        a += np.abs(term)
    u = 2.0**-24
    gamma = k * u / (1 - k * u)
    g = oracle.bf16_to_f32(got_u16).astype(np.float64)
    bound = 2.0**-8 * (np.abs(s) + gamma * a) + gamma * a
    bad = ~(np.abs(g - s) <= bound)
    assert not bad.any(), f"{int(bad.sum())} elements outside the summation bound, first at {np.argwhere(bad)[0]}"


@pytest.mark.parametrize("name", list(CONFIGS))
def test_reduce_full_size(name):
    wl = workload(name)
    cfg = wl.config
    lay = oracle_layout(name)
    y = expert_outputs(name)
    got = run_reduce(y, lay["src_token"], lay["dest_row"], wl.topk_w, cfg.T, cfg.H)
    assert_combine_close(got, oracle_out(name), exact=False)
    assert_within_sum_bound(got, y, lay["dest_row"], wl.topk_w)
    if cfg.expert == "identity":
        assert np.array_equal(oracle.bf16_to_f32(got), oracle.bf16_to_f32(wl.x))


@pytest.mark.parametrize("name", ["train", "combine_stress"])
@pytest.mark.parametrize("budget", [16, 24, 64, 256])
def test_reduce_budgets(name, budget):
    ep.ep_set_num_cus(budget)
    wl = workload(name)
    lay = oracle_layout(name)
    y = expert_outputs(name)
    got = run_reduce(y, lay["src_token"], lay["dest_row"], wl.topk_w, wl.config.T, wl.config.H)
    assert_combine_close(got, oracle_out(name), exact=False)
    assert_within_sum_bound(got, y, lay["dest_row"], wl.topk_w)


# Ragged rows (H not a multiple of 512 elements, H = 8 a single vector), any k
# (k = 11 takes the kernel with k known only at run time), and a slot removed
# from a token's routing: its receive row still names the token in
# src_token, but the token no longer lists it, so it adds nothing.
@pytest.mark.parametrize("H", [8, 520, 4104, 7176])
@pytest.mark.parametrize("k", [1, 3, 6, 8, 11])
@pytest.mark.parametrize("budget", [0, 24])
def test_reduce_ragged_rows(H, k, budget):
    ep.ep_set_num_cus(budget)
    T = 29
    wl = make_workload("combine_stress", seed=H + k, T=T, H=H, E=32, k=k)
    lay = oracle.layout(wl.topk_idx, 32)
    dest = lay["dest_row"].copy()
    dest[3, 0] = -1
    got = run_reduce(wl.y, lay["src_token"], dest, wl.topk_w, T, H)
    assert_combine_close(got, oracle.combine(wl.y, dest, wl.topk_w), exact=False)
    assert_within_sum_bound(got, wl.y, dest, wl.topk_w)


def test_reduce_identity_round_trip_ragged():
    # identity expert, weights summing to 1: exact whatever the order
    T, H, k = 300, 7176, 6
    wl = make_workload("prefill", seed=7, T=T, H=H, E=16, k=k)
    lay = oracle.layout(wl.topk_idx, 16)
    recv = oracle.dispatch(wl.x, lay["dest_row"], T * k)
    got = run_reduce(recv, lay["src_token"], lay["dest_row"], wl.topk_w, T, H)
    assert np.array_equal(oracle.bf16_to_f32(got), oracle.bf16_to_f32(wl.x))


def test_reduce_stale_src_token_entries_add_nothing():
    # out-of-range ids: ep_layout leaves src_token beyond offsets[E] unwritten
    # and gives those entries dest_row -1; the rows past offsets[E] hold junk
    T, H, k, E = 64, 1024, 4, 16
    wl = make_workload("combine_stress", seed=11, T=T, H=H, E=E, k=k)
    idx = wl.topk_idx.copy()
    idx[5, 1] = E + 3
    idx[40, 3] = -2
    lay = oracle.layout(idx, E)
    n = int(lay["offsets"][-1])
    assert n == T * k - 2
    src = lay["src_token"].copy()
    src[n:] = [5, 40]  # tokens that exist but do not list these rows
    y = wl.y.copy()
    y[n:] = 0x7F80  # +inf: any use would show
    got = run_reduce(y, src, lay["dest_row"], wl.topk_w, T, H)
    ref = oracle.combine(y, lay["dest_row"], wl.topk_w)
    assert_combine_close(got, ref, exact=False)
    src[n:] = [T + 7, -1]  # tokens outside [0, T)
    got = run_reduce(y, src, lay["dest_row"], wl.topk_w, T, H)
    assert_combine_close(got, ref, exact=False)


def test_reduce_clears_a_dirty_workspace_every_call():
    T, H, k = 128, 1024, 2
    wl = workload("tiny")
    lay = oracle_layout("tiny")
    y = expert_outputs("tiny")
    ws = torch.full((ep.ep_combine_reduce_workspace_bytes(T, H) // 4,), float("nan"), dtype=torch.float32,
                    device=DEV)
    ref = wl.x
    for _ in range(3):
        got = run_reduce(y, lay["src_token"], lay["dest_row"], wl.topk_w, T, H, workspace=ws.view(torch.uint8))
        assert np.array_equal(oracle.bf16_to_f32(got), oracle.bf16_to_f32(ref))
    assert k == wl.config.k


def test_reduce_empty_receive_buffer_gives_zeros():
    T, H, k = 5, 1024, 2
    out = torch.full((T, H), 0x7E57, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    y = torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
    src = torch.empty((0,), dtype=torch.int32, device=DEV)
    dest = torch.full((T, k), -1, dtype=torch.int32, device=DEV)
    w = torch.ones((T, k), dtype=torch.float32, device=DEV)
    ep.ep_combine_reduce(y, src, dest, w, out)
    torch.cuda.synchronize()
    assert not from_dev_bf16(out).any()


def test_reduce_unnormalised_weights_and_signed_zero():
    wl = make_workload("tiny", T=16)
    lay = oracle.layout(wl.topk_idx, 8)
    recv = oracle.dispatch(wl.x, lay["dest_row"], 32)
    recv[:4] = 0x8000  # -0.0 rows
    w = (wl.topk_w * np.float32(3.5)).astype(np.float32)
    got = run_reduce(recv, lay["src_token"], lay["dest_row"], w, 16, 1024)
    assert_combine_close(got, oracle.combine(recv, lay["dest_row"], w), exact=False)
    assert_within_sum_bound(got, recv, lay["dest_row"], w)


@pytest.mark.parametrize("name", ["tiny", "prefill"])
def test_reduce_graph_replay(name):
    """The reduce-on-store combine captured in a HIP graph (its accumulator is
    cleared by a fill kernel, not a memset node): every replay, with the
    accumulator and the output clobbered eagerly in between, gives the exact
    identity round trip."""
    wl = workload(name)
    c = wl.config
    lay = oracle_layout(name)
    y = to_dev_bf16(expert_outputs(name))
    src = to_dev(lay["src_token"])
    dest = to_dev(lay["dest_row"])
    w = to_dev(wl.topk_w)
    out = torch.empty((c.T, c.H), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(ep.ep_combine_reduce_workspace_bytes(c.T, c.H), dtype=torch.uint8, device=DEV)

    def call():
        ep.ep_combine_reduce(y, src, dest, w, out, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    want = oracle.bf16_to_f32(wl.x)
    for rep in range(4):
        out.view(torch.int16).fill_(rep)
        ws.view(torch.float32).fill_(float(rep + 1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(oracle.bf16_to_f32(from_dev_bf16(out)), want), f"replay {rep}"
