"""ep_layout_noalloc (the layout with the library's static device scratch
instead of a caller workspace) against ep_layout with a workspace, through
the C ABI: bit-identical outputs on calls in a row -- a large batch, then a
smaller one, then a larger one again, so each call finds the previous call's
scratch contents -- over the one-, two- and three-launch layout paths, with
valid and invalid ids, and the layouts checked against the oracle.  Then the
same layout inside a captured HIP graph, replayed on new routing."""

import numpy as np
import pytest
import torch

import bulk_async_tensor_amd as ep
import oracle
from synth import make_workload

from gpu_helpers import DEV, from_dev_bf16, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def routing(T, k, E, seed):
    """k distinct uniform experts per token."""
    rng = np.random.default_rng(seed)
    return np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)


def outputs(T, k, E, fill):
    i32 = dict(dtype=torch.int32, device=DEV)
    return {"counts": torch.full((E,), fill, **i32), "offsets": torch.full((E + 1,), fill, **i32),
            "dest_row": torch.full((T, k), fill, **i32), "src_token": torch.full((T * k,), fill, **i32),
            "status": torch.full((1,), fill, **i32)}


def check_same(idx_np, E, with_oracle=True):
    T, k = idx_np.shape
    print(f"no-alloc layout: T={T} k={k} E={E} scratch={ep.ep_layout_workspace_bytes(T, k, E)}", flush=True)
    idx = to_dev(idx_np)
    ws = torch.empty(max(16, ep.ep_layout_workspace_bytes(T, k, E)), dtype=torch.uint8, device=DEV)
    a = outputs(T, k, E, -7)
    b = outputs(T, k, E, -9)
    ep.ep_layout(idx, E, workspace=ws, **a)
    ep.ep_layout_noalloc(idx, E, **b)
    torch.cuda.synchronize()
    got = {key: v.cpu().numpy() for key, v in b.items()}
    ref = {key: v.cpu().numpy() for key, v in a.items()}
    n = int(ref["offsets"][-1])
    for key in ("counts", "offsets", "dest_row", "status"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    np.testing.assert_array_equal(got["src_token"][:n], ref["src_token"][:n])
    if with_oracle:
        lay = oracle.layout(idx_np, E)
        np.testing.assert_array_equal(got["counts"], lay["counts"])
        np.testing.assert_array_equal(got["offsets"], lay["offsets"])
        np.testing.assert_array_equal(got["dest_row"], lay["dest_row"])
        np.testing.assert_array_equal(got["src_token"][:n], lay["src_token"][:n])
        assert int(got["status"][0]) == lay["status"]


def test_noalloc_calls_in_a_row_shrinking_then_growing():
    wl = make_workload("prefill")
    # two launches (count table in the scratch): the prefill shape, 24.8 KB of scratch
    check_same(wl.topk_idx, wl.config.E)
    # a smaller two-launch batch right after, on the larger call's scratch contents
    check_same(routing(3000, 2, 3, 1), 3)
    # three launches: 1094 chunks x 256 experts, 1.1 MB of scratch
    check_same(routing(140000, 8, 256, 2), 256, with_oracle=False)
    # one launch, no scratch (decode shape)
    wd = make_workload("decode")
    check_same(wd.topk_idx, wd.config.E)
    # two launches again, with out-of-range and repeated ids setting status bits
    bad = routing(5000, 4, 40, 3)
    bad[7, 1] = 40
    bad[11, 2] = -3
    bad[13, 3] = bad[13, 0]
    check_same(bad, 40)


def test_noalloc_rejects_a_batch_beyond_its_scratch():
    T, k, E = 40000, 32, 1024
    assert ep.ep_layout_workspace_bytes(T, k, E) > ep.EP_LAYOUT_NOALLOC_MAX_SCRATCH
    idx = torch.zeros((T, k), dtype=torch.int32, device=DEV)
    out = outputs(T, k, E, 0)
    with pytest.raises(ep.EpError) as exc:
        ep.ep_layout_noalloc(idx, E, **out)
    assert exc.value.code == ep.EP_ERR_WORKSPACE


def test_noalloc_layout_in_a_captured_graph():
    """ep_layout_noalloc, ep_dispatch and ep_combine captured in one HIP graph,
    the use the no-allocation layout exists for.  Before each replay new
    routing is written into the captured id buffer and another batch's
    no-allocation layout runs eagerly, so the scratch holds that batch's
    table; every replay still equals the oracle."""
    wl = make_workload("prefill", seed=21, T=3000)
    c = wl.config
    assert ep.ep_layout_workspace_bytes(c.T, c.k, c.E) > 0  # the layout path that uses the scratch
    print(f"graph no-alloc step: T={c.T} k={c.k} E={c.E} H={c.H}", flush=True)
    idx = to_dev(wl.topk_idx)
    x = to_dev_bf16(wl.x)
    w = to_dev(wl.topk_w)
    R = c.T * c.k
    lay = outputs(c.T, c.k, c.E, -7)
    recv = torch.empty((R, c.H), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((c.T, c.H), dtype=torch.bfloat16, device=DEV)

    def step():
        ep.ep_layout_noalloc(idx, c.E, **lay)
        ep.ep_dispatch(x, lay["dest_row"], recv)
        ep.ep_combine(recv, lay["dest_row"], w, out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other_idx = to_dev(routing(5000, 4, 40, 9))
    other_out = outputs(5000, 4, 40, 0)
    for rep in range(4):
        routing_np = make_workload("prefill", seed=100 + rep, T=c.T).topk_idx
        idx.copy_(to_dev(routing_np))
        ep.ep_layout_noalloc(other_idx, 40, **other_out)
        recv.view(torch.int16).fill_(rep)
        out.view(torch.int16).fill_(rep)
        lay["dest_row"].fill_(-7)
        lay["src_token"].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle.layout(routing_np, c.E)
        got = {key: v.cpu().numpy() for key, v in lay.items()}
        for key in ("counts", "offsets", "dest_row"):
            np.testing.assert_array_equal(got[key], ref[key], err_msg=f"replay {rep}: {key}")
        np.testing.assert_array_equal(got["src_token"], ref["src_token"])
        assert int(got["status"][0]) == ref["status"] == 0
        np.testing.assert_array_equal(from_dev_bf16(recv), oracle.dispatch(wl.x, ref["dest_row"], R))
        # identity experts and weights summing to one: the round trip is exact
        assert np.array_equal(oracle.bf16_to_f32(from_dev_bf16(out)), oracle.bf16_to_f32(wl.x))
