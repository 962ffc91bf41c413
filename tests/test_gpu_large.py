"""Maximum-size cases: a receive buffer beyond 4 GiB (T = 40000 tokens, H =
7168, k = 8: 320,000 rows of 14 KiB = 4.59 GB), so that row offsets and byte
addresses pass 2^31 and 2^32.

The layout is compared with the oracle in full (bit-exact).  Dispatch is
compared on sampled receive rows, among them the first and the last rows of
the buffer, each against its source row x[src_token[r]].  The combine output
is checked at every token through a property that holds at any size: with
the identity expert and weights summing to 1, combine(dispatch(x)) == x
exactly (see the oracle's closed-form pin)."""

import numpy as np
import pytest
import torch

import bulk_async_tensor_amd as ep
import oracle
from synth import make_workload

from gpu_helpers import DEV, from_dev_bf16, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

T, H, E, K = 40000, 7168, 256, 8


@pytest.fixture(scope="module")
def big():
    wl = make_workload("train", seed=40, T=T, H=H, E=E, k=K)
    lay_ref = oracle.layout(wl.topk_idx, E)
    idx = to_dev(wl.topk_idx)
    lay = ep.ep_layout(idx, E)
    x = to_dev_bf16(wl.x)
    R = T * K
    recv = torch.empty((R, H), dtype=torch.bfloat16, device=DEV)
    assert recv.numel() * 2 > 2**32
    ep.ep_dispatch(x, lay["dest_row"], recv)
    torch.cuda.synchronize()
    yield wl, lay_ref, lay, x, recv
    del recv
    torch.cuda.empty_cache()


def test_layout_beyond_4gib(big):
    wl, ref, lay, _, _ = big
    np.testing.assert_array_equal(lay["counts"].cpu().numpy(), ref["counts"])
    np.testing.assert_array_equal(lay["offsets"].cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(lay["dest_row"].cpu().numpy(), ref["dest_row"])
    np.testing.assert_array_equal(lay["src_token"].cpu().numpy(), ref["src_token"])
    assert int(lay["status"].item()) == 0


def test_dispatch_rows_beyond_4gib(big):
    wl, ref, _, _, recv = big
    R = T * K
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(R - 256, R), rng.integers(0, R, 2048)]))
    got = from_dev_bf16(recv[torch.from_numpy(rows).to(DEV)])
    want = wl.x[ref["src_token"][rows]]
    np.testing.assert_array_equal(got, want)
    # the last rows lie past 2^32 bytes
    assert (R - 1) * H * 2 > 2**32


@pytest.mark.parametrize("entry", ["ep_combine", "ep_combine_reduce"])
def test_combine_round_trip_beyond_4gib(big, entry):
    wl, ref, lay, x, recv = big
    w = to_dev(wl.topk_w)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    if entry == "ep_combine":
        ep.ep_combine(recv, lay["dest_row"], w, out)
    else:
        ep.ep_combine_reduce(recv, lay["src_token"], lay["dest_row"], w, out)
    torch.cuda.synchronize()
    assert torch.equal(out.float(), x.float())
