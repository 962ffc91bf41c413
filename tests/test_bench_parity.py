"""The benchmark's same-run parity check (bench.parity_against), on the CPU:
it must call matching outputs bit-exact and catch a planted difference in each
of layout, dispatch and combine.  The 'GPU outputs' here are CPU tensors
holding the oracle's own results, then copies with one planted mistake."""

import types

import numpy as np
import torch

import bench
import oracle
from synth import make_workload


def fake_setup(lay, recv, out):
    s = types.SimpleNamespace(torch=torch)
    s.counts = torch.from_numpy(lay["counts"].copy())
    s.offsets = torch.from_numpy(lay["offsets"].copy())
    s.dest_row = torch.from_numpy(lay["dest_row"].copy())
    s.src_token = torch.from_numpy(lay["src_token"].copy())
    s.recv = torch.from_numpy(recv.copy().view(np.int16)).view(torch.bfloat16)
    s.out = torch.from_numpy(out.copy().view(np.int16)).view(torch.bfloat16)
    return s


def test_parity_check_passes_and_catches_planted_mistakes():
    wl = make_workload("tiny")
    c = wl.config
    lay = oracle.layout(wl.topk_idx, c.E)
    recv = oracle.dispatch(wl.x, lay["dest_row"], c.T * c.k)
    out = oracle.combine(recv, lay["dest_row"], wl.topk_w)

    ok = bench.parity_against(fake_setup(lay, recv, out), lay, recv, out)
    assert ok == {"layout_bit_exact": True, "dispatch_bit_exact": True,
                  "combine_bit_identical_frac": 1.0, "combine_within_gate": True, "combine_norm_rel_err": 0.0}

    s = fake_setup(lay, recv, out)
    s.dest_row.view(-1)[5] += 1
    assert bench.parity_against(s, lay, recv, out)["layout_bit_exact"] is False

    s = fake_setup(lay, recv, out)
    s.recv.view(torch.int16)[3, 7] ^= 1
    assert bench.parity_against(s, lay, recv, out)["dispatch_bit_exact"] is False

    # one bf16 ulp on one element: not bit-identical, still within the gate
    s = fake_setup(lay, recv, out)
    s.out.view(torch.int16)[0, 0] += 1
    res = bench.parity_against(s, lay, recv, out)
    assert res["combine_bit_identical_frac"] < 1.0 and res["combine_within_gate"] is True
    assert 0.0 < res["combine_norm_rel_err"] < 1e-2

    # a sign flip on a sizeable element: outside the gate
    s = fake_setup(lay, recv, out)
    r = np.abs(oracle.bf16_to_f32(out)).argmax()
    s.out.view(torch.int16).view(-1)[r] ^= np.int16(-0x8000)
    assert bench.parity_against(s, lay, recv, out)["combine_within_gate"] is False

    # the combine-only workload has no dispatch entry
    assert "dispatch_bit_exact" not in bench.parity_against(fake_setup(lay, recv, out), lay, None, out)
