"""Shared helpers of the GPU tests: host<->device bf16 transfers, cached oracle
results per workload, and the combine tolerance."""

import functools

import numpy as np
import torch

import oracle
from synth import make_workload

DEV = torch.device("cuda:0")


def to_dev_bf16(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).to(DEV).view(torch.bfloat16)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def from_dev_bf16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@functools.lru_cache(maxsize=4)
def workload(name, **overrides):
    return make_workload(name, **overrides)


@functools.lru_cache(maxsize=4)
def oracle_layout(name, **overrides):
    wl = workload(name, **overrides)
    return oracle.layout(wl.topk_idx, wl.config.E)


@functools.lru_cache(maxsize=2)
def oracle_recv(name, **overrides):
    wl = workload(name, **overrides)
    lay = oracle_layout(name, **overrides)
    return oracle.dispatch(wl.x, lay["dest_row"], wl.config.T * wl.config.k)


@functools.lru_cache(maxsize=2)
def expert_outputs(name, **overrides):
    """y of the workload's expert op, computed by the oracle from its own recv."""
    wl = workload(name, **overrides)
    if wl.config.expert == "random_y":
        return wl.y
    lay = oracle_layout(name, **overrides)
    recv = oracle_recv(name, **overrides)
    if wl.config.expert == "scale":
        return oracle.expert_scale(recv, lay["offsets"], wl.scales)
    return oracle.expert_identity(recv)


@functools.lru_cache(maxsize=2)
def oracle_out(name, **overrides):
    wl = workload(name, **overrides)
    lay = oracle_layout(name, **overrides)
    return oracle.combine(expert_outputs(name, **overrides), lay["dest_row"], wl.topk_w)


def assert_combine_close(got_u16, ref_u16, exact=True):
    """abs(g - r) <= 1e-2 * abs(r) + 1e-3 element-wise (the combine gate), and,
    when ``exact``, bit equality up to the sign of zero (no fused multiply-add
    and the same slot order on both sides make the results identical)."""
    g = oracle.bf16_to_f32(got_u16).astype(np.float64)
    r = oracle.bf16_to_f32(ref_u16).astype(np.float64)
    bad = ~(np.abs(g - r) <= 1e-2 * np.abs(r) + 1e-3)
    assert not bad.any(), f"{int(bad.sum())} elements outside tolerance, first at {np.argwhere(bad)[0]}"
    if exact:
        diff = g != r
        assert not diff.any(), f"{int(diff.sum())} of {g.size} elements not bit-exact"
