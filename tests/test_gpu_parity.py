"""GPU parity through the C ABI against the CPU oracle.

Layout and dispatch must be bit-exact; combine must be within
abs(g - r) <= 1e-2 * abs(r) + 1e-3 and is, in addition, expected bit-exact
(same slot order, no fused multiply-add, one RNE rounding on both sides).
Every workload shape runs at full size; smaller cases cover ragged chunk and
row tails, empty and degenerate routing, and every kernel variant at several
compute-unit budgets (the budgets of the benchmark among them).
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
    oracle_recv,
    to_dev,
    to_dev_bf16,
    workload,
)

pytestmark = pytest.mark.gpu

DISPATCH_CONFIGS = [n for n, c in CONFIGS.items() if c.ops != "combine"]
BUDGETS = [0, 16, 24, 32, 64, 256]


@pytest.fixture(autouse=True)
def _reset_settings():
    ep.ep_set_num_cus(0)
    ep.ep_set_variant("auto")
    ep.ep_set_slab(0)
    yield
    ep.ep_set_num_cus(0)
    ep.ep_set_variant("auto")
    ep.ep_set_slab(0)


def gpu_layout(wl):
    lay = ep.ep_layout(to_dev(wl.topk_idx), wl.config.E)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in lay.items()}


def check_layout(got, ref, T, k):
    np.testing.assert_array_equal(got["counts"], ref["counts"])
    np.testing.assert_array_equal(got["offsets"], ref["offsets"])
    np.testing.assert_array_equal(got["dest_row"].reshape(T, k), ref["dest_row"])
    n = int(ref["offsets"][-1])
    np.testing.assert_array_equal(got["src_token"][:n], ref["src_token"][:n])
    assert int(got["status"][0]) == ref["status"]


# ----------------------------------------------------------------- layout
@pytest.mark.parametrize("name", list(CONFIGS))
def test_layout_full_size(name):
    wl = workload(name)
    check_layout(gpu_layout(wl), oracle_layout(name), wl.config.T, wl.config.k)


@pytest.mark.parametrize(
    "T,E,k",
    [
        # one launch: at most four 1024-entry chunks, or up to 64 with E > 64 and T <= 12288
        (1, 1, 1), (1, 8, 8), (7, 5, 3), (171, 64, 6), (512, 256, 8), (128, 1024, 32), (513, 256, 8),
        (129, 1024, 32), (5000, 1024, 1), (8192, 256, 8), (12288, 128, 4),
        # two launches (count, then scan and rank): E <= 64 past four chunks, more than 64 chunks,
        # or more than 12288 tokens
        (513, 64, 8), (1000, 64, 6), (3000, 3, 2), (16384, 64, 1), (2047, 7, 7), (8193, 256, 8), (1024, 1024, 32),
        (12289, 256, 4), (20000, 128, 2),
        # three launches: a (chunk, expert) table too large to read in every workgroup (past 48 Ki counts)
        (140000, 256, 8), (20001, 1024, 7), (14000, 512, 8), (65536, 1024, 2),
    ],
)
def test_layout_ragged_and_extreme(T, E, k):
    wl = make_workload("prefill", seed=T * 31 + E, T=T, E=E, k=k)
    check_layout(gpu_layout(wl), oracle.layout(wl.topk_idx, E), T, k)


def test_layout_empty_batch():
    lay = ep.ep_layout(torch.zeros((0, 4), dtype=torch.int32, device=DEV), 16)
    torch.cuda.synchronize()
    assert lay["counts"].cpu().tolist() == [0] * 16
    assert lay["offsets"].cpu().tolist() == [0] * 17
    assert int(lay["status"].item()) == 0


def test_layout_flags_bad_ids():
    rng = np.random.default_rng(5)
    idx = np.array([rng.permutation(16)[:4] for _ in range(600)], dtype=np.int32)
    idx[3, 1] = 16
    idx[77, 0] = -2
    idx[500, 2] = 1 << 30
    idx[10, 3] = idx[10, 0]
    for T, want in [(600, 3), (3, 0)]:
        sub = np.ascontiguousarray(idx[:T])
        ref = oracle.layout(sub, 16)
        assert ref["status"] == want
        lay = ep.ep_layout(to_dev(sub), 16)
        torch.cuda.synchronize()
        got = {k: v.cpu().numpy() for k, v in lay.items()}
        check_layout(got, ref, T, 4)


# Odd k through the one-launch layout (a few chunks at any E, up to 64 with
# E > 64) and past it into the two launches, with a repeated expert, an id
# out of range and a negative id.
@pytest.mark.parametrize("k", [3, 5, 7])
@pytest.mark.parametrize("T,E", [(128, 64), (700, 64), (2048, 256), (9400, 256), (5000, 32)])
def test_layout_odd_k(k, T, E):
    wl = make_workload("train", seed=T + E + k, T=T, E=E, k=k, H=8)
    idx = wl.topk_idx.copy()
    idx[1, 1] = idx[1, 0]
    idx[T // 2, 0] = E
    idx[T - 1, k - 1] = -1
    ref = oracle.layout(idx, E)
    assert ref["status"] == 3
    lay = ep.ep_layout(to_dev(idx), E)
    torch.cuda.synchronize()
    check_layout({key: v.cpu().numpy() for key, v in lay.items()}, ref, T, k)


def test_layout_is_deterministic():
    wl = workload("train")
    a = gpu_layout(wl)
    b = gpu_layout(wl)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


# ----------------------------------------------------------------- dispatch
def run_dispatch(wl, dest_row_np, recv_rows, fill=0x7E57):
    x = to_dev_bf16(wl.x)
    recv = torch.full((recv_rows, wl.config.H), fill, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    ep.ep_dispatch(x, to_dev(dest_row_np), recv)
    torch.cuda.synchronize()
    return from_dev_bf16(recv)


@pytest.mark.parametrize("name", DISPATCH_CONFIGS)
def test_dispatch_full_size(name):
    wl = workload(name)
    lay = oracle_layout(name)
    got = run_dispatch(wl, lay["dest_row"], wl.config.T * wl.config.k)
    np.testing.assert_array_equal(got, oracle_recv(name))


@pytest.mark.parametrize("variant", ["vgpr", "vgpr2", "lds1", "lds2", "lds3", "pc", "vgpr_cached", "phase", "vgpr_wg"])
@pytest.mark.parametrize("budget", BUDGETS)
def test_dispatch_variants_train(variant, budget):
    ep.ep_set_variant(variant)
    ep.ep_set_num_cus(budget)
    wl = workload("train")
    got = run_dispatch(wl, oracle_layout("train")["dest_row"], wl.config.T * wl.config.k)
    np.testing.assert_array_equal(got, oracle_recv("train"))


@pytest.mark.parametrize("variant", ["vgpr", "vgpr2", "lds1", "lds2", "lds3", "pc", "phase", "vgpr_wg"])
@pytest.mark.parametrize("H", [8, 520, 1024, 4104, 7168, 7176, 8712, 16384])
@pytest.mark.parametrize("k", [2, 3, 4, 6])
@pytest.mark.parametrize("budget", [0, 24])
def test_dispatch_ragged_rows(variant, H, k, budget):
    ep.ep_set_variant(variant)
    ep.ep_set_num_cus(budget)
    T = 37
    wl = make_workload("prefill", seed=H + k, T=T, H=H, E=16, k=k)
    lay = oracle.layout(wl.topk_idx, 16)
    got = run_dispatch(wl, lay["dest_row"], T * k)
    np.testing.assert_array_equal(got, oracle.dispatch(wl.x, lay["dest_row"], T * k))


@pytest.mark.parametrize("variant", ["vgpr", "vgpr2", "lds1", "lds2", "lds3", "pc", "vgpr_wg"])
@pytest.mark.parametrize("slab", [1, 2, 4, 7, 8, 14, 16])
@pytest.mark.parametrize("budget", [0, 24])
def test_dispatch_slab_sizes(variant, slab, budget):
    ep.ep_set_variant(variant)
    ep.ep_set_slab(slab)
    ep.ep_set_num_cus(budget)
    try:
        wl = workload("train")
        got = run_dispatch(wl, oracle_layout("train")["dest_row"], wl.config.T * wl.config.k)
        np.testing.assert_array_equal(got, oracle_recv("train"))
        wr = make_workload("prefill", seed=slab, T=53, H=7176, E=16, k=6)
        lay = oracle.layout(wr.topk_idx, 16)
        got = run_dispatch(wr, lay["dest_row"], 53 * 6)
        np.testing.assert_array_equal(got, oracle.dispatch(wr.x, lay["dest_row"], 53 * 6))
    finally:
        ep.ep_set_slab(0)


# The phased dispatch's unit shapes (as for the phased combine), including a
# duplicated destination row (-1: dropped) and several units per wave.
@pytest.mark.parametrize("H", [8, 2048, 4104, 7168, 8712, 16384])
@pytest.mark.parametrize("T", [1, 29, 300])
@pytest.mark.parametrize("budget", [0, 1, 24])
def test_dispatch_phase_units(H, T, budget):
    ep.ep_set_variant("phase")
    ep.ep_set_num_cus(budget)
    k = 8 if H % 3 else 6
    wl = make_workload("prefill", seed=H + T, T=T, H=H, E=32, k=k)
    lay = oracle.layout(wl.topk_idx, 32)
    dest = lay["dest_row"].copy()
    dest[T // 2, k - 1] = -1  # a slot whose row is never written
    got = run_dispatch(wl, dest, T * k)  # receive buffer pre-filled with 0x7E57
    want = oracle.dispatch(wl.x, dest, T * k, recv=np.full((T * k, H), 0x7E57, dtype=np.uint16))
    np.testing.assert_array_equal(got, want)


# The workgroup-phased dispatch: several trips per wave with a ragged last
# trip (waves past the last unit still meet every barrier), workgroups with
# no unit at all, a dropped slot and a row outside the receive buffer.
@pytest.mark.parametrize("T,H,k", [(1, 7168, 8), (333, 7168, 6), (1000, 520, 3), (257, 8712, 8), (64, 8, 2)])
@pytest.mark.parametrize("budget", [0, 1, 3, 24, 256])
def test_dispatch_vgpr_wg_trips(T, H, k, budget):
    ep.ep_set_variant("vgpr_wg")
    ep.ep_set_num_cus(budget)
    wl = make_workload("prefill", seed=T + H + k, T=T, H=H, E=16, k=k)
    lay = oracle.layout(wl.topk_idx, 16)
    dest = lay["dest_row"].copy()
    dest[T // 2, k - 1] = -1
    dest[T - 1, 0] = 1 << 30
    got = run_dispatch(wl, dest, T * k)  # receive buffer pre-filled with 0x7E57
    want = oracle.dispatch(wl.x, dest, T * k, recv=np.full((T * k, H), 0x7E57, dtype=np.uint16))
    np.testing.assert_array_equal(got, want)


# On at least half the device the workgroup-phased dispatch issues one
# launch per trip (each launch offsets x and dest_row by the tokens before
# it): several launches with a ragged last one, a dropped slot and a row
# outside the receive buffer.
@pytest.mark.parametrize("T,k,budget", [(5000, 6, 128), (9000, 8, 0), (4097, 6, 256), (12345, 2, 192)])
def test_dispatch_vgpr_wg_launch_per_trip(T, k, budget):
    ep.ep_set_num_cus(budget)
    H = 7168
    wl = make_workload("prefill", seed=T + k, T=T, H=H, E=64, k=k)
    lay = oracle.layout(wl.topk_idx, 64)
    dest = lay["dest_row"].copy()
    dest[T // 3, k - 1] = -1
    dest[T - 1, 0] = 1 << 30
    got = run_dispatch(wl, dest, T * k)  # receive buffer pre-filled with 0x7E57
    want = oracle.dispatch(wl.x, dest, T * k, recv=np.full((T * k, H), 0x7E57, dtype=np.uint16))
    np.testing.assert_array_equal(got, want)


# Whole-row instances of the workgroup-phased dispatch for rows of 2 .. 16
# KiB other than 7 and 14 (H = 1024 .. 8192): the kernel's vectors per lane
# are the row's own, not the slab size the other kernels take.  k runs
# through 1 .. 8 with the row size (every k has its own instance).
@pytest.mark.parametrize("H", [1024, 2048, 3072, 4096, 5120, 6144, 8192])
@pytest.mark.parametrize("T,budget", [(300, 0), (300, 24), (2600, 256)])
def test_dispatch_vgpr_wg_row_sizes(H, T, budget):
    ep.ep_set_variant("vgpr_wg")
    ep.ep_set_num_cus(budget)
    k = (H // 1024) % 8 + 1
    wl = make_workload("prefill", seed=T + H, T=T, H=H, E=32, k=k)
    lay = oracle.layout(wl.topk_idx, 32)
    dest = lay["dest_row"].copy()
    dest[T // 2, k - 1] = -1
    dest[T - 1, 0] = 1 << 30
    got = run_dispatch(wl, dest, T * k)  # receive buffer pre-filled with 0x7E57
    want = oracle.dispatch(wl.x, dest, T * k, recv=np.full((T * k, H), 0x7E57, dtype=np.uint16))
    np.testing.assert_array_equal(got, want)


# Rows that are not a whole number of KiB (H a multiple of 8 but not of
# 512): the whole-row kernel loads its last KiB's tail lanes from the row's
# last vector and stores only the lanes inside the row.  The tails cover one
# vector (H = 520, 7176), most of a KiB (H = 1000, 8184) and sizes between,
# with rows of 1 .. 16 vectors per lane.
@pytest.mark.parametrize("H,k", [(8, 3), (200, 8), (520, 1), (1000, 5), (2880, 8), (5000, 2), (7176, 7), (8184, 4)])
@pytest.mark.parametrize("T,budget", [(300, 0), (300, 24), (2600, 256)])
def test_dispatch_vgpr_wg_ragged_rows(H, k, T, budget):
    ep.ep_set_variant("vgpr_wg")
    ep.ep_set_num_cus(budget)
    wl = make_workload("prefill", seed=3 * T + H + k, T=T, H=H, E=32, k=k)
    lay = oracle.layout(wl.topk_idx, 32)
    dest = lay["dest_row"].copy()
    dest[T // 2, k - 1] = -1
    dest[T - 1, 0] = 1 << 30
    got = run_dispatch(wl, dest, T * k)  # receive buffer pre-filled with 0x7E57
    want = oracle.dispatch(wl.x, dest, T * k, recv=np.full((T * k, H), 0x7E57, dtype=np.uint16))
    np.testing.assert_array_equal(got, want)


# The default dispatch on every CU around its batch-size thresholds: lds1
# below 2 tokens per CU (4 for rows of at most 8 KiB), vgpr2 on the ordinary
# grid up to 8 tokens per CU, the workgroup-phased kernel from there (the
# thresholds scale with the device's CU count; these sizes bracket them on
# a 256-CU device).  Rows of 8 to 16 KiB with a partial last KiB at k = 6
# or 8 take the workgroup-phased kernel on the ordinary grid in vgpr2's
# range (H = 4104, 5000, 7176, 8184); at k = 7 they keep vgpr2.  lds1 under
# the default stays on the ordinary grid also where its slabs are many
# (H = 5000 and 9000: 2 and 1 KiB slabs; H = 32768: 8 slabs per row).
# Rows of more than 16 vectors per lane that no slab size divides take
# 14-vector slabs in the workgroup-phased kernel (H = 9000, 11264, 15360).
# Trips of less than 32 MB run as one persistent launch of several trips
# (H = 1024, k = 1 and H = 896, k = 2: 16 and 21 MB per trip).
@pytest.mark.parametrize("H,k,T", [(7168, 8, 511), (7168, 8, 512), (7168, 8, 1536), (7168, 6, 2047), (7168, 6, 2048),
                                   (2048, 8, 1023), (2048, 8, 1024), (5120, 4, 1024), (4096, 2, 1536),
                                   (4096, 3, 1023), (4096, 3, 1024), (2880, 5, 2048), (7176, 8, 2100),
                                   (4104, 8, 511), (4104, 8, 512), (5000, 6, 1000), (7176, 8, 2047), (7176, 6, 1537),
                                   (8184, 8, 700), (5000, 7, 1000), (9000, 6, 256), (5000, 8, 511),
                                   (32768, 4, 384), (9000, 8, 2100), (11264, 2, 2048), (15360, 6, 2200),
                                   (1024, 1, 16384), (896, 2, 12000)])
def test_dispatch_default_batch_sizes(H, k, T):
    ep.ep_set_variant("auto")
    ep.ep_set_num_cus(0)
    wl = make_workload("prefill", seed=T + H + k, T=T, H=H, E=64, k=k)
    lay = oracle.layout(wl.topk_idx, 64)
    dest = lay["dest_row"].copy()
    dest[T // 2, k - 1] = -1
    got = run_dispatch(wl, dest, T * k)  # receive buffer pre-filled with 0x7E57
    want = oracle.dispatch(wl.x, dest, T * k, recv=np.full((T * k, H), 0x7E57, dtype=np.uint16))
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("name", DISPATCH_CONFIGS)
@pytest.mark.parametrize("variant,budget", [("auto", 0), ("vgpr_cached", 0), ("auto", 24), ("auto", 64)])
def test_dispatch_rows_matches(name, variant, budget):
    ep.ep_set_variant(variant)
    ep.ep_set_num_cus(budget)
    wl = workload(name)
    lay = oracle_layout(name)
    R = wl.config.T * wl.config.k
    recv = torch.full((R, wl.config.H), 0x7E57, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    ep.ep_dispatch_rows(to_bf16_x(wl), to_dev(lay["src_token"]), recv)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(from_dev_bf16(recv), oracle_recv(name))


@pytest.mark.parametrize("H", [8, 520, 7176])
def test_dispatch_rows_ragged_and_invalid(H):
    wl = make_workload("prefill", seed=H, T=41, H=H, E=16, k=3)
    lay = oracle.layout(wl.topk_idx, 16)
    src = lay["src_token"].copy()
    src[5] = -1
    src[7] = 41  # == T: out of range
    fill = 0x7E57
    recv = torch.full((41 * 3, H), fill, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    ep.ep_dispatch_rows(to_bf16_x(wl), to_dev(src), recv)
    torch.cuda.synchronize()
    # expected: the oracle's dispatch without the entries of rows 5 and 7
    dest = lay["dest_row"].copy()
    dest[np.isin(dest, [5, 7])] = -1
    ref = oracle.dispatch(wl.x, dest, 41 * 3, recv=np.full((41 * 3, H), fill, dtype=np.uint16))
    np.testing.assert_array_equal(from_dev_bf16(recv), ref)


def to_bf16_x(wl):
    return to_dev_bf16(wl.x)


def test_dispatch_skips_rows_outside_recv():
    wl = make_workload("decode", T=64)
    lay = oracle.layout(wl.topk_idx, 256)
    dest = lay["dest_row"].copy()
    dest[5, 2] = -1
    dest[9, 0] = 1 << 30
    rows = 300  # smaller than T*k: entries at or past row 300 are skipped
    fill = 0x7E57
    got = run_dispatch(wl, dest, rows, fill=fill)
    ref = oracle.dispatch(wl.x, dest, rows, recv=np.full((rows, wl.config.H), fill, dtype=np.uint16))
    np.testing.assert_array_equal(got, ref)


# ----------------------------------------------------------------- combine
def run_combine(wl, y_u16, dest_row_np):
    out = torch.empty((wl.config.T, wl.config.H), dtype=torch.bfloat16, device=DEV)
    ep.ep_combine(to_dev_bf16(y_u16), to_dev(dest_row_np), to_dev(wl.topk_w), out)
    torch.cuda.synchronize()
    return from_dev_bf16(out)


# Launches that depend on k: the persistent budget a named dispatch variant
# takes with no budget set (128 CUs at k = 1, 96 at k = 2..4, 64 from k = 5;
# lds1 here, with half-row slabs), the default dispatch (the workgroup-phased
# kernel on every CU at these sizes), and the combine's choice between the
# phased and the register kernel (by k and by how full each phased launch
# would be).  The per-expert scale is the expert.
@pytest.mark.parametrize("k,T", [(1, 4500), (2, 3100), (3, 3000), (4, 2500), (5, 2100), (6, 5461), (8, 4500)])
def test_default_launch_across_k(k, T):
    wl = make_workload("train", seed=40 + k, T=T, k=k)
    lay = oracle.layout(wl.topk_idx, wl.config.E)
    R = T * k
    ref_recv = oracle.dispatch(wl.x, lay["dest_row"], R)
    ep.ep_set_variant("lds1")
    np.testing.assert_array_equal(run_dispatch(wl, lay["dest_row"], R), ref_recv)
    ep.ep_set_variant("auto")
    np.testing.assert_array_equal(run_dispatch(wl, lay["dest_row"], R), ref_recv)
    y = oracle.expert_scale(ref_recv, lay["offsets"], wl.scales)
    assert_combine_close(run_combine(wl, y, lay["dest_row"]), oracle.combine(y, lay["dest_row"], wl.topk_w))


@pytest.mark.parametrize("name", list(CONFIGS))
def test_combine_full_size(name):
    wl = workload(name)
    got = run_combine(wl, expert_outputs(name), oracle_layout(name)["dest_row"])
    assert_combine_close(got, oracle_out(name))
    if wl.config.expert == "identity":
        # closed form: combine(dispatch(x)) == x with weights summing to 1
        assert np.array_equal(oracle.bf16_to_f32(got), oracle.bf16_to_f32(wl.x))


@pytest.mark.parametrize("variant", ["vgpr", "vgpr2", "lds1", "lds2", "vgpr_cached", "phase"])
@pytest.mark.parametrize("budget", BUDGETS)
def test_combine_variants_stress(variant, budget):
    ep.ep_set_variant(variant)
    ep.ep_set_num_cus(budget)
    name = "combine_stress"
    wl = workload(name)
    got = run_combine(wl, expert_outputs(name), oracle_layout(name)["dest_row"])
    assert_combine_close(got, oracle_out(name))


@pytest.mark.parametrize("variant", ["vgpr", "vgpr2", "lds1", "lds2", "phase"])
@pytest.mark.parametrize("budget", [0, 24])
def test_combine_variants_train(variant, budget):
    ep.ep_set_variant(variant)
    ep.ep_set_num_cus(budget)
    wl = workload("train")
    got = run_combine(wl, expert_outputs("train"), oracle_layout("train")["dest_row"])
    assert_combine_close(got, oracle_out("train"))


@pytest.mark.parametrize("variant", ["vgpr", "vgpr2", "lds1", "lds2", "phase"])
@pytest.mark.parametrize("H", [8, 520, 4104, 7176])
@pytest.mark.parametrize("k", [1, 3, 6, 8, 11])
@pytest.mark.parametrize("budget", [0, 24])
def test_combine_ragged_rows(variant, H, k, budget):
    ep.ep_set_variant(variant)
    ep.ep_set_num_cus(budget)
    T = 29
    wl = make_workload("combine_stress", seed=H + k, T=T, H=H, E=32, k=k)
    lay = oracle.layout(wl.topk_idx, 32)
    dest = lay["dest_row"].copy()
    dest[3, 0] = -1  # a slot that contributes nothing
    y = wl.y
    ref = oracle.combine(y, dest, wl.topk_w)
    got = run_combine(wl, y, dest)
    assert_combine_close(got, ref)


# The phase kernel's unit shapes: several tokens per unit in 16-wave
# workgroups (H = 8, 2048), two or three whole rows per wave in 8-wave
# workgroups (4104 ragged: 9 vectors per lane, three rows; 5000 ragged, 6144
# and 7168: two rows), a row split into segments (8712 ragged: 18 vectors per
# lane in two segments of 9; 16384: two of 16), a last unit that is only
# partly filled, and several units per wave (budget 1: one workgroup).
@pytest.mark.parametrize("H", [8, 2048, 4104, 5000, 6144, 7168, 8712, 16384])
@pytest.mark.parametrize("T", [1, 29, 300])
@pytest.mark.parametrize("budget", [0, 1, 24])
def test_combine_phase_units(H, T, budget):
    ep.ep_set_variant("phase")
    ep.ep_set_num_cus(budget)
    k = 8 if H % 3 else 6
    wl = make_workload("combine_stress", seed=H + T, T=T, H=H, E=32, k=k)
    lay = oracle.layout(wl.topk_idx, 32)
    dest = lay["dest_row"].copy()
    dest[T // 2, k - 1] = -1  # a slot that contributes nothing
    got = run_combine(wl, wl.y, dest)
    assert_combine_close(got, oracle.combine(wl.y, dest, wl.topk_w))


# At k = 2 and 4 the phase kernel reads runs of 2 vectors per source row
# where a step allows them: several tokens per unit (H = 2048), one row per
# unit with an odd vector count (4104 ragged: 9 vectors, the last step half
# used), a row split into segments of odd length (8712 ragged: 2 x 9) or
# even length (16384: 2 x 16), and single vectors where neither fits (H = 8).
@pytest.mark.parametrize("H", [8, 2048, 4104, 7168, 8712, 16384])
@pytest.mark.parametrize("T", [29, 300])
@pytest.mark.parametrize("k", [2, 4])
@pytest.mark.parametrize("budget", [0, 24])
def test_combine_phase_runs_of_two(H, T, k, budget):
    ep.ep_set_variant("phase")
    ep.ep_set_num_cus(budget)
    wl = make_workload("combine_stress", seed=H + T + k, T=T, H=H, E=32, k=k)
    lay = oracle.layout(wl.topk_idx, 32)
    dest = lay["dest_row"].copy()
    dest[T // 3, k - 1] = -1  # a slot that contributes nothing
    got = run_combine(wl, wl.y, dest)
    assert_combine_close(got, oracle.combine(wl.y, dest, wl.topk_w))


# Several launches per call: batches of whole two-row units on 256 or 128 CUs
# (4096 or 2048 tokens per launch at H = 7168), with a ragged last batch.
@pytest.mark.parametrize("T,budget", [(4097, 0), (8193, 0), (5000, 128), (2049, 192)])
@pytest.mark.parametrize("k", [6, 8])
def test_combine_phase_batches(T, budget, k):
    ep.ep_set_variant("phase")
    ep.ep_set_num_cus(budget)
    wl = make_workload("combine_stress", seed=T + k, T=T, H=7168, E=256, k=k)
    lay = oracle.layout(wl.topk_idx, 256)
    got = run_combine(wl, wl.y, lay["dest_row"])
    assert_combine_close(got, oracle.combine(wl.y, lay["dest_row"], wl.topk_w))


# The default combine with every CU on both sides of its fill thresholds for
# the phased kernel (the fraction of the grid's waves one launch gives a
# unit): 16-wave shapes take it from 9/20 at k >= 4 and 3/5 at k = 2, the
# two-row 8-wave shape from 23/25 at k = 5, 2/3 at k = 6, 3/4 at k = 7 and
# 7/10 at k = 8; in the 16-wave shape odd k takes the rule of the even k
# above it.  (H, k, T):
# H = 2048 holds four tokens per unit (16384 per full launch), H = 3072 and
# 4096 two (8192), H = 5120 and 7168 at k >= 6 two rows per wave in 8-wave
# workgroups (4096).  Rows of 9 vectors per lane (H = 4104 .. 4608) take
# three rows per wave, or two where that needs fewer passes over the grid:
# two at T = 4096 and 8192, three at T = 6144 and 12288 (a tie), with
# a ragged last vector at H = 4104 and 4160.  At k <= 4, rows of 5 and 7
# vectors per lane run padded by one vector (H = 2304 ragged, 2560 whole,
# 3584, 3000 ragged); 3 vectors (H = 1152) keep the register kernel.
@pytest.mark.parametrize(
    "H,k,T",
    [(2048, 4, 7000), (2048, 4, 8192), (4096, 8, 3686), (4096, 6, 4505), (3072, 2, 4600), (3072, 2, 4915),
     (2048, 2, 9830), (5120, 8, 2457), (5120, 8, 2800), (5120, 8, 2900), (7168, 8, 2860), (7168, 6, 2800),
     (4096, 3, 3500), (4096, 3, 3700), (2048, 1, 9600), (2048, 1, 9900), (7168, 5, 3760), (7168, 5, 3780),
     (7168, 7, 3068), (7168, 7, 3076), (4608, 8, 8192), (4160, 6, 4096), (4104, 7, 6144), (4160, 5, 12288),
     (4160, 8, 4097), (2304, 4, 8192), (2560, 3, 8191), (3584, 2, 16384), (3000, 4, 5000), (1152, 4, 8192)],
)
def test_combine_default_partial_fill(H, k, T):
    ep.ep_set_variant("auto")
    ep.ep_set_num_cus(0)
    wl = make_workload("combine_stress", seed=H + k + T, T=T, H=H, E=64, k=k)
    lay = oracle.layout(wl.topk_idx, 64)
    dest = lay["dest_row"].copy()
    dest[T // 2, k - 1] = -1  # a slot that contributes nothing
    got = run_combine(wl, wl.y, dest)
    assert_combine_close(got, oracle.combine(wl.y, dest, wl.topk_w))


# The default combine on a CU budget around its slab threshold: 1-vector
# slabs up to 32 tokens per CU of the budget, the 2- or 4-vector slabs above
# (k = 2..7 take 4), with whole and ragged rows.
@pytest.mark.parametrize("T", [24, 768, 769])
@pytest.mark.parametrize("H,k", [(7168, 8), (7168, 4), (520, 6)])
def test_combine_default_budget_slabs(T, H, k):
    ep.ep_set_variant("auto")
    ep.ep_set_num_cus(24)
    wl = make_workload("combine_stress", seed=T + H + k, T=T, H=H, E=64, k=k)
    lay = oracle.layout(wl.topk_idx, 64)
    dest = lay["dest_row"].copy()
    dest[T // 2, k - 1] = -1  # a slot that contributes nothing
    got = run_combine(wl, wl.y, dest)
    assert_combine_close(got, oracle.combine(wl.y, dest, wl.topk_w))


@pytest.mark.parametrize("variant", ["vgpr", "vgpr_cached", "lds2", "phase"])
@pytest.mark.parametrize("slab", [1, 2, 4])
@pytest.mark.parametrize("budget", [0, 24])
def test_combine_slab_sizes(variant, slab, budget):
    ep.ep_set_variant(variant)
    ep.ep_set_slab(slab)
    ep.ep_set_num_cus(budget)
    try:
        wl = workload("train")
        got = run_combine(wl, expert_outputs("train"), oracle_layout("train")["dest_row"])
        assert_combine_close(got, oracle_out("train"))
        for H, k in [(7176, 8), (4104, 3)]:
            wr = make_workload("combine_stress", seed=H + slab, T=31, H=H, E=32, k=k)
            lay = oracle.layout(wr.topk_idx, 32)
            got = run_combine(wr, wr.y, lay["dest_row"])
            assert_combine_close(got, oracle.combine(wr.y, lay["dest_row"], wr.topk_w))
    finally:
        ep.ep_set_slab(0)


@pytest.mark.parametrize("variant", ["lds3", "pc", "vgpr_wg"])
def test_combine_under_dispatch_only_variants(variant):
    # these name dispatch kernels only; combine runs its default
    ep.ep_set_variant(variant)
    wl = workload("train")
    got = run_combine(wl, expert_outputs("train"), oracle_layout("train")["dest_row"])
    assert_combine_close(got, oracle_out("train"))


def test_combine_unnormalised_weights_and_signed_zero():
    wl = make_workload("tiny", T=16)
    lay = oracle.layout(wl.topk_idx, 8)
    recv = oracle.dispatch(wl.x, lay["dest_row"], 32)
    recv[:4] = 0x8000  # -0.0 rows
    wl.topk_w = (wl.topk_w * np.float32(3.5)).astype(np.float32)
    got = run_combine(wl, recv, lay["dest_row"])
    assert_combine_close(got, oracle.combine(recv, lay["dest_row"], wl.topk_w))


@pytest.mark.parametrize(
    "T,k,variant,budget,dest",
    [
        (4096, 8, "auto", 0, "none"), (4096, 8, "phase", 0, "none"), (4096, 8, "vgpr", 0, "none"),
        (128, 8, "auto", 0, "none"), (128, 8, "phase", 0, "none"), (4096, 8, "auto", 24, "none"),
        (4096, 8, "phase", 0, "stale"), (4096, 6, "auto", 0, "stale"),
    ],
)
def test_combine_empty_receive_buffer(T, k, variant, budget, dest):
    """recv_rows == 0 (a receive buffer sized from offsets[E] = 0): y is a
    (0, H) tensor whose data pointer is NULL, and every slot is out of range,
    so the oracle's sum of no terms is +0.0 everywhere.  dest "none" routes
    every slot to -1 (what ep_layout writes for invalid ids); "stale" leaves
    row numbers that would be valid in a full buffer."""
    H = 7168
    ep.ep_set_variant(variant)
    ep.ep_set_num_cus(budget)
    rng = np.random.default_rng(T + k)
    if dest == "none":
        dest_np = np.full((T, k), -1, dtype=np.int32)
    else:
        dest_np = rng.permutation(T * k).reshape(T, k).astype(np.int32)
    w_np = rng.random((T, k), dtype=np.float32)
    y = torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
    assert y.data_ptr() == 0
    out = torch.full((T, H), 0x7E57, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    print(f"empty receive buffer: T={T} k={k} variant={variant} budget={budget} dest={dest}", flush=True)
    ep.ep_combine(y, to_dev(dest_np), to_dev(w_np), out)
    torch.cuda.synchronize()
    got = from_dev_bf16(out)
    ref = oracle.combine(np.zeros((0, H), dtype=np.uint16), dest_np, w_np)
    assert np.array_equal(got, ref)
    assert not got.any()  # +0.0, not -0.0


def test_combine_unfused_golden_cases():
    """The hand-derived cases of tests/golden/combine_unfused_cases.txt, where
    rounding each product and each sum separately gives a different bf16
    result from a fused multiply-add, through every combine kernel: 64 tokens
    alternate between the cases, every column of a row holds the case's
    value, and H = 1024 keeps several units per launch."""
    from golden_io import read_unfused_cases

    cases = read_unfused_cases()
    T, H = 64, 1024
    k = 2
    y_np = np.empty((T * k, H), dtype=np.uint16)
    w_np = np.empty((T, k), dtype=np.float32)
    want = np.empty(T, dtype=np.uint16)
    for t in range(T):
        c = cases[t % len(cases)]
        for j in range(k):
            y_np[t * k + j, :] = c["y"][j]
        w_np[t] = c["w"]
        want[t] = c["unfused"]
    dest_np = np.arange(T * k, dtype=np.int32).reshape(T, k)
    ref = oracle.combine(y_np, dest_np, w_np)
    assert np.array_equal(ref, np.repeat(want[:, None], H, axis=1))
    for variant in ("auto", "vgpr", "vgpr2", "lds1", "lds2", "phase"):
        for budget in (0, 24):
            ep.ep_set_variant(variant)
            ep.ep_set_num_cus(budget)
            out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
            ep.ep_combine(to_dev_bf16(y_np), to_dev(dest_np), to_dev(w_np), out)
            torch.cuda.synchronize()
            got = from_dev_bf16(out)
            assert np.array_equal(got, ref), (variant, budget)


# ----------------------------------------------------------------- probes
def test_inflight_probe_chase_lands_on_the_walked_index():
    """The pointer chase of ep_inflight_probe follows the chain exactly: after
    `hops` links its last index is the one a host walk reaches, with and
    without streaming waves beside it."""
    n, per = 4096, 32  # 4096 nodes of 256 bytes
    rng = np.random.default_rng(7)
    perm = rng.permutation(n)
    chain_np = np.zeros(n * per, dtype=np.int64)
    chain_np[perm * per] = np.roll(perm, -1) * per
    chain = to_dev(chain_np)
    src = torch.ones(1 << 22, dtype=torch.int32, device=DEV)
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    out = torch.zeros(4, dtype=torch.int64, device=DEV)
    for budget, waves, vec, nbytes, hops in ((1, 1, 1, 0, 777), (24, 4, 8, src.numel() * 4, 301),
                                             (0, 8, 16, src.numel() * 4, 55)):
        ep.ep_set_num_cus(budget)
        ep.ep_inflight_probe(waves, vec, src, nbytes, sink, chain, hops, out, cached=budget == 24)
        torch.cuda.synchronize()
        idx = 0
        for _ in range(hops):
            idx = int(chain_np[idx])
        o = out.cpu().tolist()
        assert o[2] == idx and o[0] > 0 and o[1] > 0
        assert int(sink.abs().sum()) == 0


def test_bw_probe_copies_and_writes():
    n = (1 << 22) + 4096
    src = torch.randint(-(1 << 31), 1 << 31, (n // 4,), dtype=torch.int32, device=DEV)
    dst = torch.zeros_like(src)
    for budget in (0, 24):
        ep.ep_set_num_cus(budget)
        dst.zero_()
        ep.ep_bw_probe(0, src, dst, n)
        torch.cuda.synchronize()
        assert torch.equal(src, dst)
        ep.ep_bw_probe(1, src, dst, n)
        ep.ep_bw_probe(2, None, dst, n)
        torch.cuda.synchronize()
        v = dst.view(-1, 4).cpu().numpy().astype(np.int64) & 0xFFFFFFFF
        idx = np.arange(v.shape[0])
        assert np.array_equal(v[:, 0], idx & 0xFFFFFFFF) and np.all(v[:, 1] == 0x5A5A5A5A)


def test_bw_probe_mixed_ratios():
    n = 1 << 22  # bytes of the larger side
    big = torch.randint(-(1 << 31), 1 << 31, (n // 4,), dtype=torch.int32, device=DEV)
    small = torch.zeros(n // 32, dtype=torch.int32, device=DEV)
    ep.ep_bw_probe(4, big, small, n)  # 8:1 -- xor of each 8 KiB chunk's vectors
    torch.cuda.synchronize()
    b = big.view(-1, 8, 64, 4).cpu().numpy()
    want = np.bitwise_xor.reduce(b, axis=1).reshape(-1)
    assert np.array_equal(small.cpu().numpy(), want)
    burst = torch.zeros(n // 32, dtype=torch.int32, device=DEV)
    ep.ep_bw_probe(6, big, burst, n)  # 8:1 in bursts -- vector i of each 8 KiB out folds 8 rounds
    torch.cuda.synchronize()
    b64 = big.view(-1, 8, 8, 64, 4).cpu().numpy()  # [chunk, round, i, lane, word]
    want = np.bitwise_xor.reduce(b64, axis=1).reshape(-1)
    assert np.array_equal(burst.cpu().numpy(), want)
    phase = torch.zeros(n // 32, dtype=torch.int32, device=DEV)
    ep.ep_bw_probe(7, big, phase, n)  # 8:1 in phases -- vector i of each 16 KiB out folds 8 blocks
    torch.cuda.synchronize()
    b16 = big.view(-1, 8, 16, 64, 4).cpu().numpy()  # [chunk, block, i, lane, word]
    want = np.bitwise_xor.reduce(b16, axis=1).reshape(-1)
    assert np.array_equal(phase.cpu().numpy(), want)
    phase.zero_()
    ep.ep_bw_probe(0x27, big, phase, n)  # the same with the bounded grid-wide wait between reads and writes
    torch.cuda.synchronize()
    assert np.array_equal(phase.cpu().numpy(), want)
    fan = torch.zeros_like(big)
    ep.ep_bw_probe(0x17, small, fan, n)  # 1:8 in phases -- each 16 KiB in written 8 times, r in the first word
    torch.cuda.synchronize()
    f = fan.view(-1, 8, 16, 64, 4).cpu().numpy()  # [chunk, copy, i, lane, word]
    s16 = small.view(-1, 16, 64, 4).cpu().numpy()
    for r in range(8):
        want = s16.copy()
        want[..., 0] ^= r
        assert np.array_equal(f[:, r], want)
    out = torch.zeros_like(big)
    ep.ep_bw_probe(5, small, out, n)  # 1:8 -- each 1 KiB chunk written 8 times (x ^ i in the first word)
    torch.cuda.synchronize()
    o = out.view(-1, 8, 64, 4).cpu().numpy()
    s = small.view(-1, 64, 4).cpu().numpy()
    for i in range(8):
        w = s.copy()
        w[:, :, 0] ^= i
        assert np.array_equal(o[:, i], w)


@pytest.mark.parametrize("budget", [16, 24, 32, 64])
def test_persistent_grid_gets_distinct_cus(budget):
    ep.ep_set_num_cus(budget)
    out = torch.full((budget, 4), -1, dtype=torch.int32, device=DEV)
    n = ep.ep_probe_placement(out, budget)
    torch.cuda.synchronize()
    assert n == budget
    rows = [tuple(r) for r in out.cpu().numpy()[:, :3].tolist()]
    assert len(set(rows)) == budget, f"workgroups shared a CU: {sorted(rows)}"
    per_xcc = np.bincount([r[0] for r in rows], minlength=8)
    print(f"budget {budget}: workgroups per XCD {per_xcc.tolist()}", flush=True)
    assert per_xcc.max() - per_xcc.min() <= 1


def test_mfma_probe_runs_and_keeps_out_untouched():
    out = torch.full((256 * 8,), 7.0, dtype=torch.float32, device=DEV)
    ep.ep_mfma_probe(8, 100, out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_cu_masked_stream_confines_work():
    n = 24
    stream = ep.ep_stream_create_cu_masked(ep.cu_mask_words(range(n)))
    try:
        out = torch.full((96, 4), -1, dtype=torch.int32, device=DEV)
        with torch.cuda.stream(stream):
            launched = ep.ep_probe_placement(out, 96, stream=stream)
        stream.synchronize()
        assert launched == 96
        rows = {tuple(r) for r in out.cpu().numpy()[:, :3].tolist()}
        per_xcc = np.bincount([r[0] for r in rows], minlength=8)
        print(f"mask of {n} CUs: {len(rows)} distinct CUs used, per XCD {per_xcc.tolist()}", flush=True)
        assert 0 < len(rows) <= n
        # the copy kernels run correctly on it, full grid or persistent
        wl = workload("train")
        for budget in (0, 24):
            ep.ep_set_num_cus(budget)
            ep.ep_set_variant("lds1")
            x = to_dev_bf16(wl.x)
            dest = to_dev(oracle_layout("train")["dest_row"])
            recv = torch.empty((wl.config.T * wl.config.k, wl.config.H), dtype=torch.bfloat16, device=DEV)
            torch.cuda.synchronize()
            ep.ep_dispatch(x, dest, recv, stream=stream)
            stream.synchronize()
            np.testing.assert_array_equal(from_dev_bf16(recv), oracle_recv("train"))
    finally:
        torch.cuda.synchronize()
        ep.ep_stream_destroy(stream)


def test_cu_mask_bits_interleave_over_the_xcds():
    """Mask bit i selects a CU of XCD i mod 8: eight consecutive bits give one
    CU on each XCD, and bits 8 apart stay on one XCD's CUs while the mask as
    a whole still reaches every XCD (masks that leave an XCD without CUs are
    refused on the host, before the runtime sees them)."""
    for bits in (range(4), [32 * i for i in range(8)]):
        with pytest.raises(ep.EpError) as exc:
            ep.ep_stream_create_cu_masked(ep.cu_mask_words(bits))
        assert exc.value.code == ep.EP_ERR_INVALID_ARG and "XCD" in str(exc.value)
    torch.zeros(16, device=DEV)  # no error was left behind for the next HIP call
    torch.cuda.synchronize()
    for bits, want in ((range(8), [1] * 8), (list(range(8)) + [8, 16, 24], [4, 1, 1, 1, 1, 1, 1, 1]),
                       (range(24), [3] * 8)):
        stream = ep.ep_stream_create_cu_masked(ep.cu_mask_words(bits))
        try:
            groups = 64
            out = torch.full((groups, 4), -1, dtype=torch.int32, device=DEV)
            ep.ep_probe_placement(out, groups, stream=stream)
            stream.synchronize()
            rows = {tuple(r) for r in out.cpu().numpy()[:, :3].tolist()}
            per_xcc = np.bincount([r[0] for r in rows], minlength=8).tolist()
            print(f"mask bits {list(bits)}: distinct CUs per XCD {per_xcc}", flush=True)
            assert per_xcc == want
        finally:
            torch.cuda.synchronize()
            ep.ep_stream_destroy(stream)


@pytest.mark.parametrize("n", [24, 128])
def test_step_on_masked_stream(n):
    """Layout, dispatch (in one launch) and combine on a stream masked to n
    CUs with no budget set: the library reads the stream's mask and sizes its
    grids and kernel choices for n CUs.  Outputs equal the oracle's."""
    stream = ep.ep_stream_create_cu_masked(ep.cu_mask_words(range(n)))
    try:
        wl = workload("train")
        c = wl.config
        ref = oracle_layout("train")
        recv = torch.empty((c.T * c.k, c.H), dtype=torch.bfloat16, device=DEV)
        out = torch.empty((c.T, c.H), dtype=torch.bfloat16, device=DEV)
        idx, x, w = to_dev(wl.topk_idx), to_dev_bf16(wl.x), to_dev(wl.topk_w)
        y = to_dev_bf16(expert_outputs("train"))
        torch.cuda.synchronize()
        lay = ep.ep_layout_dispatch(idx, c.E, x, recv, stream=stream)
        ep.ep_combine(y, lay["dest_row"], w, out, stream=stream)
        stream.synchronize()
        check_layout({k: v.cpu().numpy() for k, v in lay.items()}, ref, c.T, c.k)
        np.testing.assert_array_equal(from_dev_bf16(recv), oracle_recv("train"))
        assert_combine_close(from_dev_bf16(out), oracle_out("train"))
    finally:
        torch.cuda.synchronize()
        ep.ep_stream_destroy(stream)


def test_step_on_24_cus_beside_matrix_core_work():
    """The pages' premise in one test: the step (layout, dispatch, combine as
    separate calls) on a stream masked to 24 CUs while the matrix-core probe
    keeps the other CUs busy on a second masked stream, both launched before
    either is waited for.  The step's outputs equal the oracle's, and the
    compute kernel has not finished before the step was issued."""
    ndev = torch.cuda.get_device_properties(0).multi_processor_count
    comm = ep.ep_stream_create_cu_masked(ep.cu_mask_words(range(24)))
    comp = ep.ep_stream_create_cu_masked(ep.cu_mask_words(range(24, ndev)))
    try:
        wl = workload("train")
        c = wl.config
        ref = oracle_layout("train")
        recv = torch.empty((c.T * c.k, c.H), dtype=torch.bfloat16, device=DEV)
        out = torch.empty((c.T, c.H), dtype=torch.bfloat16, device=DEV)
        idx, x, w = to_dev(wl.topk_idx), to_dev_bf16(wl.x), to_dev(wl.topk_w)
        y = to_dev_bf16(expert_outputs("train"))
        groups = (ndev - 24) * 8
        mfma_out = torch.zeros(256 * groups, dtype=torch.float32, device=DEV)
        done = torch.cuda.Event()
        torch.cuda.synchronize()
        ep.ep_mfma_probe(groups, 4096, mfma_out, stream=comp)
        done.record(comp)
        lay = ep.ep_layout(idx, c.E, stream=comm)
        ep.ep_dispatch(x, lay["dest_row"], recv, stream=comm)
        ep.ep_combine(y, lay["dest_row"], w, out, stream=comm)
        overlapped = not done.query()
        torch.cuda.synchronize()
        check_layout({k: v.cpu().numpy() for k, v in lay.items()}, ref, c.T, c.k)
        np.testing.assert_array_equal(from_dev_bf16(recv), oracle_recv("train"))
        assert_combine_close(from_dev_bf16(out), oracle_out("train"))
        assert overlapped
        assert int((mfma_out != 0).sum()) == 0
    finally:
        torch.cuda.synchronize()
        ep.ep_stream_destroy(comm)
        ep.ep_stream_destroy(comp)


def test_k4_step_on_masked_stream():
    """k = 4 on a stream masked to 192 CUs: the one-launch layout + dispatch
    on k = 4's default budget and the phased combine with 2-vector runs, in
    launches sized for the mask.  Outputs equal the oracle's."""
    stream = ep.ep_stream_create_cu_masked(ep.cu_mask_words(range(192)))
    try:
        wl = make_workload("train", seed=44, T=8192, k=4)
        c = wl.config
        ref = oracle.layout(wl.topk_idx, c.E)
        R = c.T * c.k
        ref_recv = oracle.dispatch(wl.x, ref["dest_row"], R)
        y_np = oracle.expert_scale(ref_recv, ref["offsets"], wl.scales)
        recv = torch.empty((R, c.H), dtype=torch.bfloat16, device=DEV)
        out = torch.empty((c.T, c.H), dtype=torch.bfloat16, device=DEV)
        idx, x, w, y = to_dev(wl.topk_idx), to_dev_bf16(wl.x), to_dev(wl.topk_w), to_dev_bf16(y_np)
        torch.cuda.synchronize()
        lay = ep.ep_layout_dispatch(idx, c.E, x, recv, stream=stream)
        ep.ep_combine(y, lay["dest_row"], w, out, stream=stream)
        stream.synchronize()
        check_layout({k: v.cpu().numpy() for k, v in lay.items()}, ref, c.T, c.k)
        np.testing.assert_array_equal(from_dev_bf16(recv), ref_recv)
        assert_combine_close(from_dev_bf16(out), oracle.combine(y_np, ref["dest_row"], wl.topk_w))
    finally:
        torch.cuda.synchronize()
        ep.ep_stream_destroy(stream)


@pytest.mark.parametrize("name", ["decode", "tiny"])
def test_graph_replay_matches_eager(name):
    """The whole step captured in a HIP graph: every replay, with eager work
    and synchronisations between replays, equals the oracle."""
    wl = workload(name)
    c = wl.config
    idx = to_dev(wl.topk_idx)
    x = to_dev_bf16(wl.x)
    w = to_dev(wl.topk_w)
    R = c.T * c.k
    lay = {
        "counts": torch.empty(c.E, dtype=torch.int32, device=DEV),
        "offsets": torch.empty(c.E + 1, dtype=torch.int32, device=DEV),
        "dest_row": torch.empty((c.T, c.k), dtype=torch.int32, device=DEV),
        "src_token": torch.empty(R, dtype=torch.int32, device=DEV),
        "status": torch.empty(1, dtype=torch.int32, device=DEV),
    }
    ws = torch.empty(max(16, ep.ep_layout_workspace_bytes(c.T, c.k, c.E)), dtype=torch.uint8, device=DEV)
    recv = torch.empty((R, c.H), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((c.T, c.H), dtype=torch.bfloat16, device=DEV)

    def step():
        ep.ep_layout(idx, c.E, lay["counts"], lay["offsets"], lay["dest_row"], lay["src_token"], lay["status"], ws)
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
    ref_lay = oracle_layout(name)
    ref_recv = oracle_recv(name)
    for rep in range(4):
        # clobber the outputs eagerly so each replay must rewrite them
        recv.view(torch.int16).fill_(rep)
        out.view(torch.int16).fill_(rep)
        lay["dest_row"].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(lay["dest_row"].cpu().numpy(), ref_lay["dest_row"])
        np.testing.assert_array_equal(lay["offsets"].cpu().numpy(), ref_lay["offsets"])
        np.testing.assert_array_equal(from_dev_bf16(recv), ref_recv)
        assert np.array_equal(oracle.bf16_to_f32(from_dev_bf16(out)), oracle.bf16_to_f32(wl.x))


@pytest.mark.parametrize("name,over", [("decode", {}), ("train", dict(T=1000)), ("train", {})])
def test_graph_replay_one_launch_layout_dispatch(name, over):
    """ep_layout_dispatch (the small and the wide one-launch kernels) and
    ep_combine captured in a HIP graph: every replay, with the outputs
    clobbered eagerly in between, equals the oracle."""
    wl = make_workload(name, seed=15, **over)
    c = wl.config
    idx = to_dev(wl.topk_idx)
    x = to_dev_bf16(wl.x)
    w = to_dev(wl.topk_w)
    R = c.T * c.k
    i32 = dict(dtype=torch.int32, device=DEV)
    lay = {"counts": torch.empty(c.E, **i32), "offsets": torch.empty(c.E + 1, **i32),
           "dest_row": torch.empty((c.T, c.k), **i32), "src_token": torch.empty(R, **i32),
           "status": torch.empty(1, **i32)}
    ws = torch.empty(max(16, ep.ep_layout_workspace_bytes(c.T, c.k, c.E)), dtype=torch.uint8, device=DEV)
    recv = torch.empty((R, c.H), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((c.T, c.H), dtype=torch.bfloat16, device=DEV)

    def step():
        ep.ep_layout_dispatch(idx, c.E, x, recv, lay["counts"], lay["offsets"], lay["dest_row"], lay["src_token"],
                              lay["status"], ws)
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
    ref = oracle.layout(wl.topk_idx, c.E)
    ref_recv = oracle.dispatch(wl.x, ref["dest_row"], R)
    for rep in range(4):
        recv.view(torch.int16).fill_(rep)
        out.view(torch.int16).fill_(rep)
        lay["dest_row"].fill_(-7)
        lay["src_token"].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_layout({k: v.cpu().numpy() for k, v in lay.items()}, ref, c.T, c.k)
        np.testing.assert_array_equal(from_dev_bf16(recv), ref_recv)
        assert np.array_equal(oracle.bf16_to_f32(from_dev_bf16(out)), oracle.bf16_to_f32(wl.x))


@pytest.mark.parametrize(
    "name,over",
    [("decode", {}), ("tiny", {}), ("prefill", dict(T=170, E=64, k=6)), ("prefill", dict(T=33, H=7176, E=16, k=3)),
     ("prefill", dict(T=1, H=8, E=1, k=1)), ("prefill", dict(T=32, E=1024, k=32)),
     ("train", dict(T=300)), ("prefill", dict(T=2000, E=64, k=6)),
     ("train", dict(T=128, k=1)), ("train", dict(T=300, k=3)), ("train", dict(T=777, k=5, H=7176)),
     ("train", dict(T=512, k=7, E=100)), ("prefill", dict(T=128, E=64, k=4)), ("prefill", dict(T=170, E=32, k=5))],
)
@pytest.mark.parametrize("budget", [0, 24])
def test_layout_dispatch_matches_two_calls(name, over, budget):
    ep.ep_set_num_cus(budget)
    wl = make_workload(name, seed=7, **over)
    c = wl.config
    ref = oracle.layout(wl.topk_idx, c.E)
    R = c.T * c.k
    recv = torch.full((R, c.H), 0x7E57, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    lay = ep.ep_layout_dispatch(to_dev(wl.topk_idx), c.E, to_dev_bf16(wl.x), recv)
    torch.cuda.synchronize()
    check_layout({k: v.cpu().numpy() for k, v in lay.items()}, ref, c.T, c.k)
    np.testing.assert_array_equal(from_dev_bf16(recv), oracle.dispatch(wl.x, ref["dest_row"], R))


def test_layout_dispatch_flags_bad_ids():
    rng = np.random.default_rng(11)
    idx = np.array([rng.permutation(16)[:4] for _ in range(100)], dtype=np.int32)
    idx[3, 1] = 99
    idx[50, 2] = idx[50, 0]
    x = rng.integers(0, 2**16, size=(100, 64), dtype=np.uint32).astype(np.uint16)
    ref = oracle.layout(idx, 16)
    assert ref["status"] == 3
    recv = torch.full((400, 64), 0x7E57, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    lay = ep.ep_layout_dispatch(to_dev(idx), 16, to_dev_bf16(x), recv)
    torch.cuda.synchronize()
    check_layout({k: v.cpu().numpy() for k, v in lay.items()}, ref, 100, 4)
    want = oracle.dispatch(x, ref["dest_row"], 400, recv=np.full((400, 64), 0x7E57, dtype=np.uint16))
    np.testing.assert_array_equal(from_dev_bf16(recv), want)


# ------------------------------------------------- fused layout + dispatch, wide batches
# With k in {2, 4, 6, 8}, 65 <= E <= 256 and at most 64 Ki entries,
# ep_layout_dispatch runs as one persistent launch in which every workgroup
# histograms all ids and then ranks and copies its own token range.  These cases put T off the grid size, rows off the slab size, E at
# both ends of the range, the entry count at its limit, and several ranking
# rounds in one workgroup (the 24-CU budget at the training shape: 171
# tokens x 8 = 1368 entries per workgroup).  The last cases fall outside the
# wide path (k = 1 or 3, E = 1 or 64 or 300, past 64 Ki entries) and take the
# two separate launches.  The two after them are large enough at k = 2 and 4
# for the default budget of those k (96 CUs).
WIDE_CASES = [
    ("train", {}),
    ("train", dict(T=129)),
    ("train", dict(T=5000, H=7176)),
    ("train", dict(T=777, H=1032, E=65, k=2)),
    ("train", dict(T=4096, k=6)),
    ("train", dict(T=3000, H=512, E=256, k=4)),
    ("train", dict(T=8192)),
    ("prefill", dict(T=3001, H=4096, E=100, k=2)),
    ("train", dict(T=8193)),
    ("prefill", dict(T=6000, E=64, k=6)),
    ("prefill", dict(T=2048, H=2056, E=1, k=1)),
    ("prefill", dict(T=2000, H=1024, E=64, k=3)),
    ("train", dict(T=400, H=1024, E=300, k=8)),
    ("train", dict(T=6200, k=2)),
    ("train", dict(T=4000, k=4)),
]


def run_layout_dispatch(wl):
    c = wl.config
    ref = oracle.layout(wl.topk_idx, c.E)
    R = c.T * c.k
    recv = torch.full((R, c.H), 0x7E57, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    lay = ep.ep_layout_dispatch(to_dev(wl.topk_idx), c.E, to_dev_bf16(wl.x), recv)
    torch.cuda.synchronize()
    check_layout({k: v.cpu().numpy() for k, v in lay.items()}, ref, c.T, c.k)
    np.testing.assert_array_equal(from_dev_bf16(recv), oracle.dispatch(wl.x, ref["dest_row"], R))


# Decode-size batches (T*k <= 1024): the wide kernel where it applies, the
# small one (every workgroup lays out all entries) under another variant.
@pytest.mark.parametrize("name,over", [("decode", {}), ("decode", dict(T=1)), ("decode", dict(T=33)),
                                       ("train", dict(T=128, H=1032)), ("train", dict(T=100, E=65, k=6))])
@pytest.mark.parametrize("variant", ["auto", "vgpr"])
@pytest.mark.parametrize("budget", [0, 24])
def test_layout_dispatch_decode_sizes(name, over, variant, budget):
    ep.ep_set_variant(variant)
    ep.ep_set_num_cus(budget)
    run_layout_dispatch(make_workload(name, seed=16, **over))


# Under "lds1" the wide kernel takes every case it applies to; under "auto"
# batches of at least 8 tokens per CU of the launch run the layout and the
# default (streaming) dispatch instead.
@pytest.mark.parametrize("name,over", WIDE_CASES)
@pytest.mark.parametrize("budget", [0, 24, 256])
@pytest.mark.parametrize("variant", ["lds1", "auto"])
def test_layout_dispatch_wide(name, over, budget, variant):
    ep.ep_set_variant(variant)
    ep.ep_set_num_cus(budget)
    run_layout_dispatch(make_workload(name, seed=8, **over))


@pytest.mark.parametrize("variant", ["lds1", "auto"])
def test_layout_dispatch_wide_prefill_full_size(variant):
    ep.ep_set_variant(variant)
    run_layout_dispatch(workload("prefill"))


@pytest.mark.parametrize("slab", [2, 4, 8])
def test_layout_dispatch_wide_slabs(slab):
    ep.ep_set_slab(slab)
    try:
        run_layout_dispatch(make_workload("train", seed=9, T=1500))
    finally:
        ep.ep_set_slab(0)


@pytest.mark.parametrize("variant", ["vgpr", "lds2", "lds1"])
def test_layout_dispatch_wide_under_variants(variant):
    ep.ep_set_variant(variant)
    run_layout_dispatch(make_workload("train", seed=10, T=1200))


@pytest.mark.parametrize("E,k", [(96, 4), (256, 8)])
def test_layout_dispatch_wide_flags_bad_ids(E, k):
    rng = np.random.default_rng(12)
    T, H = 2000, 1024
    idx = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32)
    idx[3, 1] = E + 5
    idx[1500, 0] = -1
    idx[999, 2] = idx[999, 0]
    x = rng.integers(0, 2**16, size=(T, H), dtype=np.uint32).astype(np.uint16)
    ref = oracle.layout(idx, E)
    assert ref["status"] == 3
    R = T * k
    recv = torch.full((R, H), 0x7E57, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    lay = ep.ep_layout_dispatch(to_dev(idx), E, to_dev_bf16(x), recv)
    torch.cuda.synchronize()
    check_layout({kk: v.cpu().numpy() for kk, v in lay.items()}, ref, T, k)
    want = oracle.dispatch(x, ref["dest_row"], R, recv=np.full((R, H), 0x7E57, dtype=np.uint16))
    np.testing.assert_array_equal(from_dev_bf16(recv), want)


@pytest.mark.parametrize("rows", [0, 1, 4096, 20000])
def test_layout_dispatch_wide_short_receive_buffer(rows):
    # rows past the receive buffer are skipped, as in ep_dispatch
    wl = make_workload("train", seed=14, T=3000, H=1024)
    c = wl.config
    ref = oracle.layout(wl.topk_idx, c.E)
    recv = torch.full((rows, c.H), 0x7E57, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    lay = ep.ep_layout_dispatch(to_dev(wl.topk_idx), c.E, to_dev_bf16(wl.x), recv)
    torch.cuda.synchronize()
    check_layout({k: v.cpu().numpy() for k, v in lay.items()}, ref, c.T, c.k)
    want = oracle.dispatch(wl.x, ref["dest_row"], rows, recv=np.full((rows, c.H), 0x7E57, dtype=np.uint16))
    np.testing.assert_array_equal(from_dev_bf16(recv), want)


def test_layout_dispatch_wide_is_deterministic():
    wl = make_workload("train", seed=13, T=3000)
    c = wl.config
    idx, x = to_dev(wl.topk_idx), to_dev_bf16(wl.x)
    outs = []
    for _ in range(3):
        recv = torch.zeros((c.T * c.k, c.H), dtype=torch.bfloat16, device=DEV)
        lay = ep.ep_layout_dispatch(idx, c.E, x, recv)
        torch.cuda.synchronize()
        outs.append((lay["dest_row"].cpu().numpy(), lay["src_token"].cpu().numpy(), recv.view(torch.int16).cpu()))
    for o in outs[1:]:
        np.testing.assert_array_equal(o[0], outs[0][0])
        np.testing.assert_array_equal(o[1], outs[0][1])
        assert torch.equal(o[2], outs[0][2])


def test_binding_rejects_bad_device_tensors():
    """The binding's checks on device tensors: wrong dtype, non-contiguous
    views and mismatched shapes raise before anything is launched."""
    x = torch.zeros((8, 64), dtype=torch.bfloat16, device=DEV)
    dest = torch.zeros((8, 2), dtype=torch.int32, device=DEV)
    recv = torch.zeros((16, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(TypeError):
        ep.ep_dispatch(x.float(), dest, recv)
    with pytest.raises(TypeError):
        ep.ep_dispatch(x, dest.long(), recv)
    with pytest.raises(ValueError):
        ep.ep_dispatch(torch.zeros((64, 8), dtype=torch.bfloat16, device=DEV).t(), dest, recv)
    with pytest.raises(ValueError):
        ep.ep_dispatch(x, dest[:4], recv)
    w = torch.zeros((8, 2), dtype=torch.float32, device=DEV)
    out = torch.zeros((8, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(TypeError):
        ep.ep_combine(recv, dest, w.double(), out)
    with pytest.raises(ValueError):
        ep.ep_combine(recv, dest, w[:, :1], out)
    with pytest.raises(ValueError):
        ep.ep_layout(torch.zeros((2, 8), dtype=torch.int32, device=DEV).t(), 16)
    ep.ep_dispatch(x, dest, recv)  # the valid call still works
    torch.cuda.synchronize()


def _random_cases(n, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        k = int(rng.integers(1, 11)) if rng.random() < 0.8 else int(rng.integers(11, 33))
        E = int(rng.integers(max(k, 2), 300)) if rng.random() < 0.8 else int(rng.integers(max(k, 2), 1025))
        H = 8 * int(rng.integers(1, 1125))
        T = int(rng.integers(1, 3000))
        if T * k * H * 2 > 96 << 20:  # keep the oracle to a few seconds
            continue
        cases.append(dict(name=str(rng.choice(["train", "prefill"])), T=T, H=H, E=E, k=k,
                          budget=int(rng.choice([0, 0, 24, 64, 200, 256])),
                          variant=str(rng.choice(["auto", "auto", "auto", "lds1", "vgpr", "phase", "vgpr_wg", "vgpr2",
                                                  "lds2", "lds3", "pc", "vgpr_cached"])),
                          slab=int(rng.choice([0, 0, 0, 1, 2, 4, 7, 8, 14, 16])),
                          one_launch=bool(rng.integers(0, 2))))
    return cases


# Seeded random shapes through the default and forced launches: layout and
# dispatch bit-exact, combine against the oracle, with and without the
# one-launch layout + dispatch.
@pytest.mark.parametrize("case", _random_cases(150), ids=lambda c: "{name}-T{T}-H{H}-E{E}-k{k}-b{budget}-{variant}-s{slab}"
                         .format(**c) + ("-one" if c["one_launch"] else ""))
def test_random_shapes(case):
    ep.ep_set_num_cus(case["budget"])
    ep.ep_set_variant(case["variant"])
    ep.ep_set_slab(case["slab"])
    wl = make_workload(case["name"], seed=case["T"] + case["H"], T=case["T"], H=case["H"], E=case["E"],
                       k=case["k"])
    c = wl.config
    ref = oracle.layout(wl.topk_idx, c.E)
    R = c.T * c.k
    ref_recv = oracle.dispatch(wl.x, ref["dest_row"], R)
    recv = torch.full((R, c.H), 0x7E57, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    idx, x = to_dev(wl.topk_idx), to_dev_bf16(wl.x)
    if case["one_launch"]:
        lay = ep.ep_layout_dispatch(idx, c.E, x, recv)
    else:
        lay = ep.ep_layout(idx, c.E)
        ep.ep_dispatch(x, lay["dest_row"], recv)
    torch.cuda.synchronize()
    check_layout({k: v.cpu().numpy() for k, v in lay.items()}, ref, c.T, c.k)
    np.testing.assert_array_equal(from_dev_bf16(recv), ref_recv)
    # the gather form on the library's own src_token
    recv.view(torch.int16).fill_(0x7E57)
    ep.ep_dispatch_rows(x, lay["src_token"], recv)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(from_dev_bf16(recv), ref_recv)
    y = oracle.expert_identity(ref_recv) if wl.config.expert != "scale" else \
        oracle.expert_scale(ref_recv, ref["offsets"], wl.scales)
    got = run_combine(wl, y, ref["dest_row"])
    assert_combine_close(got, oracle.combine(y, ref["dest_row"], wl.topk_w))
