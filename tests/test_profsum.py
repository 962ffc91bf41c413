"""The rocprofv3 summariser (bulk_async_tensor_amd/profsum.py) on small
hand-made counter files: kernel classification, the copy-probe scaling of
FETCH_SIZE and WRITE_SIZE, the per-call sum of a multi-launch kernel, and
the source hash that bench.py checks before it reports the traffic."""

import csv

from bulk_async_tensor_amd import profsum
from bulk_async_tensor_amd.build import kernel_source_hash

import bench

COLS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def write_counters(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=COLS)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_kind_of_classifies_our_kernels():
    k = profsum.kind_of
    assert k("void ep::(anonymous namespace)::layout_fused_kernel<8>(int const*)") == "layout"
    assert k("void ep::(anonymous namespace)::layout_dispatch_wide_kernel<7, 8, true>(int const*)") == "layout_dispatch"
    assert k("void ep::(anonymous namespace)::layout_dispatch_kernel<2, 8, true>(int const*)") == "layout_dispatch"
    assert k("void ep::(anonymous namespace)::dispatch_lds1_kernel<7, 8, true, true>(x)") == "dispatch"
    assert k("void ep::(anonymous namespace)::combine_phase_kernel<8, 1, 4, 28, true, 512>(x)") == "combine"
    assert k("void ep::(anonymous namespace)::reduce_scatter_kernel<8, true>(x)") == "combine_reduce"
    assert k("void ep::(anonymous namespace)::bw_kernel<0, 8, 0>(x)") == "copy_probe"
    assert k("void at::native::vectorized_elementwise_kernel<4>(x)") is None


def test_hbm_scales_by_the_copy_probe_and_sums_launches(tmp_path):
    comb = "void ep::(anonymous namespace)::combine_phase_kernel<6, 1, 4, 28, true, 512>(x)"
    probe = "void ep::(anonymous namespace)::bw_kernel<0, 8, 0>(x)"
    copy = 256 << 20
    # FETCH_SIZE reads half the true bytes, WRITE_SIZE all of them (KiB per dispatch)
    write_counters(tmp_path / "f.csv", "FETCH_SIZE", [(comb, 1000.0), (comb, 1002.0), (comb, 998.0), (probe, copy / 2048)])
    write_counters(tmp_path / "w.csv", "WRITE_SIZE", [(comb, 100.0), (comb, 100.0), (comb, 100.0), (probe, copy / 1024)])
    out = tmp_path / "combine_x_hbm_counters.txt"
    profsum.main(["hbm", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "--kernel", "combine", "--workload", "x",
                  "--out", str(out), "--algorithmic", str(4 * 2200 * 1024), "--launches-per-call", "4"])
    fields = dict(line.split(": ", 1) for line in out.read_text().splitlines() if not line.startswith("#"))
    assert float(fields["fetch_scale"]) == 2.0 and float(fields["write_scale"]) == 1.0
    assert int(fields["hbm_bytes_per_launch"]) == (1000 * 2 + 100) * 1024  # medians, scaled
    assert int(fields["hbm_bytes_per_call"]) == 4 * (1000 * 2 + 100) * 1024
    assert abs(float(fields["traffic_over_algorithmic"]) - 2100 / 2200) < 1e-4
    assert fields["kernel_sources"] == kernel_source_hash("combine")


def test_bench_reads_traffic_per_call_and_checks_the_source_hash(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    good = prof / "combine_w_hbm_counters.txt"
    good.write_text(f"kernel_sources: {kernel_source_hash('combine')}\nhbm_bytes_per_launch: 10\n"
                    f"hbm_bytes_per_call: 40\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.read_traffic("combine", "w") == 40.0
    good.write_text("kernel_sources: 0000000000000000\nhbm_bytes_per_launch: 10\n")
    assert bench.read_traffic("combine", "w") is None
    assert bench.read_traffic("dispatch", "w") is None


def test_sweep_table_lists_step_records(tmp_path, capsys):
    import json

    path = tmp_path / "s.jsonl"
    recs = [{"kind": "probe", "mode": "write", "GBs": 5000.0},
            {"kind": "step", "shape": {"T": 16384, "H": 7168, "E": 256, "k": 2}, "variant": "lds1", "slab": 0, "num_cus": "96",
             "GBs": {"layout": 40.0, "dispatch": 7012.4, "combine": 5401.0}},
            {"kind": "step", "shape": {"T": 128, "H": 7168, "E": 256, "k": 8}, "variant": "vgpr", "slab": 2, "num_cus": "0",
             "GBs": {"layout": 40.0, "dispatch": None, "combine": 812.0}}]
    path.write_text("\n".join(json.dumps(r) for r in recs) + "\n")
    profsum.main(["sweep", str(path), "--title", "t", "--command", "c1", "--command", "c2"])
    out = capsys.readouterr().out.splitlines()
    assert out[:3] == ["# t", "# command: c1", "# command: c2"]
    rows = [line.split() for line in out if line and line[0] != "#" and not line.lstrip().startswith("k ")]
    assert rows == [["2", "16384", "7168", "256", "lds1", "0", "96", "7012", "5401", "-", "-", "-"],
                    ["8", "128", "7168", "256", "vgpr", "2", "0", "-", "812", "-", "-", "-"]]


def test_bench_shape_overrides():
    import pytest

    assert bench.parse_shape("k=2,T=16384") == {"k": 2, "T": 16384}
    assert bench.parse_shape(None) == {}
    for bad in ("q=3", "k=two", "k"):
        with pytest.raises(SystemExit):
            bench.parse_shape(bad)


def test_latency_table_formats_every_record_kind(tmp_path, capsys):
    from bulk_async_tensor_amd import profsum

    recs = [
        {"kind": "unloaded", "level": "HBM", "set_MiB": 4096, "chase_ns_per_hop": 420.0,
         "chase_cycles_per_hop": 1000.0, "clock_GHz": 2.4},
        {"kind": "loaded", "cus": 24, "waves_per_cu": 8, "vectors_per_lane": 8,
         "requested_KiB_in_flight_per_cu": [64, 128], "GBs": 1387.4, "GBs_per_cu": 57.81,
         "B_per_clk_per_cu": 23.91, "latency_ns": 621.2, "littles_law_KiB_in_flight_per_cu": 35.1},
        {"kind": "residency", "cus": 24, "waves_per_cu": 16, "vectors_per_lane": 8, "source": "Infinity Cache",
         "loads": "cacheable", "MiB": 128, "GBs": 2065.2, "GBs_per_cu": 86.05, "B_per_clk_per_cu": 35.69,
         "chase_ns_per_hop": 563.0},
    ]
    path = tmp_path / "lat.jsonl"
    path.write_text("\n".join(__import__("json").dumps(r) for r in recs) + "\n")
    profsum.main(["latency", str(path), "--title", "t", "--command", "c"])
    text = capsys.readouterr().out
    assert "# command: c" in text
    assert "420.0" in text and "1387.4" in text and "35.1" in text and "86.05" in text


def test_budgets_table_scales_sums_per_call(tmp_path, capsys):
    """Per-budget counter table: FETCH/WRITE sums per kind over the calls,
    scaled by the copy probe's reading, and SQ medians per kind."""
    import json

    from bulk_async_tensor_amd import profsum

    disp = "void ep::(anonymous namespace)::dispatch_vgpr2_kernel<14, 6, true, true>(args)"
    copy = "void ep::(anonymous namespace)::bw_kernel<0, 8, 0>(args)"

    def counters(path, name, rows):
        with open(path, "w") as fh:
            fh.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
            for i, (kern, val) in enumerate(rows):
                fh.write(f'{i},"{kern}",{name},{val}\n')

    f = tmp_path / "f.csv"
    w = tmp_path / "w.csv"
    q = tmp_path / "q.csv"
    # copy probe: FETCH reads half the true 256 MiB, WRITE reads it exactly
    counters(f, "FETCH_SIZE", [(copy, 131072.0), (disp, 100.0), (disp, 300.0)])
    counters(w, "WRITE_SIZE", [(copy, 262144.0), (disp, 1000.0), (disp, 1000.0)])
    with open(q, "w") as fh:
        fh.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i in (1, 2):
            for name, val in (("GRBM_GUI_ACTIVE", 8000.0), ("SQ_LDS_BANK_CONFLICT", 0.0),
                              ("SQ_ACTIVE_INST_VALU", 256000.0 * i)):
                fh.write(f'{i},"{disp}",{name},{val}\n')
    log = tmp_path / "b.log"
    log.write_text(json.dumps({"cold_only": True, "steps": 1, "warmup": 1, "bytes": {"dispatch": 4096000}}) + "\n")
    profsum.main(["budgets", "--run", f"all:256:{f}:{w}:{q}:{log}", "--title", "t"])
    row = [line.split() for line in capsys.readouterr().out.splitlines() if line.startswith("all ")][0]
    # (400 KiB x 2 + 2000 KiB x 1) x 1024 / 2 calls = 1,433,600 bytes -> 1.43 MB, ratio 0.35
    assert row[:8] == ["all", "dispatch", "1", "0.41", "1.02", "1.43", "4.10", "0.3500"]
    # VALU busy: median of 256000 and 512000 over 256 CUs and GUI 1000 -> 150%
    assert row[9] == "150.00"
