"""Summaries of rocprofv3 output for the profiles/ directory.

  python -m bulk_async_tensor_amd.profsum trace <kernel_stats.csv> <bench.log> --command "..."
      kernel-trace statistics of our kernels beside the per-launch times the
      benchmark measured with HIP events in the same run.

  python -m bulk_async_tensor_amd.profsum sweep <sweep.jsonl>... --title "..." --command "..."
      the step records of bench.py --sweep files as one table (dispatch and
      combine GB/s per shape, variant and CU budget).

  python -m bulk_async_tensor_amd.profsum latency <latency.jsonl> --title "..." --command "..."
      the pointer-chase latencies and bytes-in-flight tables of bench.py --latency.

  python -m bulk_async_tensor_amd.profsum hbm <fetch_counter_collection.csv> <write_counter_collection.csv>
          --kernel dispatch|combine|layout|layout_dispatch --workload NAME --out FILE --command "..."
      HBM bytes per launch from FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
      each scaled by what the same counter reads for the copy probe, which
      reads and writes exactly --copy-bytes (default 256 MiB).
"""

import argparse
import csv
import json
import statistics
import sys

from .build import kernel_source_hash

# first match wins: the one-launch layout + dispatch kernels before the layout ones
KINDS = {
    "layout_dispatch": ("layout_dispatch",),
    "layout": ("layout_",),
    "dispatch": ("dispatch_",),
    "combine": ("combine_",),
    "combine_reduce": ("reduce_zero", "reduce_scatter", "reduce_convert"),
    "copy_probe": ("bw_kernel<0",),
}


def kind_of(name):
    short = name.replace("(anonymous namespace)", "anon").split("(")[0]
    if "ep::" not in short:
        return None
    for kind, keys in KINDS.items():
        if any(k in short for k in keys):
            return kind
    return None


def trace(args):
    rows = list(csv.DictReader(open(args.stats)))
    bench = None
    for line in open(args.bench_log):
        line = line.strip()
        if line.startswith("{") and ('"metric"' in line or '"cold_only"' in line):
            bench = json.loads(line)
    out = [f"# rocprofv3 kernel trace: {args.title}", f"# command: {args.command}", "",
           f"{'kernel':<60s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
    for r in rows:
        k = kind_of(r["Name"])
        if k is None:
            continue
        nm = r["Name"].replace("ep::(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        out.append(f"{nm[:60]:<60s} {r['Calls']:>6s} {float(r['AverageNs']) / 1e3:9.2f} "
                   f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f}")
    if bench and bench.get("cold_only"):
        out += ["", "same run, HIP events on the launch stream (bench.py --cold-only: every call after a 1 GiB "
                    "write, us per call; a phased combine call is several launches):"]
        for op, st in bench.get("us_per_op", {}).items():
            out.append(f"  {op}: {json.dumps(st)}")
    elif bench:
        out += ["", "same run, HIP events on the launch stream (bench.py, ms per launch):"]
        out.append("  " + json.dumps(bench.get("kernel_ms")))
        out.append(f"  roofline: {json.dumps(bench.get('roofline'))}")
    sys.stdout.write("\n".join(out) + "\n")


def per_kind(path, counter):
    vals = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        k = kind_of(r["Kernel_Name"])
        if k is not None:
            vals.setdefault(k, []).append(float(r["Counter_Value"]))
    return {k: statistics.median(v) for k, v in vals.items()}, {k: len(v) for k, v in vals.items()}


def hbm(args):
    fetch, nf = per_kind(args.fetch, "FETCH_SIZE")
    write, nw = per_kind(args.write, "WRITE_SIZE")
    copy_kib = args.copy_bytes / 1024.0
    f_scale = copy_kib / fetch["copy_probe"]
    w_scale = copy_kib / write["copy_probe"]
    k = args.kernel
    read_b = fetch[k] * f_scale * 1024.0
    write_b = write[k] * w_scale * 1024.0
    lines = [
        f"# HBM traffic per launch of ep_{k} on the {args.workload} workload (rocprofv3 --pmc)",
        f"# command (FETCH_SIZE pass): {args.command_fetch}",
        f"# command (WRITE_SIZE pass): {args.command_write}",
        f"# summarised by: python -m bulk_async_tensor_amd.profsum hbm ...",
        f"kernel: ep_{k}",
        f"workload: {args.workload}",
        f"kernel_sources: {kernel_source_hash(k)}",
        f"launches_fetch: {nf.get(k, 0)}",
        f"launches_write: {nw.get(k, 0)}",
        f"fetch_kib_per_launch: {fetch[k]:.1f}",
        f"write_kib_per_launch: {write[k]:.1f}",
        f"copy_probe_bytes: {args.copy_bytes}",
        f"copy_probe_fetch_kib: {fetch['copy_probe']:.1f}",
        f"copy_probe_write_kib: {write['copy_probe']:.1f}",
        f"fetch_scale: {f_scale:.5f}",
        f"write_scale: {w_scale:.5f}",
        f"hbm_read_bytes_per_launch: {read_b:.0f}",
        f"hbm_write_bytes_per_launch: {write_b:.0f}",
        f"hbm_bytes_per_launch: {read_b + write_b:.0f}",
    ]
    n = args.launches_per_call
    if n > 1:
        # one library call runs n launches of equal share (the phased combine on large batches)
        lines.append(f"launches_per_call: {n}")
        lines.append(f"hbm_bytes_per_call: {(read_b + write_b) * n:.0f}")
    if args.algorithmic:
        lines.append(f"algorithmic_bytes_per_call: {args.algorithmic}")
        lines.append(f"traffic_over_algorithmic: {(read_b + write_b) * n / args.algorithmic:.4f}")
    with open(args.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def sq(args):
    """LDS bank conflicts and VALU busy per kernel from one SQ counter pass.
    The CSV reports GRBM_GUI_ACTIVE summed over the XCDs; the busy-cycle
    denominator is that sum / xcds (the per-XCD value), as the derived
    metrics use the maximum over instances."""
    per = {}
    for r in csv.DictReader(open(args.counters)):
        k = kind_of(r["Kernel_Name"])
        if k is None:
            continue
        nm = r["Kernel_Name"].replace("ep::(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        per.setdefault((nm, r["Dispatch_Id"]), {})[r["Counter_Name"]] = float(r["Counter_Value"])
    by_kernel = {}
    for (nm, _), c in per.items():
        by_kernel.setdefault(nm, []).append(c)
    out = [f"# SQ counters per launch: {args.title}", f"# command: {args.command}",
           f"# LDSBankConflict% = 100*SQ_LDS_BANK_CONFLICT/GUI/CUs; conflict ratio = conflicts/(SQ_LDS_IDX_ACTIVE-"
           f"conflicts); VALUBusy% = 100*SQ_ACTIVE_INST_VALU/CUs/GUI; GUI = GRBM_GUI_ACTIVE/{args.xcds}; "
           f"CUs = {args.cus}", "",
           f"{'kernel':<46s} {'launches':>8s} {'LDS_conf%':>9s} {'conf_ratio':>10s} {'VALUBusy%':>9s} "
           f"{'VALU_insts':>11s} {'LDS_insts':>10s} {'waves':>7s}"]
    for nm, cs in by_kernel.items():
        med = {key: statistics.median(c.get(key, 0.0) for c in cs) for key in cs[0]}
        gui = med["GRBM_GUI_ACTIVE"] / args.xcds
        conf = med["SQ_LDS_BANK_CONFLICT"]
        idx = med["SQ_LDS_IDX_ACTIVE"]
        ratio = conf / (idx - conf) if idx > conf else 0.0
        out.append(f"{nm[:46]:<46s} {len(cs):8d} {100 * conf / gui / args.cus:9.3f} {ratio:10.3f} "
                   f"{100 * med['SQ_ACTIVE_INST_VALU'] / args.cus / gui:9.2f} {med['SQ_INSTS_VALU']:11.0f} "
                   f"{med['SQ_INSTS_LDS']:10.0f} {med['SQ_WAVES']:7.0f}")
    sys.stdout.write("\n".join(out) + "\n")


def sweep_table(args):
    """Step records of `bench.py --sweep` files as one table: dispatch and
    combine GB/s per shape, variant, slab setting (0: the kernels' default)
    and CU budget (0: the default launch)."""
    out = [f"# {args.title}"] + [f"# command: {c}" for c in args.command] + [
        "# GB/s are algorithmic bytes over the HIP-event time per launch; slab 0 = the kernels' default; "
        "CUs 0 = the library's default launch", "",
        f"{'k':>2s} {'T':>6s} {'H':>5s} {'E':>4s} {'variant':<8s} {'slab':>4s} {'CUs':>4s} {'dispatch GB/s':>14s} "
        f"{'combine GB/s':>13s} {'cold disp GB/s':>15s} {'cold comb GB/s':>15s} {'cold step GB/s':>15s}"]
    for path in args.jsonl:
        for line in open(path):
            r = json.loads(line)
            if r.get("kind") != "step":
                continue
            sh = r.get("shape") or {}
            g = r.get("GBs") or {}
            cell = lambda v, w: f"{v:{w}.0f}" if v else f"{'-':>{w}s}"
            c = (r.get("cold") or {}).get("GBs_p50") or {}
            cstep = (r.get("cold") or {}).get("value")
            out.append(f"{sh.get('k', 0):2d} {sh.get('T', 0):6d} {sh.get('H', 0):5d} {sh.get('E', 0):4d} "
                       f"{r['variant']:<8s} {r.get('slab', 0):4d} {r['num_cus']:>4s} {cell(g.get('dispatch'), 14)} "
                       f"{cell(g.get('combine'), 13)} {cell(c.get('dispatch'), 15)} {cell(c.get('combine'), 15)} "
                       f"{cell(cstep, 15)}")
    sys.stdout.write("\n".join(out) + "\n")


def budgets_table(args):
    """HBM bytes per call, LDS bank conflicts and VALU busy per kernel kind
    across CU budgets, from one FETCH_SIZE, one WRITE_SIZE and one SQ pass
    per budget over bench.py --cold-only.  Each --run is
    LABEL:CUS:FETCH_CSV:WRITE_CSV:SQ_CSV:BENCH_LOG; the bench log's last
    line gives the algorithmic bytes and the number of calls (steps plus
    warm-up).  Counters are scaled by what they read for the 256 MiB copy
    probe of the same pass."""
    out = [f"# {args.title}"] + [f"# command: {c}" for c in args.command] + [
        "# HBM MB = (FETCH_SIZE x fetch scale + WRITE_SIZE x write scale) summed over a kind's launches, per call",
        "# (launches / launches per call, the latter rounded from launches / calls);",
        "# ratio = HBM bytes / algorithmic bytes; LDS_conf% and VALUBusy% are medians over the kind's launches,",
        "# over the budget's CUs (GUI = GRBM_GUI_ACTIVE / 8).", "",
        f"{'budget':<8s} {'kernel':<10s} {'launches/call':>13s} {'read MB':>9s} {'write MB':>9s} {'HBM MB':>9s} "
        f"{'alg MB':>9s} {'ratio':>7s} {'LDS_conf%':>9s} {'VALUBusy%':>9s}"]
    for spec in args.run:
        label, cus, fetch_csv, write_csv, sq_csv, log = spec.split(":")
        cus = int(cus)
        bench = None
        for line in open(log):
            if line.strip().startswith("{") and '"cold_only"' in line:
                bench = json.loads(line)
        calls = bench["steps"] + bench.get("warmup", 0)
        fsum, fn = sums_of(fetch_csv, "FETCH_SIZE")
        wsum, _ = sums_of(write_csv, "WRITE_SIZE")
        copy_kib = args.copy_bytes / 1024.0
        f_scale = copy_kib / (fsum["copy_probe"] / fn["copy_probe"])
        w_scale = copy_kib / (wsum["copy_probe"] / fn["copy_probe"])
        sq = sq_of(sq_csv)
        for kind in ("layout", "dispatch", "combine"):
            if kind not in fsum:
                continue
            # launches per call from the counts (the setup's own first
            # launches of layout and dispatch make a few more than calls x n)
            per_call = max(1, round(fn[kind] / calls))
            ncalls = fn[kind] / per_call
            rd = fsum[kind] * f_scale * 1024.0 / ncalls
            wr = wsum.get(kind, 0.0) * w_scale * 1024.0 / ncalls
            hbm = rd + wr
            alg = bench["bytes"].get(kind) or 0
            q = sq.get(kind, {})
            gui = q.get("GRBM_GUI_ACTIVE", 0.0) / args.xcds
            conf = 100 * q.get("SQ_LDS_BANK_CONFLICT", 0.0) / gui / cus if gui else 0.0
            valu = 100 * q.get("SQ_ACTIVE_INST_VALU", 0.0) / cus / gui if gui else 0.0
            out.append(f"{label:<8s} {kind:<10s} {per_call:13d} {rd / 1e6:9.2f} {wr / 1e6:9.2f} "
                       f"{hbm / 1e6:9.2f} {alg / 1e6:9.2f} {(hbm / alg if alg else 0.0):7.4f} {conf:9.3f} {valu:9.2f}")
    sys.stdout.write("\n".join(out) + "\n")


def sums_of(path, counter):
    """Sum of a counter and launch count per kernel kind."""
    tot, cnt = {}, {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        k = kind_of(r["Kernel_Name"])
        if k is not None:
            tot[k] = tot.get(k, 0.0) + float(r["Counter_Value"])
            cnt[k] = cnt.get(k, 0) + 1
    return tot, cnt


def sq_of(path):
    """Median per kind of each SQ/GRBM counter over the kind's launches."""
    per = {}
    for r in csv.DictReader(open(path)):
        k = kind_of(r["Kernel_Name"])
        if k is None:
            continue
        per.setdefault(k, {}).setdefault(r["Dispatch_Id"], {})[r["Counter_Name"]] = float(r["Counter_Value"])
    out = {}
    for k, launches in per.items():
        names = set().union(*[set(c) for c in launches.values()])
        out[k] = {n: statistics.median(c.get(n, 0.0) for c in launches.values()) for n in names}
    return out


def overlap_table(args):
    """The records of bench.py --overlap: the step on n masked CUs beside the
    computation on the other CUs, each alone on its partition and both
    together, and both together without a partition."""
    out = [f"# {args.title}"] + [f"# command: {c}" for c in args.command] + [""]
    for path in args.jsonl:
        for line in open(path):
            r = json.loads(line)
            if r["kind"] == "overlap_base":
                out.append(f"{r['compute']} computation alone on all CUs: {r['gemm_ms_all_cus']:.3f} ms "
                           f"({r['gemm_TFLOPs_all_cus']:.0f} TFLOP/s); step ({r['workload']}) alone on all CUs: "
                           f"{r['step_ms_all_cus'] * 1e3:.1f} us")
                out.append(f"  {'copy/compute CUs':<17s} {'compute alone':>14s} {'compute with step':>18s} "
                           f"{'slowdown':>9s} {'step alone us':>14s} {'step with compute us':>21s} {'slowdown':>9s} "
                           f"{'step GB/s':>10s}")
            elif r.get("partition") == "none":
                out.append(f"  {'none (shared)':<17s} {'-':>14s} {r['gemm_ms'] * 1e3:15.1f} us {r['gemm_slowdown']:9.3f} "
                           f"{'-':>14s} {r['step_ms'] * 1e3:21.1f} {r['step_slowdown']:9.3f} {'-':>10s}")
            else:
                out.append(f"  {r['partition']:<17s} {r['gemm_ms_alone_on_rest'] * 1e3:11.1f} us "
                           f"{r['gemm_ms'] * 1e3:15.1f} us {r['gemm_slowdown_vs_alone_on_rest']:9.3f} "
                           f"{r['step_ms_alone_on_n'] * 1e3:14.1f} {r['step_ms'] * 1e3:21.1f} "
                           f"{r['step_slowdown_vs_alone_on_n']:9.3f} {r['step_GBs_concurrent']:10.0f}")
        out.append("")
    sys.stdout.write("\n".join(out) + "\n")


def probes_table(args):
    """The streaming-probe matrix of bench.py --probe-sweep: GB/s per
    operation, depth and load policy (rows) at each CU budget (columns)."""
    recs = [json.loads(line) for path in args.jsonl for line in open(path) if line.strip()]
    budgets = sorted({r["num_cus"] for r in recs}, key=lambda b: (b == 0, b))
    keys = []
    for r in recs:
        k = (r["op"], r["depth"], r["policy"])
        if k not in keys:
            keys.append(k)
    val = {(r["op"], r["depth"], r["policy"], r["num_cus"]): r["GBs"] for r in recs}
    out = [f"# {args.title}"] + [f"# command: {c}" for c in args.command] + [
        "# GB/s of bytes moved (copy: read + write; mixes: both sides), 1 GiB buffers, mean of 10 launches; "
        "budget 0 = the probe's ordinary grid on every CU", "",
        f"{'op':<9s} {'depth':>5s} {'policy':<7s} " + " ".join(f"{('all' if b == 0 else str(b)):>7s}" for b in budgets)]
    for op, d, pol in keys:
        out.append(f"{op:<9s} {d:5d} {pol:<7s} " + " ".join(
            f"{val[(op, d, pol, b)]:7.0f}" if (op, d, pol, b) in val else f"{'-':>7s}" for b in budgets))
    sys.stdout.write("\n".join(out) + "\n")


def latency_table(args):
    """The records of bench.py --latency as three tables: unloaded chase
    latency per memory level; read GB/s against requested bytes in flight at
    the CU budgets, with the loaded latency and Little's-law bytes in flight;
    and the per-CU rate by where the streamed data lives."""
    recs = [json.loads(line) for path in args.jsonl for line in open(path) if line.strip()]
    out = [f"# {args.title}"] + [f"# command: {c}" for c in args.command] + [""]
    out.append("unloaded latency (one wave, random chain of 256-byte nodes, nothing else running):")
    out.append(f"  {'level':<22s} {'set MiB':>8s} {'ns/hop':>8s} {'cycles/hop':>11s} {'clock GHz':>10s}")
    for r in recs:
        if r["kind"] == "unloaded":
            out.append(f"  {r['level']:<22s} {r['set_MiB']:8d} {r['chase_ns_per_hop']:8.1f} "
                       f"{r['chase_cycles_per_hop']:11.1f} {r['clock_GHz']:10.3f}")
    out += ["", "streaming nt reads of 2 GiB from HBM beside a pointer chase on a streaming CU (fresh 4 GiB chain):",
            f"  {'CUs':>4s} {'waves/CU':>8s} {'vec/lane':>8s} {'req KiB/CU':>11s} {'GB/s':>8s} {'GB/s/CU':>8s} "
            f"{'B/clk/CU':>8s} {'lat ns':>7s} {'Little KiB/CU':>13s}"]
    for r in recs:
        if r["kind"] == "loaded":
            req = r["requested_KiB_in_flight_per_cu"]
            out.append(f"  {r['cus']:4d} {r['waves_per_cu']:8d} {r['vectors_per_lane']:8d} {req[0]:>5d}-{req[1]:<5d} "
                       f"{r['GBs']:8.1f} {r['GBs_per_cu']:8.2f} {r['B_per_clk_per_cu']:8.2f} {r['latency_ns']:7.1f} "
                       f"{r['littles_law_KiB_in_flight_per_cu']:13.1f}")
    out += ["", "per-CU read rate by where the data lives (same depth; the chase on a fresh HBM chain):",
            f"  {'CUs':>4s} {'waves/CU':>8s} {'vec/lane':>8s} {'source':<26s} {'loads':<9s} {'MiB':>5s} {'GB/s':>8s} "
            f"{'GB/s/CU':>8s} {'B/clk/CU':>8s} {'chase ns':>8s}"]
    for r in recs:
        if r["kind"] == "residency":
            out.append(f"  {r['cus']:4d} {r['waves_per_cu']:8d} {r['vectors_per_lane']:8d} {r['source']:<26s} "
                       f"{r['loads']:<9s} {r['MiB']:5d} {r['GBs']:8.1f} {r['GBs_per_cu']:8.2f} "
                       f"{r['B_per_clk_per_cu']:8.2f} {r['chase_ns_per_hop']:8.1f}")
    sys.stdout.write("\n".join(out) + "\n")


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats")
    t.add_argument("bench_log")
    t.add_argument("--title", default="")
    t.add_argument("--command", default="")
    h = sub.add_parser("hbm")
    h.add_argument("fetch")
    h.add_argument("write")
    h.add_argument("--kernel", required=True, choices=["layout", "dispatch", "combine", "layout_dispatch"])
    h.add_argument("--workload", required=True)
    h.add_argument("--out", required=True)
    h.add_argument("--copy-bytes", type=int, default=256 << 20)
    h.add_argument("--algorithmic", type=int, default=0, help="algorithmic bytes of one library call")
    h.add_argument("--launches-per-call", type=int, default=1)
    h.add_argument("--command-fetch", default="")
    h.add_argument("--command-write", default="")
    q = sub.add_parser("sq")
    q.add_argument("counters")
    q.add_argument("--title", default="")
    q.add_argument("--command", default="")
    q.add_argument("--xcds", type=int, default=8)
    q.add_argument("--cus", type=int, default=256)
    w = sub.add_parser("sweep")
    w.add_argument("jsonl", nargs="+")
    w.add_argument("--title", default="")
    w.add_argument("--command", action="append", default=[])
    bu = sub.add_parser("budgets")
    bu.add_argument("--run", action="append", required=True,
                    help="LABEL:CUS:FETCH_CSV:WRITE_CSV:SQ_CSV:BENCH_LOG, one per budget")
    bu.add_argument("--title", default="")
    bu.add_argument("--command", action="append", default=[])
    bu.add_argument("--copy-bytes", type=int, default=256 << 20)
    bu.add_argument("--xcds", type=int, default=8)
    ov = sub.add_parser("overlap")
    ov.add_argument("jsonl", nargs="+")
    ov.add_argument("--title", default="")
    ov.add_argument("--command", action="append", default=[])
    pr = sub.add_parser("probes")
    pr.add_argument("jsonl", nargs="+")
    pr.add_argument("--title", default="")
    pr.add_argument("--command", action="append", default=[])
    lt = sub.add_parser("latency")
    lt.add_argument("jsonl", nargs="+")
    lt.add_argument("--title", default="")
    lt.add_argument("--command", action="append", default=[])
    args = p.parse_args(argv)
    {"trace": trace, "hbm": hbm, "sq": sq, "sweep": sweep_table, "latency": latency_table,
     "budgets": budgets_table, "overlap": overlap_table, "probes": probes_table}[args.mode](args)


if __name__ == "__main__":
    main()
