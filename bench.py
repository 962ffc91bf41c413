"""Benchmark of the MoE row-movement hot path on one MI355X.

One step = ep_layout + ep_dispatch + ep_combine over one batch of the chosen
workload (default: the prefill shape, T=16384 tokens, H=7168 bf16, E=64
experts, top-6 with Zipf(1.0) routing, the largest of the workloads),
inputs resident in HBM.  The expert op between dispatch and combine is
applied once before timing and is not part of a step.

Headline (``value``): every op timed alone with cold caches -- before each
call 1 GiB of other memory is written, which evicts the L2s and the 256 MB
Infinity Cache, and the call sits between two HIP events on its stream --
over max(steps, --cold) such steps; value = algorithmic bytes of a step /
(median layout + median dispatch + median combine).  The roofline entry is
the dominant kernel's algorithmic bytes over its mean cold time.  Warm
(back-to-back) figures, the training shape and a 24-CU budget are reported
as labelled extra keys, with the CPU oracle timed on the host.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--variant V]
  python bench.py --cold-only     # only the cold-protocol steps (for rocprofv3)
  python bench.py --sweep FILE   # CU-budget x variant sweep + copy ceilings, JSONL
"""

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dispatch+combine HBM GB/s and tokens/s on 1 MI355X at 24 CUs and all CUs"
HBM_PEAK_GBS = 8000.0


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--cold", type=int, default=50,
                   help="least number of cold-protocol steps (each op after a 1 GiB cache flush); "
                        "max(--steps, --cold) are timed")
    p.add_argument("--cold-only", action="store_true",
                   help="only the cold-protocol steps of the workload (a profiling run)")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the warm, 24-CU, training-shape and reduce-on-store extras")
    p.add_argument("--cold-study", action="store_true",
                   help="also time single launches with no flush and with write / read / write+read flushes")
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="prefill")
    p.add_argument("--variant", default="auto")
    p.add_argument("--budget", type=int, default=24, help="the restricted CU budget reported beside all CUs")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--sweep", default=None, help="write a CU x variant sweep as JSONL to this file")
    p.add_argument("--sweep-budgets", default="16,24,32,64,128,256,0")
    p.add_argument("--sweep-variants", default="vgpr,vgpr2,lds1,lds2,vgpr_cached")
    p.add_argument("--sweep-slabs", default="0", help="slab sizes (vectors per lane) to sweep; 0 = default")
    p.add_argument("--shape", default=None,
                   help="--sweep and --kernels-only: override the workload's sizes, e.g. k=2,T=16384 (keys T, H, E, k)")
    p.add_argument("--no-probes", action="store_true", help="skip the streaming probes in --sweep")
    p.add_argument("--sweep-cold", type=int, default=0,
                   help="--sweep: also time this many cold-protocol steps per budget and variant")
    p.add_argument("--only-all", action="store_true", help="time only the all-CU configuration")
    p.add_argument("--graph", action="store_true", help="also time the step captured in a HIP graph")
    p.add_argument("--fused", action="store_true", help="layout and dispatch through ep_layout_dispatch")
    p.add_argument("--overlap", default=None,
                   help="CU-partitioned overlap with computation, JSONL to this file (budgets from --sweep-budgets)")
    p.add_argument("--overlap-compute", default="gemm", choices=["gemm", "mfma"],
                   help="the computation beside the copies: a torch bf16 GEMM or the matrix-core probe")
    p.add_argument("--kernels-only", action="store_true",
                   help="a few launches of each kernel and of a 256 MiB copy probe (for counter passes)")
    p.add_argument("--probe-sweep", default=None, help="write a streaming-probe matrix as JSONL to this file")
    p.add_argument("--no-reduce", action="store_true", help="skip timing the reduce-on-store combine")
    p.add_argument("--latency", default=None,
                   help="pointer-chase latencies and the bytes-in-flight vs read GB/s table at --budget CUs, "
                        "JSONL to this file")
    return p.parse_args()


class Setup:
    """Device buffers of one workload and the step that runs on them."""

    def __init__(self, name, stream=None, shape=None):
        import numpy as np
        import torch

        import bulk_async_tensor_amd as ep
        from synth import algorithmic_bytes, make_workload

        self.ep = ep
        self.torch = torch
        self.stream = stream
        self.gather = False  # True: dispatch through ep_dispatch_rows (gather form)
        self.fused = False   # True: layout and dispatch through ep_layout_dispatch
        dev = torch.device("cuda:0")
        wl = make_workload(name, **(shape or {}))
        self.wl = wl
        c = self.cfg = wl.config
        self.T, self.H, self.E, self.k = c.T, c.H, c.E, c.k
        R = c.T * c.k
        self.idx = torch.from_numpy(wl.topk_idx).to(dev)
        self.w = torch.from_numpy(wl.topk_w).to(dev)
        i32 = dict(dtype=torch.int32, device=dev)
        self.counts = torch.empty(c.E, **i32)
        self.offsets = torch.empty(c.E + 1, **i32)
        self.dest_row = torch.empty((c.T, c.k), **i32)
        self.src_token = torch.empty(R, **i32)
        self.status = torch.empty(1, **i32)
        self.ws = torch.empty(max(16, ep.ep_layout_workspace_bytes(c.T, c.k, c.E)), dtype=torch.uint8, device=dev)
        self.out = torch.empty((c.T, c.H), dtype=torch.bfloat16, device=dev)
        self.do_dispatch = c.ops != "combine"
        self.layout()
        if self.do_dispatch:
            self.x = torch.from_numpy(wl.x.view(np.int16)).to(dev).view(torch.bfloat16)
            self.recv = torch.empty((R, c.H), dtype=torch.bfloat16, device=dev)
            ep.ep_dispatch(self.x, self.dest_row, self.recv)
            if c.expert == "scale":
                # expert op (not timed): y[r] = bf16(s_e * recv[r]) for the expert e of row r
                s = torch.from_numpy(wl.scales).to(dev)
                row_scale = torch.repeat_interleave(s, self.counts.long(), output_size=R)
                self.y = (self.recv.float() * row_scale[:, None]).to(torch.bfloat16)
            else:
                self.y = self.recv  # identity expert: combine reads what dispatch wrote
        else:
            self.y = torch.from_numpy(wl.y.view(np.int16)).to(dev).view(torch.bfloat16)
        torch.cuda.synchronize()
        if int(self.status.item()) != 0:
            raise RuntimeError("layout flagged the routing as invalid")
        self.bytes = algorithmic_bytes(c.T, c.H, c.k, c.E)
        if not self.do_dispatch:
            self.bytes["dispatch"] = 0
        self.step_bytes = sum(self.bytes.values())

    def layout(self):
        if self.fused and self.do_dispatch:
            self.ep.ep_layout_dispatch(self.idx, self.E, self.x, self.recv, self.counts, self.offsets,
                                       self.dest_row, self.src_token, self.status, self.ws, stream=self.stream)
            return
        self.ep.ep_layout(self.idx, self.E, self.counts, self.offsets, self.dest_row, self.src_token, self.status,
                          self.ws, stream=self.stream)

    def dispatch(self):
        if self.do_dispatch and not self.fused:
            if self.gather:
                self.ep.ep_dispatch_rows(self.x, self.src_token, self.recv, stream=self.stream)
            else:
                self.ep.ep_dispatch(self.x, self.dest_row, self.recv, stream=self.stream)

    def combine(self):
        self.ep.ep_combine(self.y, self.dest_row, self.w, self.out, stream=self.stream)

    def kernel_ms(self, fn, reps):
        """ms per launch of one kernel: `reps` back-to-back launches captured
        in a HIP graph and replayed once between two HIP events on the
        launch stream, so that the binding's per-call host cost (a few us)
        does not stretch short kernels.  Falls back to eager launches if the
        capture fails."""
        torch = self.torch
        stream = self.stream if self.stream is not None else torch.cuda.current_stream()
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        try:
            with torch.cuda.graph(g, stream=self.stream):
                for _ in range(reps):
                    fn()
        except Exception:  # pragma: no cover - depends on the runtime
            g = None
            torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            if g is not None:
                g.replay()  # warm
            e0.record(stream)
            if g is not None:
                g.replay()
            else:
                for _ in range(reps):
                    fn()
            e1.record(stream)
        torch.cuda.synchronize()
        self.kernel_timing = "hip graph of back-to-back launches" if g is not None else "eager back-to-back launches"
        del g
        return e0.elapsed_time(e1) / reps

    def run(self, steps, warmup):
        """Whole steps: `steps` back-to-back steps between two synchronisations
        (no events inside the loop).  Per kernel: kernel_ms() over `steps`
        launches of that kernel alone; returns ms per step and ms per launch."""
        torch = self.torch
        for _ in range(warmup):
            self.layout()
            self.dispatch()
            self.combine()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.layout()
            self.dispatch()
            self.combine()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        per = {}
        for name, fn in (("layout", self.layout), ("dispatch", self.dispatch), ("combine", self.combine)):
            if name == "dispatch" and (not self.do_dispatch or self.fused):
                per[name] = 0.0
                continue
            per[name] = self.kernel_ms(fn, steps)
        return ms, per


def cold_times(s, iters, flush_mode="write"):
    """Per-launch times with cold caches: before each launch 1 GiB of other
    memory is written (torch fill), read (the read probe) or both, which
    evicts the L2s and the 256 MB Infinity Cache ("none": no flush, one launch
    at a time); one launch sits between two HIP events on its stream.
    Returns {kernel: [p10, median, p90]} in us."""
    import bulk_async_tensor_amd as ep

    torch = s.torch
    stream = s.stream if s.stream is not None else torch.cuda.current_stream()
    flush = torch.empty(1 << 28, dtype=torch.int32, device="cuda:0")
    sink = torch.empty(4, dtype=torch.int32, device="cuda:0")
    flush.fill_(1)
    out = {}
    for name, fn in (("layout", s.layout), ("dispatch", s.dispatch), ("combine", s.combine)):
        if name == "dispatch" and not s.do_dispatch:
            continue
        fn()
        evs = []
        for i in range(iters):
            if "write" in flush_mode:
                with torch.cuda.stream(stream):
                    flush.fill_(i)
            if "read" in flush_mode:
                ep.ep_bw_probe(1, flush, sink, flush.numel() * 4, stream=stream)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        pick = lambda q: us[min(len(us) - 1, int(q * (len(us) - 1) + 0.5))]
        out[name] = [round(pick(0.1), 2), round(pick(0.5), 2), round(pick(0.9), 2)]
    del flush
    return out


def cold_steps(s, iters, warmup=3):
    """The cold-cache protocol: in every step each op (layout, dispatch,
    combine) runs once right after 1 GiB of other memory has been written (a
    torch fill on the launch stream, which evicts the L2s and the 256 MB
    Infinity Cache), between two HIP events on the launch stream.  `warmup`
    such steps run first and are not recorded.  Returns {op: [us per call]}."""
    torch = s.torch
    stream = s.stream if s.stream is not None else torch.cuda.current_stream()
    flush = torch.empty(1 << 28, dtype=torch.int32, device="cuda:0")
    ops = [("layout", s.layout)]
    if s.do_dispatch and not s.fused:
        ops.append(("dispatch", s.dispatch))
    ops.append(("combine", s.combine))
    evs = {name: [] for name, _ in ops}
    for i in range(warmup + iters):
        for name, fn in ops:
            with torch.cuda.stream(stream):
                flush.fill_(i)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            if i >= warmup:
                evs[name].append((e0, e1))
    torch.cuda.synchronize()
    del flush
    return {name: [a.elapsed_time(b) * 1e3 for a, b in v] for name, v in evs.items()}


def summarize(us):
    """p10 / p50 / p90 / mean of a list of times (us)."""
    v = sorted(us)
    pick = lambda q: v[min(len(v) - 1, int(q * (len(v) - 1) + 0.5))]
    return {"p10": round(pick(0.1), 2), "p50": round(pick(0.5), 2), "p90": round(pick(0.9), 2),
            "mean": round(sum(v) / len(v), 2), "n": len(v)}


def cold_report(s, iters, warmup):
    """Cold-protocol steps of Setup s: per-op statistics, the step time (sum
    of the per-op medians), step GB/s and tokens/s."""
    raw = cold_steps(s, iters, warmup)
    st = {op: summarize(v) for op, v in raw.items()}
    t_us = sum(v["p50"] for v in st.values())
    return {
        "us_per_op": st,
        "GBs_p50": {op: round(s.bytes[op] / (v["p50"] * 1e3), 1) for op, v in st.items() if s.bytes[op]},
        "step_us": round(t_us, 2),
        "value": round(s.step_bytes / (t_us * 1e3), 2),
        "tokens_per_s": round(s.T / (t_us * 1e-6), 1),
    }


def budget_probes(budget):
    """Streaming ceilings (GB/s of bytes moved) on a persistent grid of
    `budget` CUs: a plain copy (read and written bytes both counted), nt
    reads, 8 and 32 KiB-per-wave writes, the phased 8:1 mix (combine's ratio)
    and the 1:8 mix (dispatch's).  Best of three timings of 10 launches over
    1 GiB."""
    import torch

    import bulk_async_tensor_amd as ep

    n = 1 << 30
    a = torch.empty(n // 4, dtype=torch.int32, device="cuda:0")
    b = torch.empty_like(a)
    once = min(n, budget * 16 * (128 << 10))
    out = {}
    ep.ep_set_num_cus(budget)
    try:
        for mode, label, nb in ((0, "copy", n), (1, "read", n), (2, "write", n), (0x22, "write32", n),
                                (5, "mix1to8", n), (7, "mix8to1_phase_once", once)):
            for _ in range(3):
                ep.ep_bw_probe(mode, a, b, nb)
            best = None
            for _ in range(3):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(10):
                    ep.ep_bw_probe(mode, a, b, nb)
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / 10
                best = ms if best is None else min(best, ms)
            moved = 2 * nb if mode == 0 else nb + nb // 8 if mode in (5, 7) else nb
            out[label] = round(moved / best / 1e6, 1)
    finally:
        ep.ep_set_num_cus(0)
    del a, b
    return out


def cpu_model():
    """The first processor's model name from /proc/cpuinfo, with its family,
    model and stepping numbers (a virtual machine may report a short name)."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if not line.strip():
                    break  # end of the first processor's block
                key, _, val = line.partition(":")
                fields.setdefault(key.strip(), val.strip())
    except OSError:  # pragma: no cover - non-Linux
        return None
    name = fields.get("model name")
    if name is None:
        return None
    ids = [f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields]
    return f"{name} ({', '.join(ids)})" if ids else name


def reduce_times(s, steps, budgets):
    """ep_combine_reduce (zero fill, scatter-add with fp32 atomics, bf16
    conversion: three launches) on the workload's expert outputs: `steps`
    back-to-back calls between two HIP events on the launch stream, per CU
    budget.  GB/s uses the combine's algorithmic bytes, so the figure compares
    directly with ep_combine's."""
    torch, ep = s.torch, s.ep
    ws = torch.empty(max(16, ep.ep_combine_reduce_workspace_bytes(s.T, s.H)), dtype=torch.uint8, device="cuda:0")
    out = torch.empty_like(s.out)
    stream = torch.cuda.current_stream()

    def call():
        ep.ep_combine_reduce(s.y, s.src_token, s.dest_row, s.w, out, workspace=ws, stream=stream)

    res = {}
    for b in budgets:
        ep.ep_set_num_cus(b)
        for _ in range(3):
            call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        res["all" if b == 0 else f"cu{b}"] = {"ms": round(ms, 5), "GBs": round(s.bytes["combine"] / (ms * 1e6), 1)}
    ep.ep_set_num_cus(0)
    # the same inputs through ep_combine: share of bit-identical elements and
    # the largest absolute difference (the orders of the k additions differ)
    s.combine()
    torch.cuda.synchronize()
    a, b = out.float(), s.out.float()
    res["bit_identical_frac_vs_ep_combine"] = round(float((a == b).float().mean().item()), 6) if a.numel() else 1.0
    res["max_abs_diff_vs_ep_combine"] = float((a - b).abs().max().item()) if a.numel() else 0.0
    del ws
    return res


def read_traffic(kernel, workload):
    """HBM bytes per library call (one launch, or the several of a phased
    combine) from the committed counter summary, or None when it is missing
    or was taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            m = re.match(r"^([a-z_]+):\s*(\S+)", line.strip())
            if m:
                fields[m.group(1)] = m.group(2)
    from bulk_async_tensor_amd.build import kernel_source_hash

    if fields.get("kernel_sources") != kernel_source_hash(kernel):
        return None
    try:
        return float(fields.get("hbm_bytes_per_call", fields["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(name, seconds, gpu=None):
    """The oracle as it stands, on the host, over the whole workload, repeated
    until about `seconds` of CPU work; reported in the metric's unit.  With
    `gpu` (the Setup whose step was timed), the oracle's outputs of the last
    pass are also compared with the GPU's outputs of the same inputs."""
    import oracle
    from synth import algorithmic_bytes, make_workload

    wl = make_workload(name)
    c = wl.config
    y_fixed = wl.y
    scales = wl.scales
    passes = 0
    t_total = 0.0
    # one core: this process pinned to a single CPU, BLAS / OpenMP pools at one thread
    from threadpoolctl import threadpool_limits

    cores_before = os.sched_getaffinity(0)
    pinned = min(cores_before)
    os.sched_setaffinity(0, {pinned})
    try:
        with threadpool_limits(limits=1):
            t_start = time.perf_counter()
            while True:
                t0 = time.perf_counter()
                lay = oracle.layout(wl.topk_idx, c.E)
                if c.ops != "combine":
                    recv = oracle.dispatch(wl.x, lay["dest_row"], c.T * c.k)
                t1 = time.perf_counter()
                # the expert op sits between the two and is not part of a step
                if c.ops == "combine":
                    y = y_fixed
                elif c.expert == "scale":
                    y = oracle.expert_scale(recv, lay["offsets"], scales)
                else:
                    y = recv
                t2 = time.perf_counter()
                out = oracle.combine(y, lay["dest_row"], wl.topk_w)
                t3 = time.perf_counter()
                t_total += (t1 - t0) + (t3 - t2)
                passes += 1
                if time.perf_counter() - t_start >= seconds:
                    break
    finally:
        os.sched_setaffinity(0, cores_before)
    per_step = t_total / passes
    parity = None if gpu is None else parity_against(gpu, lay, recv if c.ops != "combine" else None, out)
    parity_fused = None
    if gpu is not None and c.ops != "combine":
        # layout and dispatch once more through the one-launch entry point, on
        # outputs overwritten with sentinels first
        for t in (gpu.counts, gpu.offsets, gpu.dest_row, gpu.src_token):
            t.fill_(-7)
        gpu.recv.view(gpu.torch.int16).fill_(0x7E57)
        gpu.fused = True
        gpu.layout()
        gpu.fused = False
        gpu.torch.cuda.synchronize()
        parity_fused = {k: v for k, v in parity_against(gpu, lay, recv, out).items() if not k.startswith("combine")}
    b = algorithmic_bytes(c.T, c.H, c.k, c.E)
    step_bytes = b["layout"] + b["combine"] + (b["dispatch"] if c.ops != "combine" else 0)
    return {
        "value": round(step_bytes / per_step / 1e9, 3),
        "unit": "GB/s",
        "tokens_per_s": round(c.T / per_step, 1),
        "s_per_step": round(per_step, 4),
        "cores": 1,
        "kind": "oracle",
        "sample": f"whole {name} workload (T={c.T}), {passes} pass(es) of layout+dispatch+combine, "
                  f"single-threaded numpy/Python pinned to CPU {pinned} with BLAS/OpenMP pools at 1 thread",
        "cpu_model": cpu_model(),
        "host_cpus_available": len(cores_before),
        "parity_of_timed_gpu_outputs": parity,
        "parity_of_one_launch_layout_dispatch": parity_fused,
    }


_ORACLE_WORKER = {}


def _oracle_worker_task(task):
    """One token slice of dispatch or combine, by the oracle's own functions,
    written into the shared output.  The worker maps the shared arrays (files
    named in the task) on first use."""
    import numpy as np

    import oracle

    spec, op, a, b = task
    W = _ORACLE_WORKER
    if W.get("spec") != spec:
        W.clear()
        for key, (path, shape, dtype) in spec.items():
            W[key] = np.memmap(path, dtype=dtype, mode="r+", shape=tuple(shape))
        W["spec"] = spec
    if op == "dispatch":
        oracle.dispatch(W["x"][a:b], W["dest"][a:b], W["recv"].shape[0], recv=W["recv"])
    else:
        W["out"][a:b] = oracle.combine(W["y"], W["dest"][a:b], W["w"][a:b])
    return b - a


def oracle_pool(workers):
    """Processes for the all-cores oracle leg.  Started before this process
    touches the GPU: they are new interpreters (spawn) that import no GPU
    library."""
    import multiprocessing as mp

    return mp.get_context("spawn").Pool(workers)


def cpu_baseline_parallel(name, seconds, pool, workers):
    """The same oracle functions on `workers` host processes: the layout as
    it stands in this process (its counting pass runs over the tokens in
    order), then dispatch and combine over token slices in a process pool,
    each slice writing its own rows of arrays shared through files
    (`pool` from oracle_pool(workers)).  The expert op is computed once beforehand (it is not part of a step).
    The last pass's outputs are compared with the one-process oracle's."""
    import shutil
    import tempfile

    import numpy as np

    import oracle
    from synth import algorithmic_bytes, make_workload

    wl = make_workload(name)
    c = wl.config
    R = c.T * c.k
    dispatch_too = c.ops != "combine"
    lay = oracle.layout(wl.topk_idx, c.E)
    recv1 = oracle.dispatch(wl.x, lay["dest_row"], R) if dispatch_too else None
    if not dispatch_too:
        y1 = wl.y
    elif c.expert == "scale":
        y1 = oracle.expert_scale(recv1, lay["offsets"], wl.scales)
    else:
        y1 = None  # identity: combine reads the shared receive buffer itself
    out1 = oracle.combine(y1 if y1 is not None else recv1, lay["dest_row"], wl.topk_w)

    tmp = tempfile.mkdtemp(prefix="ep_oracle_")
    try:
        arrays = {}

        def shared(key, shape, dtype, init=None):
            path = os.path.join(tmp, key)
            m = np.memmap(path, dtype=dtype, mode="w+", shape=shape)
            if init is not None:
                m[...] = init
            m.flush()
            arrays[key] = m
            return (path, list(shape), np.dtype(dtype).str)

        spec = {"dest": shared("dest", (c.T, c.k), np.int32, lay["dest_row"]),
                "w": shared("w", (c.T, c.k), np.float32, wl.topk_w),
                "out": shared("out", (c.T, c.H), np.uint16)}
        if dispatch_too:
            spec["x"] = shared("x", (c.T, c.H), np.uint16, wl.x)
            spec["recv"] = shared("recv", (R, c.H), np.uint16)
        if y1 is not None:
            spec["y"] = shared("y", (R, c.H), np.uint16, y1)
        else:
            spec["y"] = spec["recv"]
        chunks = max(1, workers * 4)
        bounds = np.linspace(0, c.T, chunks + 1).astype(int)
        slices = [(int(a), int(b)) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
        passes = 0
        t_total = 0.0
        pool.map(_oracle_worker_task, [(spec, "combine", 0, 1)] * (4 * workers))  # arrays mapped
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            lay_p = oracle.layout(wl.topk_idx, c.E)
            arrays["dest"][...] = lay_p["dest_row"]
            if dispatch_too:
                pool.map(_oracle_worker_task, [(spec, "dispatch", a, b) for a, b in slices])
            pool.map(_oracle_worker_task, [(spec, "combine", a, b) for a, b in slices])
            t_total += time.perf_counter() - t0
            passes += 1
            if time.perf_counter() - t_start >= seconds:
                break
        same = bool(np.array_equal(arrays["out"], out1) and
                    (not dispatch_too or np.array_equal(arrays["recv"], recv1)))
        arrays.clear()
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    per_step = t_total / passes
    b = algorithmic_bytes(c.T, c.H, c.k, c.E)
    step_bytes = b["layout"] + b["combine"] + (b["dispatch"] if dispatch_too else 0)
    return {
        "value": round(step_bytes / per_step / 1e9, 3),
        "unit": "GB/s",
        "tokens_per_s": round(c.T / per_step, 1),
        "s_per_step": round(per_step, 4),
        "cores": workers,
        "kind": "oracle",
        "sample": f"whole {name} workload (T={c.T}), {passes} pass(es); layout in one process, dispatch and "
                  f"combine over {len(slices)} token slices on {workers} processes",
        "matches_one_process_oracle": same,
    }


def host_threads(cap=16):
    """Host cores this process may use, at most `cap` (the CPU share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def parity_against(s, lay, recv, out):
    """The GPU outputs of the timed step (layout, dispatch, combine on the
    workload's inputs) against the oracle's: bit-exact flags for layout and
    dispatch; for combine the bit-identical fraction, the gate
    abs(g - r) <= 1e-2 abs(r) + 1e-3 and the norm-relative error
    ||g - r|| / ||r||."""
    import numpy as np

    import oracle

    res = {}
    n = int(lay["offsets"][-1])
    got = {k: getattr(s, k).cpu().numpy().reshape(-1) for k in ("counts", "offsets", "dest_row", "src_token")}
    res["layout_bit_exact"] = bool(
        np.array_equal(got["counts"], lay["counts"]) and np.array_equal(got["offsets"], lay["offsets"])
        and np.array_equal(got["dest_row"], lay["dest_row"].reshape(-1))
        and np.array_equal(got["src_token"][:n], lay["src_token"][:n]))
    if recv is not None:
        g = s.recv.contiguous().view(s.torch.int16).cpu().numpy().view(np.uint16)
        res["dispatch_bit_exact"] = bool(np.array_equal(g, recv))
    go = oracle.bf16_to_f32(s.out.contiguous().view(s.torch.int16).cpu().numpy().view(np.uint16))
    ro = oracle.bf16_to_f32(out)
    res["combine_bit_identical_frac"] = round(float(np.mean(go == ro)), 6)
    res["combine_within_gate"] = bool(np.all(np.abs(go.astype(np.float64) - ro) <= 1e-2 * np.abs(ro) + 1e-3))
    rn = float(np.linalg.norm(ro.astype(np.float64)))
    dn = float(np.linalg.norm(go.astype(np.float64) - ro))
    res["combine_norm_rel_err"] = dn / rn if rn > 0 else dn
    return res


def parse_budget(tok):
    """'24' -> persistent grid of 24 workgroups; 'm24' -> ordinary grid on a
    stream masked to the first 24 CUs; '0' -> ordinary grid, whole device."""
    tok = str(tok).strip()
    if tok.startswith("m"):
        return "mask", int(tok[1:])
    return "grid", int(tok)


def parse_shape(text):
    """"k=2,T=16384" -> {"k": 2, "T": 16384}: size overrides of a named workload."""
    if not text:
        return {}
    out = {}
    for item in text.split(","):
        key, _, val = item.partition("=")
        if key not in ("T", "H", "E", "k") or not val.isdigit():
            raise SystemExit(f"bench.py: bad --shape item {item!r} (keys T, H, E, k with integer values)")
        out[key] = int(val)
    return out


def sweep(path, name, steps, warmup, budgets, variants, slabs, probes=True, shape=None, cold=0):
    """CU budget x variant x slab over the workload, plus the streaming-probe
    ceilings.  With cold > 0, each record also carries the cold-protocol
    per-op statistics (every call after a 1 GiB write) over `cold` steps."""
    import torch

    import bulk_async_tensor_amd as ep

    s = Setup(name, shape=shape)
    n = 1 << 30
    ndev = torch.cuda.get_device_properties(0).multi_processor_count
    a = torch.empty(n // 4, dtype=torch.int32, device="cuda:0")
    bb = torch.empty_like(a)
    with open(path, "a") as fh:
        for tok in budgets:
            kind, budget = parse_budget(tok)
            stream = None
            if kind == "mask":
                stream = ep.ep_stream_create_cu_masked(ep.cu_mask_words(range(budget)))
                ep.ep_set_num_cus(0)
            else:
                ep.ep_set_num_cus(budget)
            s.stream = stream
            st = stream if stream is not None else torch.cuda.current_stream()
            ceiling = {}  # probe GB/s at this budget, by probe name
            # operation 7 once per wave: 128 KiB read by each of 16 waves on every CU of the grid
            once = min(n, (budget if budget > 0 else ndev) * 16 * (128 << 10))
            for mode, label, nb in ([(0, "copy", n), (1, "read", n), (2, "write", n), (0x20 | 2, "write32", n),
                                     (4, "mix8to1", n), (6, "mix8to1_burst", n), (7, "mix8to1_phase", n),
                                     (7, "mix8to1_phase_once", once), (5, "mix1to8", n),
                                     (0x27, "mix8to1_phase_once_barrier", once),
                                     (0x17, "mix1to8_phase", n), (0x17, "mix1to8_phase_once", once)]
                                    if probes else []):
                for _ in range(3):
                    ep.ep_bw_probe(mode, a, bb, nb, stream=st)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(st)
                for _ in range(10):
                    ep.ep_bw_probe(mode, a, bb, nb, stream=st)
                e1.record(st)
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / 10
                moved = 2 * nb if mode == 0 else (nb + nb // 8) if mode in (4, 5, 6, 7, 0x17, 0x27) else nb
                rec = {"kind": "probe", "mode": label, "num_cus": str(tok), "ms": ms, "GBs": moved / ms / 1e6,
                       "bytes": nb}
                ceiling[label] = rec["GBs"]
                fh.write(json.dumps(rec) + "\n")
                print(json.dumps(rec), flush=True)
            for v in variants:
                for slab in slabs:
                    # "rows" / "rows_nt": the gather-form dispatch (cacheable / streaming x loads)
                    s.gather = v.startswith("rows")
                    ep.ep_set_variant({"rows": "auto", "rows_nt": "vgpr_cached"}.get(v, v))
                    ep.ep_set_slab(slab)
                    cold_rep = cold_report(s, cold, 2) if cold > 0 and not s.gather else None
                    ms, per = s.run(steps, warmup)
                    gbs = {k: (s.bytes[k] / (per[k] * 1e6) if per[k] > 0 else None) for k in per}
                    # streaming ceilings at this budget: dispatch (8/9 writes) against the
                    # better write probe, combine against the probe with its phased 8:1 mix
                    writes = [ceiling[m] for m in ("write", "write32") if m in ceiling]
                    ref = {"dispatch": max(writes) if writes else None,
                           "combine": ceiling.get("mix8to1_phase_once")}
                    rec = {"kind": "step", "workload": name, "seed": s.wl.seed,
                           "shape": {"T": s.T, "H": s.H, "E": s.E, "k": s.k}, "variant": v, "slab": slab,
                           "num_cus": str(tok), "ms_per_step": ms, "tokens_per_s": s.T / (ms * 1e-3),
                           "kernel_ms": per, "kernel_timing": getattr(s, "kernel_timing", None), "GBs": gbs,
                           "frac_of_hbm_peak": {k: (g / HBM_PEAK_GBS if g else None) for k, g in gbs.items()},
                           "frac_of_probe": {k: (gbs[k] / ref[k] if gbs.get(k) and ref.get(k) else None)
                                             for k in ("dispatch", "combine")},
                           "probe_ref": {"dispatch": "max(write, write32)", "combine": "mix8to1_phase_once"}}
                    if cold_rep is not None:
                        rec["cold"] = cold_rep
                    fh.write(json.dumps(rec) + "\n")
                    print(json.dumps(rec), flush=True)
            ep.ep_set_slab(0)
            s.gather = False
            s.stream = None
            if stream is not None:
                torch.cuda.synchronize()
                ep.ep_stream_destroy(stream)
    ep.ep_set_num_cus(0)
    ep.ep_set_variant("auto")


def probe_sweep(path, budgets):
    """Streaming-probe matrix: operation x in-flight depth x load cache policy
    at each CU budget (1 GiB buffers, 10 timed launches each)."""
    import torch

    import bulk_async_tensor_amd as ep

    n = 1 << 30
    ndev = torch.cuda.get_device_properties(0).multi_processor_count
    a = torch.empty(n // 4, dtype=torch.int32, device="cuda:0")
    b = torch.empty_like(a)
    cases = [(0, d, 0) for d in range(3)] + [(2, d, 0) for d in range(3)]
    cases += [(1, d, p) for d in range(3) for p in range(6)] + [(3, 0, p) for p in range(6)]
    cases += [(4, 0, 0), (5, 0, 0)]
    names = {0: "copy", 1: "read", 2: "write", 3: "read_lds", 4: "mix8to1", 5: "mix1to8"}
    pols = {0: "nt", 1: "none", 2: "sc0", 3: "sc1", 4: "sc0sc1", 5: "nt_buf"}
    with open(path, "a") as fh:
        for budget in budgets:
            ep.ep_set_num_cus(budget)
            for op, d, p in cases:
                mode = op | (d << 4) | (p << 8)
                for _ in range(2):
                    ep.ep_bw_probe(mode, a, b, n)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(10):
                    ep.ep_bw_probe(mode, a, b, n)
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / 10
                moved = 2 * n if op == 0 else (n + n // 8) if op >= 4 else n
                rec = {"kind": "probe", "op": names[op], "depth": 8 << d, "policy": pols[p], "num_cus": budget,
                       "ms": round(ms, 4), "GBs": round(moved / ms / 1e6, 1)}
                fh.write(json.dumps(rec) + "\n")
                print(json.dumps(rec), flush=True)
    ep.ep_set_num_cus(0)


def latency_study(path, budget):
    """Load latency and the per-CU read ceiling (ep_inflight_probe).

    Every measured walk follows a fresh random cyclic chain of 256-byte
    nodes (rebuilt from a new seed), so no hop finds its node in a cache it
    did not get there itself:
    1. Unloaded, one wave, nothing else running: an L2 hit (a 1 MiB chain
       walked twice, the second walk reported); an Infinity Cache hit (a
       128 MiB chain read once with cacheable loads, which thrashes the 4 MB
       L2 but leaves the chain in the 256 MB Infinity Cache); HBM (a 4 GiB
       chain after a 1 GiB write that evicts both).
    2. Loaded, at `budget` CUs: waves_per_cu x vectors_per_lane of streaming
       nt reads over 2 GiB while wave 0 of workgroup 0 chases a fresh 4 GiB
       chain from HBM on its CU, which its other waves keep streaming.  Read
       GB/s over the streaming waves, latency per hop, the clock from the
       chase's shader-cycle and real-time counters, and the bytes in flight
       per CU that Little's law gives (per-CU GB/s x latency).
    3. The same at every CU with the deepest settings."""
    import torch

    import bulk_async_tensor_amd as ep

    dev = "cuda:0"
    sink = torch.empty(4, dtype=torch.int32, device=dev)
    out = torch.zeros(4, dtype=torch.int64, device=dev)
    src = torch.empty(1 << 29, dtype=torch.int32, device=dev)  # 2 GiB
    src.fill_(3)
    flush = torch.empty(1 << 28, dtype=torch.int32, device=dev)
    ndev = torch.cuda.get_device_properties(0).multi_processor_count
    node = 256
    per = node // 8
    big = torch.zeros((4 << 30) // 8, dtype=torch.int64, device=dev)

    def chain_of(set_bytes, seed):
        n = set_bytes // node
        chain = big[: n * per]
        chain.zero_()
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)
        perm = torch.randperm(n, device=dev, generator=gen)
        chain[perm * per] = torch.roll(perm, -1) * per
        return chain

    def walk(waves, vec, nbytes, chain, hops, cached=False):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ep.ep_inflight_probe(waves, vec, src, nbytes, sink, chain, hops, out, cached=cached)
        e1.record()
        torch.cuda.synchronize()
        o = out.cpu().tolist()
        ns = o[0] * 10.0  # 100 MHz ticks
        return {"kernel_us": round(e0.elapsed_time(e1) * 1e3, 2), "chase_ns_per_hop": round(ns / hops, 1),
                "chase_cycles_per_hop": round(o[1] / hops, 1), "clock_GHz": round(o[1] / ns, 3) if ns > 0 else None,
                "chase_us": round(ns / 1e3, 2), "chase_xcc": o[3] >> 32}

    seed = [100]

    def fresh(set_bytes, evict=True):
        seed[0] += 1
        chain = chain_of(set_bytes, seed[0])
        if evict:
            flush.fill_(seed[0])
        torch.cuda.synchronize()
        return chain

    with open(path, "w") as fh:
        def emit(rec):
            fh.write(json.dumps(rec) + "\n")
            fh.flush()
            print(json.dumps(rec), flush=True)

        ep.ep_set_num_cus(1)
        chain = fresh(1 << 20)
        walk(1, 1, 0, chain, 4000)
        emit({"kind": "unloaded", "level": "L2 hit", "set_MiB": 1, "hops": 4000, **walk(1, 1, 0, chain, 4000)})
        chain = fresh(128 << 20)
        ep.ep_set_num_cus(0)
        ep.ep_bw_probe(1 | (1 << 8), chain, sink, chain.numel() * 8)  # cacheable read of the whole chain
        torch.cuda.synchronize()
        ep.ep_set_num_cus(1)
        emit({"kind": "unloaded", "level": "Infinity Cache hit", "set_MiB": 128, "hops": 2000,
              **walk(1, 1, 0, chain, 2000)})
        for set_bytes in (1 << 30, 4 << 30):
            chain = fresh(set_bytes)
            emit({"kind": "unloaded", "level": "HBM", "set_MiB": set_bytes >> 20, "hops": 1500,
                  **walk(1, 1, 0, chain, 1500)})
        nbytes = src.numel() * 4
        for cus, hops, grid in ((budget, 100, [(w, v) for w in (1, 2, 4, 8, 16) for v in (1, 2, 4, 8, 16)]),
                                (ndev, 60, [(16, 8), (8, 16), (16, 4), (4, 8)])):
            ep.ep_set_num_cus(cus)
            for w, v in grid:
                if v == 16 and w > 8:
                    continue
                chain = fresh(4 << 30)
                r = walk(w, v, nbytes, chain, hops)
                gbs = nbytes / (r["kernel_us"] * 1e3)
                per_cu = gbs / cus
                lat_ns = r["chase_ns_per_hop"]
                emit({"kind": "loaded", "cus": cus, "waves_per_cu": w, "vectors_per_lane": v,
                      "requested_KiB_in_flight_per_cu": [w * v, 2 * w * v], "streaming_waves": cus * w - 1,
                      "GBs": round(gbs, 1), "GBs_per_cu": round(per_cu, 2),
                      "B_per_clk_per_cu": round(per_cu / r["clock_GHz"], 2) if r["clock_GHz"] else None,
                      "latency_ns": lat_ns, "littles_law_KiB_in_flight_per_cu": round(per_cu * lat_ns / 1024, 1),
                      "chase_shorter_than_stream": r["chase_us"] < r["kernel_us"], **r})
        # where the streamed data lives: HBM (nt or cacheable loads, after a flush) or the Infinity Cache
        # (a 128 MiB source read once with cacheable loads first), at the same depth.  A per-CU cap that
        # rises when the data comes from closer (lower latency) is a limit on outstanding misses; one that
        # does not is a throughput limit of the CU's vector memory path.
        small = 128 << 20
        for cus in (budget, ndev):
            ep.ep_set_num_cus(cus)
            for w, v in ((16, 8), (8, 8), (4, 8)):
                for where, nb, cached, warm in (("HBM", nbytes, False, False), ("HBM", nbytes, True, False),
                                                ("Infinity Cache", small, True, True),
                                                ("Infinity Cache (nt loads)", small, False, True)):
                    chain = fresh(4 << 30)
                    if warm:
                        walk(w, v, nb, chain, 1, cached=True)
                    r = walk(w, v, nb, chain, 40, cached=cached)
                    gbs = nb / (r["kernel_us"] * 1e3)
                    emit({"kind": "residency", "cus": cus, "waves_per_cu": w, "vectors_per_lane": v, "source": where,
                          "loads": "cacheable" if cached else "nt", "MiB": nb >> 20, "GBs": round(gbs, 1),
                          "GBs_per_cu": round(gbs / cus, 2),
                          "B_per_clk_per_cu": round(gbs / cus / r["clock_GHz"], 2) if r["clock_GHz"] else None,
                          "chase_ns_per_hop": r["chase_ns_per_hop"], "kernel_us": r["kernel_us"]})
    ep.ep_set_num_cus(0)


def graph_step(s, steps, warmup):
    """One whole step captured in a HIP graph (torch.cuda.CUDAGraph) and
    replayed: the step's device time without per-launch host overhead.
    Returns (ms per replayed step, ms per eager step)."""
    import torch

    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            s.layout()
            s.dispatch()
            s.combine()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s.layout()
        s.dispatch()
        s.combine()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    ms_graph = (time.perf_counter() - t0) * 1e3 / steps
    # many steps per graph (a decode loop reusing its buffers): the graph
    # launch is paid once per `per_graph` steps
    per_graph = 16
    gm = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gm):
        for _ in range(per_graph):
            s.layout()
            s.dispatch()
            s.combine()
    reps = max(1, steps // per_graph)
    for _ in range(max(1, warmup // per_graph)):
        gm.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        gm.replay()
    torch.cuda.synchronize()
    ms_graph_many = (time.perf_counter() - t0) * 1e3 / (reps * per_graph)
    t0 = time.perf_counter()
    for _ in range(steps):
        s.layout()
        s.dispatch()
        s.combine()
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t0) * 1e3 / steps
    return ms_graph, ms_eager, ms_graph_many, per_graph


def kernels_only(s, launches=5, copy_bytes=256 << 20):
    """Short run for counter passes: `launches` of each kernel of the step,
    then of a copy probe that reads and writes exactly `copy_bytes`."""
    import torch

    import bulk_async_tensor_amd as ep

    for _ in range(launches):
        s.layout()
    for _ in range(launches):
        s.dispatch()
    for _ in range(launches):
        s.combine()
    if s.do_dispatch:
        s.fused = True
        for _ in range(launches):
            s.layout()
        s.fused = False
    a = torch.empty(copy_bytes // 4, dtype=torch.int32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(launches):
        ep.ep_bw_probe(0, a, b, copy_bytes)
    torch.cuda.synchronize()
    print(json.dumps({"kernels_only": True, "launches": launches, "copy_bytes": copy_bytes,
                      "bytes": s.bytes}), flush=True)


def overlap(path, name, comm_cus_list, steps, gemm_n=8192, gemm_reps=None, compute="gemm", mfma_iters=16384):
    """Row movement on a stream masked to n CUs beside computation on a stream
    masked to the other CUs (the pages' premise: the copy kernels leave the
    remaining units to computation).  Each side alone and concurrently; also
    both concurrently without a partition.  compute = "gemm": a bf16 GEMM
    through torch (hipBLASLt, whose grid is sized for the whole device);
    "mfma": ep_mfma_probe, a matrix-core loop sized to its share of CUs,
    whose throughput follows the CUs it gets."""
    import torch

    import bulk_async_tensor_amd as ep

    s = Setup(name)
    dev = torch.device("cuda:0")
    n_all = torch.cuda.get_device_properties(0).multi_processor_count
    if compute == "mfma":
        A = B = C = None
        sink = torch.empty(256 * 8 * n_all, dtype=torch.float32, device=dev)
    else:
        A = torch.randn((gemm_n, gemm_n), device=dev, dtype=torch.bfloat16)
        B = torch.randn((gemm_n, gemm_n), device=dev, dtype=torch.bfloat16)
        C = torch.empty((gemm_n, gemm_n), device=dev, dtype=torch.bfloat16)
    share = {"cus": n_all}  # CUs the computation is sized for

    # the matrix-core probe runs 8 short workgroups per CU of its share, so
    # that the dispatcher can even out a partition whose shader engines hold
    # unequal numbers of CUs (with two long workgroups per CU the most loaded
    # CU set the time: 1.5x on 240 of 256 CUs)
    groups_per_cu, iters_per_group = 8, max(1, mfma_iters // 4)

    def flop_per_call():
        if compute == "mfma":
            return 2.0 * share["cus"] * groups_per_cu * 4 * iters_per_group * 4 * 16384
        return 2.0 * gemm_n ** 3

    def timed(jobs):
        """jobs: list of (stream, fn, reps); all start together; returns ms per stream."""
        torch.cuda.synchronize()
        evs = []
        for st, fn, reps in jobs:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            evs.append((e0, e1))
        # record the starts first so the streams begin together
        for (st, fn, reps), (e0, _) in zip(jobs, evs):
            e0.record(st)
        for (st, fn, reps), (_, e1) in zip(jobs, evs):
            with torch.cuda.stream(st):
                for _ in range(reps):
                    fn(st)
            e1.record(st)
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) for e0, e1 in evs]

    def gemm(st):
        if compute == "mfma":
            ep.ep_mfma_probe(groups_per_cu * share["cus"], iters_per_group, sink, stream=st)
        else:
            torch.matmul(A, B, out=C)

    def step(st):
        s.stream = st
        s.layout()
        s.dispatch()
        s.combine()

    default = torch.cuda.current_stream()
    for _ in range(3):
        gemm(default)
        step(default)
    g_full = timed([(default, gemm, 10)])[0] / 10
    s_full = timed([(default, step, steps)])[0] / steps
    reps_g = gemm_reps or max(4, int(round(steps * s_full / g_full)))
    recs = []
    with open(path, "a") as fh:
        base = {"kind": "overlap_base", "workload": name, "compute": compute,
                "gemm_n": gemm_n if compute == "gemm" else None, "gemm_ms_all_cus": g_full,
                "gemm_TFLOPs_all_cus": flop_per_call() / g_full / 1e9, "step_ms_all_cus": s_full}
        fh.write(json.dumps(base) + "\n")
        print(json.dumps(base), flush=True)
        # no partition: both on ordinary streams at once
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        t_g, t_s = timed([(s1, gemm, reps_g), (s2, step, steps)])
        rec = {"kind": "overlap", "partition": "none", "gemm_ms": t_g / reps_g, "step_ms": t_s / steps,
               "gemm_slowdown": (t_g / reps_g) / g_full, "step_slowdown": (t_s / steps) / s_full}
        fh.write(json.dumps(rec) + "\n")
        print(json.dumps(rec), flush=True)
        for n in comm_cus_list:
            comm = ep.ep_stream_create_cu_masked(ep.cu_mask_words(range(n)))
            comp = ep.ep_stream_create_cu_masked(ep.cu_mask_words(range(n, n_all)))
            share["cus"] = n_all - n
            for _ in range(2):
                step(comm)
                with torch.cuda.stream(comp):
                    gemm(comp)
            g_alone = timed([(comp, gemm, reps_g)])[0] / reps_g
            s_alone = timed([(comm, step, steps)])[0] / steps
            t_g, t_s = timed([(comp, gemm, reps_g), (comm, step, steps)])
            rec = {"kind": "overlap", "partition": f"{n}/{n_all - n}", "comm_cus": n,
                   "gemm_ms_alone_on_rest": g_alone, "step_ms_alone_on_n": s_alone,
                   "gemm_ms": t_g / reps_g, "step_ms": t_s / steps,
                   "gemm_slowdown_vs_alone_on_rest": (t_g / reps_g) / g_alone,
                   "gemm_slowdown_vs_all_cus": (t_g / reps_g) / g_full,
                   "step_slowdown_vs_alone_on_n": (t_s / steps) / s_alone,
                   "step_GBs_concurrent": s.step_bytes / (t_s / steps) / 1e6,
                   "gemm_TFLOPs_alone_on_rest": flop_per_call() / g_alone / 1e9,
                   "gemm_TFLOPs_concurrent": flop_per_call() / (t_g / reps_g) / 1e9}
            fh.write(json.dumps(rec) + "\n")
            print(json.dumps(rec), flush=True)
            torch.cuda.synchronize()
            s.stream = None
            ep.ep_stream_destroy(comm)
            ep.ep_stream_destroy(comp)
            share["cus"] = n_all
    s.stream = None


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only; --gpus {args.gpus} is not supported "
              "(a single-GPU kernel library with no collectives)", file=sys.stderr)
        sys.exit(2)
    # the all-cores oracle's processes start before anything touches the GPU
    pool = None
    if not args.no_cpu and not (args.probe_sweep or args.overlap or args.sweep or args.kernels_only or args.cold_only
                                or args.latency):
        pool = oracle_pool(host_threads())
    import torch

    import bulk_async_tensor_amd as ep

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)
    ep.lib()
    budgets = args.sweep_budgets.split(",")
    if args.probe_sweep:
        probe_sweep(args.probe_sweep, [int(b) for b in budgets])
        return
    if args.latency:
        latency_study(args.latency, args.budget)
        return
    if args.overlap:
        overlap(args.overlap, args.workload, [int(b) for b in budgets], max(20, args.steps // 4),
                compute=args.overlap_compute)
        return
    if args.sweep:
        sweep(args.sweep, args.workload, max(20, args.steps // 4), 5, budgets, args.sweep_variants.split(","),
              [int(v) for v in args.sweep_slabs.split(",")], probes=not args.no_probes, shape=parse_shape(args.shape),
              cold=args.sweep_cold)
        return
    if args.shape and not (args.kernels_only or args.cold_only):
        raise SystemExit("bench.py: --shape applies to --sweep, --kernels-only and --cold-only; the benchmark line "
                         "runs the named workload")

    ep.ep_set_variant(args.variant)
    s = Setup(args.workload, shape=parse_shape(args.shape))
    s.fused = args.fused
    if args.kernels_only:
        kernels_only(s)
        return
    iters = max(args.steps, args.cold)
    if args.cold_only:
        rep = cold_report(s, iters, args.warmup)
        # the copy probe that moves exactly 256 MiB each way: the calibration
        # kernel of the counter passes
        a = torch.empty((256 << 20) // 4, dtype=torch.int32, device="cuda:0")
        for _ in range(3):
            ep.ep_bw_probe(0, a, torch.empty_like(a), 256 << 20)
        torch.cuda.synchronize()
        print(json.dumps({"cold_only": True, "workload": args.workload, "steps": iters, "warmup": args.warmup,
                          "bytes": s.bytes, **rep}), flush=True)
        return

    # ---- headline: the cold-cache protocol on all CUs (the library's default launches)
    cold = cold_report(s, iters, args.warmup)
    kernels = ["dispatch", "combine"] if (s.do_dispatch and not s.fused) else ["combine"]
    st = cold["us_per_op"]
    dom = max(kernels, key=lambda k: st[k]["mean"])
    achieved = s.bytes[dom] / (st[dom]["mean"] * 1e3)
    kname = {"dispatch": "ep_dispatch", "combine": "ep_combine"}[dom]
    traffic = read_traffic(dom, args.workload)
    probes_all = budget_probes(torch.cuda.get_device_properties(0).multi_processor_count)
    ref_all = {"dispatch": max(probes_all["mix1to8"], probes_all["write"]), "combine": probes_all["mix8to1_phase_once"]}

    line = {
        "metric": METRIC,
        "value": cold["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(cold["step_us"] / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "T": s.T, "H": s.H, "E": s.E, "k": s.k, "num_cus": "all",
                   "variant": ep.ep_get_variant(),
                   "step": "layout_dispatch+combine" if args.fused else "layout+dispatch+combine",
                   "timing": f"cold caches: each op after a 1 GiB write, between HIP events; {iters} steps; "
                             "step time = sum of per-op medians"},
        "tokens_per_s": cold["tokens_per_s"],
        "cold_us_per_op": st,
        "cold_GBs_p50": cold["GBs_p50"],
        "probe_ceilings_GBs": probes_all,
        "frac_of_probe": {k: round(s.bytes[k] / (st[k]["p50"] * 1e3) / ref_all[k], 4) for k in kernels},
        "frac_of_probe_against": {"dispatch": "max(mix1to8, write)", "combine": "mix8to1_phase_once"},
        "frac_of_copy_probe": {k: round(s.bytes[k] / (st[k]["p50"] * 1e3) / probes_all["copy"], 4) for k in kernels},
        "roofline": {
            "kernel": kname,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes": s.bytes[dom],
            "time": "mean of the cold-protocol calls (HIP events on the launch stream)",
        },
    }

    if not args.no_extras:
        # ---- the same workload at a restricted CU budget (persistent grid), cold and warm
        b = args.budget
        ep.ep_set_num_cus(b)
        cold_b = cold_report(s, iters, args.warmup)
        ms_b, per_b = s.run(args.steps, args.warmup)
        ep.ep_set_num_cus(0)
        probes_b = budget_probes(b)
        ref_b = {"dispatch": max(probes_b["mix1to8"], probes_b["write"]), "combine": probes_b["read"]}
        line[f"cu{b}"] = {
            "cold": cold_b,
            "warm": {"ms_per_step": round(ms_b, 5), "value": round(s.step_bytes / (ms_b * 1e6), 2),
                     "kernel_ms": {k: round(v, 5) for k, v in per_b.items()}},
            "probe_ceilings_GBs": probes_b,
            "frac_of_probe_cold_p50": {k: round(s.bytes[k] / (cold_b["us_per_op"][k]["p50"] * 1e3) / ref_b[k], 4)
                                       for k in kernels},
            "frac_of_probe_against": {"dispatch": "max(mix1to8, write)", "combine": "read"},
            "frac_of_copy_probe_cold_p50": {k: round(s.bytes[k] / (cold_b["us_per_op"][k]["p50"] * 1e3) / probes_b["copy"], 4)
                                            for k in kernels},
            "frac_of_hbm_peak_cold": round(cold_b["value"] / HBM_PEAK_GBS, 4),
        }
        # ---- the same budget as a CU-masked stream with ordinary grids (warm)
        mask_stream = ep.ep_stream_create_cu_masked(ep.cu_mask_words(range(b)))
        s.stream = mask_stream
        ms_m, per_m = s.run(args.steps, args.warmup)
        s.stream = None
        torch.cuda.synchronize()
        ep.ep_stream_destroy(mask_stream)
        line[f"cu{b}_masked_stream_warm"] = {"ms_per_step": round(ms_m, 5),
                                             "value": round(s.step_bytes / (ms_m * 1e6), 2),
                                             "kernel_ms": {k: round(v, 5) for k, v in per_m.items()}}
        # ---- warm: back-to-back launches on all CUs (inputs partly in the Infinity Cache)
        ms_w, per_w = s.run(args.steps, args.warmup)
        line["warm_all_cus"] = {
            "ms_per_step": round(ms_w, 5), "value": round(s.step_bytes / (ms_w * 1e6), 2),
            "kernel_ms": {k: round(v, 5) for k, v in per_w.items()},
            "kernel_timing": getattr(s, "kernel_timing", None),
            "kernel_GBs": {k: round(s.bytes[k] / (per_w[k] * 1e6), 1) for k in per_w if per_w[k] > 0 and s.bytes[k]},
        }
        if s.do_dispatch and not args.fused:
            # the staged dispatch on 64 CUs, fastest while x is cache-resident
            ep.ep_set_variant("lds1")
            cold_l = cold_steps(s, max(20, iters // 2), 2)["dispatch"]
            ms_l, per_l = s.run(args.steps, args.warmup)
            ep.ep_set_variant(args.variant)
            line["dispatch_lds1_64cus"] = {"cold": summarize(cold_l), "warm_us": round(per_l["dispatch"] * 1e3, 2)}
            # layout and dispatch in one launch (ep_layout_dispatch), warm
            s.fused = True
            ms_f, per_f = s.run(args.steps, args.warmup)
            s.fused = False
            line["fused_step_warm"] = {"step": "layout_dispatch+combine", "ms_per_step": round(ms_f, 5),
                                       "value": round(s.step_bytes / (ms_f * 1e6), 2),
                                       "kernel_ms": {"layout_dispatch": round(per_f["layout"], 5),
                                                     "combine": round(per_f["combine"], 5)}}
        if not args.no_reduce:
            line["combine_reduce_warm"] = reduce_times(s, min(args.steps, 50), [0])
        if args.graph:
            ms_g, ms_e, ms_m2, per_graph = graph_step(s, args.steps, args.warmup)
            line["graph_replay"] = {"ms_per_step": round(ms_g, 5), "eager_ms_per_step": round(ms_e, 5),
                                    "value": round(s.step_bytes / (ms_g * 1e-3) / 1e9, 2), "unit": "GB/s",
                                    "tokens_per_s": round(s.T / (ms_g * 1e-3), 1),
                                    "steps_per_graph": {"steps": per_graph, "ms_per_step": round(ms_m2, 5),
                                                        "tokens_per_s": round(s.T / (ms_m2 * 1e-3), 1)}}
        # ---- the training shape (T=4096, E=256, k=8), cold and warm
        if args.workload != "train" and not args.shape:
            t = Setup("train")
            cold_t = cold_report(t, iters, args.warmup)
            ms_t, per_t = t.run(args.steps, args.warmup)
            line["train"] = {"cold": cold_t,
                             "warm": {"ms_per_step": round(ms_t, 5), "value": round(t.step_bytes / (ms_t * 1e6), 2),
                                      "kernel_ms": {k: round(v, 5) for k, v in per_t.items()}}}
            del t
            torch.cuda.empty_cache()
    if args.cold_study:
        for mode in ("none", "write", "read", "write_read"):
            print(json.dumps({"kind": "cold_study", "workload": args.workload, "flush": mode,
                              "us_p10_p50_p90": cold_times(s, args.cold or 50, mode)}), flush=True)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_seconds, gpu=s)
        line["cpu_baseline"]["all_cores"] = cpu_baseline_parallel(args.workload, args.cpu_seconds / 2, pool,
                                                                  host_threads())
        pool.close()
        pool.join()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
