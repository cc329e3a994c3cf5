#!/usr/bin/env python3
"""Benchmark of the MoE expert-parallel dispatch/combine path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
route (softmax/top-k), dispatch (count, scan, pack, exchange), expert stub,
combine (reverse exchange, weighted reduction).  The default workload is the
decode-shaped H=7168 / E=256 / top-8 batch (8 logical ranks x 16 tokens);
``--config`` selects another of the five workloads.

Prints ONE JSON line: tokens/s over K back-to-back steps with the inputs
resident in HBM, the per-phase split, the roofline of the dominant kernel
(algorithmic bytes per launch / its mean HIP-event duration, against the
8 TB/s HBM peak) and the CPU oracle's rate on a bounded sample of the same
workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "dispatch+combine tokens/s and achieved HBM GB/s vs peak, H=7168 E=256 k=8"

KERNEL_SOURCES = {
    "route_topk": "route.hip", "count": "count.hip", "scan": "count.hip", "pack": "pack.hip",
    "exchange": "exchange.hip", "stub": "stub.hip", "reverse_exchange": "exchange.hip", "reduce": "reduce.hip",
    "pack_direct": "pack.hip", "reduce_direct": "reduce.hip", "count_pack": "pack.hip", "count_pack_direct": "pack.hip",
    "allgather": "pack.hip", "handles": "pack.hip", "count_handles": "pack.hip", "select": "exchange.hip",
}
PHASE_OF = {
    "route_topk": "route", "count": "dispatch", "scan": "dispatch", "pack": "dispatch", "exchange": "dispatch",
    "stub": "expert_stub", "reverse_exchange": "combine", "reduce": "combine",
    "pack_direct": "dispatch", "reduce_direct": "combine", "count_pack": "dispatch", "count_pack_direct": "dispatch",
    "allgather": "dispatch", "handles": "dispatch", "count_handles": "dispatch", "select": "dispatch",
}


def kernel_bytes(w) -> dict:
    """Algorithmic bytes one launch of each kernel moves (payload model: hidden rows,
    FP8 scales and routing data; the 16-byte handle records and int32 position
    arrays are metadata, counted separately)."""
    T, E, k, H = w.tokens, w.num_experts, w.top_k, w.hidden
    Na = T * k
    D = (H + 4 * (H // 128)) if w.dispatch_dtype != "bf16" else 2 * H   # dispatched row incl. scales
    pack = 2 * H * T + Na * D
    count = 8 * Na + 12 * w.num_ranks * E
    return {
        "route_topk": 4 * T * E + 8 * T * k,
        "count": count,
        "scan": 12 * w.num_ranks * E,
        "pack": pack,
        "exchange": 2 * Na * D,
        "stub": Na * D + Na * 2 * H,
        "reverse_exchange": 2 * Na * 2 * H,
        "reduce": Na * 2 * H + 2 * H * T,
        "pack_direct": pack,                         # rows land straight in the receive buffer
        "reduce_direct": Na * 2 * H + 2 * H * T,    # reads the expert output through the handle
        "count_pack": count + pack,                  # small problems: the pack kernel counts by itself
        "count_pack_direct": count + pack,
        "allgather": 2 * H * T + w.num_ranks * T * D,   # every rank's copy of every token
        "handles": 8 * Na,                           # positions and records only (metadata)
        "count_handles": count,
        "select": 2 * Na * D,                        # each rank's pick from its own copy
    }


def metadata_bytes(w) -> int:
    Na = w.tokens * w.top_k
    # pack writes 16 B record + 4 B map per row and 8 B of positions per assignment;
    # the exchange moves the record; the reverse exchange reads it
    return Na * (16 + 4 + 8) + 2 * Na * 16 + Na * 16


def logical_payload_bytes(w) -> int:
    """The bytes that cross the links once each way: every assignment's dispatched row
    (the FP8 codes without their scales, else 2H) and its bf16 combine row."""
    row = w.hidden if w.dispatch_dtype != "bf16" else 2 * w.hidden
    return w.tokens * w.top_k * (row + 2 * w.hidden)


def source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "combine_router_softmax_expert_amd", "csrc")
    for f in (KERNEL_SOURCES[kernel], "device.hpp"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(config: str, kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current source of the kernel; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    rec = data.get(config, {}).get(kernel)
    if not rec or rec.get("source_sha") != source_sha(kernel):
        return None
    return int(rec["fetch_bytes"] + rec["write_bytes"])


KERNEL_NAME_PATTERNS = (   # rocprofv3 kernel name fragment -> kernel of the path
    ("route_topk", "route_topk"), ("count_scan_single_kernel", "count"), ("count_kernel", "count"),
    ("scan_kernel", "scan"), ("count_pack_kernel", "count_pack"), ("pack_kernel", "pack"),
    ("allgather_kernel", "allgather"), ("handle_kernel", "handles"), ("select_kernel", "select"),
    ("select_scatter_kernel", "select"), ("reverse_exchange_", "reverse_exchange"),
    ("exchange_kernel", "exchange"), ("exchange_affine_kernel", "exchange"), ("stub_kernel", "stub"),
    ("stub_affine_kernel", "stub"), ("reduce_kernel", "reduce"),
)


# template argument that marks the direct form: position in the argument list
DIRECT_TEMPLATE_ARG = {"count_pack": 1, "pack": 3, "reduce": 2}


def path_kernel(rocprof_name: str):
    for frag, k in KERNEL_NAME_PATTERNS:
        if frag in rocprof_name:
            i = DIRECT_TEMPLATE_ARG.get(k)
            if i is not None:
                args = [a.strip() for a in rocprof_name.split(frag + "<", 1)[1].split(">", 1)[0].split(",")]
                if k == "count_pack" and len(args) > 4 and args[4] == "false":
                    return "count_handles"          # the all-gather dispatcher's position pass (no rows)
                if args[i] == "true":
                    k += "_direct"
            return k
    return None


def _counter_means(d: str, counter: str) -> dict:
    """Mean value per dispatch of one counter for every kernel in a rocprofv3 --pmc csv output dir."""
    import csv
    import glob
    sums, cnts = {}, {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") != counter:
                    continue
                name = r["Kernel_Name"]
                sums[name] = sums.get(name, 0.0) + float(r["Counter_Value"])
                cnts[name] = cnts.get(name, 0) + 1
    return {n: sums[n] / cnts[n] for n in sums}


def ingest_counters(config: str, fetch_dir: str, write_dir: str, copy_fetch_dir: str, copy_write_dir: str,
                    copy_bytes: int, command: str, path: str = os.path.join(ROOT, "profiles", "traffic.json")):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the path's kernels, each scaled by
    known bytes / counter reading of a plain copy, into ``path`` (profiles/traffic.json)."""
    fetch, write = _counter_means(fetch_dir, "FETCH_SIZE"), _counter_means(write_dir, "WRITE_SIZE")
    cf = max(_counter_means(copy_fetch_dir, "FETCH_SIZE").values())
    cw = max(_counter_means(copy_write_dir, "WRITE_SIZE").values())
    f_fac, w_fac = copy_bytes / (cf * 1024.0), copy_bytes / (cw * 1024.0)
    data = json.load(open(path)) if os.path.exists(path) else {}
    rec = {}
    for name, kib in fetch.items():
        k = path_kernel(name)
        if k is None or name not in write:
            continue
        rec[k] = {"fetch_bytes": round(kib * 1024 * f_fac), "write_bytes": round(write[name] * 1024 * w_fac),
                  "fetch_kib_per_dispatch": round(kib, 1), "write_kib_per_dispatch": round(write[name], 1),
                  "copy_factor_fetch": round(f_fac, 4), "copy_factor_write": round(w_fac, 4),
                  "source_sha": source_sha(k), "command": command}
    data[config] = rec
    with open(path, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
    print(json.dumps({"config": config, "copy_factor_fetch": f_fac, "copy_factor_write": w_fac,
                      "kernels": {k: v["fetch_bytes"] + v["write_bytes"] for k, v in rec.items()}}))


def copy_calibration(nbytes: int = 1 << 30, reps: int = 5):
    """A plain device copy of known size (read nbytes, write nbytes) for counter calibration."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)                      # warm
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        torch.neg(src, out=dst)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / reps
    # the copy's own rate: a practical ceiling for the path's copy kernels on this GPU
    print(json.dumps({"copy_bytes": nbytes, "reps": reps + 1, "ms_per_copy": round(ms, 4),
                      "copy_tbps": round(2 * nbytes / (ms * 1e-3) / 1e12, 3)}))


def routing_stats(ids, num_ranks: int, num_experts: int) -> dict:
    """The routing's shape from the expert ids [T, k]: per-expert load imbalance
    (max / mean), empty experts, the share the hottest tenth of the experts takes,
    per-destination-rank imbalance and the share of assignments that stay on the
    source rank."""
    import numpy as np
    T, k = ids.shape
    n_e = np.bincount(ids.ravel(), minlength=num_experts)
    Ep = num_experts // num_ranks
    dst = ids // Ep
    src = np.repeat(np.arange(T) // (T // num_ranks), k).reshape(T, k)
    n_r = np.bincount(dst.ravel(), minlength=num_ranks)
    top = np.sort(n_e)[::-1][:max(1, num_experts // 10)]
    return {
        "expert_imbalance": round(float(n_e.max() / n_e.mean()), 3),
        "empty_experts": int((n_e == 0).sum()),
        "top10pct_expert_share": round(float(top.sum() / n_e.sum()), 4),
        "rank_imbalance": round(float(n_r.max() / n_r.mean()), 3),
        "local_share": round(float((dst == src).mean()), 4),
    }


def host_info() -> dict:
    import platform
    import torch
    cpu = platform.processor()
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((line.split(":", 1)[1].strip() for line in f if line.startswith("model name")), cpu)
    except OSError:
        pass
    props = torch.cuda.get_device_properties(0)
    return {"gpu": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "hip": torch.version.hip, "host_cpu": cpu,
            "host_cores": os.cpu_count()}


def cpu_baseline(w, inp, budget_s: float) -> dict:
    """The oracle, as it stands, on one host core over a bounded sample of the workload."""
    import numpy as np
    from oracle import oracle as orc

    # size the sample: whole workload if one pass fits the budget, else the first
    # tokens of every rank (same ranks, experts, top-k and hidden size)
    P, Tp = w.num_ranks, w.tokens_per_rank
    probe_tp = max(1, min(Tp, 4))
    old = os.sched_getaffinity(0)
    core = min(old)
    os.sched_setaffinity(0, {core})
    try:
        def sub(tp):
            sel = np.concatenate([np.arange(r * Tp, r * Tp + tp) for r in range(P)])
            return orc.Shape(P, P * tp, w.num_experts, w.top_k, w.hidden, w.dispatch_dtype != "bf16"), \
                np.ascontiguousarray(inp["x"][sel]), np.ascontiguousarray(inp["logits"][sel])

        sh, x, lg = sub(probe_tp)
        t0 = time.perf_counter()
        orc.run(sh, x, lg)
        per_token = (time.perf_counter() - t0) / sh.T
        tp = int(min(Tp, max(1, budget_s / 3 / (per_token * P))))
        sh, x, lg = sub(tp)
        reps, t0 = 0, time.perf_counter()
        while True:
            orc.run(sh, x, lg)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= 1000:
                break
    finally:
        os.sched_setaffinity(0, old)
    flags = ""
    with open(os.path.join(ROOT, "oracle", "Makefile")) as fh:     # how the timed oracle was compiled
        for line in fh:
            if line.startswith("CFLAGS"):
                flags = line.split("=", 1)[1].strip()
    return {
        "value": reps * sh.T / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
        "build": f"{os.environ.get('CC', 'gcc')} {flags}",
        "sample": (f"{'whole workload' if tp == Tp else f'first {tp} of {Tp} tokens on each of {P} ranks'}"
                   f" ({sh.T} tokens), route+dispatch+stub+combine, {reps} passes in {el:.1f} s, "
                   f"single-threaded C oracle pinned to host core {core}"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 1000 steps: at decode size one step is ~31 us, and a timed region of a few
    # ms let one host or GPU hiccup move the mean by 10-20%
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="c2", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--mode", default="base", choices=["base", "direct"],
                    help="base: pack into send buffers + exchange copies; direct: pack straight into the "
                         "receive rows and reduce straight from the expert output")
    ap.add_argument("--ranks", type=int, default=0,
                    help="comparison runs only: the workload with this many logical ranks instead of its own")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush-run", action="store_true", help="skip the cache-flushed per-step run")
    ap.add_argument("--core-only", action="store_true",
                    help="only the timed steps, dispatch+combine and the per-kernel pass (for kernel traces: no "
                         "other forms, micro-batches or graphs whose launches would mix into the statistics)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--ingest-counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="turn rocprofv3 --pmc outputs into profiles/traffic.json for --config")
    ap.add_argument("--counter-command", default="", help="command recorded with --ingest-counters")
    args = ap.parse_args()

    if args.ingest_counters:
        ingest_counters(args.config, *args.ingest_counters, copy_bytes=1 << 30, command=args.counter_command)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the expert-parallel ranks are emulated in one HBM "
              "and nothing here uses a second GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch

    from combine_router_softmax_expert_amd import binding as B
    from combine_router_softmax_expert_amd import workloads as wl

    w = wl.WORKLOADS[args.config]
    if args.ranks:
        w = wl.custom(f"{w.name}-as-ep{args.ranks}", args.ranks, w.tokens, w.num_experts, w.top_k, w.hidden,
                      w.dispatch_dtype, w.seed, w.zipf)
    inp = wl.make_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ctx = B.Context.for_workload(w)
    bufs = ctx.allocate(dev)
    x = torch.from_numpy(inp["x"].view(np.int16)).to(dev)
    logits = torch.from_numpy(inp["logits"]).to(dev)
    stream = torch.cuda.current_stream()

    direct = args.mode == "direct"

    # Each form's calls with their arguments checked and marshalled once (binding.PreparedPath):
    # the same library calls and kernels as binding.run_path without its per-call Python work,
    # which at decode size cost more host time per step than the GPU needs for the step.
    paths = {d: B.PreparedPath(ctx, bufs, x, logits, stream, direct=d) for d in (False, True)}
    dcs = {d: B.PreparedPath(ctx, bufs, x, None, stream, direct=d, stages="dispatch_combine") for d in (False, True)}

    def step(direct=direct):
        paths[direct]()

    def dispatch_combine(direct=direct):
        """Dispatch and combine alone (routing ids/weights and expert outputs from earlier steps)."""
        dcs[direct]()

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, n):
        """Mean ms of n back-to-back calls, bracketed by synchronize + events on the launch stream."""
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(n):
            fn()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K back-to-back steps of the whole path
    ms_per_step = timed(step, args.steps)
    # dispatch + combine alone, K times back to back
    dc_ms = timed(dispatch_combine, args.steps)

    def latency_percentiles(fn, n):
        """Median, p95 and p99 of n back-to-back calls, each bracketed by its own events."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) for a, b in evs])
        return {"median": round(float(np.median(t)), 5), "p95": round(float(np.percentile(t, 95)), 5),
                "p99": round(float(np.percentile(t, 99)), 5)}

    latency_ms = {"step": latency_percentiles(step, args.steps),
                  "dispatch_combine": latency_percentiles(dispatch_combine, args.steps)}

    # the same K steps with every kernel bracketed by HIP events on its stream
    # (the library records them around each launch), for per-kernel durations;
    # each event pair adds launch-to-launch overhead, so these read high for
    # kernels of a few microseconds
    B.moe_timing_begin(ctx)
    ms_with_events = timed(step, args.steps)
    kt = B.moe_timing_end(ctx)

    extras = not args.core_only
    other_ms = other_dc_ms = ag_dc_ms = None
    kt_other, kt_ag, graph, micro = {}, {}, None, None
    if extras:
        # the other form of dispatch/combine on the same data, for comparison
        other = not direct
        for _ in range(args.warmup):
            step(other)
        other_ms = timed(lambda: step(other), args.steps)
        other_dc_ms = timed(lambda: dispatch_combine(other), args.steps)
        B.moe_timing_begin(ctx)
        step(other)                      # once, for the names of the kernels it runs
        kt_other = B.moe_timing_end(ctx)
        step()   # leave the buffers as the measured form wrote them

        # the all-gather dispatcher (with the base combine) on the same data
        gathered, gathered_scales = ctx.allocate_gathered(dev)

        allgather_dc = B.PreparedPath(ctx, bufs, x, None, stream, stages="dispatch_combine", gathered=gathered,
                                      gathered_scales=gathered_scales)

        for _ in range(args.warmup):
            allgather_dc()
        ag_dc_ms = timed(allgather_dc, args.steps)
        B.moe_timing_begin(ctx)
        timed(allgather_dc, args.steps)
        kt_ag = B.moe_timing_end(ctx)
        del allgather_dc, gathered, gathered_scales
        step()   # leave the buffers as the measured form wrote them

    # per-step times with the caches flushed before each step (a 1 GiB write)
    cold_ms = None
    if extras and not args.no_flush_run:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        times = []
        for _ in range(min(args.steps, 30)):
            flush.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        cold_ms = float(np.median(times))
        del flush

    if extras:
        # the step captured once in a HIP graph and replayed (no per-call host work)
        def graph_ms(direct):
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                B.run_path(ctx, bufs, x, logits, None, direct=direct)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                B.run_path(ctx, bufs, x, logits, None, direct=direct)
            for _ in range(args.warmup):
                g.replay()
            ms = timed(g.replay, args.steps)
            del g
            return ms

        graph = {}
        for mode, d in (("base", False), ("direct", True)):
            ms = graph_ms(d)
            graph[mode] = {"ms_per_step": round(ms, 5), "tokens_per_s": round(w.tokens / (ms * 1e-3), 1)}
        # two micro-batches through the split phases: the expert stage of one on a
        # second stream overlaps the other's dispatch and combine (vs one stream)
        fp8 = w.dispatch_dtype != "bf16"
        parts = []
        for c in range(2):
            rows = torch.from_numpy(wl.micro_batch_rows(w.num_ranks, w.tokens_per_rank, 2, c)).to(dev)
            cc = B.Context(w.num_ranks, w.tokens_per_rank // 2, w.num_experts, w.top_k, w.hidden, fp8)
            parts.append((cc, cc.allocate(dev), x[rows].contiguous(), logits[rows].contiguous()))

        def micro_batches_ms(same_stream):
            """Eager launches: the host issues 12 calls per step, so at decode sizes this
            measures the host; large problems measure the GPU."""
            comm = torch.cuda.Stream()
            compute = comm if same_stream else torch.cuda.Stream()

            def go():
                comm.wait_stream(stream)
                compute.wait_stream(stream)
                B.run_overlapped(parts, comm, compute)
                stream.wait_stream(comm)
                stream.wait_stream(compute)

            for _ in range(args.warmup):
                go()
            return timed(go, args.steps)

        mb_two, mb_one = micro_batches_ms(False), micro_batches_ms(True)
        micro = {"parts": 2, "eager": True, "ms_two_streams": round(mb_two, 5), "ms_one_stream": round(mb_one, 5),
                 "tokens_per_s_two_streams": round(w.tokens / (mb_two * 1e-3), 1)}
        del parts
        step()   # leave the buffers as the measured form wrote them

    kb = kernel_bytes(w)
    per_kernel = {}
    phases = {}
    for name, (launches, tot) in kt.items():
        avg = tot / launches
        per_kernel[name] = {"launches": launches, "avg_us": round(avg * 1e3, 3),
                            "algorithmic_bytes": kb[name],
                            "gbps": round(kb[name] / (avg * 1e-3) / 1e9, 1)}
        phases[PHASE_OF[name]] = phases.get(PHASE_OF[name], 0.0) + tot / launches
    dom = max(kt, key=lambda n: kt[n][1])
    dom_avg_s = kt[dom][1] / kt[dom][0] * 1e-3
    achieved = kb[dom] / dom_avg_s / 1e9
    traffic = load_traffic(args.config, dom)

    T = w.tokens
    dc_bytes = sum(kb[n] for n in kt if PHASE_OF[n] in ("dispatch", "combine"))
    other_dc_bytes = sum(kb[n] for n in kt_other if PHASE_OF[n] in ("dispatch", "combine"))
    step_bytes = sum(kb[n] for n in kt)
    out = {
        "metric": METRIC,
        "value": round(T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dispatch_dtype == "bf16" else "fp8_e4m3+bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "ranks": w.num_ranks, "tokens": T, "experts": w.num_experts,
                   "top_k": w.top_k, "hidden": w.hidden, "dispatch": w.dispatch_dtype,
                   "parallelism": f"ep{w.num_ranks} emulated on 1 GPU", "mode": args.mode},
        "step_gbps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "dispatch_combine": {
            "ms": round(dc_ms, 5), "tokens_per_s": round(T / (dc_ms * 1e-3), 1),
            "algorithmic_bytes": dc_bytes, "gbps": round(dc_bytes / (dc_ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(dc_bytes / (dc_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "logical_payload_bytes": logical_payload_bytes(w),
            "logical_payload_gbps": round(logical_payload_bytes(w) / (dc_ms * 1e-3) / 1e9, 1),
        },
        "other_mode": None if not extras else {
            "mode": "base" if direct else "direct",
            "ms_per_step": round(other_ms, 5), "tokens_per_s": round(T / (other_ms * 1e-3), 1),
            "dispatch_combine_ms": round(other_dc_ms, 5),
            "dispatch_combine_tokens_per_s": round(T / (other_dc_ms * 1e-3), 1),
            "dispatch_combine_gbps": round(other_dc_bytes / (other_dc_ms * 1e-3) / 1e9, 1),
        },
        "allgather_dispatch": None if not extras else {
            "dispatch_combine_ms": round(ag_dc_ms, 5), "dispatch_combine_tokens_per_s": round(T / (ag_dc_ms * 1e-3), 1),
            "algorithmic_bytes": sum(kb[n] for n in kt_ag if PHASE_OF[n] in ("dispatch", "combine")),
            "kernels_ms": {n: round(v[1] / v[0], 5) for n, v in kt_ag.items()},
        },
        "graph_replay": graph,
        "micro_batches": micro,
        "phases_ms": {k: round(v, 5) for k, v in phases.items()},
        "kernels": per_kernel,
        "latency_ms": latency_ms,
        "ms_per_step_with_kernel_events": round(ms_with_events, 5),
        "ms_per_step_cache_flushed": None if cold_ms is None else round(cold_ms, 5),
        "metadata_bytes_per_step": metadata_bytes(w),
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic},
        "routing": routing_stats(bufs["topk_ids"].cpu().numpy(), w.num_ranks, w.num_experts),
        "hardware": host_info(),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
