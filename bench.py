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
    """Hash of what a kernel's machine code is built from: its source, the device helpers, the launch
    constants and shared layouts, and the build script with its compiler flags."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "combine_router_softmax_expert_amd")
    for f in (os.path.join("csrc", KERNEL_SOURCES[kernel]), os.path.join("csrc", "device.hpp"),
              os.path.join("csrc", "kernels.hpp"), "_build.py"):
        with open(os.path.join(pkg, f), "rb") as fh:
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


# rocprofv3 kernel name fragment -> kernel of the path, and the position of the template argument that marks
# the direct form (None: the kernel has no direct form of its own)
KERNEL_NAME_PATTERNS = (
    ("route_topk", "route_topk", None), ("count_scan_single_kernel", "count", None), ("count_kernel", "count", None),
    ("scan_kernel", "scan", None), ("scan_spread_kernel", "scan", None), ("count_pack_kernel", "count_pack", 1),
    ("pack_kernel", "pack", 3),
    ("allgather_kernel", "allgather", None), ("handle_kernel", "handles", None), ("select_kernel", "select", None),
    ("select_scatter_kernel", "select", None), ("reverse_exchange_", "reverse_exchange", None),
    ("exchange_kernel", "exchange", None), ("exchange_affine_kernel", "exchange", None), ("stub_kernel", "stub", None),
    ("stub_affine_kernel", "stub", None), ("reduce_kernel", "reduce", 2), ("reduce_affine_kernel", "reduce", 0),
)


def path_kernel(rocprof_name: str):
    for frag, k, i in KERNEL_NAME_PATTERNS:
        if frag in rocprof_name:
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


def eviction_probe(dev, stream, nbytes: int = 117_440_512, reps: int = 20) -> dict:
    """Median µs of single 117 MB probe reads and copies (moe_probe_read / moe_probe_copy, temporal), each after
    one pass on the launch stream: none (the host's launch is timed too), a 0.2 ms GPU spin (warm), a 1 GiB write
    (evicts the caches and leaves the Infinity Cache full of dirty lines), a 1 GiB temporal read (evicts with
    clean lines), a 1 GiB nontemporal read, and the write followed by the read.  It separates what a cold cache
    costs a call from what the write-back of a flush's own dirty lines costs it."""
    import numpy as np
    import torch

    from combine_router_softmax_expert_amd import binding as B
    flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    cyc = _spin_cycles_per_ms(stream)

    def fill():
        with torch.cuda.stream(stream):
            flush.fill_(1)

    def spin():
        with torch.cuda.stream(stream):
            torch.cuda._sleep(int(0.2 * cyc))

    passes = {
        "none": lambda: None,
        "spin_0.2ms": spin,
        "write_1GiB": fill,
        "read_1GiB": lambda: B.moe_probe_read(flush, sink, False, stream),
        "read_nt_1GiB": lambda: B.moe_probe_read(flush, sink, True, stream),
        "write_then_read_1GiB": lambda: (fill(), B.moe_probe_read(flush, sink, False, stream)),
    }
    ops = {"read_117MB": lambda: B.moe_probe_read(src, sink, False, stream),
           "copy_117MB": lambda: B.moe_probe_copy(src, dst, 0, stream)}
    out = {}
    for op_name, op in ops.items():
        op()
        for name, pre in passes.items():
            times = []
            for _ in range(reps):
                pre()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                op()
                b.record(stream)
                torch.cuda.synchronize()
                times.append(a.elapsed_time(b) * 1e3)
            out.setdefault(op_name, {})[name] = round(float(np.median(times)), 2)
    return {"eviction_probe_us": out, "reps": reps, "bytes": nbytes}


CEILING_SIZES = (("1GiB", 1 << 30, 10), ("940MB", 939_524_096, 10), ("117MB", 117_440_512, 50),
                 ("14.7MB", 14_680_064, 500))


def _spin_cycles_per_ms(stream) -> float:
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    torch.cuda._sleep(10_000_000)
    b.record(stream)
    torch.cuda.synchronize()
    return 10_000_000 / max(a.elapsed_time(b), 1e-3)


def gated_ms(fn, n: int, stream, cycles_per_ms: float, chunk: int = 50, gate_ms: float = 40.0) -> float:
    """Mean ms per call of n calls of fn, enqueued in chunks behind a GPU spin (torch.cuda._sleep), so
    that the GPU runs each chunk back to back whatever the host's pace; events on `stream`."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    total, done = 0.0, 0
    while done < n:
        m = min(chunk, n - done)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(gate_ms * cycles_per_ms))
        a.record(stream)
        for _ in range(m):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        total += a.elapsed_time(b)
        done += m
    return total / n


def ceilings(dev, stream, reps_scale: float = 1.0) -> dict:
    """The library's probe kernels (16-byte units, one per lane, as in the row kernels): a plain copy and a
    streaming read, temporal, nontemporal or (copies) with write-through stores, at the sizes of the
    workloads' row buffers (1 GiB as the HBM reference; 940 MB and 117 MB are the skewed workload's expert
    output and hidden rows; 14.7 MB the decode workload's row buffers, which stay in the Infinity Cache).
    Rates in TB/s of bytes moved (a copy moves 2x its size).  Each figure is the mean of launches the GPU
    runs back to back (enqueued behind a GPU spin, so the host's pace does not enter).  Then four dependent
    copies that move the decode workload's dispatch+combine bytes: contiguous, and as row gathers through a
    random permutation or the identity (microseconds per four copies); and the skewed workload's streaming row
    gather (65,536 rows of 14 KiB through a random permutation or the identity, TB/s)."""
    import torch

    from combine_router_softmax_expert_amd import binding as B

    out = {}
    cpm = _spin_cycles_per_ms(stream)
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    for label, nbytes, reps in CEILING_SIZES:
        reps = max(2, int(reps * reps_scale))
        src = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for policy, tag in ((B.PROBE_TEMPORAL, "temporal"), (B.PROBE_NONTEMPORAL, "nt"),
                            (B.PROBE_WRITE_THROUGH, "write_through")):
            for kind in ("copy", "read"):
                if kind == "read" and policy == B.PROBE_WRITE_THROUGH:
                    continue                     # no stores to write through
                def call():
                    if kind == "copy":
                        B.moe_probe_copy(src, dst, policy, stream)
                    else:
                        B.moe_probe_read(src, sink, policy == B.PROBE_NONTEMPORAL, stream)
                call()
                call()
                ms = gated_ms(call, reps, stream, cpm, chunk=min(reps, 100))
                moved = (2 if kind == "copy" else 1) * nbytes
                out[f"{kind}_{tag}_{label}"] = round(moved / (ms * 1e-3) / 1e12, 3)
        del src, dst
    # the floor of the decode workload's dispatch+combine as four back-to-back kernels: plain contiguous
    # copies moving the bytes of its four kernels (pack 16.5 MB, exchange 29.4 MB, reverse exchange
    # 29.4 MB, reduction 16.5 MB), each reading the buffer the copy before it wrote
    from combine_router_softmax_expert_amd import workloads as wl
    kb = kernel_bytes(wl.WORKLOADS["c2"])
    sizes = [kb[k] // 2 // 16 * 16 for k in ("count_pack", "exchange", "reverse_exchange", "reduce")]
    bufs = [torch.zeros(max(sizes), dtype=torch.uint8, device=dev) for _ in range(5)]
    views = [(bufs[i][:n], bufs[i + 1][:n]) for i, n in enumerate(sizes)]
    for policy, tag in ((B.PROBE_TEMPORAL, "temporal"), (B.PROBE_NONTEMPORAL, "nt"),
                        (B.PROBE_WRITE_THROUGH, "write_through")):
        def chain():
            for s_, d_ in views:
                B.moe_probe_copy(s_, d_, policy, stream)
        for _ in range(5):
            chain()
        us = gated_ms(chain, max(2, int(500 * reps_scale)), stream, cpm, chunk=25) * 1e3
        out[f"decode_dc_four_copies_{tag}_us"] = round(us, 3)
        out[f"decode_dc_four_copies_{tag}_frac_of_8tbps"] = round(2 * sum(sizes) / (us * 1e-6) / 8e12, 4)
    del bufs, views
    # the same four copies in rows of the decode workload's hidden size (577, 1024, 1024 and 576 rows of
    # 14 KiB), each reading its rows through a seeded random permutation of what the copy before it wrote,
    # as the path's kernels do (a row is read on another XCD than the one that wrote it 7 times in 8); and
    # through the identity, which keeps each row on its writer's XCD
    import numpy as np
    row = 2 * wl.WORKLOADS["c2"].hidden
    rows = [n // row for n in sizes]
    rbufs = [torch.zeros((max(rows), row), dtype=torch.uint8, device=dev) for _ in range(5)]
    rng = np.random.default_rng(20)
    perms = {"permuted": [torch.from_numpy(rng.permutation(max(rows))[:n].astype(np.int32)).to(dev) for n in rows],
             "identity": [torch.arange(n, dtype=torch.int32, device=dev) for n in rows]}
    for order, policies in (("permuted", ((B.PROBE_TEMPORAL, "temporal"), (B.PROBE_NONTEMPORAL, "nt"),
                                          (B.PROBE_WRITE_THROUGH, "write_through"))),
                            ("identity", ((B.PROBE_WRITE_THROUGH, "write_through"),))):
        for policy, tag in policies:
            def chain():
                for i, n in enumerate(rows):
                    B.moe_probe_gather(rbufs[i], rbufs[i + 1][:n], perms[order][i], policy, stream)
            for _ in range(5):
                chain()
            us = gated_ms(chain, max(2, int(500 * reps_scale)), stream, cpm, chunk=25) * 1e3
            out[f"decode_dc_four_row_copies_{order}_{tag}_us"] = round(us, 3)
    del rbufs, perms
    # the skewed workload's row gather: 65,536 rows of 14 KiB (940 MB), nontemporal, each destination row read
    # from a source row through a seeded random permutation (the streaming reverse exchange's pattern), and
    # through the identity (a plain row copy of the same shape); TB/s of bytes moved
    w5 = wl.WORKLOADS["c5"]
    n5, row5 = w5.tokens * w5.top_k, 2 * w5.hidden
    src5 = torch.zeros((n5, row5), dtype=torch.uint8, device=dev)
    dst5 = torch.empty_like(src5)
    perm5 = {"permuted": torch.from_numpy(np.random.default_rng(21).permutation(n5).astype(np.int32)).to(dev),
             "identity": torch.arange(n5, dtype=torch.int32, device=dev)}
    for order, perm in perm5.items():
        def gather():
            B.moe_probe_gather(src5, dst5, perm, B.PROBE_NONTEMPORAL, stream)
        gather()
        ms = gated_ms(gather, max(2, int(10 * reps_scale)), stream, cpm, chunk=10)
        out[f"skewed_row_gather_{order}_nt_940MB"] = round(2 * n5 * row5 / (ms * 1e-3) / 1e12, 3)
    del src5, dst5, perm5
    torch.cuda.empty_cache()
    return out


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


# ---------------------------------------------------------------------------
# summaries of rocprofv3 outputs (profiles/*.md)
# ---------------------------------------------------------------------------

def _short_kernel(name: str) -> str:
    return name.replace("void ", "").replace("moe::(anonymous namespace)::", "").split("(", 1)[0]


def summarize_trace(config: str, trace_dir: str, command: str) -> str:
    """Markdown table of a `rocprofv3 --kernel-trace` run of `bench.py --core-only`: per path kernel, the
    launches of the gated per-kernel pass (those after the first GPU spin, which the pass uses as its gate)
    and, for comparison, all launches, which include the passes whose host pace the profiler slows."""
    import csv
    from combine_router_softmax_expert_amd import workloads as wl

    w = wl.WORKLOADS[config]
    kb = kernel_bytes(w)
    rows = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    gated, every, names = {}, {}, {}
    markers = 0                          # probe copies seen (trace_marker brackets the per-kernel pass)
    for r in rows:
        if "probe_copy_kernel" in r["Kernel_Name"]:
            markers += 1
            continue
        k = path_kernel(r["Kernel_Name"])
        if k is None:
            continue
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        names[k] = _short_kernel(r["Kernel_Name"])
        every.setdefault(k, []).append(d)
        if markers == 1:
            gated.setdefault(k, []).append(d)
    if not gated:
        raise SystemExit("summarize_trace: no per-kernel pass bracketed by two probe copies in this trace")
    lines = [f"# Kernel durations: {w.name}", "", f"Workload: {w.describe()}.", "",
             "Commands (from the repository root, on one MI355X):", "", "```", command,
             f"python3 bench.py --config {config} --summarize-trace <dir>", "```", "",
             "Per-kernel durations from `run_kernel_trace.csv`. The \"gated\" columns take the launches of the "
             "benchmark's per-kernel pass, which enqueues its calls behind a GPU spin so that kernels run back to back, "
             "each with its own start and stop events (the launches between the two 16-byte `probe_copy_kernel` "
             "markers that bracket the pass); these are the durations the benchmark's `kernels` table and `roofline` "
             "report, measured there with HIP events. \"All launches\" adds the other passes: those the host sets "
             "the pace of, where the profiler's per-dispatch work lets kernels start on an idle GPU, and the gated "
             "passes without per-kernel events, where a kernel's recorded start can precede the end of the one "
             "before it.", "",
             "| kernel | path step | gated calls | gated avg us | gated min us | gated max us | all launches avg us | "
             "algorithmic MB / launch | GB/s at gated avg | of 8 TB/s |", "|---|---|---|---|---|---|---|---|---|---|"]
    order = sorted(gated, key=lambda k: -sum(gated[k]) / len(gated[k]))
    total = 0.0
    for k in order:
        g = gated[k]
        avg = sum(g) / len(g)
        total += avg
        b = kb[k]
        lines.append(f"| `{names[k]}` | {k} | {len(g)} | {avg:.3f} | {min(g):.3f} | {max(g):.3f} | "
                     f"{sum(every[k]) / len(every[k]):.3f} | {b / 1e6:.2f} | {b / avg / 1e3:.0f} | "
                     f"{b / avg / 1e3 / HBM_PEAK_GBPS:.3f} |")
    dc = [k for k in order if PHASE_OF[k] in ("dispatch", "combine")]
    dom = max(dc, key=lambda k: sum(gated[k]) / len(gated[k]))
    avg = sum(gated[dom]) / len(gated[dom])
    lines += ["", f"Sum of the gated per-kernel averages: {total:.2f} us per step.", "",
              f"Roofline kernel (the dispatch or combine kernel with the largest mean): {dom}, {kb[dom]:,} algorithmic "
              f"bytes per launch / {avg:.3f} us = {kb[dom] / avg / 1e3:.1f} GB/s, "
              f"{kb[dom] / avg / 1e3 / HBM_PEAK_GBPS:.4f} of 8 TB/s.", ""]
    return "\n".join(lines)


def summarize_traffic(config: str) -> str:
    """Markdown table of profiles/traffic.json for one workload (calibrated FETCH_SIZE + WRITE_SIZE)."""
    from combine_router_softmax_expert_amd import workloads as wl

    w = wl.WORKLOADS[config]
    kb = kernel_bytes(w)
    t = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))[config]
    any_rec = next(iter(t.values()))
    core = f"python3 bench.py --no-cpu-baseline --core-only --config {config} --steps 3 --warmup 1"
    lines = [f"# HBM traffic per kernel launch: {w.name}", "", f"Workload: {w.describe()}.", "",
             "Commands (one counter per run, from the repository root, on one MI355X):", "", "```",
             f"timeout -s KILL 90 rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch_dir> -o run -- {core}",
             f"timeout -s KILL 90 rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write_dir> -o run -- {core}",
             "timeout -s KILL 90 rocprofv3 --pmc FETCH_SIZE --output-format csv -d <copy_fetch_dir> -o run -- "
             "python3 bench.py --copy-calibration",
             "timeout -s KILL 90 rocprofv3 --pmc WRITE_SIZE --output-format csv -d <copy_write_dir> -o run -- "
             "python3 bench.py --copy-calibration",
             f"python3 bench.py --config {config} --ingest-counters <fetch_dir> <write_dir> <copy_fetch_dir> "
             "<copy_write_dir>",
             f"python3 bench.py --config {config} --summarize-traffic", "```", "",
             "Calibration: a plain copy of 1 GiB (`torch.neg` on int32, 1 GiB read + 1 GiB written) reads FETCH_SIZE "
             f"x {any_rec['copy_factor_fetch']} and WRITE_SIZE x {any_rec['copy_factor_write']} of its known bytes; "
             "every kernel's counters are scaled by these factors. FETCH_SIZE / WRITE_SIZE count L2 <-> fabric "
             "traffic: bytes the Infinity Cache serves count as fetched.", "",
             "| kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | traffic MB/launch (calibrated) | "
             "algorithmic MB/launch | traffic / algorithmic |", "|---|---|---|---|---|---|"]
    for k, r in sorted(t.items(), key=lambda kv: -(kv[1]["fetch_bytes"] + kv[1]["write_bytes"])):
        tot = r["fetch_bytes"] + r["write_bytes"]
        lines.append(f"| {k} | {r['fetch_kib_per_dispatch']} | {r['write_kib_per_dispatch']} | {tot / 1e6:.2f} | "
                     f"{kb[k] / 1e6:.2f} | {tot / kb[k]:.3f} |")
    lines += ["", "Source hashes the figures were taken on (bench.py drops `traffic` once a kernel's source changes): "
              + ", ".join(f"{k} `{r['source_sha']}`" for k, r in sorted(t.items())), ""]
    return "\n".join(lines)


COUNTER_PASSES = (
    ("l2", "TCC_HIT_sum TCC_MISS_sum TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_DRAM_sum"),
    ("lat", "TCC_EA0_WRREQ_sum TCC_EA0_WRREQ_DRAM_sum TCP_TCC_READ_REQ_sum TCP_TCC_READ_REQ_LATENCY_sum "
            "TCP_TCC_WRITE_REQ_sum TCP_TCC_WRITE_REQ_LATENCY_sum"),
    ("occ", "OccupancyPercent MeanOccupancyPerCU SQ_WAVES GRBM_GUI_ACTIVE"),
)


def _counters_by(d: str, key) -> dict:
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            k = key(r)
            if k is None:
                continue
            vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in vals.items()}


def summarize_ceilings(bench_json: str) -> str:
    """Markdown summary of the ceilings_tbps block of a bench.py output line (the default run, or --ceilings)."""
    line = [x for x in open(bench_json).read().splitlines() if x.startswith("{")][-1]
    c = json.loads(line)["ceilings_tbps"]
    sizes = [label for label, _, _ in CEILING_SIZES]
    moved = 91.8e6
    out = ["# Probe ceilings: plain copy, streaming read, and four dependent copies of the decode bytes", "",
           "Kernels: `probe_copy_kernel<policy>`, `probe_read_kernel<nontemporal>` and `probe_gather_kernel<policy>` in "
           "`combine_router_softmax_expert_amd/csrc/probe.hip`, built like the path's kernels (kernel arguments "
           "preloaded). Copy and read: one 16-byte unit per lane, consecutive lanes on consecutive units, 256-thread "
           "workgroups (the row kernels' access pattern without the permutation). Gather: destination row r takes "
           "source row perm[r], one unit per lane, the slices of a row adjacent (the streaming exchange's pattern).", "",
           "Commands (from the repository root, on one MI355X):", "", "```",
           "python3 bench.py --ceilings > <json>        # or the default python3 bench.py line",
           "python3 bench.py --summarize-ceilings <json>", "```", "",
           "Every figure is the mean of launches the GPU runs back to back: the host enqueues them behind a GPU spin, "
           "so its pace does not enter.", "",
           "TB/s of bytes moved (a copy moves twice its size); 10 launches at 1 GiB and 940 MB, 50 at 117 MB, 500 at "
           "14.7 MB:", "",
           "| size | copy, temporal | copy, nontemporal | copy, write-through stores | read, temporal | read, nontemporal |",
           "|---|---|---|---|---|---|"]
    for sz in sizes:
        out.append(f"| {sz} | {c['copy_temporal_' + sz]} | {c['copy_nt_' + sz]} | {c['copy_write_through_' + sz]} | "
                   f"{c['read_temporal_' + sz]} | {c['read_nt_' + sz]} |")
    out += ["", "Four dependent copies that move the decode workload's dispatch+combine bytes (8.27, 14.68, 14.68 and "
            "8.26 MB copied, 91.8 MB moved in all; each copy reads the buffer the copy before it wrote into), 500 "
            "repetitions:", "", "| copies | store policy | us per four copies | of 8 TB/s |", "|---|---|---|---|"]
    names = (("temporal", "write-back"), ("nt", "nontemporal"), ("write_through", "write-through"))
    for tag, name in names:
        us = c[f"decode_dc_four_copies_{tag}_us"]
        out.append(f"| flat, contiguous | {name} | {us} | {moved / (us * 1e-6) / 8e12:.3f} |")
    us = c["decode_dc_four_row_copies_identity_write_through_us"]
    out.append(f"| rows of 14 KiB, identity order | write-through | {us} | {moved / (us * 1e-6) / 8e12:.3f} |")
    for tag, name in names:
        us = c[f"decode_dc_four_row_copies_permuted_{tag}_us"]
        out.append(f"| rows of 14 KiB, random permutation | {name} | {us} | {moved / (us * 1e-6) / 8e12:.3f} |")
    out += ["", "The row copies move 577, 1,024, 1,024 and 576 rows of 14 KiB; each takes its rows through a seeded "
            "random permutation of the 1,024 rows of the buffer the copy before it wrote into (a row is read on another "
            "XCD than the one that wrote it 7 times in 8, as in the path), or through the identity, which keeps each "
            "row on its writer's XCD.", ""]
    if "skewed_row_gather_permuted_nt_940MB" in c:
        out += ["The skewed workload's streaming row gather: 65,536 rows of 14 KiB (940 MB), nontemporal loads and "
                "stores, one-wave workgroups (as the library's streaming row kernels), 10 launches; each destination "
                "row reads the source row a seeded random permutation names (the streaming reverse exchange's "
                "pattern), or the same row (the identity):", "",
                "| order | TB/s of bytes moved | of 8 TB/s |", "|---|---|---|"]
        for order in ("identity", "permuted"):
            v = c[f"skewed_row_gather_{order}_nt_940MB"]
            out.append(f"| {order} | {v} | {v / 8:.3f} |")
        out.append("")
    return "\n".join(out)


def summarize_counters(config: str, path_dirs: list, probe_dirs: list) -> str:
    """Markdown table of the cache, latency and occupancy counters (COUNTER_PASSES) of the path's kernels,
    next to the probe copies and reads of the same sizes, per dispatch."""
    from combine_router_softmax_expert_amd import workloads as wl

    w = wl.WORKLOADS[config]

    def path_key(r):
        return path_kernel(r["Kernel_Name"])

    def probe_key(r):
        n = r["Kernel_Name"]
        if "probe_" not in n:
            return None
        pol = n.split("<", 1)[1].split(">", 1)[0]
        label = {"0": "temporal", "1": "nontemporal", "2": "write-through", "false": "temporal",
                 "true": "nontemporal"}[pol]
        mb = int(r["Grid_Size"]) * 16 / 1e6
        kind = "copy" if "probe_copy" in n else "row gather" if "probe_gather" in n else "read"
        return f"probe {kind} {mb:.1f} MB, {label}"

    def merged(dirs, key):
        out = {}
        for d in dirs:
            for k, cs in _counters_by(d, key).items():
                out.setdefault(k, {}).update(cs)
        return out

    rows = list(merged(path_dirs, path_key).items()) + sorted(merged(probe_dirs, probe_key).items())
    core = f"python3 bench.py --no-cpu-baseline --core-only --config {config} --steps 3 --warmup 1"
    probe = "python3 bench.py --ceilings --reps-scale 0.02"
    lines = [f"# Cache, latency and occupancy counters: {w.name} and the probe kernels", "",
             f"Workload: {w.describe()}.", "", "Commands (one pass per line, each for the path and for the probes; from "
             "the repository root, on one MI355X):", "", "```"]
    for name, counters in COUNTER_PASSES:
        lines.append(f"timeout -s KILL 120 rocprofv3 --pmc {counters} --output-format csv -d <{name}_dir> -o run -- "
                     f"{core}")
        lines.append(f"timeout -s KILL 120 rocprofv3 --pmc {counters} --output-format csv -d <{name}_probe_dir> -o "
                     f"run -- {probe}")
    lines += [f"python3 bench.py --config {config} --summarize-counters <l2_dir> <lat_dir> <occ_dir> "
              "<l2_probe_dir> <lat_probe_dir> <occ_probe_dir>", "```", "",
              "Per dispatch, mean over the dispatches of each kernel (the probes: per size and policy). L2 hit rate = "
              "TCC_HIT / (TCC_HIT + TCC_MISS). EA reads and writes are the L2's requests to the fabric (64 or 128 "
              "bytes each); every one is counted as destined for DRAM, because the Infinity Cache sits on the memory "
              "side of the fabric and gfx950 exposes no counter that splits its hits from HBM accesses. Latencies "
              "are TCP_TCC_*_REQ_LATENCY / TCP_TCC_*_REQ, in cycles, from the vector cache to the L2 and back. "
              "Occupancy is rocprofv3's derived OccupancyPercent and MeanOccupancyPerCU (waves resident per CU, of "
              "32); under counter collection each dispatch's GRBM_GUI_ACTIVE window includes the profiler's own "
              "overhead, so these read low in absolute terms and compare kernels of similar size.", "",
              "| kernel | L2 hit % | EA read req | EA write req | read latency (cycles) | write latency (cycles) | "
              "waves | mean waves / CU | occupancy % |", "|---|---|---|---|---|---|---|---|---|"]
    for k, c in rows:
        hit, miss = c.get("TCC_HIT_sum", 0.0), c.get("TCC_MISS_sum", 0.0)
        rq, wq = c.get("TCP_TCC_READ_REQ_sum", 0.0), c.get("TCP_TCC_WRITE_REQ_sum", 0.0)
        rl = c.get("TCP_TCC_READ_REQ_LATENCY_sum", 0.0) / rq if rq else 0.0
        wlat = c.get("TCP_TCC_WRITE_REQ_LATENCY_sum", 0.0) / wq if wq else 0.0
        lines.append(f"| {k} | {100 * hit / max(hit + miss, 1):.1f} | {c.get('TCC_EA0_RDREQ_sum', 0):.0f} | "
                     f"{c.get('TCC_EA0_WRREQ_sum', 0):.0f} | {rl:.0f} | {wlat:.0f} | {c.get('SQ_WAVES', 0):.0f} | "
                     f"{c.get('MeanOccupancyPerCU', 0):.2f} | {c.get('OccupancyPercent', 0):.1f} |")
    lines.append("")
    return "\n".join(lines)


class Runner:
    """One workload's buffers and prepared calls on cuda:0, and the ways it is timed.

    Every timing is a pair of HIP events on the launch stream around back-to-back
    calls.  ``gated`` first spins the stream for a few tens of milliseconds
    (torch.cuda._sleep) so that the host enqueues a chunk of calls ahead of the
    GPU, which then runs them back to back: with per-kernel events each launch
    costs the host ~15-20 us, more than a decode-sized kernel takes, and without
    the gate every kernel would start on an idle GPU."""

    CHUNK = 50          # calls enqueued behind one gate
    GATE_MS = 40.0

    def __init__(self, w, dev, stream, direct=False):
        import numpy as np
        import torch

        from combine_router_softmax_expert_amd import binding as B
        from combine_router_softmax_expert_amd import workloads as wl

        self.B, self.torch, self.np = B, torch, np
        self.w, self.dev, self.stream, self.direct = w, dev, stream, direct
        self.inp = wl.make_inputs(w)
        self.ctx = B.Context.for_workload(w)
        self.bufs = self.ctx.allocate(dev)
        self.x = torch.from_numpy(self.inp["x"].view(np.int16)).to(dev)
        self.logits = torch.from_numpy(self.inp["logits"]).to(dev)
        # each form's calls with their arguments checked and marshalled once (binding.PreparedPath): the
        # same library calls and kernels as binding.run_path without its per-call Python work
        self.paths = {d: B.PreparedPath(self.ctx, self.bufs, self.x, self.logits, stream, direct=d)
                      for d in (False, True)}
        self.dcs = {d: B.PreparedPath(self.ctx, self.bufs, self.x, None, stream, direct=d, stages="dispatch_combine")
                    for d in (False, True)}
        self.ev0 = torch.cuda.Event(enable_timing=True)
        self.ev1 = torch.cuda.Event(enable_timing=True)
        self._cycles_per_ms = None

    def step(self, direct=None):
        self.paths[self.direct if direct is None else direct]()

    def dispatch_combine(self, direct=None):
        """Dispatch and combine alone (routing ids/weights and expert outputs from earlier steps)."""
        self.dcs[self.direct if direct is None else direct]()

    def timed(self, fn, n):
        """Mean ms of n back-to-back calls, bracketed by synchronize + events on the launch stream."""
        torch = self.torch
        torch.cuda.synchronize()
        self.ev0.record(self.stream)
        for _ in range(n):
            fn()
        self.ev1.record(self.stream)
        torch.cuda.synchronize()
        return self.ev0.elapsed_time(self.ev1) / n

    def gated(self, fn, n):
        """Mean ms per call of n calls, in chunks that the host enqueues behind a GPU spin."""
        if self._cycles_per_ms is None:       # the spin's clock, once
            self._cycles_per_ms = _spin_cycles_per_ms(self.stream)
        return gated_ms(fn, n, self.stream, self._cycles_per_ms, chunk=self.CHUNK, gate_ms=self.GATE_MS)

    def kernel_times(self, fn, n, ctxs=None):
        """Per-kernel mean durations (ms) of n gated calls: every launch carries a start and a stop
        event in its own dispatch (moe_timing_*).  Returns ({kernel: (launches, total_ms)}, ms per call)."""
        ctxs = ctxs or [self.ctx]
        for c in ctxs:
            self.B.moe_timing_begin(c)
        ms = self.gated(fn, n)
        kt = {}
        for c in ctxs:
            for name, (launches, tot) in self.B.moe_timing_end(c).items():
                a, b = kt.get(name, (0, 0.0))
                kt[name] = (a + launches, b + tot)
        return kt, ms

    def flushed(self, fn, n, evict="write"):
        """Median ms of n single calls, each after a pass on the launch stream that keeps the GPU busy while the
        host enqueues the call (so the host's launch is not timed): "write" writes 1 GiB, which evicts the L2s
        and the 256 MB Infinity Cache and leaves the latter full of dirty lines that the measured call's own
        misses then have to write back; "read" reads 1 GiB (temporal loads), which evicts with clean lines;
        "none" spins for 0.2 ms and touches no memory (the warm single-call time)."""
        torch, np = self.torch, self.np
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=self.dev) if evict != "none" else None
        sink = torch.zeros(256, dtype=torch.int32, device=self.dev)
        if flush is not None:
            flush.fill_(1)
        elif self._cycles_per_ms is None:
            self._cycles_per_ms = _spin_cycles_per_ms(self.stream)
        times = []
        for _ in range(n):
            if evict == "write":
                with torch.cuda.stream(self.stream):
                    flush.fill_(1)
            elif evict == "read":
                self.B.moe_probe_read(flush, sink, False, self.stream)
            else:
                with torch.cuda.stream(self.stream):
                    torch.cuda._sleep(int(0.2 * self._cycles_per_ms))
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(self.stream)
            fn()
            b.record(self.stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        del flush
        return float(np.median(times))


def per_kernel_table(kt, kb) -> dict:
    out = {}
    for name, (launches, tot) in kt.items():
        avg = tot / launches
        out[name] = {"launches": launches, "avg_us": round(avg * 1e3, 3), "algorithmic_bytes": kb[name],
                     "gbps": round(kb[name] / (avg * 1e-3) / 1e9, 1)}
    return out


def roofline_of(kt, kb, config: str) -> dict:
    """The dispatch/combine kernel with the largest mean duration: its algorithmic bytes per launch
    over that duration, against the 8 TB/s HBM peak; traffic from committed counter runs."""
    dc = {n: v for n, v in kt.items() if PHASE_OF[n] in ("dispatch", "combine")}
    dom = max(dc, key=lambda n: dc[n][1] / dc[n][0])
    avg_ms = dc[dom][1] / dc[dom][0]
    achieved = kb[dom] / (avg_ms * 1e-3) / 1e9
    return {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": load_traffic(config, dom),
            "avg_us": round(avg_ms * 1e3, 3), "bytes_per_launch": kb[dom]}


def dc_block(w, ms, kb, kt) -> dict:
    dc_bytes = sum(kb[n] for n in kt if PHASE_OF[n] in ("dispatch", "combine"))
    return {"ms": round(ms, 5), "tokens_per_s": round(w.tokens / (ms * 1e-3), 1), "algorithmic_bytes": dc_bytes,
            "gbps": round(dc_bytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(dc_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}


def trace_marker(r: "Runner") -> None:
    """A 16-byte probe copy on the launch stream: two of them bracket the per-kernel pass in a kernel
    trace, so that summarize_trace can take that pass's launches apart from the other gated passes."""
    buf = r.torch.zeros(32, dtype=r.torch.uint8, device=r.dev)
    r.B.moe_probe_copy(buf[:16], buf[16:], r.B.PROBE_TEMPORAL, r.stream)


def measure_core(r: "Runner", steps: int, flush_runs: int, config: str, other_form: bool = True) -> dict:
    """The figures every H=7168 workload reports: whole steps, dispatch+combine (warm and cache-flushed),
    the direct form, per-kernel durations and the roofline of the dominant dispatch/combine kernel."""
    w = r.w
    kb = kernel_bytes(w)
    ms_step = r.timed(r.step, steps)
    step_gated_ms = r.gated(r.step, steps)
    dc_ms = r.timed(r.dispatch_combine, steps)
    dc_gated_ms = r.gated(r.dispatch_combine, steps)
    trace_marker(r)                      # the per-kernel pass, bracketed for summarize_trace
    kt, ms_with_events = r.kernel_times(r.step, steps)
    trace_marker(r)
    dc_single = r.flushed(r.dispatch_combine, flush_runs, "none") if flush_runs else None
    dc_flushed = r.flushed(r.dispatch_combine, flush_runs) if flush_runs else None
    dc_flushed_clean = r.flushed(r.dispatch_combine, flush_runs, "read") if flush_runs else None
    other = not r.direct
    other_block = None
    if other_form:
        for _ in range(5):
            r.step(other)
        other_dc_ms = r.timed(lambda: r.dispatch_combine(other), steps)
        r.B.moe_timing_begin(r.ctx)
        r.step(other)                    # once, for the names of the kernels the other form runs
        kt_other = r.B.moe_timing_end(r.ctx)
        r.step()                         # leave the buffers as the measured form wrote them
        other_block = dict(dc_block(w, other_dc_ms, kb, kt_other), mode="base" if r.direct else "direct")
    phases = {}
    for name, (launches, tot) in kt.items():
        phases[PHASE_OF[name]] = phases.get(PHASE_OF[name], 0.0) + tot / launches
    out = {
        "workload": w.name, "mode": "direct" if r.direct else "base",
        "ms_per_step": round(ms_step, 5), "tokens_per_s": round(w.tokens / (ms_step * 1e-3), 1),
        "ms_per_step_gated": round(step_gated_ms, 5),
        "dispatch_combine": dict(dc_block(w, dc_ms, kb, kt), gated_ms=round(dc_gated_ms, 5)),
        "dispatch_combine_single_call": None if dc_single is None else dc_block(w, dc_single, kb, kt),
        "dispatch_combine_cache_flushed": None if dc_flushed is None else dc_block(w, dc_flushed, kb, kt),
        "dispatch_combine_cache_flushed_clean": None if dc_flushed_clean is None else dc_block(w, dc_flushed_clean,
                                                                                              kb, kt),
        "other_mode_dispatch_combine": other_block,
        "kernels": per_kernel_table(kt, kb),
        "phases_ms": {k: round(v, 5) for k, v in phases.items()},
        "ms_per_step_with_kernel_events": round(ms_with_events, 5),
        "roofline": roofline_of(kt, kb, config),
    }
    return out


def micro_batch_figures(r: "Runner", steps: int, parts: int = 2) -> dict:
    """Micro-batches through the split phases: the expert stage of one on a second stream overlaps the
    dispatch and combine of the others, the streams ordered by the library's events.  Wall time on two
    streams and on one (stream order alone, no events), eagerly and with the host enqueued ahead (gated),
    against the sum of the schedule's kernel durations (the phases end to end)."""
    B, torch, w = r.B, r.torch, r.w
    from combine_router_softmax_expert_amd import workloads as wl

    fp8 = w.dispatch_dtype != "bf16"
    mb = []
    for c in range(parts):
        rows = torch.from_numpy(wl.micro_batch_rows(w.num_ranks, w.tokens_per_rank, parts, c)).to(r.dev)
        cc = B.Context(w.num_ranks, w.tokens_per_rank // parts, w.num_experts, w.top_k, w.hidden, fp8)
        mb.append((cc, cc.allocate(r.dev), r.x[rows].contiguous(), r.logits[rows].contiguous()))
    comm, compute = torch.cuda.Stream(), torch.cuda.Stream()
    fork, join = B.OrderEvent(), [B.OrderEvent(), B.OrderEvent()]

    def schedule(same_stream):
        cs = comm if same_stream else compute

        def go():                  # the schedule between the launch stream's work before and after it
            fork.record(r.stream)
            fork.wait(comm)
            if not same_stream:
                fork.wait(cs)
            B.run_overlapped(mb, comm, cs)
            join[0].record(comm)
            join[0].wait(r.stream)
            if not same_stream:
                join[1].record(cs)
                join[1].wait(r.stream)
        return go

    two, one = schedule(False), schedule(True)
    for _ in range(5):
        two()
        one()
    out = {"parts": parts,
           "eager_ms_two_streams": round(r.timed(two, steps), 5), "eager_ms_one_stream": round(r.timed(one, steps), 5),
           "gated_ms_two_streams": round(r.gated(two, steps), 5), "gated_ms_one_stream": round(r.gated(one, steps), 5)}
    kt, _ = r.kernel_times(one, min(steps, 100), ctxs=[m[0] for m in mb])
    # the phases end to end: every kernel of the schedule, one after another
    out["sum_of_kernel_ms"] = round(sum(tot / min(steps, 100) for _, tot in kt.values()), 5)
    out["saved_by_second_stream_ms"] = round(out["gated_ms_one_stream"] - out["gated_ms_two_streams"], 5)
    out["tokens_per_s_two_streams"] = round(w.tokens / (out["gated_ms_two_streams"] * 1e-3), 1)
    del mb
    return out


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
    ap.add_argument("--no-flush-run", action="store_true", help="skip the cache-flushed runs")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the blocks of the other H=7168 workloads (byte-model and skewed)")
    ap.add_argument("--core-only", action="store_true",
                    help="only the headline workload's timed steps, dispatch+combine and per-kernel pass (for kernel "
                         "traces: no other forms, workloads, micro-batches or graphs whose launches would mix in)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--ceilings", action="store_true",
                    help="only run the copy and streaming-read probes and print their rates")
    ap.add_argument("--eviction-probe", action="store_true",
                    help="only time single 117 MB probe reads and copies after each cache-eviction pass")
    ap.add_argument("--reps-scale", type=float, default=1.0,
                    help="scale the probes' repetitions (short runs under a counter profiler)")
    ap.add_argument("--ingest-counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="turn rocprofv3 --pmc outputs into profiles/traffic.json for --config")
    ap.add_argument("--counter-command", default="", help="command recorded with --ingest-counters")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="print the markdown summary of a rocprofv3 --kernel-trace run of bench.py --core-only")
    ap.add_argument("--trace-command", default="", help="command recorded with --summarize-trace")
    ap.add_argument("--summarize-traffic", action="store_true",
                    help="print the markdown summary of profiles/traffic.json for --config")
    ap.add_argument("--summarize-ceilings", metavar="BENCH_JSON",
                    help="print the markdown summary of the ceilings in a bench.py output (default run or --ceilings)")
    ap.add_argument("--summarize-counters", nargs=6, metavar=("L2", "LAT", "OCC", "L2_PROBE", "LAT_PROBE", "OCC_PROBE"),
                    help="print the markdown summary of the cache, latency and occupancy counter passes")
    args = ap.parse_args()

    if args.summarize_trace:
        print(summarize_trace(args.config, args.summarize_trace, args.trace_command))
        return
    if args.summarize_traffic:
        print(summarize_traffic(args.config))
        return
    if args.summarize_ceilings:
        print(summarize_ceilings(args.summarize_ceilings))
        return

    if args.summarize_counters:
        print(summarize_counters(args.config, list(args.summarize_counters[:3]), list(args.summarize_counters[3:])))
        return

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

    if args.eviction_probe:
        import torch
        torch.cuda.set_device(0)
        print(json.dumps(eviction_probe(torch.device("cuda:0"), torch.cuda.current_stream())), flush=True)
        return

    if args.ceilings:
        import torch
        torch.cuda.set_device(0)
        print(json.dumps({"ceilings_tbps": ceilings(torch.device("cuda:0"), torch.cuda.current_stream(),
                                                    args.reps_scale)}), flush=True)
        return

    import numpy as np
    import torch

    from combine_router_softmax_expert_amd import workloads as wl

    w = wl.WORKLOADS[args.config]
    if args.ranks:
        w = wl.custom(f"{w.name}-as-ep{args.ranks}", args.ranks, w.tokens, w.num_experts, w.top_k, w.hidden,
                      w.dispatch_dtype, w.seed, w.zipf)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    r = Runner(w, dev, stream, direct=args.mode == "direct")
    B = r.B
    extras = not args.core_only
    flush_runs = 0 if args.no_flush_run else 30

    for _ in range(args.warmup):
        r.step()
    torch.cuda.synchronize()

    # timed region: K back-to-back steps of the whole path (the headline value)
    ms_per_step = r.timed(r.step, args.steps)

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

    core = measure_core(r, args.steps, 0 if args.core_only else flush_runs, args.config, other_form=extras)
    latency_ms = None
    ag = graph = micro = cold_ms = cold_clean_ms = None
    if extras:
        latency_ms = {"step": latency_percentiles(r.step, args.steps),
                      "dispatch_combine": latency_percentiles(r.dispatch_combine, args.steps)}
        # the all-gather dispatcher (with the base combine) on the same data
        gathered, gathered_scales = r.ctx.allocate_gathered(dev)
        allgather_dc = B.PreparedPath(r.ctx, r.bufs, r.x, None, stream, stages="dispatch_combine",
                                      gathered=gathered, gathered_scales=gathered_scales)
        for _ in range(args.warmup):
            allgather_dc()
        ag_ms = r.timed(allgather_dc, args.steps)
        kt_ag, _ = r.kernel_times(allgather_dc, min(args.steps, 200))
        ag = dict(dc_block(w, ag_ms, kernel_bytes(w), kt_ag),
                  kernels_us={n: round(v[1] / v[0] * 1e3, 3) for n, v in kt_ag.items()})
        del allgather_dc, gathered, gathered_scales
        r.step()   # leave the buffers as the measured form wrote them
        if flush_runs:
            cold_ms = r.flushed(r.step, flush_runs)
            cold_clean_ms = r.flushed(r.step, flush_runs, "read")

        # the step captured once in a HIP graph and replayed (no per-call host work)
        def graph_ms(direct):
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                B.run_path(r.ctx, r.bufs, r.x, r.logits, None, direct=direct)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                B.run_path(r.ctx, r.bufs, r.x, r.logits, None, direct=direct)
            for _ in range(args.warmup):
                g.replay()
            ms = r.timed(g.replay, args.steps)
            gated = r.gated(g.replay, args.steps)   # replays enqueued ahead: the GPU's own time per replay
            del g
            return ms, gated

        graph = {}
        for mode, d in (("base", False), ("direct", True)):
            ms, gated = graph_ms(d)
            graph[mode] = {"ms_per_step": round(ms, 5), "tokens_per_s": round(w.tokens / (ms * 1e-3), 1),
                           "gated_ms_per_step": round(gated, 5)}
        micro = micro_batch_figures(r, min(args.steps, 300))
        r.step()   # leave the buffers as the measured form wrote them

    T = w.tokens
    kb = kernel_bytes(w)
    step_bytes = sum(kb[n] for n in core["kernels"])
    out = {
        "metric": METRIC,
        "value": round(T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_gated": core["ms_per_step_gated"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dispatch_dtype == "bf16" else "fp8_e4m3+bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "ranks": w.num_ranks, "tokens": T, "experts": w.num_experts,
                   "top_k": w.top_k, "hidden": w.hidden, "dispatch": w.dispatch_dtype,
                   "parallelism": f"ep{w.num_ranks} emulated on 1 GPU", "mode": args.mode},
        "value_is": "whole step (route, dispatch, expert stub, combine); dispatch_combine.tokens_per_s is the "
                    "dispatch and combine alone",
        "step_gbps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "dispatch_combine": dict(core["dispatch_combine"],
                                 logical_payload_bytes=logical_payload_bytes(w),
                                 logical_payload_gbps=round(logical_payload_bytes(w) / (core["dispatch_combine"]["ms"]
                                                                                        * 1e-3) / 1e9, 1)),
        "dispatch_combine_single_call": core["dispatch_combine_single_call"],
        "dispatch_combine_cache_flushed": core["dispatch_combine_cache_flushed"],
        "dispatch_combine_cache_flushed_clean": core["dispatch_combine_cache_flushed_clean"],
        "other_mode": core["other_mode_dispatch_combine"],
        "allgather_dispatch": ag,
        "graph_replay": graph,
        "micro_batches": micro,
        "phases_ms": core["phases_ms"],
        "kernels": core["kernels"],
        "kernel_timing": "per-kernel HIP events in each launch, the host enqueued ahead of a GPU spin (gated)",
        "latency_ms": latency_ms,
        "ms_per_step_with_kernel_events": core["ms_per_step_with_kernel_events"],
        "ms_per_step_cache_flushed": None if cold_ms is None else round(cold_ms, 5),
        "ms_per_step_cache_flushed_clean": None if cold_clean_ms is None else round(cold_clean_ms, 5),
        "metadata_bytes_per_step": metadata_bytes(w),
        "roofline": core["roofline"],
        "h7168_workloads": None,
        "ceilings_tbps": None,
        "routing": routing_stats(r.bufs["topk_ids"].cpu().numpy(), w.num_ranks, w.num_experts),
        "hardware": host_info(),
        "cpu_baseline": None,
    }
    inp = r.inp
    del r
    torch.cuda.empty_cache()
    if extras and not args.no_other_configs and not args.ranks:
        # the other H=7168 workloads the target applies to, each in its own buffers
        blocks = {}
        for name in ("c2", "c3", "c5"):
            if name == args.config:
                continue
            o = Runner(wl.WORKLOADS[name], dev, stream, direct=args.mode == "direct")
            for _ in range(10):
                o.step()
            blocks[name] = measure_core(o, min(args.steps, 300), min(flush_runs, 10), name)
            del o
            torch.cuda.empty_cache()
        out["h7168_workloads"] = blocks
    if extras:
        out["ceilings_tbps"] = ceilings(dev, stream)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
