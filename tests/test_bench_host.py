"""Host logic of bench.py (no GPU): the single-GPU refusal, the algorithmic byte
model against its closed form, rocprof kernel-name mapping, the counter
calibration arithmetic and the kernel-trace summary's choice of launches."""

import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402
from combine_router_softmax_expert_amd import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT)
    assert r.returncode == 2 and "exactly one GPU" in r.stderr


@pytest.mark.parametrize("name,total", [("c1", 1_835_008), ("c2", 91_750_400), ("c3", 325_713_920),
                                        ("c4", 1_879_048_192), ("c5", 4_506_779_648)])
def test_dispatch_combine_bytes_match_the_closed_form(name, total):
    # 2HT + 3 N_a D + 3 N_a 2H + 2HT with D the dispatched row including FP8 scales
    # (the totals of the byte model the measurement is defined by); the count's
    # metadata bytes (8 N_a + 12 P E) are counted on top
    w = wl.WORKLOADS[name]
    kb = bench.kernel_bytes(w)
    payload = kb["pack"] + kb["exchange"] + kb["reverse_exchange"] + kb["reduce"]
    assert payload == total
    H, T, Na = w.hidden, w.tokens, w.tokens * w.top_k
    D = H + 4 * (H // 128) if w.dispatch_dtype != "bf16" else 2 * H
    assert kb["pack_direct"] + kb["reduce_direct"] == 2 * H * T + Na * D + Na * 2 * H + 2 * H * T
    assert kb["count_pack"] == kb["count"] + kb["pack"]


def test_routing_stats_on_a_known_routing():
    # 2 ranks, 4 experts (2 per rank), 4 tokens (2 per rank), top-2
    ids = np.array([[0, 1], [0, 2], [3, 0], [2, 3]], dtype=np.int32)
    s = bench.routing_stats(ids, 2, 4)
    # expert loads 3, 1, 2, 2 (mean 2); rank loads 4, 4; tokens 0-1 on rank 0, 2-3 on rank 1:
    # local assignments: (0,0) (0,1) (1,0) for rank 0 and (2,3) (3,2) (3,3) for rank 1 -> 6 of 8
    assert s == {"expert_imbalance": 1.5, "empty_experts": 0, "top10pct_expert_share": 0.375,
                 "rank_imbalance": 1.0, "local_share": 0.75}


def test_byte_model_example_payload():
    # the logical payload of the byte-model workload: N_a * H * (1 + 2) bytes
    w = wl.WORKLOADS["c3"]
    assert w.tokens * w.top_k * w.hidden * (1 + 2) == 88_080_384
    assert bench.logical_payload_bytes(w) == 88_080_384
    # bf16 dispatch: 2H out and 2H back per assignment (decode workload: 29,360,128 B)
    assert bench.logical_payload_bytes(wl.WORKLOADS["c2"]) == 29_360_128


@pytest.mark.parametrize("rocprof_name,kernel", [
    ("void moe::(anonymous namespace)::count_pack_kernel<false, false, 4, 1, true>(x)", "count_pack"),
    ("void moe::(anonymous namespace)::count_pack_kernel<true, true, 16, 2, true>(x)", "count_pack_direct"),
    ("moe::(anonymous namespace)::pack_kernel<true, true, false, false>(x)", "pack"),
    ("moe::(anonymous namespace)::pack_kernel<false, false, false, true>(x)", "pack_direct"),
    ("reduce_kernel<true, true, true>(x)", "reduce_direct"),
    ("reduce_kernel<false, false, false>(x)", "reduce"),
    ("reduce_affine_kernel<true>(x)", "reduce_direct"), ("reduce_affine_kernel<false>(x)", "reduce"),
    ("reverse_exchange_affine_kernel(x)", "reverse_exchange"), ("exchange_affine_kernel(x)", "exchange"),
    ("stub_affine_kernel(x)", "stub"),
    ("reverse_exchange_gather_kernel(x)", "reverse_exchange"), ("reverse_exchange_scatter_kernel(x)",
                                                                "reverse_exchange"),
    ("exchange_kernel<true>(x)", "exchange"), ("count_scan_single_kernel(x)", "count"), ("scan_kernel(x)", "scan"),
    ("scan_spread_kernel(x)", "scan"),
    ("allgather_kernel<true, false, false>(x)", "allgather"), ("select_scatter_kernel<false>(x)", "select"),
    ("select_kernel<true>(x)", "select"), ("handle_kernel(x)", "handles"),
    ("count_pack_kernel<false, true, 8, 1, false>(x)", "count_handles"),
    ("route_topk_wave_kernel<4>(x)", "route_topk"), ("stub_kernel<true, true, false>(x)", "stub"),
    ("at::native::vectorized_elementwise_kernel(x)", None),
])
def test_rocprof_names_map_to_path_steps(rocprof_name, kernel):
    assert bench.path_kernel(rocprof_name) == kernel


def _counter_csv(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, value in rows:
            wr.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_counter_ingestion_scales_by_the_copy_calibration(tmp_path):
    copy_bytes = 1 << 30
    # the copy reads FETCH_SIZE = half its bytes and WRITE_SIZE = all of them (KiB)
    _counter_csv(tmp_path / "cf", "FETCH_SIZE", [("copy", copy_bytes / 2048)])
    _counter_csv(tmp_path / "cw", "WRITE_SIZE", [("copy", copy_bytes / 1024)])
    name = "moe::(anonymous namespace)::exchange_kernel<false>(x)"
    _counter_csv(tmp_path / "f", "FETCH_SIZE", [(name, 100.0), (name, 300.0)])   # mean 200 KiB
    _counter_csv(tmp_path / "w", "WRITE_SIZE", [(name, 400.0)])
    out = tmp_path / "traffic.json"
    bench.ingest_counters("cX", str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"), str(tmp_path / "cw"),
                          copy_bytes, "cmd", path=str(out))
    rec = json.load(open(out))["cX"]["exchange"]
    assert rec["fetch_bytes"] == 2 * 200 * 1024 and rec["write_bytes"] == 400 * 1024
    assert rec["source_sha"] == bench.source_sha("exchange")


def test_trace_summary_takes_the_bracketed_pass_only(tmp_path):
    # launches before the first marker (ungated passes), between the two markers (the per-kernel pass)
    # and after the second: only the middle ones count as gated
    rows, t = [], 0
    def launch(name, us):
        nonlocal t
        rows.append({"Kernel_Name": name, "Start_Timestamp": str(t), "End_Timestamp": str(t + int(us * 1000))})
        t += int(us * 1000) + 500
    ex = "void moe::(anonymous namespace)::exchange_kernel<false>(x)"
    launch("at::cuda::(anonymous namespace)::spin_kernel(long)", 50.0)
    launch(ex, 9.0)
    launch("void moe::(anonymous namespace)::probe_copy_kernel<0>(x)", 1.0)
    launch(ex, 5.0)
    launch(ex, 7.0)
    launch("void moe::(anonymous namespace)::probe_copy_kernel<0>(x)", 1.0)
    launch(ex, 20.0)
    os.makedirs(tmp_path / "tr")
    with open(tmp_path / "tr" / "run_kernel_trace.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        wr.writeheader()
        wr.writerows(rows)
    md = bench.summarize_trace("c2", str(tmp_path / "tr"), "cmd")
    line = next(x for x in md.splitlines() if x.startswith("| `exchange_kernel"))
    cells = [c.strip() for c in line.split("|")]
    assert cells[3] == "2" and cells[4] == "6.000"          # gated calls and mean of the bracketed pair
    assert cells[7] == "10.250"                            # all four launches
    os.remove(tmp_path / "tr" / "run_kernel_trace.csv")
    with open(tmp_path / "tr" / "run_kernel_trace.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        wr.writeheader()
        wr.writerows([r for r in rows if "probe_copy" not in r["Kernel_Name"]])
    with pytest.raises(SystemExit):                        # no bracketed pass: refused, not guessed
        bench.summarize_trace("c2", str(tmp_path / "tr"), "cmd")


def test_cpu_baseline_reports_its_sample_cores_and_build(orc):
    import bench
    from combine_router_softmax_expert_amd import workloads as wl
    w = wl.WORKLOADS["c1"]
    r = bench.cpu_baseline(w, wl.make_inputs(w), 0.2)
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["unit"] == "tokens/s" and r["value"] > 0
    assert "-ffp-contract=off" in r["build"]
    # the sample is sized by a timing probe: the whole workload, or the first tokens of each of the 4 ranks
    import re
    m = re.match(r"(?:whole workload|first (\d+) of 64 tokens on each of 4 ranks) \((\d+) tokens\)", r["sample"])
    assert m, r["sample"]
    assert int(m.group(2)) == (256 if m.group(1) is None else 4 * int(m.group(1)))


def test_ceilings_summary_renders_every_probe(tmp_path):
    # a bench line with every ceiling key (values made up): the summary names each size and policy,
    # the decode chains and, when present, the skewed row gather
    c = {}
    for label, _, _ in bench.CEILING_SIZES:
        for kind in ("copy", "read"):
            for tag in ("temporal", "nt", "write_through"):
                c[f"{kind}_{tag}_{label}"] = 6.5
    for tag in ("temporal", "nt", "write_through"):
        c[f"decode_dc_four_copies_{tag}_us"] = 15.0
        c[f"decode_dc_four_row_copies_permuted_{tag}_us"] = 17.5
    c["decode_dc_four_row_copies_identity_write_through_us"] = 16.0
    path = tmp_path / "bench.json"
    path.write_text(json.dumps({"ceilings_tbps": c}) + "\n")
    text = bench.summarize_ceilings(str(path))
    for label, _, _ in bench.CEILING_SIZES:
        assert f"| {label} |" in text
    assert "random permutation | write-through | 17.5 |" in text
    assert "skewed workload's streaming row gather" not in text
    c["skewed_row_gather_identity_nt_940MB"] = 6.8
    c["skewed_row_gather_permuted_nt_940MB"] = 6.3
    path.write_text(json.dumps({"ceilings_tbps": c}) + "\n")
    text = bench.summarize_ceilings(str(path))
    assert "| permuted | 6.3 | 0.787 |" in text and "| identity | 6.8 | 0.850 |" in text
