"""Many steps back to back must keep giving the first step's bytes.

Every cross-kernel hand-off in the path (rows, FP8 scales and handle records
written through, scalar loads of maps and weights, counts read by the next
launch) relies on the kernel boundary for visibility.  These tests run the
whole path hundreds of times in a row on one stream, with no host
synchronisation in between, and after every step compare all of its outputs
with the first step's on the GPU (a mismatch counter that only the end of the
run reads back).  The first step itself is checked against the individual
library calls bit for bit by test_gpu_prepared, and those against the oracle
by test_gpu_parity."""

import numpy as np
import pytest

from combine_router_softmax_expert_amd import workloads as wl
from gpu_helpers import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,direct,steps", [("c2", False, 400), ("c2", True, 400), ("c3", False, 200),
                                               ("c5", False, 20)])
def test_back_to_back_steps_stay_bit_identical(name, direct, steps):
    import torch
    from combine_router_softmax_expert_amd import binding as B

    log(f"[repeat] {name} direct={direct} steps={steps}")
    w = wl.WORKLOADS[name]
    ctx = B.Context.for_workload(w)
    bufs = ctx.allocate()
    inp = wl.make_inputs(w)
    x = torch.from_numpy(inp["x"].view(np.int16)).cuda()
    logits = torch.from_numpy(inp["logits"]).cuda()
    path = B.PreparedPath(ctx, bufs, x, logits, direct=direct)
    path()
    torch.cuda.synchronize()
    keys = ["topk_ids", "topk_w", "recv", "expert_out", "y"] + ([] if direct else ["send", "comb"])
    if bufs["recv_scales"] is not None:
        keys.append("recv_scales")
    # int32 words of each output (every buffer is a whole number of 4-byte words)
    words = {k: bufs[k].view(torch.uint8).view(torch.int32) for k in keys}
    first = {k: v.clone() for k, v in words.items()}
    mismatches = torch.zeros((), dtype=torch.int64, device="cuda")
    for _ in range(steps):
        path()
        for k in keys:
            mismatches += (words[k] != first[k]).sum()
    torch.cuda.synchronize()
    assert int(mismatches.item()) == 0, (name, direct, int(mismatches.item()))
    ctx.close()


@pytest.mark.parametrize("name,parts,reps", [("c2", 2, 100), ("c3", 2, 50)])
def test_two_stream_schedule_repeated_stays_bit_identical(name, parts, reps):
    """The micro-batch schedule orders its two streams with the library's events; run many times back to
    back (each run waits only for the comparisons of the one before), every micro-batch's routing, expert
    outputs and y must keep the first run's bytes."""
    import torch
    from combine_router_softmax_expert_amd import binding as B

    log(f"[repeat] two streams {name} parts={parts} reps={reps}")
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    x = torch.from_numpy(inp["x"].view(np.int16)).cuda()
    logits = torch.from_numpy(inp["logits"]).cuda()
    P, Tp = w.num_ranks, w.tokens_per_rank
    fp8 = w.dispatch_dtype != "bf16"
    run = []
    for c in range(parts):
        rows = torch.from_numpy(wl.micro_batch_rows(P, Tp, parts, c)).cuda()
        cc = B.Context(P, Tp // parts, w.num_experts, w.top_k, w.hidden, fp8)
        run.append((cc, cc.allocate(), x[rows].contiguous(), logits[rows].contiguous()))
    comm, compute = torch.cuda.Stream(), torch.cuda.Stream()
    main = torch.cuda.current_stream()

    def once():
        comm.wait_stream(main)                # the comparisons of the run before have read the outputs
        compute.wait_stream(main)
        B.run_overlapped(run, comm, compute)
        main.wait_stream(comm)
        main.wait_stream(compute)

    keys = ("topk_ids", "topk_w", "expert_out", "y")
    once()
    torch.cuda.synchronize()
    words = [{k: cb[k].view(torch.uint8).view(torch.int32) for k in keys} for _, cb, _, _ in run]
    first = [{k: v.clone() for k, v in ws.items()} for ws in words]
    mismatches = torch.zeros((), dtype=torch.int64, device="cuda")
    for _ in range(reps):
        once()
        for ws, fs in zip(words, first):
            for k in keys:
                mismatches += (ws[k] != fs[k]).sum()
    torch.cuda.synchronize()
    assert int(mismatches.item()) == 0, (name, int(mismatches.item()))
    for cc, _, _, _ in run:
        cc.close()
