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
