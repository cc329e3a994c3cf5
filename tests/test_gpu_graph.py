"""The whole path captured in a HIP graph (torch.cuda.CUDAGraph on the caller's
stream) and replayed ([A2A] 9: a low-latency decode path keeps host work and
synchronisation off the step).  With new inputs copied into the captured buffers,
the outputs poisoned before each replay and eager work and synchronisations
between replays, every replay must give the oracle's outputs for its inputs
(ids, integer parts, rows, scales, expert outputs and combine rows bit for bit,
weights and y to the parity tolerances) and, bit for bit, what eager calls give
on the same inputs.  The library only enqueues kernel launches on the caller's
stream (no allocation, no memset, no host synchronisation), which is what makes
the capture valid."""

import numpy as np
import pytest

from combine_router_softmax_expert_amd import workloads as wl
from gpu_helpers import compare_with_oracle, log, oracle_path, read_back

pytestmark = pytest.mark.gpu


def _snapshot(bufs, direct):
    import torch
    keys = ["topk_ids", "topk_w", "recv", "expert_out", "y"] + ([] if direct else ["send", "comb"])
    if bufs["recv_scales"] is not None:
        keys.append("recv_scales")
    return {key: bufs[key].view(torch.uint8).clone() for key in keys}   # raw bytes: bit-exact comparison


@pytest.mark.parametrize("name,direct", [("c1", False), ("c2", False), ("c2", True), ("c3", True)])
def test_graph_replays_match_the_oracle(orc, name, direct):
    import torch
    from combine_router_softmax_expert_amd import binding as B

    log(f"[graph] {name} direct={direct}")
    w = wl.WORKLOADS[name]
    sh = orc.Shape.of(w)
    ctx = B.Context.for_workload(w)
    bufs = ctx.allocate()
    inputs = [wl.make_inputs(w)]
    for seed in (11, 12, 13):     # three more input sets of the same shape for the replays
        inputs.append({"x": wl.make_hidden(seed, w.tokens, w.hidden), "logits": wl.make_logits(seed, w.tokens,
                                                                                              w.num_experts)})
    oracle = [oracle_path(orc, sh, i["x"], logits=i["logits"]) for i in inputs]
    xs = [torch.from_numpy(i["x"].view(np.int16)).cuda() for i in inputs]
    ls = [torch.from_numpy(i["logits"]).cuda() for i in inputs]
    x = xs[0].clone()
    logits = ls[0].clone()

    # eager results for every input set
    expected = []
    for xi, li in zip(xs, ls):
        x.copy_(xi)
        logits.copy_(li)
        B.run_path(ctx, bufs, x, logits, direct=direct)
        torch.cuda.synchronize()
        expected.append(_snapshot(bufs, direct))

    # capture one step (warmed up on the capture stream first, as torch asks)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.run_path(ctx, bufs, x, logits, direct=direct)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        h = B.run_path(ctx, bufs, x, logits, direct=direct)   # the handle's arrays: fixed workspace addresses
    torch.cuda.synchronize()

    for rep in range(2):
        for i, (xi, li) in enumerate(zip(xs, ls)):
            x.copy_(xi)
            logits.copy_(li)
            for t in bufs.values():          # poison the outputs: the replay must rewrite them
                if t is not None and t is not bufs["workspace"]:
                    t.view(torch.uint8).fill_(0xA5)
            graph.replay()
            scratch = torch.randn(1 << 16, device="cuda").sum()   # eager work between replays
            torch.cuda.synchronize()
            got = _snapshot(bufs, direct)
            for key, want in expected[i].items():
                assert torch.equal(got[key], want), (name, direct, rep, i, key)
            g = read_back(sh, ctx, bufs, h, direct=direct)
            compare_with_oracle(orc, sh, g, inputs[i]["x"], logits=inputs[i]["logits"], o=oracle[i])
            del scratch
