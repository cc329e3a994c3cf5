"""Split phases and the two-stream micro-batch schedule: each micro-batch's
tokens, run through moe_dispatch_send/recv, the expert stage on a second
stream and moe_combine_send/recv, must give bit for bit the outputs the whole
batch gives for those tokens in one eager pass (routing, weights and y depend
on the token alone; positions are per micro-batch)."""

import numpy as np
import pytest

from combine_router_softmax_expert_amd import workloads as wl
from gpu_helpers import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,parts,same_stream", [("c1", 2, False), ("c2", 2, False), ("c2", 4, False),
                                                    ("c3", 2, False), ("c3", 2, True)])
def test_micro_batches_on_two_streams_match_the_whole_batch(name, parts, same_stream):
    import torch
    from combine_router_softmax_expert_amd import binding as B

    log(f"[overlap] {name} parts={parts} same_stream={same_stream}")
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    ctx = B.Context.for_workload(w)
    bufs = ctx.allocate()
    x = torch.from_numpy(inp["x"].view(np.int16)).cuda()
    logits = torch.from_numpy(inp["logits"]).cuda()
    B.run_path(ctx, bufs, x, logits)
    torch.cuda.synchronize()
    want_y = bufs["y"].view(torch.int16).cpu().numpy()
    want_ids = bufs["topk_ids"].cpu().numpy()
    want_w = bufs["topk_w"].cpu().numpy()

    P, Tp = w.num_ranks, w.tokens_per_rank
    fp8 = w.dispatch_dtype != "bf16"
    run = []
    for c in range(parts):
        rows = wl.micro_batch_rows(P, Tp, parts, c)
        cc = B.Context(P, Tp // parts, w.num_experts, w.top_k, w.hidden, fp8)
        cb = cc.allocate()
        for t in cb.values():
            if t is not None:
                t.view(torch.uint8).fill_(0xA5)
        run.append((cc, cb, x[torch.from_numpy(rows).cuda()].contiguous(),
                    logits[torch.from_numpy(rows).cuda()].contiguous(), rows))
    comm = torch.cuda.Stream()
    compute = comm if same_stream else torch.cuda.Stream()
    comm.wait_stream(torch.cuda.current_stream())
    compute.wait_stream(torch.cuda.current_stream())
    B.run_overlapped([r[:4] for r in run], comm, compute)
    torch.cuda.synchronize()
    for cc, cb, _, _, rows in run:
        assert np.array_equal(cb["topk_ids"].cpu().numpy(), want_ids[rows])
        assert np.array_equal(cb["topk_w"].cpu().numpy(), want_w[rows])
        assert np.array_equal(cb["y"].view(torch.int16).cpu().numpy(), want_y[rows])
