"""Split phases and the two-stream micro-batch schedule ([PPLX] dispatch and combine
as send and receive halves; [A2A] 7: overlap needs independent work to hide behind).
Each micro-batch is itself a rank-blocked EP problem; its outputs after
moe_dispatch_send/recv, the expert stage on a second stream and
moe_combine_send/recv must equal the oracle's whole path on that micro-batch's
tokens (ids, integer parts, rows, scales, expert outputs and combine rows bit for
bit, weights and y to the parity tolerances), and routing, weights and y must also
equal, bit for bit, what the whole batch gives for those tokens."""

import ctypes

import numpy as np
import pytest

from combine_router_softmax_expert_amd import workloads as wl
from gpu_helpers import compare_with_oracle, log, read_back

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,parts,same_stream", [("c1", 2, False), ("c2", 2, False), ("c2", 4, False),
                                                    ("c3", 2, False), ("c3", 2, True)])
def test_micro_batches_on_two_streams_match_the_oracle(orc, name, parts, same_stream):
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
    whole_y = bufs["y"].view(torch.int16).cpu().numpy()
    whole_ids = bufs["topk_ids"].cpu().numpy()
    whole_w = bufs["topk_w"].cpu().numpy()

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
    handles = B.run_overlapped([r[:4] for r in run], comm, compute)
    torch.cuda.synchronize()
    for (cc, cb, _, _, rows), h in zip(run, handles):
        sh = orc.Shape(P, P * (Tp // parts), w.num_experts, w.top_k, w.hidden, fp8)
        g = read_back(sh, cc, cb, h)
        compare_with_oracle(orc, sh, g, inp["x"][rows], logits=inp["logits"][rows])
        assert np.array_equal(g["ids"], whole_ids[rows])
        assert np.array_equal(g["w"].view(np.uint32), whole_w[rows].view(np.uint32))
        assert np.array_equal(g["y"].view(np.int16), whole_y[rows])


def test_run_overlapped_refuses_stream_capture():
    """The micro-batch schedule forks work onto two streams and orders them with the library's
    events; it is not built for graph capture, so it refuses to run while the caller's stream,
    or either of its own, is capturing, before it enqueues anything.  The events refuse a
    capturing stream by themselves too."""
    import torch
    from combine_router_softmax_expert_amd import binding as B

    w = wl.WORKLOADS["c1"]
    inp = wl.make_inputs(w)
    ctx = B.Context.for_workload(w)
    bufs = ctx.allocate()
    x = torch.from_numpy(inp["x"].view(np.int16)).cuda()
    logits = torch.from_numpy(inp["logits"]).cuda()
    comm, compute = torch.cuda.Stream(), torch.cuda.Stream()
    side = torch.cuda.Stream()
    counter = torch.zeros(1, device="cuda")
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        graph.capture_begin()
        try:
            counter.add_(1.0)           # one captured node, so the graph is not empty
            with pytest.raises(RuntimeError, match="capturing"):
                B.run_overlapped([(ctx, bufs, x, logits)], comm, compute)
            ev = B.OrderEvent()
            assert B.lib.moe_event_record(ev.handle, ctypes.c_void_p(side.cuda_stream)) == -2
            assert b"capturing" in B.lib.moe_last_error()
            assert B.lib.moe_stream_wait_event(ctypes.c_void_p(side.cuda_stream), ev.handle) == -2
        finally:
            graph.capture_end()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    assert counter.item() == 1.0        # the capture holds the add alone: nothing of the schedule ran or was captured
    del graph


def test_order_event_orders_two_streams():
    """Work enqueued on a stream after OrderEvent.wait starts only after the work the other stream had
    enqueued before OrderEvent.record: a copy on the waiting stream reads what a kernel on the recording
    stream wrote after a long GPU spin (without the wait it would read the old contents), on every one of
    several rounds that reuse the same event."""
    import torch
    from combine_router_softmax_expert_amd import binding as B

    a, b = torch.cuda.Stream(), torch.cuda.Stream()
    ev = B.OrderEvent()
    src = torch.zeros(1 << 20, dtype=torch.int32, device="cuda")
    for r in range(1, 4):
        torch.cuda.synchronize()
        with torch.cuda.stream(a):
            torch.cuda._sleep(20_000_000)         # a few milliseconds of spinning on stream a
            src.fill_(r)
        ev.record(a)
        ev.wait(b)
        with torch.cuda.stream(b):
            dst = src.clone()
        torch.cuda.synchronize()
        assert bool((dst == r).all()), f"round {r}: the copy did not wait for the fill"
