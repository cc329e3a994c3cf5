"""binding.PreparedPath (the arguments checked and marshalled once, the calls
replayed) must produce, bit for bit, what the individual calls of run_path
produce on the same inputs: the whole path and dispatch+combine alone, in both
forms, over several calls with new inputs copied into the same tensors."""

import numpy as np
import pytest

from combine_router_softmax_expert_amd import workloads as wl
from gpu_helpers import log

pytestmark = pytest.mark.gpu


def _snapshot(bufs, direct):
    import torch
    keys = ["topk_ids", "topk_w", "recv", "expert_out", "y"] + ([] if direct else ["send", "comb"])
    if bufs["recv_scales"] is not None:
        keys.append("recv_scales")
    return {key: bufs[key].view(torch.uint8).clone() for key in keys}   # raw bytes: bit-exact comparison


@pytest.mark.parametrize("name,direct", [("c1", False), ("c1", True), ("c2", False), ("c2", True), ("c3", False),
                                         ("c3", True)])
def test_prepared_path_matches_run_path(name, direct):
    import torch
    from combine_router_softmax_expert_amd import binding as B

    log(f"[prepared] {name} direct={direct}")
    w = wl.WORKLOADS[name]
    ctx = B.Context.for_workload(w)
    ref, bufs = ctx.allocate(), ctx.allocate()
    inputs = [wl.make_inputs(w)] + [{"x": wl.make_hidden(s, w.tokens, w.hidden),
                                     "logits": wl.make_logits(s, w.tokens, w.num_experts)} for s in (21, 22)]
    x = torch.from_numpy(inputs[0]["x"].view(np.int16)).cuda()
    logits = torch.from_numpy(inputs[0]["logits"]).cuda()
    path = B.PreparedPath(ctx, bufs, x, logits, direct=direct)
    dc = B.PreparedPath(ctx, bufs, x, None, direct=direct, stages="dispatch_combine")
    for i, inp in enumerate(inputs):
        x.copy_(torch.from_numpy(inp["x"].view(np.int16)))
        logits.copy_(torch.from_numpy(inp["logits"]))
        B.run_path(ctx, ref, x, logits, direct=direct)
        torch.cuda.synchronize()
        want = _snapshot(ref, direct)
        for t in bufs.values():          # poison the outputs: the prepared calls must rewrite them
            if t is not None and t is not bufs["workspace"]:
                t.view(torch.uint8).fill_(0xA5)
        h = path()
        torch.cuda.synchronize()
        got = _snapshot(bufs, direct)
        for key in want:
            assert torch.equal(got[key], want[key]), (name, direct, i, "path", key)
        assert h.generation > 0
        # dispatch+combine alone, on the ids, weights and expert outputs now in bufs
        bufs["y"].view(torch.uint8).fill_(0xA5)
        dc()
        torch.cuda.synchronize()
        assert torch.equal(bufs["y"].view(torch.uint8), want["y"]), (name, direct, i, "dispatch_combine")
    torch.cuda.synchronize()
    ctx.close()                          # the cached ctx pointer is gone: no call may reach the library
    with pytest.raises(ValueError, match="closed"):
        path()


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_prepared_allgather_matches_individual_calls(name):
    import torch
    from combine_router_softmax_expert_amd import binding as B

    log(f"[prepared allgather] {name}")
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    ctx = B.Context.for_workload(w)
    ref, bufs = ctx.allocate(), ctx.allocate()
    x = torch.from_numpy(inp["x"].view(np.int16)).cuda()
    logits = torch.from_numpy(inp["logits"]).cuda()
    g_ref, gs_ref = ctx.allocate_gathered()
    g, gs = ctx.allocate_gathered()
    B.run_path(ctx, ref, x, logits)                  # ids, weights, expert outputs
    h = B.moe_dispatch_allgather(ctx, x, ref["topk_ids"], ref["topk_w"], ref["workspace"], g_ref, gs_ref,
                                 ref["recv"], ref["recv_scales"])
    B.moe_combine(ctx, h, ref["expert_out"], ref["topk_w"], ref["comb"], ref["y"])
    torch.cuda.synchronize()
    for key in ("topk_ids", "topk_w", "expert_out"):
        bufs[key].copy_(ref[key])
    for key in ("recv", "comb", "y"):
        bufs[key].view(torch.uint8).fill_(0xA5)
    ag = B.PreparedPath(ctx, bufs, x, None, stages="dispatch_combine", gathered=g, gathered_scales=gs)
    ag()
    ag()
    torch.cuda.synchronize()
    for key in ("recv", "comb", "y"):
        assert torch.equal(bufs[key].view(torch.uint8), ref[key].view(torch.uint8)), (name, key)
    assert torch.equal(g.view(torch.uint8), g_ref.view(torch.uint8)), name
    with pytest.raises(ValueError):
        B.PreparedPath(ctx, bufs, x, None, direct=True, stages="dispatch_combine", gathered=g, gathered_scales=gs)


def test_prepared_path_rejects_bad_tensors():
    import torch
    from combine_router_softmax_expert_amd import binding as B

    w = wl.WORKLOADS["c1"]
    ctx = B.Context.for_workload(w)
    bufs = ctx.allocate()
    x = torch.empty(w.tokens, w.hidden, dtype=torch.int16, device="cuda")
    with pytest.raises(ValueError):      # logits missing for the whole path
        B.PreparedPath(ctx, bufs, x, None)
    with pytest.raises(ValueError):      # wrong dtype, as the individual calls check it
        B.PreparedPath(ctx, bufs, x.float(), torch.empty(w.tokens, w.num_experts, device="cuda"))
    with pytest.raises(ValueError):
        B.PreparedPath(ctx, bufs, x, None, stages="route")
