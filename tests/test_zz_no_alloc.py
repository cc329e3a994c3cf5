"""moe_dispatch_noalloc: moe_dispatch with the library's static workspace instead of a
caller buffer, for callers that cannot allocate.  Through the C ABI, two calls in a
row (the skewed 32-rank FP8 workload, then a smaller bf16 one on another ctx) must
give, bit for bit, what moe_dispatch with a caller workspace gives on the same
inputs: send and receive rows and scales, every array of the handle, and, through
the stub and the combine that read the handle, the expert outputs, combine rows
and y.  A handle whose static arrays a later call has reused is refused (the
host-side argument and size checks run on the CPU, in test_abi.py)."""

import ctypes

import numpy as np
import pytest

from combine_router_softmax_expert_amd import workloads as wl
from gpu_helpers import log

pytestmark = pytest.mark.gpu

HANDLE_ARRAYS = (   # field, int32 elements (or 16-byte records) as a function of (P, T, E, k)
    ("expert_counts", lambda P, T, E, k: 4 * E), ("expert_offsets", lambda P, T, E, k: 4 * (E + 1)),
    ("rank_recv_offsets", lambda P, T, E, k: 4 * (P + 1)), ("count_matrix", lambda P, T, E, k: 4 * P * P),
    ("rank_expert_counts", lambda P, T, E, k: 4 * P * E), ("send_offsets", lambda P, T, E, k: 4 * P * E),
    ("recv_offsets", lambda P, T, E, k: 4 * P * E), ("send_pos", lambda P, T, E, k: 4 * T * k),
    ("recv_pos", lambda P, T, E, k: 4 * T * k), ("send_meta", lambda P, T, E, k: 16 * T * k),
    ("recv_meta", lambda P, T, E, k: 16 * T * k),
)


def _device_bytes(ptr, nbytes):
    """Copy nbytes at a device address to the host (the HIP runtime torch and the library share)."""
    hip = ctypes.CDLL("libamdhip64.so.7")
    out = np.empty(nbytes, np.uint8)
    rc = hip.hipMemcpy(ctypes.c_void_p(out.ctypes.data), ctypes.c_void_p(ptr), ctypes.c_size_t(nbytes),
                       ctypes.c_int(2))   # hipMemcpyDeviceToHost
    assert rc == 0, rc
    return out


def _run(w, noalloc):
    import torch
    from combine_router_softmax_expert_amd import binding as B

    inp = wl.make_inputs(w)
    ctx = B.Context.for_workload(w)
    bufs = ctx.allocate()
    for key, t in bufs.items():
        if t is not None:
            t.view(torch.uint8).fill_(0xFF)
    x = torch.from_numpy(inp["x"].view(np.int16)).cuda()
    logits = torch.from_numpy(inp["logits"]).cuda()
    B.moe_route_topk(ctx, logits, bufs["topk_ids"], bufs["topk_w"])
    if noalloc:
        h = B.moe_dispatch_noalloc(ctx, x, bufs["topk_ids"], bufs["topk_w"], bufs["send"], bufs["send_scales"],
                                   bufs["recv"], bufs["recv_scales"])
    else:
        h = B.moe_dispatch(ctx, x, bufs["topk_ids"], bufs["topk_w"], bufs["workspace"], bufs["send"],
                           bufs["send_scales"], bufs["recv"], bufs["recv_scales"])
    B.moe_expert_stub(ctx, h, bufs["recv"], bufs["recv_scales"], bufs["expert_out"])
    B.moe_combine(ctx, h, bufs["expert_out"], bufs["topk_w"], bufs["comb"], bufs["y"])
    torch.cuda.synchronize()
    P, T, E, k = w.num_ranks, w.tokens, w.num_experts, w.top_k
    out = {name: _device_bytes(getattr(h, name), size(P, T, E, k)) for name, size in HANDLE_ARRAYS}
    for key in ("topk_ids", "topk_w", "send", "recv", "send_scales", "recv_scales", "expert_out", "comb", "y"):
        if bufs[key] is not None:
            out[key] = bufs[key].view(torch.uint8).cpu().numpy()
    ws = bufs["workspace"]
    in_caller_ws = ws.data_ptr() <= h.recv_pos < ws.data_ptr() + ws.numel()
    return out, ctx, bufs, h, in_caller_ws


def _check_same(w):
    log(f"[noalloc] {w.describe()}")
    got, ctx, bufs, h, in_ws = _run(w, noalloc=True)
    want, *_ = _run(w, noalloc=False)
    assert not in_ws        # the handle points into the library's static workspace
    assert got.keys() == want.keys()
    for key in want:
        assert np.array_equal(got[key], want[key]), key
    return ctx, bufs, h


def test_noalloc_dispatch_matches_the_workspace_dispatch_twice():
    from combine_router_softmax_expert_amd import binding as B

    big = wl.WORKLOADS["c5"]                 # 65536 assignments: about 3.4 MB of the 8 MiB
    small = wl.WORKLOADS["c1"]               # then a smaller problem on another ctx
    ctx_big, bufs_big, h_big = _check_same(big)
    _check_same(small)
    # the second call reused the static workspace the first handle points into
    with pytest.raises(B.MoeError) as err:
        B.moe_combine(ctx_big, h_big, bufs_big["expert_out"], bufs_big["topk_w"], bufs_big["comb"], bufs_big["y"])
    assert err.value.status == B.MOE_ERR_STALE_HANDLE
