"""Shared pieces of the GPU parity tests: run the HIP path through the C ABI and
read every output back, and compare it with the oracle."""

from __future__ import annotations

import sys

import numpy as np

W_REL_TOL = 2.0 ** -19          # routing weights: two exp implementations + roundings
Y_REL_TOL = 2.0 ** -8           # combined bf16 output vs the oracle's fp32 sum
Y_ABS_TOL = 1e-6


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def _ws_view(ws, base_ptr, ptr, nbytes, dtype):
    off = ptr - base_ptr
    assert 0 <= off and off + nbytes <= ws.numel()
    return ws[off:off + nbytes].cpu().numpy().view(dtype)


def run_gpu(shape, x, logits=None, ids=None, w=None, sentinel=True, repeat=1, read_payload=True, direct=False,
            allgather=False):
    """Run route (unless ids/w are given), dispatch, stub and combine on cuda:0
    (the direct forms, or the all-gather dispatch with the base combine, if
    asked); returns numpy copies of every output."""
    import torch
    from combine_router_softmax_expert_amd import binding as B
    from oracle.oracle import META_DTYPE

    P, T, E, k, H = shape.P, shape.T, shape.E, shape.k, shape.H
    ctx = B.Context(P, T // P, E, k, H, shape.fp8)
    bufs = ctx.allocate()
    if allgather:
        bufs["gathered"], bufs["gathered_scales"] = ctx.allocate_gathered()
    if sentinel:
        for key, t in bufs.items():
            if t is not None and key not in ("workspace",):
                t.view(torch.uint8).fill_(0xFF)
        bufs["workspace"].fill_(0xFF)
    xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    if ids is None:
        ld = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).cuda()
    else:
        bufs["topk_ids"].copy_(torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)))
        bufs["topk_w"].copy_(torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)))
    h = None
    for _ in range(repeat):
        if ids is None:
            B.moe_route_topk(ctx, ld, bufs["topk_ids"], bufs["topk_w"])
        if allgather:
            h = B.moe_dispatch_allgather(ctx, xd, bufs["topk_ids"], bufs["topk_w"], bufs["workspace"],
                                         bufs["gathered"], bufs["gathered_scales"], bufs["recv"], bufs["recv_scales"])
        elif direct:
            h = B.moe_dispatch_direct(ctx, xd, bufs["topk_ids"], bufs["topk_w"], bufs["workspace"], bufs["recv"],
                                      bufs["recv_scales"])
        else:
            h = B.moe_dispatch(ctx, xd, bufs["topk_ids"], bufs["topk_w"], bufs["workspace"], bufs["send"],
                               bufs["send_scales"], bufs["recv"], bufs["recv_scales"])
        B.moe_expert_stub(ctx, h, bufs["recv"], bufs["recv_scales"], bufs["expert_out"])
        if direct:
            B.moe_combine_direct(ctx, h, bufs["expert_out"], bufs["topk_w"], bufs["y"])
        else:
            B.moe_combine(ctx, h, bufs["expert_out"], bufs["topk_w"], bufs["comb"], bufs["y"])
    torch.cuda.synchronize()

    ws = bufs["workspace"]
    base = ws.data_ptr()
    Na = T * k
    out = {
        "ids": bufs["topk_ids"].cpu().numpy(), "w": bufs["topk_w"].cpu().numpy(),
        "N": _ws_view(ws, base, h.expert_counts, 4 * E, np.int32),
        "expert_off": _ws_view(ws, base, h.expert_offsets, 4 * (E + 1), np.int32),
        "rank_recv_off": _ws_view(ws, base, h.rank_recv_offsets, 4 * (P + 1), np.int32),
        "C": _ws_view(ws, base, h.count_matrix, 4 * P * P, np.int32).reshape(P, P),
        "n": _ws_view(ws, base, h.rank_expert_counts, 4 * P * E, np.int32).reshape(P, E),
        "send_off": _ws_view(ws, base, h.send_offsets, 4 * P * E, np.int32).reshape(P, E),
        "recv_off": _ws_view(ws, base, h.recv_offsets, 4 * E * P, np.int32).reshape(P, E).T,
        "send_pos": _ws_view(ws, base, h.send_pos, 4 * Na, np.int32).reshape(T, k),
        "recv_pos": _ws_view(ws, base, h.recv_pos, 4 * Na, np.int32).reshape(T, k),
        "send_meta": None if (direct or allgather) else _ws_view(ws, base, h.send_meta, 16 * Na, META_DTYPE),
        "recv_meta": _ws_view(ws, base, h.recv_meta, 16 * Na, META_DTYPE),
    }
    if read_payload:
        out.update({
            "send_rows": None if (direct or allgather) else bufs["send"].cpu().numpy(),
            "recv_rows": bufs["recv"].cpu().numpy(),
            "send_scales": bufs["send_scales"].cpu().numpy() if shape.fp8 and not (direct or allgather) else None,
            "recv_scales": bufs["recv_scales"].cpu().numpy() if shape.fp8 else None,
            "expert_out": bufs["expert_out"].view(torch.int16).cpu().numpy().view(np.uint16),
            "comb": None if direct else bufs["comb"].view(torch.int16).cpu().numpy().view(np.uint16),
            "y": bufs["y"].view(torch.int16).cpu().numpy().view(np.uint16),
        })
        if allgather:
            out["gathered"] = bufs["gathered"].cpu().numpy()
            out["gathered_scales"] = bufs["gathered_scales"].cpu().numpy() if shape.fp8 else None
    else:
        out["_bufs"] = bufs
    out["_ctx"] = ctx
    return out


def bf16_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def assert_weights_close(w_gpu, w_ref):
    # |dw| <= 2^-19 |w| (a weight of exactly 0, from a -inf logit, must stay 0)
    err = np.abs(w_gpu.astype(np.float64) - w_ref)
    bad = err > W_REL_TOL * np.abs(w_ref)
    assert not bad.any(), f"{bad.sum()} weights outside 2^-19 relative, worst abs error {err.max():.3e}"


def assert_y_close(y_gpu_bits, y32_ref):
    y = bf16_to_f32(y_gpu_bits).astype(np.float64)
    ref = y32_ref.astype(np.float64)
    err = np.abs(y - ref)
    bad = err > Y_REL_TOL * np.abs(ref) + Y_ABS_TOL
    assert not bad.any(), f"{bad.sum()} outputs outside |d| <= 2^-8|ref| + 1e-6, worst {err.max():.3e}"


INT_KEYS = ("N", "expert_off", "rank_recv_off", "C", "n", "send_off", "recv_off", "send_pos", "recv_pos")


def assert_integer_parts_equal(g, o):
    for key in INT_KEYS:
        assert np.array_equal(g[key], o[key]), key
    for key in ("send_meta", "recv_meta"):
        if g[key] is None:            # the direct dispatch keeps no send-side records
            continue
        for f in ("src_rank", "src_token", "slot", "local_expert"):
            assert np.array_equal(g[key][f], o[key][f]), (key, f)
