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
    return read_back(shape, ctx, bufs, h, read_payload=read_payload, direct=direct, allgather=allgather)


def read_back(shape, ctx, bufs, h, read_payload=True, direct=False, allgather=False, send_side=None):
    """numpy copies of every output of one pass: routing, the handle's arrays (through the
    handle's pointers into the workspace), rows, scales, expert outputs, combine rows and y.
    ``send_side`` (default: the base form) says whether the pass kept a send buffer."""
    import torch
    from oracle.oracle import META_DTYPE

    P, T, E, k = shape.P, shape.T, shape.E, shape.k
    if send_side is None:
        send_side = not (direct or allgather)
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
        "send_meta": _ws_view(ws, base, h.send_meta, 16 * Na, META_DTYPE) if send_side else None,
        "recv_meta": _ws_view(ws, base, h.recv_meta, 16 * Na, META_DTYPE),
    }
    if read_payload:
        out.update({
            "send_rows": bufs["send"].cpu().numpy() if send_side else None,
            "recv_rows": bufs["recv"].cpu().numpy(),
            "send_scales": bufs["send_scales"].cpu().numpy() if shape.fp8 and send_side else None,
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


def _finite_positions(got, ref, what):
    """Non-finite values must sit at the same positions on both sides, NaN against NaN
    and each infinity against the same infinity; returns the mask of the finite
    positions, which the caller compares with its tolerance."""
    got_nf, ref_nf = ~np.isfinite(got), ~np.isfinite(ref)
    moved = got_nf != ref_nf
    assert not moved.any(), (f"{what}: {moved.sum()} positions finite on one side only "
                             f"(first at flat index {int(np.flatnonzero(moved)[0])})")
    if ref_nf.any():
        g, r = got[ref_nf], ref[ref_nf]
        same = (np.isnan(g) & np.isnan(r)) | (g == r)
        assert same.all(), f"{what}: {(~same).sum()} non-finite values differ (NaN against inf, or the inf's sign)"
    return ~ref_nf


def assert_weights_close(w_gpu, w_ref):
    # |dw| <= 2^-19 |w| on finite weights (a weight of exactly 0, from a -inf logit,
    # must stay 0); non-finite weights (rows holding NaN) must match in place and kind
    w_gpu = np.asarray(w_gpu, dtype=np.float32)
    w_ref = np.asarray(w_ref, dtype=np.float32)
    fin = _finite_positions(w_gpu, w_ref, "weights")
    err = np.abs(w_gpu[fin].astype(np.float64) - w_ref[fin].astype(np.float64))
    bad = err > W_REL_TOL * np.abs(w_ref[fin].astype(np.float64))
    assert not bad.any(), f"{bad.sum()} weights outside 2^-19 relative, worst abs error {err.max():.3e}"


def assert_y_close(y_gpu_bits, y32_ref, y_ref_bits):
    """y (bf16 bits) against the oracle's unrounded fp32 sum y32: |d| <= 2^-8 |y32| + 1e-6
    where the oracle's bf16 y is finite; where it is not (an infinity or NaN from the
    stub's overflow, or an overflow of the rounding itself), the GPU's y must hold the
    same non-finite value."""
    y = bf16_to_f32(y_gpu_bits)
    fin = _finite_positions(y, bf16_to_f32(y_ref_bits), "y")
    y64 = y[fin].astype(np.float64)
    ref = np.asarray(y32_ref, dtype=np.float32)[fin].astype(np.float64)
    err = np.abs(y64 - ref)
    bad = err > Y_REL_TOL * np.abs(ref) + Y_ABS_TOL
    assert not bad.any(), f"{bad.sum()} outputs outside |d| <= 2^-8|ref| + 1e-6, worst {err.max():.3e}"


def assert_bf16_equal(got_bits, ref_bits, what="y"):
    """Bit for bit, except that any NaN equals any NaN (the sign and payload of a NaN
    are not part of the contract)."""
    got_bits, ref_bits = np.asarray(got_bits, dtype=np.uint16), np.asarray(ref_bits, dtype=np.uint16)
    both_nan = np.isnan(bf16_to_f32(got_bits)) & np.isnan(bf16_to_f32(ref_bits))
    same = both_nan | (got_bits == ref_bits)
    assert same.all(), f"{what}: {(~same).sum()} values differ bit for bit"


def weights_equal(a, b) -> bool:
    return np.array_equal(np.asarray(a, dtype=np.float32), np.asarray(b, dtype=np.float32), equal_nan=True)


def record_weights_match(meta, w, pos):
    """The weight in each row's record is a bit copy of its assignment's routing weight."""
    rec = np.ascontiguousarray(meta["weight"]).view(np.uint32)
    want = np.ascontiguousarray(np.asarray(w, dtype=np.float32).ravel()[np.argsort(np.asarray(pos).ravel())])
    return np.array_equal(rec, want.view(np.uint32))


INT_KEYS = ("N", "expert_off", "rank_recv_off", "C", "n", "send_off", "recv_off", "send_pos", "recv_pos")


def assert_integer_parts_equal(g, o):
    for key in INT_KEYS:
        assert np.array_equal(g[key], o[key]), key
    for key in ("send_meta", "recv_meta"):
        if g[key] is None:            # the direct dispatch keeps no send-side records
            continue
        for f in ("src_rank", "src_token", "slot", "local_expert"):
            assert np.array_equal(g[key][f], o[key][f]), (key, f)


def oracle_path(orc, sh, x, logits=None, ids=None, w=None):
    """The oracle's whole path: routing from the logits, or the given ids and weights."""
    if ids is None:
        ids, w = orc.route(sh, logits)
    return orc.run(sh, x, ids=ids, w=w)


def compare_with_oracle(orc, sh, g, x, logits=None, ids=None, w=None, o=None):
    """Every output in ``g`` (read_back's dict) against the oracle's whole path on the same
    inputs (``o`` if it was computed already): ids and integer parts, rows, scales, expert
    outputs and combine rows bit for bit, weights within 2^-19 relative (bit for bit when
    given), y within |d| <= 2^-8 |y32| + 1e-6 and bit for bit when both sides used the same
    weights.  Returns the oracle's dict."""
    if o is None:
        o = oracle_path(orc, sh, x, logits=logits, ids=ids, w=w)
    o_ids, o_w = o["ids"], o["w"]
    assert np.array_equal(g["ids"], o_ids)
    if ids is None:
        assert_weights_close(g["w"], o_w)
    else:
        assert weights_equal(g["w"], o_w)
    assert_integer_parts_equal(g, o)
    for key in ("send_rows", "recv_rows", "send_scales", "recv_scales", "expert_out", "comb"):
        if o[key] is None or g.get(key) is None:
            continue
        assert np.array_equal(g[key].view(np.uint8), o[key].view(np.uint8)), key
    assert record_weights_match(g["recv_meta"], g["w"], g["recv_pos"])
    if g["send_meta"] is not None:
        assert record_weights_match(g["send_meta"], g["w"], g["send_pos"])
    assert_y_close(g["y"], o["y32"], o["y"])
    if weights_equal(g["w"], o_w):
        assert_bf16_equal(g["y"], o["y"])
    return o
