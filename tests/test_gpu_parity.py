"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Integer and byte outputs (ids, counts, offsets, count
matrix, positions, handle records, send/receive rows, FP8 codes and scales,
expert outputs, combine rows) must match bit for bit; routing weights within
2^-19 relative; combined outputs within |d| <= 2^-8 |ref| + 1e-6 of the
oracle's fp32 sum, and bit for bit when both sides use the same weights."""

import zlib

import numpy as np
import pytest

from combine_router_softmax_expert_amd import workloads as wl
from gpu_helpers import (assert_integer_parts_equal, assert_weights_close, assert_y_close, bf16_to_f32, log,
                         run_gpu)

pytestmark = pytest.mark.gpu


def _full_parity(orc, sh, x, logits=None, ids=None, w=None, label="", direct=False, allgather=False):
    log(f"[parity] {label} P={sh.P} T={sh.T} E={sh.E} k={sh.k} H={sh.H} fp8={sh.fp8} "
        f"{'route' if ids is None else 'given ids'}{' direct' if direct else ''}")
    if ids is None:
        o_ids, o_w = orc.route(sh, logits)
    else:
        o_ids, o_w = ids, w
    g = run_gpu(sh, x, logits=logits, ids=ids, w=w, direct=direct, allgather=allgather)
    assert np.array_equal(g["ids"], o_ids)
    if ids is None:
        assert_weights_close(g["w"], o_w)
    else:
        assert np.array_equal(g["w"], o_w)
    o = orc.run(sh, x, ids=o_ids, w=o_w)
    assert_integer_parts_equal(g, o)
    for key in ("send_rows", "recv_rows", "send_scales", "recv_scales", "expert_out", "comb"):
        if o[key] is None or g[key] is None:
            continue
        assert np.array_equal(g[key].view(np.uint8), o[key].view(np.uint8)), key
    assert np.array_equal(g["recv_meta"]["weight"], g["w"].ravel()[np.argsort(g["recv_pos"].ravel())])
    if g["send_meta"] is not None:
        assert np.array_equal(g["send_meta"]["weight"], g["w"].ravel()[np.argsort(g["send_pos"].ravel())])
    assert_y_close(g["y"], o["y32"])
    if np.array_equal(g["w"], o_w):
        assert np.array_equal(g["y"], o["y"])
    if allgather:
        # every rank's copy holds every token in its dispatched form
        if sh.fp8:
            rows = [orc.quantize_row(sh.H, x[t]) for t in range(sh.T)]
            codes = np.stack([r[0] for r in rows])
            scales = np.stack([r[1] for r in rows])
        else:
            codes = np.ascontiguousarray(x).view(np.uint8).reshape(sh.T, 2 * sh.H)
        for r in range(sh.P):
            assert np.array_equal(g["gathered"][r * sh.T:(r + 1) * sh.T], codes), ("gathered rows", r)
            if sh.fp8:
                assert np.array_equal(g["gathered_scales"][r * sh.T:(r + 1) * sh.T].view(np.uint32),
                                      scales.view(np.uint32)), ("gathered scales", r)
    return g, o


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_workload_parity(orc, name):
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    _full_parity(orc, orc.Shape.of(w), inp["x"], logits=inp["logits"], label=name)


@pytest.mark.parametrize("policy,name", [("streaming", "c1"), ("streaming", "c3"), ("temporal", "c4")])
def test_workload_parity_other_cache_policy(orc, monkeypatch, policy, name):
    # the size-based choice picks one form per kernel; force the other one
    # (streaming: gather-form exchanges and nontemporal accesses) on the same data
    monkeypatch.setenv("MOE_EP_CACHE_POLICY", policy)
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    _full_parity(orc, orc.Shape.of(w), inp["x"], logits=inp["logits"], label=f"{name} {policy}")


@pytest.mark.parametrize("layout,name,direct", [("rows", "c1", False), ("rows", "c2", False), ("rows", "c2", True),
                                                ("tokens", "c4", False), ("tokens", "c4", True)])
def test_workload_parity_other_layout(orc, monkeypatch, layout, name, direct):
    # cache-resident bf16 problems serve each token's rows on the XCD that packed
    # them (token-affine layout), larger ones walk rows; force the other layout
    monkeypatch.setenv("MOE_EP_LAYOUT", layout)
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    _full_parity(orc, orc.Shape.of(w), inp["x"], logits=inp["logits"], label=f"{name} {layout} layout",
                 direct=direct)


@pytest.mark.parametrize("name,direct", [("c1", False), ("c1", True), ("c2", False), ("c2", True), ("c3", False)])
def test_workload_parity_separate_count(orc, monkeypatch, name, direct):
    # small problems rank their assignments inside the pack kernel; force the
    # count (and scan) kernels on the same data
    monkeypatch.setenv("MOE_EP_COUNT_PATH", "separate")
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    _full_parity(orc, orc.Shape.of(w), inp["x"], logits=inp["logits"], label=f"{name} separate count",
                 direct=direct)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_workload_parity_allgather(orc, name):
    # every rank gathers every token and picks its own assignments; same receive side
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    _full_parity(orc, orc.Shape.of(w), inp["x"], logits=inp["logits"], label=f"{name} allgather", allgather=True)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_workload_parity_direct(orc, name):
    # pack straight into the receive rows, reduce straight from the expert output
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    _full_parity(orc, orc.Shape.of(w), inp["x"], logits=inp["logits"], label=name, direct=True)


def test_workload_parity_with_oracle_routing(orc):
    # the oracle's ids and weights fed to the GPU dispatch: everything bit-exact
    w = wl.WORKLOADS["c3"]
    sh = orc.Shape.of(w)
    inp = wl.make_inputs(w)
    ids, wt = orc.route(sh, inp["logits"])
    g, o = _full_parity(orc, sh, inp["x"], ids=ids, w=wt, label="c3 oracle routing")
    assert np.array_equal(g["y"], o["y"])


@pytest.mark.parametrize("mode", ["base", "direct", "allgather"])
def test_skewed_workload_full_size_sampled(orc, mode):
    # c5 at its full size, in the launch configuration the benchmark times: all
    # routing, counts, offsets, positions and handle records in full; payload,
    # stub and combine on sampled tokens that the oracle computes one by one
    w = wl.WORKLOADS["c5"]
    sh = orc.Shape.of(w)
    direct, allgather = mode == "direct", mode == "allgather"
    log(f"[parity] c5 full size {mode}, generating inputs")
    inp = wl.make_inputs(w)
    o_ids, o_w = orc.route(sh, inp["logits"])
    g = run_gpu(sh, inp["x"], logits=inp["logits"], direct=direct, allgather=allgather)
    assert np.array_equal(g["ids"], o_ids)
    assert_weights_close(g["w"], o_w)
    o = orc.dispatch(sh, inp["x"], o_ids, o_w, payload=False)
    assert_integer_parts_equal(g, o)
    n = np.sort(o["N"])[::-1]
    assert 0.40 <= n[: w.num_experts // 10].sum() / n.sum() <= 0.50
    rng = np.random.default_rng(5)
    tokens = np.unique(np.concatenate([[0, sh.T - 1], rng.integers(0, sh.T, 48)]))
    nb = sh.H // 128
    stub_rows = np.empty((len(tokens), sh.k, sh.H), np.uint16)
    for r, t in enumerate(tokens):
        q, sc = orc.quantize_row(sh.H, inp["x"][t])
        for j in range(sh.k):
            p, qq = o["send_pos"][t, j], o["recv_pos"][t, j]
            assert np.array_equal(g["recv_rows"][qq], q) and np.array_equal(g["recv_scales"][qq], sc)
            if mode == "base":
                assert np.array_equal(g["send_rows"][p], q) and np.array_equal(g["send_scales"][p], sc)
            if allgather:               # the token in every rank's copy
                for rr in range(sh.P):
                    assert np.array_equal(g["gathered"][rr * sh.T + t], q)
                    assert np.array_equal(g["gathered_scales"][rr * sh.T + t], sc)
            e = int(o_ids[t, j])
            stub_rows[r, j] = orc.stub_row(sh, e, q, sc)
            assert np.array_equal(g["expert_out"][qq], stub_rows[r, j])
            if not direct:              # the base combine also serves the all-gather dispatch
                assert np.array_equal(g["comb"][t * sh.k + j], stub_rows[r, j])
    red = orc.reduce_tokens(sh, tokens, stub_rows, o_w)
    assert_y_close(g["y"][tokens], red["y32"])
    if np.array_equal(g["w"][tokens], o_w[tokens]):
        assert np.array_equal(g["y"][tokens], red["y"])
    del nb


def test_worked_example_on_gpu(orc):
    from conftest import read_golden
    recs = read_golden("ep_top2_worked_example.txt")
    ids = np.array([[int(v) for v in r[2:]] for r in recs if r[0] == "route"], np.int32)
    T, k = ids.shape
    sh = orc.Shape(4, T, 8, k, 8, False)
    x = np.repeat(wl.float32_to_bf16_bits(np.arange(1, T + 1, dtype=np.float32))[:, None], 8, axis=1)
    g, _ = _full_parity(orc, sh, x, ids=ids, w=np.full((T, k), 0.5, np.float32), label="worked example")
    for r in recs:
        if r[0] == "recv":
            e, toks = int(r[2]), [int(v) for v in r[3:]]
            seg = g["recv_meta"][g["expert_off"][e]:g["expert_off"][e + 1]]
            assert [int(m["src_rank"]) * 2 + int(m["src_token"]) for m in seg] == toks


# --------------------------------------------------------------------------
# edge cases of the page's correctness list: all local, all to one remote
# rank, extreme skew, empty experts, token counts that are not a multiple of
# any tile, top-1 / top-2 / top-8, plus sizes and formats
# --------------------------------------------------------------------------

EDGE = [
    # name, P, Tp, E, k, H, fp8
    ("all-local-P1", 1, 33, 8, 2, 256, False),
    ("ragged-Tp1", 4, 1, 8, 2, 136, False),
    ("ragged-Tp7-top1", 3, 7, 6, 1, 64, False),
    ("ragged-Tp257-top8", 8, 257, 64, 8, 384, True),
    ("tiny-H8", 2, 5, 4, 4, 8, False),
    ("k-equals-E", 2, 9, 4, 4, 128, True),
    ("count-chunks-Tp3000", 2, 3000, 256, 8, 64, False),
    ("E1024-top32", 4, 40, 1024, 32, 128, True),
    ("E1024-top32-wide-rows", 4, 4, 1024, 32, 7168, False),
    ("two-tokens-per-block", 6, 342, 12, 3, 4096, False),
    ("four-tokens-per-block-fp8", 4, 1024, 8, 2, 8192, True),
    ("E-odd-96", 3, 50, 96, 5, 520, False),
    ("six-slices-ragged-row", 2, 6, 8, 2, 10248, False),   # 1281 units: 6 workgroups of 256, the last partial
    ("three-slices-fp8", 2, 5, 8, 2, 24576, True),         # 1536 code units (3 x 512), 3072 output units (6 x 512)
]


@pytest.mark.parametrize("policy,count,direct,layout", [("auto", "auto", False, "auto"),
                                                        ("streaming", "auto", False, "auto"),
                                                        ("streaming", "auto", True, "auto"),
                                                        ("auto", "auto", True, "auto"),
                                                        ("auto", "separate", False, "auto"),
                                                        ("auto", "fused", True, "auto"),
                                                        ("auto", "auto", "allgather", "auto"),
                                                        ("streaming", "separate", "allgather", "auto"),
                                                        ("auto", "auto", False, "rows"),
                                                        ("auto", "separate", True, "rows"),
                                                        ("auto", "auto", False, "tokens"),
                                                        ("auto", "separate", True, "tokens")])
@pytest.mark.parametrize("name,P,Tp,E,k,H,fp8", EDGE, ids=[e[0] for e in EDGE])
def test_edge_shapes(orc, monkeypatch, name, P, Tp, E, k, H, fp8, policy, count, direct, layout):
    monkeypatch.setenv("MOE_EP_CACHE_POLICY", policy)
    monkeypatch.setenv("MOE_EP_COUNT_PATH", count)
    monkeypatch.setenv("MOE_EP_LAYOUT", layout)
    allgather = direct == "allgather"
    direct = direct is True
    sh = orc.Shape(P, P * Tp, E, k, H, fp8)
    seed = zlib.crc32(name.encode())
    x = wl.make_hidden(seed, sh.T, H)
    logits = wl.make_logits(seed, sh.T, E)
    _full_parity(orc, sh, x, logits=logits, label=name, direct=direct, allgather=allgather)


def test_all_tokens_to_one_remote_rank_and_empty_experts(orc):
    P, Tp, E, k, H = 4, 20, 16, 2, 256
    sh = orc.Shape(P, P * Tp, E, k, H, False)
    T = sh.T
    ids = np.stack([np.full(T, E - 1), np.full(T, E - 2)], axis=1).astype(np.int32)  # all to rank P-1
    w = np.tile(np.float32([0.75, 0.25]), (T, 1))
    g, _ = _full_parity(orc, sh, wl.make_hidden(3, T, H), ids=ids, w=w, label="one remote rank")
    assert np.count_nonzero(g["N"]) == 2 and g["C"][:, P - 1].sum() == T * k


@pytest.mark.parametrize("E,k", [(32, 4), (96, 8), (256, 8)])
def test_extreme_skew_and_ties_in_logits(orc, E, k):
    # both router shapes (lane groups for E <= 32, whole waves above)
    P, Tp, H = 4, 64, 128
    sh = orc.Shape(P, P * Tp, E, k, H, True)
    rng = np.random.default_rng(9)
    logits = rng.integers(-2, 3, size=(sh.T, E)).astype(np.float32)   # many exact ties
    logits[:, :3] += 8.0                                              # three hot experts
    logits[::7] = 0.0                                                 # whole rows of ties
    logits[1, 5] = -0.0                                               # -0 ties with +0
    logits[2, 1:] = -np.inf                                           # masked experts
    logits[3, ::2] = -np.inf
    _full_parity(orc, sh, wl.make_hidden(4, sh.T, H), logits=logits, label=f"skew+ties E={E}")


def test_fp8_special_blocks(orc):
    # zero blocks (scale 0, signed zeros), blocks whose amax is 448 (scale exactly
    # 1, so every e4m3 tie is decided by the rounding rule), tiny and huge values
    P, Tp, E, k, H = 2, 8, 4, 2, 512
    sh = orc.Shape(P, P * Tp, E, k, H, True)
    T = sh.T
    x = wl.make_hidden(5, T, H)
    x[0, :128] = 0
    x[0, 5] = 0x8000
    codes = np.arange(0x00, 0x7F, dtype=np.uint8)
    import torch
    vals = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    row = np.concatenate([mids, -mids[:1], [448.0]]).astype(np.float32)[:128]
    x[1, 128:256] = wl.float32_to_bf16_bits(row)
    x[1, 255] = wl.float32_to_bf16_bits(np.float32([448.0]))[0]
    x[2, 256:384] = wl.float32_to_bf16_bits(np.full(128, 1e-30, np.float32))
    x[3, 384:512] = wl.float32_to_bf16_bits(np.linspace(-3e38, 3e38, 128).astype(np.float32))
    # both sides of amax = 2^-64, where the kernel switches between the reciprocal
    # and the divided quotient, and bf16 subnormals under a large amax
    g = np.random.default_rng(7).standard_normal(128).astype(np.float32)
    x[4, 0:128] = wl.float32_to_bf16_bits(g / np.abs(g).max() * np.float32(2.0 ** -64))
    x[5, 128:256] = wl.float32_to_bf16_bits(g / np.abs(g).max() * np.float32(2.0 ** -64 * (1 - 2 ** -7)))
    x[6, 256:384] = (np.arange(128, dtype=np.uint16) % 0x80) | np.where(np.arange(128) % 2, 0x8000, 0).astype(np.uint16)
    x[6, 300] = wl.float32_to_bf16_bits(np.float32([1e30]))[0]
    x[7, 384:512] = (np.arange(128, dtype=np.uint16) % 0x80)
    logits = wl.make_logits(6, T, E)
    _full_parity(orc, sh, x, logits=logits, label="fp8 special blocks")


def test_deterministic_and_sentinel_free(orc):
    w = wl.WORKLOADS["c1"]
    sh = orc.Shape.of(w)
    inp = wl.make_inputs(w)
    a = run_gpu(sh, inp["x"], logits=inp["logits"], sentinel=True)
    b = run_gpu(sh, inp["x"], logits=inp["logits"], sentinel=False, repeat=2)
    for key in ("ids", "w", "send_rows", "recv_rows", "expert_out", "comb", "y", "send_pos", "recv_pos"):
        assert np.array_equal(a[key], b[key]), key


def test_combine_identity_top1_expert0(orc):
    P, Tp, E, H = 4, 33, 8, 136
    sh = orc.Shape(P, P * Tp, E, 1, H, False)
    x = wl.make_hidden(8, sh.T, H)
    g = run_gpu(sh, x, ids=np.zeros((sh.T, 1), np.int32), w=np.ones((sh.T, 1), np.float32))
    assert np.array_equal(g["y"], x)


def test_misaligned_buffers_are_refused_after_a_dispatch(orc):
    """With a live handle the stub and combine calls refuse byte-offset buffers
    before launching anything; the path then completes with the oracle's y."""
    import ctypes
    import torch
    from combine_router_softmax_expert_amd import binding as B

    w = wl.WORKLOADS["c1"]
    inp = wl.make_inputs(w)
    sh = orc.Shape.of(w)
    ids, wt = orc.route(sh, inp["logits"])
    log("[align] c1 base, given ids")
    ctx = B.Context.for_workload(w)
    bufs = ctx.allocate()
    bufs["topk_ids"].copy_(torch.from_numpy(ids))
    bufs["topk_w"].copy_(torch.from_numpy(wt))
    x = torch.from_numpy(inp["x"].view(np.int16)).cuda()
    h = B.moe_dispatch(ctx, x, bufs["topk_ids"], bufs["topk_w"], bufs["workspace"], bufs["send"], None,
                       bufs["recv"], None)

    def at(key, off=0):
        return ctypes.c_void_p(bufs[key].data_ptr() + off)

    c, hp = ctx.handle_ptr, ctypes.byref(h)
    assert B.lib.moe_expert_stub(c, hp, at("recv", 8), None, at("expert_out"), None) == -1
    assert b"16-byte" in B.lib.moe_last_error()
    assert B.lib.moe_combine(c, hp, at("expert_out"), at("topk_w", 2), at("comb"), at("y"), None) == -1
    assert b"4-byte" in B.lib.moe_last_error()
    assert B.lib.moe_combine_send(c, hp, at("expert_out"), at("comb", 8), None) == -1
    assert B.lib.moe_combine_direct(c, hp, at("expert_out", 8), at("topk_w"), at("y"), None) == -1
    B.moe_expert_stub(ctx, h, bufs["recv"], None, bufs["expert_out"])
    B.moe_combine(ctx, h, bufs["expert_out"], bufs["topk_w"], bufs["comb"], bufs["y"])
    torch.cuda.synchronize()
    o = orc.run(sh, inp["x"], ids=ids, w=wt)
    assert np.array_equal(bufs["y"].view(torch.int16).cpu().numpy().view(np.uint16), o["y"].view(np.uint16))


def test_zero_tokens(orc):
    from combine_router_softmax_expert_amd import binding as B
    import torch
    ctx = B.Context(4, 0, 8, 2, 256, False)
    bufs = ctx.allocate()
    h = B.moe_dispatch(ctx, torch.empty((0, 256), dtype=torch.bfloat16, device="cuda"), bufs["topk_ids"],
                       bufs["topk_w"], bufs["workspace"], bufs["send"], None, bufs["recv"], None)
    B.moe_expert_stub(ctx, h, bufs["recv"], None, bufs["expert_out"])
    B.moe_combine(ctx, h, bufs["expert_out"], bufs["topk_w"], bufs["comb"], bufs["y"])
    torch.cuda.synchronize()


def _random_shapes(n, seed):
    """Seeded random shapes over the ranges of the test plan: P in {1, 2, 3, 4, 8, 32}, E a multiple of P,
    k <= min(E, 8), H in {8, 128, 136, 7168} (FP8: {128, 7168}), T/P in 1..300, capped so the oracle
    stays within a second."""
    rng = np.random.default_rng(seed)
    shapes = []
    for i in range(n):
        P = int(rng.choice([1, 2, 3, 4, 8, 32]))
        E = P * int(rng.integers(1, 9))
        k = int(rng.integers(1, min(E, 8) + 1))
        fp8 = bool(rng.integers(0, 2))
        H = int(rng.choice([128, 7168] if fp8 else [8, 128, 136, 7168]))
        Tp = min(int(rng.integers(1, 301)), max(1, (1 << 20) // (P * H)))
        mode = ("base", "direct", "allgather")[i % 3]
        shapes.append((f"rand{i}-P{P}-Tp{Tp}-E{E}-k{k}-H{H}-{'fp8' if fp8 else 'bf16'}-{mode}", P, Tp, E, k, H, fp8,
                       mode))
    return shapes


RANDOM_SHAPES = _random_shapes(18, 20261202)


@pytest.mark.parametrize("name,P,Tp,E,k,H,fp8,mode", RANDOM_SHAPES, ids=[s[0] for s in RANDOM_SHAPES])
def test_random_shapes(orc, name, P, Tp, E, k, H, fp8, mode):
    sh = orc.Shape(P, P * Tp, E, k, H, fp8)
    seed = zlib.crc32(name.encode())
    x = wl.make_hidden(seed, sh.T, H)
    logits = wl.make_logits(seed, sh.T, E)
    _full_parity(orc, sh, x, logits=logits, label=name, direct=mode == "direct", allgather=mode == "allgather")


GUARD = 4096   # bytes of 0xA5 on each side of every buffer (keeps the 256-byte workspace alignment)


def _guarded(t):
    """A buffer of t's shape and dtype in the middle of a larger one whose edges hold a known pattern."""
    import torch
    if t is None:
        return None, None
    n = t.numel() * t.element_size()
    big = torch.full((n + 2 * GUARD,), 0xA5, dtype=torch.uint8, device=t.device)
    return big[GUARD:GUARD + n].view(t.dtype).view(t.shape), big


@pytest.mark.parametrize("name,P,Tp,E,k,H,fp8", [("guard-bf16", 4, 33, 8, 2, 136, False),
                                                 ("guard-fp8-ragged", 3, 7, 6, 3, 384, True),
                                                 ("guard-counting-pack", 8, 16, 64, 8, 1024, False)])
@pytest.mark.parametrize("mode", ["base", "direct", "allgather"])
@pytest.mark.parametrize("count", ["auto", "separate"])
def test_no_writes_outside_buffers(orc, monkeypatch, name, P, Tp, E, k, H, fp8, mode, count):
    """Every output buffer sits between guard bands; after the whole path the bands are intact and y matches
    the oracle, so no kernel writes past either end of a caller's buffer."""
    import torch
    from combine_router_softmax_expert_amd import binding as B

    monkeypatch.setenv("MOE_EP_COUNT_PATH", count)
    log(f"[guard] {name} {mode} count={count}")
    ctx = B.Context(P, Tp, E, k, H, fp8)
    bufs, bigs = {}, {}
    plain = ctx.allocate()
    if mode == "allgather":
        plain["gathered"], plain["gathered_scales"] = ctx.allocate_gathered()
    for key, t in plain.items():
        bufs[key], bigs[key] = _guarded(t)
    sh = orc.Shape(P, P * Tp, E, k, H, fp8)
    seed = zlib.crc32(name.encode())
    x_np = wl.make_hidden(seed, sh.T, H)
    logits_np = wl.make_logits(seed, sh.T, E)
    x = torch.from_numpy(x_np.view(np.int16)).cuda()
    logits = torch.from_numpy(logits_np).cuda()
    B.moe_route_topk(ctx, logits, bufs["topk_ids"], bufs["topk_w"])
    if mode == "allgather":
        h = B.moe_dispatch_allgather(ctx, x, bufs["topk_ids"], bufs["topk_w"], bufs["workspace"], bufs["gathered"],
                                     bufs["gathered_scales"], bufs["recv"], bufs["recv_scales"])
    elif mode == "direct":
        h = B.moe_dispatch_direct(ctx, x, bufs["topk_ids"], bufs["topk_w"], bufs["workspace"], bufs["recv"],
                                  bufs["recv_scales"])
    else:
        h = B.moe_dispatch(ctx, x, bufs["topk_ids"], bufs["topk_w"], bufs["workspace"], bufs["send"],
                           bufs["send_scales"], bufs["recv"], bufs["recv_scales"])
    B.moe_expert_stub(ctx, h, bufs["recv"], bufs["recv_scales"], bufs["expert_out"])
    if mode == "direct":
        B.moe_combine_direct(ctx, h, bufs["expert_out"], bufs["topk_w"], bufs["y"])
    else:
        B.moe_combine(ctx, h, bufs["expert_out"], bufs["topk_w"], bufs["comb"], bufs["y"])
    torch.cuda.synchronize()
    for key, big in bigs.items():
        if big is None:
            continue
        edges = torch.cat([big[:GUARD], big[-GUARD:]]).cpu().numpy()
        assert (edges == 0xA5).all(), (name, mode, key)
    o_ids, o_w = orc.route(sh, logits_np)
    assert np.array_equal(bufs["topk_ids"].cpu().numpy(), o_ids)
    o = orc.run(sh, x_np, ids=o_ids, w=bufs["topk_w"].cpu().numpy())
    assert np.array_equal(bufs["y"].view(torch.int16).cpu().numpy().view(np.uint16), o["y"].view(np.uint16))


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_direct_dispatch_with_either_combine(orc, name):
    """After a direct dispatch (token-affine layout at these sizes) both combines, the base one through the
    combine buffer and the direct one through recv_pos, give y bit for bit equal to the oracle's."""
    import torch
    from combine_router_softmax_expert_amd import binding as B

    log(f"[direct+either combine] {name}")
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    sh = orc.Shape.of(w)
    ctx = B.Context.for_workload(w)
    bufs = ctx.allocate()
    x = torch.from_numpy(inp["x"].view(np.int16)).cuda()
    logits = torch.from_numpy(inp["logits"]).cuda()
    B.moe_route_topk(ctx, logits, bufs["topk_ids"], bufs["topk_w"])
    h = B.moe_dispatch_direct(ctx, x, bufs["topk_ids"], bufs["topk_w"], bufs["workspace"], bufs["recv"],
                              bufs["recv_scales"])
    B.moe_expert_stub(ctx, h, bufs["recv"], bufs["recv_scales"], bufs["expert_out"])
    B.moe_combine(ctx, h, bufs["expert_out"], bufs["topk_w"], bufs["comb"], bufs["y"])
    torch.cuda.synchronize()
    y_base = bufs["y"].view(torch.int16).cpu().numpy().copy()
    comb = bufs["comb"].view(torch.int16).cpu().numpy().copy()
    bufs["y"].view(torch.uint8).fill_(0xFF)
    B.moe_combine_direct(ctx, h, bufs["expert_out"], bufs["topk_w"], bufs["y"])
    torch.cuda.synchronize()
    y_direct = bufs["y"].view(torch.int16).cpu().numpy()
    ids, wt = bufs["topk_ids"].cpu().numpy(), bufs["topk_w"].cpu().numpy()
    o = orc.run(sh, inp["x"], ids=ids, w=wt)
    assert np.array_equal(comb.view(np.uint16), o["comb"].view(np.uint16).reshape(comb.shape))
    assert np.array_equal(y_base.view(np.uint16), o["y"].view(np.uint16))
    assert np.array_equal(y_direct.view(np.uint16), o["y"].view(np.uint16))
