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
from gpu_helpers import (INT_KEYS, assert_bf16_equal, assert_integer_parts_equal, assert_weights_close, assert_y_close,
                         bf16_to_f32, compare_with_oracle, log, record_weights_match, run_gpu, weights_equal)

pytestmark = pytest.mark.gpu


def _full_parity(orc, sh, x, logits=None, ids=None, w=None, label="", direct=False, allgather=False):
    log(f"[parity] {label} P={sh.P} T={sh.T} E={sh.E} k={sh.k} H={sh.H} fp8={sh.fp8} "
        f"{'route' if ids is None else 'given ids'}{' direct' if direct else ''}")
    g = run_gpu(sh, x, logits=logits, ids=ids, w=w, direct=direct, allgather=allgather)
    o = compare_with_oracle(orc, sh, g, x, logits=logits, ids=ids, w=w)
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


@pytest.fixture(scope="module")
def skewed_oracle(orc):
    """c5 at its full size through the whole oracle path, once for the three forms below."""
    w = wl.WORKLOADS["c5"]
    sh = orc.Shape.of(w)
    log("[parity] c5 full size: inputs and the oracle's whole path")
    inp = wl.make_inputs(w)
    ids, wt = orc.route(sh, inp["logits"])
    o = orc.run(sh, inp["x"], ids=ids, w=wt)
    return w, sh, inp, o


@pytest.mark.parametrize("mode", ["base", "direct", "allgather"])
def test_skewed_workload_full_parity(skewed_oracle, mode):
    """c5 (32 ranks, 8192 tokens, E=256, top-8, H=7168, FP8, Zipf-skewed routing) at its full size, in
    the launch configuration the benchmark times, element by element against the oracle: every
    routing id and weight, count, offset, position and handle record, every send and receive row
    with its scales, every expert output and combine row, every y, and in the all-gather form every
    rank's copy of every token."""
    w, sh, inp, o = skewed_oracle
    direct, allgather = mode == "direct", mode == "allgather"
    log(f"[parity] c5 full size {mode}")
    g = run_gpu(sh, inp["x"], logits=inp["logits"], direct=direct, allgather=allgather)
    assert np.array_equal(g["ids"], o["ids"])
    assert_weights_close(g["w"], o["w"])
    assert_integer_parts_equal(g, o)
    n = np.sort(o["N"])[::-1]
    assert 0.40 <= n[: w.num_experts // 10].sum() / n.sum() <= 0.50
    for key in ("send_rows", "recv_rows", "send_scales", "recv_scales", "expert_out", "comb"):
        if g[key] is None:             # the direct and all-gather forms keep no send side; direct no comb
            assert (key.startswith("send") and (direct or allgather)) or (key == "comb" and direct), key
            continue
        assert np.array_equal(g[key].view(np.uint8), o[key].view(np.uint8)), key
        g[key] = None                   # keep the host copies of a 4 GB problem bounded
    assert record_weights_match(g["recv_meta"], g["w"], g["recv_pos"])
    assert_y_close(g["y"], o["y32"], o["y"])
    if weights_equal(g["w"], o["w"]):
        assert_bf16_equal(g["y"], o["y"])
    if allgather:
        # token t's dispatched codes and scales are the oracle's receive row of its slot 0
        q0 = o["recv_pos"][:, 0]
        codes, scales = o["recv_rows"][q0], o["recv_scales"][q0]
        for r in range(sh.P):
            assert np.array_equal(g["gathered"][r * sh.T:(r + 1) * sh.T], codes), ("gathered rows", r)
            assert np.array_equal(g["gathered_scales"][r * sh.T:(r + 1) * sh.T].view(np.uint32),
                                  scales.view(np.uint32)), ("gathered scales", r)


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


@pytest.mark.parametrize("strength", [0.4, 1.0])
def test_zipf_prior_in_identity_order(orc, strength):
    """The skewed workload's Zipf log-prior -s*ln(1 + e) with the identity rank order: the hottest experts are
    the lowest ids, which the contiguous placement puts on the first ranks, so one rank receives most of the
    rows (at the skewed workload's strength 0.4: rank 0 about 7x the mean; at full strength 1.0 about 19x,
    with many experts receiving nothing)."""
    P, Tp, E, k, H = 32, 32, 256, 8, 256
    sh = orc.Shape(P, P * Tp, E, k, H, True)
    z = wl.normals(wl.stream_seed(0x5EED0007, wl.STREAM_LOGITS), sh.T * E).reshape(sh.T, E)
    logits = (z - strength * np.log1p(np.arange(E, dtype=np.float64))[None, :]).astype(np.float32)
    g, _ = _full_parity(orc, sh, wl.make_hidden(7, sh.T, H), logits=logits, label=f"zipf identity s={strength}")
    per_rank = np.asarray(g["N"]).reshape(P, E // P).sum(axis=1)
    assert per_rank[0] == per_rank.max() and per_rank[0] > 5 * per_rank.mean()
    if strength == 1.0:
        assert np.count_nonzero(np.asarray(g["N"]) == 0) > 50


@pytest.mark.parametrize("E,k", [(8, 2), (32, 8), (96, 8), (256, 8)])
def test_route_nan_logits(orc, E, k):
    """NaN logits rank below every number and tie with each other (lower id first), in
    both router shapes; the rows that hold one get NaN weights on both sides, and the
    whole path then carries those NaNs to the same y positions as the oracle."""
    P, Tp, H = 4, 32, 128
    sh = orc.Shape(P, P * Tp, E, k, H, False)
    rng = np.random.default_rng(23)
    logits = rng.integers(-3, 4, size=(sh.T, E)).astype(np.float32)
    logits[rng.random((sh.T, E)) < 0.05] = np.nan
    logits[0] = np.nan                        # a whole row of NaN
    logits[1, 0] = np.nan                     # NaN before every number
    logits[2] = -np.inf
    logits[2, E - 1] = np.nan                 # NaN after a row of -inf
    logits[3, : E - k + 1] = np.nan           # fewer numbers than slots
    logits[4] = rng.normal(size=E)            # no NaN at all
    logits[5, 3] = np.frombuffer(np.uint32(0xFFC00000).tobytes(), np.float32)[0]   # a negative NaN
    _full_parity(orc, sh, wl.make_hidden(11, sh.T, H), logits=logits, label=f"NaN logits E={E}")


def test_fp8_hardware_conversions(orc):
    """The FP8 encoder (v_cvt_pk_fp8_f32) and decoder (v_cvt_pk_f32_fp8) against the oracle's
    E4M3 conversions written from the format's definition.  Every bf16 value of magnitude <= 448
    sits in a block whose maximum is 448, so the scale is exactly 1 and the code is the plain
    nearest-even E4M3 of the value; those codes cover all 254 finite codes, and the expert stub
    of expert 0 (multiplier exactly 1) writes each code's decoded value back, so expert_out
    checks the decoder.  Two more rows of normal values quantise under arbitrary scales."""
    H = 7168
    per_block = 127
    mags = np.arange(0x0000, 0x43E1, dtype=np.uint16)                 # bf16 0 .. 448
    vals = np.concatenate([mags, mags | np.uint16(0x8000)])           # and their negatives
    nblk = -(-len(vals) // per_block)
    rows = -(-nblk // (H // 128))
    P, Tp = 2, (rows + 2 + 1) // 2
    T = P * Tp
    x = wl.make_hidden(29, T, H)
    blocks = np.zeros((rows * (H // 128), 128), np.uint16)
    padded = np.zeros(nblk * per_block, np.uint16)
    padded[: len(vals)] = vals
    blocks[:nblk, :per_block] = padded.reshape(nblk, per_block)
    blocks[:, per_block] = 0x43E0                                     # 448: amax 448, scale exactly 1
    x[:rows] = blocks.reshape(rows, H)
    sh = orc.Shape(P, T, 4, 1, H, True)
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    g, o = _full_parity(orc, sh, x, ids=ids, w=w, label="fp8 hardware conversions")
    assert np.all(g["recv_scales"][g["recv_pos"][:rows, 0]] == 1.0)
    codes = g["recv_rows"][g["recv_pos"][:rows, 0]]
    finite = np.setdiff1d(np.arange(256), [0x7F, 0xFF])
    assert np.array_equal(np.unique(codes), finite), "not every finite E4M3 code was produced"
    # each code's decoded value: the stub of expert 0 multiplies by exactly 1
    dec = bf16_to_f32(g["expert_out"][g["recv_pos"][:rows, 0]])
    assert np.array_equal(dec.view(np.uint32), orc.e4m3_to_f32(codes).view(np.uint32))
    assert np.array_equal(codes, orc.e4m3_from_double(bf16_to_f32(x[:rows]).astype(np.float64)))


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


@pytest.mark.parametrize("name,mode", [("c1", "base"), ("c2", "base"), ("c2", "direct"), ("c3", "base"),
                                       ("c4", "base"), ("c5", "base"), ("c5", "direct")])
def test_deterministic_and_sentinel_free(orc, name, mode):
    """Two runs of the same workload, one over buffers pre-filled with 0xFF and one over
    whatever the allocator hands out, run twice in a row, give identical bytes in every
    output: no result depends on scheduling, on earlier buffer contents or on a previous call."""
    w = wl.WORKLOADS[name]
    sh = orc.Shape.of(w)
    inp = wl.make_inputs(w)
    log(f"[determinism] {name} {mode}")
    direct = mode == "direct"
    a = run_gpu(sh, inp["x"], logits=inp["logits"], sentinel=True, direct=direct)
    b = run_gpu(sh, inp["x"], logits=inp["logits"], sentinel=False, repeat=2, direct=direct)
    keys = ("ids", "w", "send_meta", "recv_meta", "send_rows", "recv_rows", "send_scales", "recv_scales",
            "expert_out", "comb", "y") + INT_KEYS
    for key in keys:
        if a[key] is None:
            assert b[key] is None, key
            continue
        assert np.array_equal(np.ascontiguousarray(a[key]).view(np.uint8),
                              np.ascontiguousarray(b[key]).view(np.uint8)), key


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
