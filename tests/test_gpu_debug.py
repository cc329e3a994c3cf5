"""Debug mode (MOE_EP_DEBUG=1): dispatch checks the expert ids on the device
before launching anything else and refuses ids out of range or repeated within
a token; valid input gives exactly the normal results.  Invalid ids are only
ever passed with the check on, which stops them before any kernel that would
index with them."""

import numpy as np
import pytest

from combine_router_softmax_expert_amd import workloads as wl
from gpu_helpers import assert_integer_parts_equal, log, run_gpu

pytestmark = pytest.mark.gpu


def _dispatch(B, ctx, bufs, x, direct):
    if direct:
        return B.moe_dispatch_direct(ctx, x, bufs["topk_ids"], bufs["topk_w"], bufs["workspace"], bufs["recv"],
                                     bufs["recv_scales"])
    return B.moe_dispatch(ctx, x, bufs["topk_ids"], bufs["topk_w"], bufs["workspace"], bufs["send"],
                          bufs["send_scales"], bufs["recv"], bufs["recv_scales"])


@pytest.mark.parametrize("direct", [False, True])
def test_debug_mode_refuses_invalid_ids(monkeypatch, direct):
    import torch
    from combine_router_softmax_expert_amd import binding as B

    monkeypatch.setenv("MOE_EP_DEBUG", "1")
    P, Tp, E, k, H = 4, 8, 8, 2, 64
    ctx = B.Context(P, Tp, E, k, H, False)
    bufs = ctx.allocate()
    T = P * Tp
    x = torch.from_numpy(wl.make_hidden(3, T, H).view(np.int16)).cuda()
    good = np.stack([np.random.default_rng(t).permutation(E)[:k] for t in range(T)]).astype(np.int32)
    bufs["topk_w"].fill_(0.5)
    cases = {
        "above range": (5, 1, E),
        "negative": (17, 0, -1),
        "repeated in a token": (9, 1, None),
    }
    for label, (t, j, value) in cases.items():
        ids = good.copy()
        ids[t, j] = ids[t, 0] if value is None else value
        log(f"[debug] {label} direct={direct}")
        bufs["topk_ids"].copy_(torch.from_numpy(ids))
        with pytest.raises(B.MoeError) as err:
            _dispatch(B, ctx, bufs, x, direct)
        assert err.value.status == -1
        assert b"out of range or repeated" in B.lib.moe_last_error()
    # the ctx stays usable: valid ids dispatch normally afterwards
    bufs["topk_ids"].copy_(torch.from_numpy(good))
    h = _dispatch(B, ctx, bufs, x, direct)
    torch.cuda.synchronize()
    assert h.generation == 1


def test_debug_mode_results_equal_normal_mode(orc, monkeypatch):
    w = wl.WORKLOADS["c1"]
    inp = wl.make_inputs(w)
    sh = orc.Shape.of(w)
    ids, wt = orc.route(sh, inp["logits"])
    plain = run_gpu(sh, inp["x"], ids=ids, w=wt)
    monkeypatch.setenv("MOE_EP_DEBUG", "1")
    checked = run_gpu(sh, inp["x"], ids=ids, w=wt)
    assert_integer_parts_equal(checked, plain)
    for key in ("recv_rows", "expert_out", "y"):
        assert np.array_equal(checked[key], plain[key]), key
