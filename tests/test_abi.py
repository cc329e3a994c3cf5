"""The C ABI on the CPU: the library loads, exports every declared symbol, and
its host-side validation returns the documented codes.  No call here reaches a
kernel launch (every case fails or finishes before one)."""

import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "moe_ep.h")


@pytest.fixture(scope="module")
def b():
    from combine_router_softmax_expert_amd import binding
    return binding


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(b):
    names = _declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(b.lib, n), n


def _create(b, P=4, Tp=16, E=8, k=2, H=256, dt=0):
    s = b.MoeShape(P, Tp, E, k, H, dt)
    h = ctypes.c_void_p()
    st = b.lib.moe_ctx_create(ctypes.byref(s), ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("args,code", [
    (dict(P=0), -1), (dict(Tp=-1), -1), (dict(E=6, P=4), -1), (dict(k=0), -1), (dict(k=9, E=8), -1),
    (dict(H=4), -1), (dict(H=260), -1), (dict(dt=2), -1),
    (dict(E=2048, P=4), -2), (dict(k=33, E=64), -2), (dict(dt=1, H=200), -2), (dict(H=131072), -2),
    (dict(P=1, Tp=1 << 28, k=8), -2), (dict(P=1, Tp=8_400_000, k=1, H=8), -2),
])
def test_ctx_create_rejects_bad_shapes(b, args, code):
    st, h = _create(b, **args)
    assert st == code and not h.value


def test_ctx_sizes(b):
    st, h = _create(b, P=8, Tp=16, E=256, k=8, H=7168, dt=0)
    assert st == 0
    try:
        assert b.lib.moe_dispatch_row_bytes(h) == 2 * 7168
        assert b.lib.moe_scales_per_row(h) == 0
        assert b.lib.moe_num_assignments(h) == 128 * 8
        ws = b.lib.moe_workspace_bytes(h)
        # counts/offsets + 4 int32 arrays of N_a + 2 handle records of 16 B per assignment
        assert ws >= 4 * (3 * 8 * 256 + 256 + 257 + 9 + 64) + 4 * 4 * 1024 + 2 * 16 * 1024
        assert ws % 256 == 0
    finally:
        b.lib.moe_ctx_destroy(h)
    st, h = _create(b, P=8, Tp=256, E=64, k=2, H=7168, dt=1)
    assert st == 0
    assert b.lib.moe_dispatch_row_bytes(h) == 7168 and b.lib.moe_scales_per_row(h) == 56
    b.lib.moe_ctx_destroy(h)


def test_status_strings(b):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert b.lib.moe_status_string(code)
    assert len({b.lib.moe_status_string(c) for c in range(-6, 1)}) == 7
    assert b.lib.moe_status_string(7) == b"unknown status"


def test_misaligned_pointers_are_refused_before_any_launch(b):
    """Row buffers need 16-byte alignment, the 4-byte arrays 4 bytes (CPU: every case fails before a launch)."""
    st, h = _create(b, dt=1)
    try:
        a = 1 << 20
        ok, row8, word2 = ctypes.c_void_p(a), ctypes.c_void_p(a + 8), ctypes.c_void_p(a + 2)
        ws = b.lib.moe_workspace_bytes(h)
        assert b.lib.moe_route_topk(h, word2, ok, ok, None) == -1
        assert b"4-byte" in b.lib.moe_last_error()
        hd = b.MoeHandle()
        # moe_dispatch: x, topk_ids, topk_w, workspace, bytes, send, send_scales, recv, recv_scales
        cases = [(row8, ok, ok, ok, ok, b"16-byte"), (ok, word2, ok, ok, ok, b"4-byte"),
                 (ok, ok, row8, ok, ok, b"16-byte"), (ok, ok, ok, word2, ok, b"4-byte"),
                 (ok, ok, ok, ok, row8, b"16-byte")]
        for x, ids, send, send_sc, recv, why in cases:
            assert b.lib.moe_dispatch(h, x, ids, ok, ok, ws, send, send_sc, recv, ok, ctypes.byref(hd), None) == -1
            assert why in b.lib.moe_last_error()
            assert hd.generation == 0                      # nothing was published
        assert b.lib.moe_dispatch_direct(h, row8, ok, ok, ok, ws, ok, ok, ctypes.byref(hd), None) == -1
        assert b.lib.moe_dispatch_allgather(h, ok, ok, ok, ok, ws, row8, ok, ok, ok, ctypes.byref(hd), None) == -1
        assert b.lib.moe_dispatch_send(h, ok, ok, word2, ok, ws, ok, ok, ctypes.byref(hd), None) == -1
        assert b"4-byte" in b.lib.moe_last_error() and hd.generation == 0
    finally:
        b.lib.moe_ctx_destroy(h)


def test_last_error_is_per_thread(b):
    """Each thread reads the reason of its own latest call, whatever another thread did meanwhile."""
    import threading
    st, h = _create(b)
    assert st == 0
    gate = threading.Barrier(2)
    seen = {}

    def worker(name, fail):
        fail()
        gate.wait()          # both threads have failed their call before either reads
        gate.wait()
        seen[name] = b.lib.moe_last_error()

    fake = ctypes.c_void_p(1 << 20)
    t1 = threading.Thread(target=worker, args=("route", lambda: b.lib.moe_route_topk(h, None, fake, fake, None)))
    t2 = threading.Thread(target=worker, args=("ws", lambda: b.lib.moe_dispatch(
        h, fake, fake, fake, fake, 0, fake, None, fake, None, ctypes.byref(b.MoeHandle()), None)))
    try:
        t1.start()
        t2.start()
        t1.join(30)
        t2.join(30)
        assert b"logits" in seen["route"] and b"workspace_bytes" in seen["ws"]
    finally:
        b.lib.moe_ctx_destroy(h)


def test_last_error_names_the_latest_calls_reason(b):
    """Each failing call leaves its own reason; every call clears the previous one."""
    st, h = _create(b, dt=1)            # FP8 dispatch: scales are required
    assert st == 0 and b.lib.moe_last_error() == b""
    try:
        fake = ctypes.c_void_p(1 << 20)
        ws = b.lib.moe_workspace_bytes(h)
        hd = b.MoeHandle()
        assert b.lib.moe_dispatch(h, fake, fake, fake, fake, ws - 1, fake, fake, fake, fake, ctypes.byref(hd),
                                  None) == -3
        assert b"workspace_bytes" in b.lib.moe_last_error()
        assert b.lib.moe_dispatch(h, fake, fake, fake, ctypes.c_void_p((1 << 20) + 8), ws, fake, fake, fake, fake,
                                  ctypes.byref(hd), None) == -1
        assert b"aligned" in b.lib.moe_last_error()
        assert b.lib.moe_dispatch(h, fake, fake, fake, fake, ws, fake, None, fake, fake, ctypes.byref(hd),
                                  None) == -1
        assert b"scales" in b.lib.moe_last_error()
        assert b.lib.moe_expert_stub(h, ctypes.byref(hd), fake, fake, fake, None) == -4
        assert b"latest dispatch" in b.lib.moe_last_error()
        assert b.lib.moe_route_topk(h, None, fake, fake, None) == -1
        assert b"logits" in b.lib.moe_last_error()
        assert b.lib.moe_timing_begin(h) == 0 and b.lib.moe_last_error() == b""   # cleared by a call that succeeds
        n = ctypes.c_int32(-1)
        assert b.lib.moe_timing_end(h, None, 0, ctypes.byref(n)) == 0 and b.lib.moe_last_error() == b""
        bad = b.MoeShape(4, 16, 6, 2, 256, 0)                                       # E not a multiple of P
        out = ctypes.c_void_p()
        assert b.lib.moe_ctx_create(ctypes.byref(bad), ctypes.byref(out)) == -1 and not out.value
        assert b"multiple of num_ranks" in b.lib.moe_last_error()
        # the Python error carries the reason for any status
        with pytest.raises(b.MoeError, match=r"invalid argument \(.*multiple of num_ranks"):
            b._check(-1, "moe_ctx_create")
    finally:
        b.lib.moe_ctx_destroy(h)


def test_null_arguments(b):
    assert b.lib.moe_ctx_create(None, None) == -1
    st, h = _create(b)
    fake = ctypes.c_void_p(1 << 20)  # an aligned non-null address that is never dereferenced
    handle = b.MoeHandle()
    assert b.lib.moe_route_topk(None, fake, fake, fake, None) == -1
    assert b.lib.moe_route_topk(h, None, fake, fake, None) == -1
    ws = b.lib.moe_workspace_bytes(h)
    D = b.lib.moe_dispatch
    assert D(None, fake, fake, fake, fake, ws, fake, None, fake, None, ctypes.byref(handle), None) == -1
    assert D(h, fake, fake, fake, fake, ws, fake, None, fake, None, None, None) == -1
    assert D(h, None, fake, fake, fake, ws, fake, None, fake, None, ctypes.byref(handle), None) == -1
    assert D(h, fake, fake, fake, None, ws, fake, None, fake, None, ctypes.byref(handle), None) == -1
    # misaligned workspace
    assert D(h, fake, fake, fake, ctypes.c_void_p((1 << 20) + 4), ws, fake, None, fake, None,
             ctypes.byref(handle), None) == -1
    # workspace too small
    assert D(h, fake, fake, fake, fake, ws - 1, fake, None, fake, None, ctypes.byref(handle), None) == -3
    # bf16 dispatch must not be given scales
    assert D(h, fake, fake, fake, fake, ws, fake, fake, fake, fake, ctypes.byref(handle), None) == -1
    b.lib.moe_ctx_destroy(h)
    st, h8 = _create(b, dt=1)
    ws8 = b.lib.moe_workspace_bytes(h8)
    # e4m3 dispatch needs both scale arrays
    assert b.lib.moe_dispatch(h8, fake, fake, fake, fake, ws8, fake, None, fake, fake,
                              ctypes.byref(handle), None) == -1
    b.lib.moe_ctx_destroy(h8)


def test_direct_forms_validate_arguments(b):
    st, h = _create(b)
    fake = ctypes.c_void_p(1 << 20)
    ws = b.lib.moe_workspace_bytes(h)
    handle = b.MoeHandle()
    D = b.lib.moe_dispatch_direct
    assert D(None, fake, fake, fake, fake, ws, fake, None, ctypes.byref(handle), None) == -1
    assert D(h, fake, fake, fake, fake, ws, None, None, ctypes.byref(handle), None) == -1
    assert D(h, fake, fake, fake, fake, ws - 1, fake, None, ctypes.byref(handle), None) == -3
    assert D(h, fake, fake, fake, fake, ws, fake, fake, ctypes.byref(handle), None) == -1   # bf16 takes no scales
    assert b.lib.moe_combine_direct(h, ctypes.byref(b.MoeHandle()), fake, fake, fake, None) == -4
    b.lib.moe_ctx_destroy(h)
    st, h0 = _create(b, Tp=0)
    h1 = b.MoeHandle()
    assert b.lib.moe_dispatch_direct(h0, None, None, None, fake, b.lib.moe_workspace_bytes(h0), None, None,
                                     ctypes.byref(h1), None) == 0
    assert h1.generation == 1 and not h1.send_meta
    assert b.lib.moe_combine_direct(h0, ctypes.byref(h1), None, None, None, None) == 0
    b.lib.moe_ctx_destroy(h0)


def test_noalloc_dispatch_validates_arguments(b):
    """moe_dispatch_noalloc checks its arguments and the size of the static workspace on the
    host, before it looks up that workspace or enqueues anything."""
    fake = ctypes.c_void_p(1 << 20)
    handle = b.MoeHandle()
    D = b.lib.moe_dispatch_noalloc
    st, h = _create(b)
    assert D(None, fake, fake, fake, fake, None, fake, None, ctypes.byref(handle), None) == -1
    assert D(h, fake, fake, fake, fake, None, fake, None, None, None) == -1
    assert D(h, fake, fake, fake, None, None, fake, None, ctypes.byref(handle), None) == -1    # no send_buf
    assert D(h, fake, fake, fake, fake, None, None, None, ctypes.byref(handle), None) == -1    # no recv_buf
    assert D(h, fake, fake, fake, fake, fake, fake, fake, ctypes.byref(handle), None) == -1    # bf16 takes no scales
    assert D(h, fake, fake, fake, ctypes.c_void_p((1 << 20) + 8), None, fake, None, ctypes.byref(handle), None) == -1
    assert b"16-byte" in b.lib.moe_last_error()
    b.lib.moe_ctx_destroy(h)
    st, h8 = _create(b, dt=1)
    assert D(h8, fake, fake, fake, fake, None, fake, fake, ctypes.byref(handle), None) == -1   # e4m3 needs both
    b.lib.moe_ctx_destroy(h8)
    # 262144 assignments need more than the 8 MiB the library holds: refused first
    st, big = _create(b, P=32, Tp=1024, E=256, k=8, H=128)
    assert st == 0 and b.lib.moe_workspace_bytes(big) > 8 << 20
    assert D(big, fake, fake, fake, fake, None, fake, None, ctypes.byref(handle), None) == -3
    assert b"8 MiB" in b.lib.moe_last_error()
    b.lib.moe_ctx_destroy(big)
    # the largest workloads here fit: the skewed 32-rank one needs about 3.4 MB
    st, c5 = _create(b, P=32, Tp=256, E=256, k=8, H=7168, dt=1)
    assert b.lib.moe_workspace_bytes(c5) < 8 << 20
    b.lib.moe_ctx_destroy(c5)


def test_probes_validate_arguments(b):
    fake = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 8)
    assert b.lib.moe_probe_copy(None, fake, 16, 0, None) == -1
    assert b.lib.moe_probe_copy(fake, None, 16, 1, None) == -1
    assert b.lib.moe_probe_copy(fake, fake, 17, 0, None) == -1
    assert b.lib.moe_probe_copy(odd, fake, 16, 0, None) == -1
    assert b"16-byte" in b.lib.moe_last_error()
    assert b.lib.moe_probe_read(fake, 16, None, 0, None) == -1
    assert b.lib.moe_probe_read(None, 16, fake, 0, None) == -1
    assert b.lib.moe_probe_read(fake, 24, fake, 1, None) == -1
    assert b.lib.moe_probe_copy(fake, fake, 16, 3, None) == -1    # policies 0..2 only
    assert b.lib.moe_probe_copy(fake, fake, 0, 0, None) == 0     # nothing to move: nothing enqueued
    G = b.lib.moe_probe_gather
    assert G(None, 4, fake, fake, 4, 64, 0, None) == -1             # src, dst and perm must be given
    assert G(fake, 4, fake, None, 4, 64, 0, None) == -1
    assert G(fake, 4, fake, fake, 4, 40, 0, None) == -1             # rows of whole 16-byte units
    assert G(fake, 4, fake, fake, 4, 0, 0, None) == -1
    assert G(fake, 0, fake, fake, 4, 64, 0, None) == -1             # a source to clamp into
    assert G(fake, 4, fake, fake, -1, 64, 0, None) == -1
    assert G(fake, 4, fake, fake, 4, 64, 3, None) == -1             # policies 0..2 only
    assert G(odd, 4, fake, fake, 4, 64, 0, None) == -1
    assert G(fake, 4, fake, fake, 1 << 30, 1 << 12, 0, None) == -2  # beyond one grid dimension
    assert G(fake, 4, fake, fake, 0, 64, 1, None) == 0              # no rows: nothing enqueued


def test_order_events_validate_arguments(b):
    assert b.lib.moe_event_create(None) == -1                 # nowhere to return the event
    assert b.lib.moe_event_destroy(None) == 0                 # nothing to destroy
    assert b.lib.moe_event_record(None, None) == -1
    assert b"event is NULL" in b.lib.moe_last_error()
    assert b.lib.moe_stream_wait_event(None, None) == -1


def test_stale_and_foreign_handles(b):
    st, h = _create(b)
    st2, h2 = _create(b)
    fake = ctypes.c_void_p(1 << 20)
    blank = b.MoeHandle()
    assert b.lib.moe_expert_stub(h, ctypes.byref(blank), fake, None, fake, None) == -4
    assert b.lib.moe_combine(h, ctypes.byref(blank), fake, fake, fake, fake, None) == -4
    assert b.lib.moe_expert_stub(h, None, fake, None, fake, None) == -1
    # a handle of another context is foreign
    other = b.MoeHandle()
    other.ctx = h2.value
    other.generation = 1
    assert b.lib.moe_combine(h, ctypes.byref(other), fake, fake, fake, fake, None) == -4
    b.lib.moe_ctx_destroy(h)
    b.lib.moe_ctx_destroy(h2)


def test_zero_tokens_is_a_noop_and_generations_advance(b):
    st, h = _create(b, Tp=0)
    assert st == 0
    fake = ctypes.c_void_p(1 << 20)
    ws = b.lib.moe_workspace_bytes(h)
    assert b.lib.moe_route_topk(h, None, None, None, None) == 0
    h1, h2 = b.MoeHandle(), b.MoeHandle()
    assert b.lib.moe_dispatch(h, None, None, None, fake, ws, None, None, None, None, ctypes.byref(h1), None) == 0
    assert h1.generation == 1 and h1.ctx == h.value
    assert b.lib.moe_expert_stub(h, ctypes.byref(h1), None, None, None, None) == 0
    assert b.lib.moe_combine(h, ctypes.byref(h1), None, None, None, None, None) == 0
    assert b.lib.moe_dispatch(h, None, None, None, fake, ws, None, None, None, None, ctypes.byref(h2), None) == 0
    assert h2.generation == 2
    # the first handle is stale once a newer dispatch reused the workspace
    assert b.lib.moe_combine(h, ctypes.byref(h1), None, None, None, None, None) == -4
    assert b.lib.moe_combine(h, ctypes.byref(h2), None, None, None, None, None) == 0
    b.lib.moe_ctx_destroy(h)


def test_timing_without_launches(b):
    st, h = _create(b)
    assert b.lib.moe_timing_begin(h) == 0
    recs = (b.MoeKernelTime * 4)()
    n = ctypes.c_int32(-1)
    assert b.lib.moe_timing_end(h, recs, 4, ctypes.byref(n)) == 0 and n.value == 0
    b.lib.moe_ctx_destroy(h)


def test_split_phases_enforce_their_order(b):
    """The host refuses a stage whose earlier half was not issued (T = 0: nothing is launched)."""
    st, h = _create(b, Tp=0)
    fake = ctypes.c_void_p(1 << 20)
    ws = b.lib.moe_workspace_bytes(h)
    hd = b.MoeHandle()
    assert b.lib.moe_dispatch_send(h, None, None, None, fake, ws, None, None, ctypes.byref(hd), None) == 0
    # the expert stage and the combine need the receive half first
    assert b.lib.moe_expert_stub(h, ctypes.byref(hd), None, None, None, None) == -1
    assert b"moe_dispatch_recv" in b.lib.moe_last_error()
    assert b.lib.moe_combine(h, ctypes.byref(hd), None, None, None, None, None) == -1
    assert b.lib.moe_dispatch_recv(h, ctypes.byref(hd), None, None, None, None, None) == 0
    assert b.lib.moe_dispatch_recv(h, ctypes.byref(hd), None, None, None, None, None) == -1   # only once
    assert b.lib.moe_expert_stub(h, ctypes.byref(hd), None, None, None, None) == 0
    # the combine's receive half needs its send half
    assert b.lib.moe_combine_recv(h, ctypes.byref(hd), None, None, None, None) == -1
    assert b.lib.moe_combine_send(h, ctypes.byref(hd), None, None, None) == 0
    assert b.lib.moe_combine_recv(h, ctypes.byref(hd), None, None, None, None) == 0
    # a direct dispatch has no separate receive half
    hdir = b.MoeHandle()
    assert b.lib.moe_dispatch_direct(h, None, None, None, fake, ws, None, None, ctypes.byref(hdir), None) == 0
    assert b.lib.moe_dispatch_recv(h, ctypes.byref(hdir), None, None, None, None, None) == -1
    assert b.lib.moe_combine_direct(h, ctypes.byref(hdir), None, None, None, None) == 0
    # a newer dispatch makes the older handle stale for every half
    assert b.lib.moe_dispatch_recv(h, ctypes.byref(hd), None, None, None, None, None) == -4
    b.lib.moe_ctx_destroy(h)


def test_split_phases_validate_arguments(b):
    st, h = _create(b)
    fake = ctypes.c_void_p(1 << 20)
    ws = b.lib.moe_workspace_bytes(h)
    hd = b.MoeHandle()
    S = b.lib.moe_dispatch_send
    assert S(h, fake, fake, fake, fake, ws, None, None, ctypes.byref(hd), None) == -1      # no send buffer
    assert S(h, fake, fake, fake, fake, ws, fake, fake, ctypes.byref(hd), None) == -1      # bf16 takes no scales
    assert S(h, fake, fake, fake, fake, ws - 1, fake, None, ctypes.byref(hd), None) == -3
    assert b.lib.moe_dispatch_recv(h, ctypes.byref(b.MoeHandle()), fake, None, fake, None, None) == -4
    assert b.lib.moe_combine_send(h, ctypes.byref(b.MoeHandle()), fake, fake, None) == -4
    assert b.lib.moe_combine_recv(h, ctypes.byref(b.MoeHandle()), fake, fake, fake, None) == -4
    b.lib.moe_ctx_destroy(h)


def test_allgather_dispatch_validates_arguments(b):
    st, h = _create(b)
    fake = ctypes.c_void_p(1 << 20)
    ws = b.lib.moe_workspace_bytes(h)
    hd = b.MoeHandle()
    A = b.lib.moe_dispatch_allgather
    assert A(h, fake, fake, fake, fake, ws, None, None, fake, None, ctypes.byref(hd), None) == -1    # no gathered buffer
    assert A(h, fake, fake, fake, fake, ws, fake, fake, fake, None, ctypes.byref(hd), None) == -1    # bf16 takes no scales
    assert A(h, fake, fake, fake, fake, ws - 1, fake, None, fake, None, ctypes.byref(hd), None) == -3
    assert A(h, fake, fake, fake, fake, ws, fake, None, fake, None, None, None) == -1
    b.lib.moe_ctx_destroy(h)
    st, hbig = _create(b, P=2, Tp=2_250_000, E=2, k=1, H=8)     # P * T * (H/8 + 512) >= 2^32 gathered work-items
    assert st == 0
    assert b.lib.moe_dispatch_allgather(hbig, fake, fake, fake, fake, b.lib.moe_workspace_bytes(hbig), fake, None,
                                        fake, None, ctypes.byref(hd), None) == -2
    b.lib.moe_ctx_destroy(hbig)
    st, h0 = _create(b, Tp=0)
    h1 = b.MoeHandle()
    assert b.lib.moe_dispatch_allgather(h0, None, None, None, fake, b.lib.moe_workspace_bytes(h0), None, None, None,
                                        None, ctypes.byref(h1), None) == 0
    assert not h1.send_meta and b.lib.moe_combine(h0, ctypes.byref(h1), None, None, None, None, None) == 0
    b.lib.moe_ctx_destroy(h0)


def test_prepared_path_refuses_a_closed_context(b):
    # the cached calls hold the ctx pointer; after close() they must not reach the library
    ctx = b.Context(2, 4, 4, 2, 64)
    path = b.PreparedPath.__new__(b.PreparedPath)
    path._ctx, path._calls, path.handle = ctx, [(b.lib.moe_timing_begin, (ctx.handle_ptr,), "moe_timing_begin")], None
    path()                                         # open: the cached call runs
    ctx.close()
    with pytest.raises(ValueError, match="closed"):
        path()


def test_prepared_path_checks_its_tensors_once_without_a_gpu(b):
    # the prepared calls run the same checks as the individual functions at set-up:
    # tensors that are not on the GPU, an unknown stage list, missing logits and the
    # all-gather dispatcher's missing direct form are refused before any library call
    import torch
    ctx = b.Context(2, 4, 4, 2, 64)
    T, E, k, H, Na = 8, 4, 2, 64, 16
    bufs = {"topk_ids": torch.zeros(T, k, dtype=torch.int32), "topk_w": torch.zeros(T, k),
            "workspace": torch.zeros(ctx.workspace_bytes, dtype=torch.uint8),
            "send": torch.zeros(Na, 2 * H, dtype=torch.uint8), "recv": torch.zeros(Na, 2 * H, dtype=torch.uint8),
            "send_scales": None, "recv_scales": None, "expert_out": torch.zeros(Na, H, dtype=torch.int16),
            "comb": torch.zeros(Na, H, dtype=torch.int16), "y": torch.zeros(T, H, dtype=torch.int16)}
    x = torch.zeros(T, H, dtype=torch.int16)
    logits = torch.zeros(T, E)
    with pytest.raises(ValueError, match="GPU tensor"):
        b.PreparedPath(ctx, bufs, x, logits)
    with pytest.raises(ValueError, match="stages"):
        b.PreparedPath(ctx, bufs, x, logits, stages="combine")
    with pytest.raises(ValueError, match="logits"):
        b.PreparedPath(ctx, bufs, x, None)
    with pytest.raises(ValueError, match="direct form"):
        b.PreparedPath(ctx, bufs, x, None, direct=True, stages="dispatch_combine", gathered=torch.zeros(1))
