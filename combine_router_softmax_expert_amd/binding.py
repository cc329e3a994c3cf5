"""Thin ctypes binding of libmoe_ep.so (the C ABI in include/moe_ep.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Tensors are torch tensors on the GPU (torch supplies device memory
and streams); pointers and sizes go straight to the C calls.  If the library
is missing this module raises on import: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_ep.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_STALE_HANDLE = -4
MOE_ERR_HIP = -5
MOE_ERR_NO_MEMORY = -6

MOE_DTYPE_BF16 = 0
MOE_DTYPE_FP8_E4M3 = 1

FP8_BLOCK = 128


class MoeShape(ctypes.Structure):
    _fields_ = [("num_ranks", ctypes.c_int32), ("tokens_per_rank", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("dispatch_dtype", ctypes.c_int32)]


class MoeMeta(ctypes.Structure):
    _fields_ = [("src_rank", ctypes.c_int32), ("src_token", ctypes.c_int32), ("slot", ctypes.c_int16),
                ("local_expert", ctypes.c_int16), ("weight", ctypes.c_float)]


class MoeHandle(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "expert_counts", "expert_offsets", "rank_recv_offsets", "count_matrix", "rank_expert_counts",
        "send_offsets", "recv_offsets", "send_pos", "recv_pos", "send_meta", "recv_meta", "ctx")] + [
        ("generation", ctypes.c_uint64)]


class MoeKernelTime(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char_p), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_float)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                           "(hipcc --offload-arch=gfx950) first")
    # torch first: the library and torch must share one HIP runtime, and torch ships
    # its own.  Loaded first, the library would bring in the system's runtime under
    # the same soname, and torch would then run on a runtime it was not built with
    # (its calls then find no device).
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "moe_ctx_create": (I32, [ctypes.POINTER(MoeShape), ctypes.POINTER(P)]),
        "moe_ctx_destroy": (None, [P]),
        "moe_workspace_bytes": (SZ, [P]),
        "moe_dispatch_row_bytes": (SZ, [P]),
        "moe_scales_per_row": (I32, [P]),
        "moe_num_assignments": (I64, [P]),
        "moe_route_topk": (I32, [P, P, P, P, P]),
        "moe_dispatch": (I32, [P, P, P, P, P, SZ, P, P, P, P, ctypes.POINTER(MoeHandle), P]),
        "moe_expert_stub": (I32, [P, ctypes.POINTER(MoeHandle), P, P, P, P]),
        "moe_combine": (I32, [P, ctypes.POINTER(MoeHandle), P, P, P, P, P]),
        "moe_dispatch_direct": (I32, [P, P, P, P, P, SZ, P, P, ctypes.POINTER(MoeHandle), P]),
        "moe_dispatch_noalloc": (I32, [P, P, P, P, P, P, P, P, ctypes.POINTER(MoeHandle), P]),
        "moe_combine_direct": (I32, [P, ctypes.POINTER(MoeHandle), P, P, P, P]),
        "moe_dispatch_allgather": (I32, [P, P, P, P, P, SZ, P, P, P, P, ctypes.POINTER(MoeHandle), P]),
        "moe_dispatch_send": (I32, [P, P, P, P, P, SZ, P, P, ctypes.POINTER(MoeHandle), P]),
        "moe_dispatch_recv": (I32, [P, ctypes.POINTER(MoeHandle), P, P, P, P, P]),
        "moe_combine_send": (I32, [P, ctypes.POINTER(MoeHandle), P, P, P]),
        "moe_combine_recv": (I32, [P, ctypes.POINTER(MoeHandle), P, P, P, P]),
        "moe_probe_copy": (I32, [P, P, SZ, I32, P]),
        "moe_probe_read": (I32, [P, SZ, P, I32, P]),
        "moe_probe_gather": (I32, [P, I32, P, P, I32, I32, I32, P]),
        "moe_event_create": (I32, [ctypes.POINTER(ctypes.c_void_p)]),
        "moe_event_destroy": (I32, [P]),
        "moe_event_record": (I32, [P, P]),
        "moe_stream_wait_event": (I32, [P, P]),
        "moe_status_string": (ctypes.c_char_p, [I32]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_timing_begin": (I32, [P]),
        "moe_timing_end": (I32, [P, ctypes.POINTER(MoeKernelTime), I32, ctypes.POINTER(I32)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib.moe_status_string(status).decode()
        extra = lib.moe_last_error().decode()   # the failing call's reason, "" if it gave none
        super().__init__(f"{where}: {msg}" + (f" ({extra})" if extra else ""))
        self.status = status


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def _ptr(t, dtype=None, numel=None, name="tensor"):
    """Device pointer of a contiguous CUDA/HIP tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() * t.element_size() < numel:
        raise ValueError(f"{name} is too small: {t.numel() * t.element_size()} < {numel} bytes")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class Context:
    """Owns a moe_ctx (host object; no device memory)."""

    def __init__(self, num_ranks: int, tokens_per_rank: int, num_experts: int, top_k: int, hidden: int,
                 fp8: bool = False):
        self.shape = MoeShape(num_ranks, tokens_per_rank, num_experts, top_k, hidden,
                              MOE_DTYPE_FP8_E4M3 if fp8 else MOE_DTYPE_BF16)
        h = ctypes.c_void_p()
        _check(lib.moe_ctx_create(ctypes.byref(self.shape), ctypes.byref(h)), "moe_ctx_create")
        self._h = h
        self.P, self.Tp, self.E, self.k, self.H, self.fp8 = num_ranks, tokens_per_rank, num_experts, top_k, hidden, fp8
        self.T = num_ranks * tokens_per_rank

    @classmethod
    def for_workload(cls, w) -> "Context":
        return cls(w.num_ranks, w.tokens_per_rank, w.num_experts, w.top_k, w.hidden, w.dispatch_dtype != "bf16")

    @property
    def handle_ptr(self):
        return self._h

    @property
    def workspace_bytes(self) -> int:
        return lib.moe_workspace_bytes(self._h)

    @property
    def row_bytes(self) -> int:
        return lib.moe_dispatch_row_bytes(self._h)

    @property
    def scales_per_row(self) -> int:
        return lib.moe_scales_per_row(self._h)

    @property
    def num_assignments(self) -> int:
        return lib.moe_num_assignments(self._h)

    def close(self):
        if self._h:
            lib.moe_ctx_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def allocate_gathered(self, device="cuda"):
        """The all-gather dispatcher's per-rank copies of every token (rows and FP8 scales)."""
        import torch
        rows = self.P * self.T
        return (torch.empty((rows, self.row_bytes), dtype=torch.uint8, device=device),
                torch.empty((rows, self.scales_per_row), dtype=torch.float32, device=device) if self.fp8 else None)

    def allocate(self, device="cuda"):
        """Caller-owned device buffers of the sizes the calls expect (torch.empty: contents undefined)."""
        import torch
        Na, H, T, k = self.num_assignments, self.H, self.T, self.k
        nb = self.scales_per_row
        b = {
            "topk_ids": torch.empty((T, k), dtype=torch.int32, device=device),
            "topk_w": torch.empty((T, k), dtype=torch.float32, device=device),
            "workspace": torch.empty(max(self.workspace_bytes, 1), dtype=torch.uint8, device=device),
            "send": torch.empty((Na, self.row_bytes), dtype=torch.uint8, device=device),
            "recv": torch.empty((Na, self.row_bytes), dtype=torch.uint8, device=device),
            "send_scales": torch.empty((Na, nb), dtype=torch.float32, device=device) if self.fp8 else None,
            "recv_scales": torch.empty((Na, nb), dtype=torch.float32, device=device) if self.fp8 else None,
            "expert_out": torch.empty((Na, H), dtype=torch.bfloat16, device=device),
            "comb": torch.empty((Na, H), dtype=torch.bfloat16, device=device),
            "y": torch.empty((T, H), dtype=torch.bfloat16, device=device),
        }
        return b


def moe_route_topk(ctx: Context, logits, topk_ids, topk_w, stream=None):
    import torch
    T, E, k = ctx.T, ctx.E, ctx.k
    _check(lib.moe_route_topk(ctx.handle_ptr, _ptr(logits, torch.float32, 4 * T * E, "logits"),
                              _ptr(topk_ids, torch.int32, 4 * T * k, "topk_ids"),
                              _ptr(topk_w, torch.float32, 4 * T * k, "topk_w"), _stream(stream)),
           "moe_route_topk")


def moe_dispatch(ctx: Context, x, topk_ids, topk_w, workspace, send_buf, send_scales, recv_buf, recv_scales,
                 stream=None) -> MoeHandle:
    import torch
    T, H, k, Na = ctx.T, ctx.H, ctx.k, ctx.num_assignments
    rb, nb = ctx.row_bytes, ctx.scales_per_row
    h = MoeHandle()
    ws = _ptr(workspace, None, ctx.workspace_bytes, "workspace")
    _check(lib.moe_dispatch(ctx.handle_ptr, _ptr(x, (torch.bfloat16, torch.int16), 2 * T * H, "x"),
                            _ptr(topk_ids, torch.int32, 4 * T * k, "topk_ids"),
                            _ptr(topk_w, torch.float32, 4 * T * k, "topk_w"),
                            ws, workspace.numel() * workspace.element_size(),
                            _ptr(send_buf, None, Na * rb, "send_buf"),
                            _ptr(send_scales, torch.float32, 4 * Na * nb, "send_scales"),
                            _ptr(recv_buf, None, Na * rb, "recv_buf"),
                            _ptr(recv_scales, torch.float32, 4 * Na * nb, "recv_scales"),
                            ctypes.byref(h), _stream(stream)), "moe_dispatch")
    return h


def moe_expert_stub(ctx: Context, handle: MoeHandle, recv_buf, recv_scales, expert_out, stream=None):
    import torch
    Na, H, rb, nb = ctx.num_assignments, ctx.H, ctx.row_bytes, ctx.scales_per_row
    _check(lib.moe_expert_stub(ctx.handle_ptr, ctypes.byref(handle), _ptr(recv_buf, None, Na * rb, "recv_buf"),
                               _ptr(recv_scales, torch.float32, 4 * Na * nb, "recv_scales"),
                               _ptr(expert_out, (torch.bfloat16, torch.int16), 2 * Na * H, "expert_out"),
                               _stream(stream)), "moe_expert_stub")


def moe_combine(ctx: Context, handle: MoeHandle, expert_out, topk_w, comb_buf, y, stream=None):
    import torch
    Na, H, T, k = ctx.num_assignments, ctx.H, ctx.T, ctx.k
    _check(lib.moe_combine(ctx.handle_ptr, ctypes.byref(handle),
                           _ptr(expert_out, (torch.bfloat16, torch.int16), 2 * Na * H, "expert_out"),
                           _ptr(topk_w, torch.float32, 4 * T * k, "topk_w"),
                           _ptr(comb_buf, (torch.bfloat16, torch.int16), 2 * Na * H, "comb_buf"),
                           _ptr(y, (torch.bfloat16, torch.int16), 2 * T * H, "y"), _stream(stream)),
           "moe_combine")


def moe_dispatch_noalloc(ctx: Context, x, topk_ids, topk_w, send_buf, send_scales, recv_buf, recv_scales,
                         stream=None) -> MoeHandle:
    """moe_dispatch with the library's static workspace in place of a caller buffer."""
    import torch
    T, H, k, Na = ctx.T, ctx.H, ctx.k, ctx.num_assignments
    rb, nb = ctx.row_bytes, ctx.scales_per_row
    h = MoeHandle()
    _check(lib.moe_dispatch_noalloc(ctx.handle_ptr, _ptr(x, (torch.bfloat16, torch.int16), 2 * T * H, "x"),
                                    _ptr(topk_ids, torch.int32, 4 * T * k, "topk_ids"),
                                    _ptr(topk_w, torch.float32, 4 * T * k, "topk_w"),
                                    _ptr(send_buf, None, Na * rb, "send_buf"),
                                    _ptr(send_scales, torch.float32, 4 * Na * nb, "send_scales"),
                                    _ptr(recv_buf, None, Na * rb, "recv_buf"),
                                    _ptr(recv_scales, torch.float32, 4 * Na * nb, "recv_scales"),
                                    ctypes.byref(h), _stream(stream)), "moe_dispatch_noalloc")
    return h


def moe_dispatch_direct(ctx: Context, x, topk_ids, topk_w, workspace, recv_buf, recv_scales,
                        stream=None) -> MoeHandle:
    import torch
    T, H, k, Na = ctx.T, ctx.H, ctx.k, ctx.num_assignments
    rb, nb = ctx.row_bytes, ctx.scales_per_row
    h = MoeHandle()
    ws = _ptr(workspace, None, ctx.workspace_bytes, "workspace")
    _check(lib.moe_dispatch_direct(ctx.handle_ptr, _ptr(x, (torch.bfloat16, torch.int16), 2 * T * H, "x"),
                                   _ptr(topk_ids, torch.int32, 4 * T * k, "topk_ids"),
                                   _ptr(topk_w, torch.float32, 4 * T * k, "topk_w"),
                                   ws, workspace.numel() * workspace.element_size(),
                                   _ptr(recv_buf, None, Na * rb, "recv_buf"),
                                   _ptr(recv_scales, torch.float32, 4 * Na * nb, "recv_scales"),
                                   ctypes.byref(h), _stream(stream)), "moe_dispatch_direct")
    return h


def moe_combine_direct(ctx: Context, handle: MoeHandle, expert_out, topk_w, y, stream=None):
    import torch
    Na, H, T, k = ctx.num_assignments, ctx.H, ctx.T, ctx.k
    _check(lib.moe_combine_direct(ctx.handle_ptr, ctypes.byref(handle),
                                  _ptr(expert_out, (torch.bfloat16, torch.int16), 2 * Na * H, "expert_out"),
                                  _ptr(topk_w, torch.float32, 4 * T * k, "topk_w"),
                                  _ptr(y, (torch.bfloat16, torch.int16), 2 * T * H, "y"), _stream(stream)),
           "moe_combine_direct")


def moe_dispatch_allgather(ctx: Context, x, topk_ids, topk_w, workspace, gathered, gathered_scales, recv_buf,
                           recv_scales, stream=None) -> MoeHandle:
    import torch
    T, H, k, Na, P = ctx.T, ctx.H, ctx.k, ctx.num_assignments, ctx.P
    rb, nb = ctx.row_bytes, ctx.scales_per_row
    h = MoeHandle()
    ws = _ptr(workspace, None, ctx.workspace_bytes, "workspace")
    _check(lib.moe_dispatch_allgather(ctx.handle_ptr, _ptr(x, (torch.bfloat16, torch.int16), 2 * T * H, "x"),
                                      _ptr(topk_ids, torch.int32, 4 * T * k, "topk_ids"),
                                      _ptr(topk_w, torch.float32, 4 * T * k, "topk_w"),
                                      ws, workspace.numel() * workspace.element_size(),
                                      _ptr(gathered, None, P * T * rb, "gathered"),
                                      _ptr(gathered_scales, torch.float32, 4 * P * T * nb, "gathered_scales"),
                                      _ptr(recv_buf, None, Na * rb, "recv_buf"),
                                      _ptr(recv_scales, torch.float32, 4 * Na * nb, "recv_scales"),
                                      ctypes.byref(h), _stream(stream)), "moe_dispatch_allgather")
    return h


def moe_dispatch_send(ctx: Context, x, topk_ids, topk_w, workspace, send_buf, send_scales, stream=None) -> MoeHandle:
    import torch
    T, H, k, Na = ctx.T, ctx.H, ctx.k, ctx.num_assignments
    rb, nb = ctx.row_bytes, ctx.scales_per_row
    h = MoeHandle()
    ws = _ptr(workspace, None, ctx.workspace_bytes, "workspace")
    _check(lib.moe_dispatch_send(ctx.handle_ptr, _ptr(x, (torch.bfloat16, torch.int16), 2 * T * H, "x"),
                                 _ptr(topk_ids, torch.int32, 4 * T * k, "topk_ids"),
                                 _ptr(topk_w, torch.float32, 4 * T * k, "topk_w"),
                                 ws, workspace.numel() * workspace.element_size(),
                                 _ptr(send_buf, None, Na * rb, "send_buf"),
                                 _ptr(send_scales, torch.float32, 4 * Na * nb, "send_scales"),
                                 ctypes.byref(h), _stream(stream)), "moe_dispatch_send")
    return h


def moe_dispatch_recv(ctx: Context, handle: MoeHandle, send_buf, send_scales, recv_buf, recv_scales, stream=None):
    import torch
    Na, rb, nb = ctx.num_assignments, ctx.row_bytes, ctx.scales_per_row
    _check(lib.moe_dispatch_recv(ctx.handle_ptr, ctypes.byref(handle), _ptr(send_buf, None, Na * rb, "send_buf"),
                                 _ptr(send_scales, torch.float32, 4 * Na * nb, "send_scales"),
                                 _ptr(recv_buf, None, Na * rb, "recv_buf"),
                                 _ptr(recv_scales, torch.float32, 4 * Na * nb, "recv_scales"), _stream(stream)),
           "moe_dispatch_recv")


def moe_combine_send(ctx: Context, handle: MoeHandle, expert_out, comb_buf, stream=None):
    import torch
    Na, H = ctx.num_assignments, ctx.H
    _check(lib.moe_combine_send(ctx.handle_ptr, ctypes.byref(handle),
                                _ptr(expert_out, (torch.bfloat16, torch.int16), 2 * Na * H, "expert_out"),
                                _ptr(comb_buf, (torch.bfloat16, torch.int16), 2 * Na * H, "comb_buf"),
                                _stream(stream)), "moe_combine_send")


def moe_combine_recv(ctx: Context, handle: MoeHandle, comb_buf, topk_w, y, stream=None):
    import torch
    Na, H, T, k = ctx.num_assignments, ctx.H, ctx.T, ctx.k
    _check(lib.moe_combine_recv(ctx.handle_ptr, ctypes.byref(handle),
                                _ptr(comb_buf, (torch.bfloat16, torch.int16), 2 * Na * H, "comb_buf"),
                                _ptr(topk_w, torch.float32, 4 * T * k, "topk_w"),
                                _ptr(y, (torch.bfloat16, torch.int16), 2 * T * H, "y"), _stream(stream)),
           "moe_combine_recv")


PROBE_TEMPORAL, PROBE_NONTEMPORAL, PROBE_WRITE_THROUGH = 0, 1, 2


def moe_probe_copy(src, dst, policy: int, stream=None):
    """Measurement aid: dst = src (both contiguous GPU tensors of the same byte size); policy
    PROBE_TEMPORAL, PROBE_NONTEMPORAL or PROBE_WRITE_THROUGH."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("src and dst differ in size")
    _check(lib.moe_probe_copy(_ptr(src, name="src"), _ptr(dst, name="dst"), n, int(policy), _stream(stream)),
           "moe_probe_copy")


def moe_probe_read(src, sink, nontemporal: bool, stream=None):
    """Measurement aid: reads every byte of src; sink is a GPU tensor of at least 256 int32."""
    import torch
    n = src.numel() * src.element_size()
    _check(lib.moe_probe_read(_ptr(src, name="src"), n, _ptr(sink, (torch.int32, torch.uint32), 1024, "sink"),
                              int(nontemporal), _stream(stream)), "moe_probe_read")


def moe_probe_gather(src, dst, perm, policy: int, stream=None):
    """Measurement aid: row r of dst = row perm[r] of src.  src [src_rows, row_bytes] and dst [rows,
    row_bytes] are 2-D uint8 GPU tensors with the same row size; perm holds rows int32 (entries outside
    [0, src_rows) are clamped into it)."""
    import torch
    if src.dim() != 2 or dst.dim() != 2 or src.dtype != torch.uint8 or dst.dtype != torch.uint8:
        raise ValueError("src and dst must be 2-D uint8 tensors")
    if src.shape[1] != dst.shape[1]:
        raise ValueError("src and dst rows differ in size")
    rows, row_bytes = dst.shape
    _check(lib.moe_probe_gather(_ptr(src, name="src"), src.shape[0], _ptr(dst, name="dst"),
                                _ptr(perm, torch.int32, 4 * rows, "perm"), rows, row_bytes, int(policy),
                                _stream(stream)), "moe_probe_gather")


def moe_timing_begin(ctx: Context):
    _check(lib.moe_timing_begin(ctx.handle_ptr), "moe_timing_begin")


def moe_timing_end(ctx: Context) -> dict:
    recs = (MoeKernelTime * 64)()
    n = ctypes.c_int32()
    _check(lib.moe_timing_end(ctx.handle_ptr, recs, 64, ctypes.byref(n)), "moe_timing_end")
    return {recs[i].kernel.decode(): (recs[i].launches, recs[i].total_ms) for i in range(min(n.value, 64))}


def run_path(ctx: Context, bufs: dict, x, logits, stream=None, direct: bool = False) -> MoeHandle:
    """One pass of the whole path: route, dispatch, expert stub, combine (direct forms if asked)."""
    moe_route_topk(ctx, logits, bufs["topk_ids"], bufs["topk_w"], stream)
    if direct:
        h = moe_dispatch_direct(ctx, x, bufs["topk_ids"], bufs["topk_w"], bufs["workspace"], bufs["recv"],
                                bufs["recv_scales"], stream)
    else:
        h = moe_dispatch(ctx, x, bufs["topk_ids"], bufs["topk_w"], bufs["workspace"], bufs["send"],
                         bufs["send_scales"], bufs["recv"], bufs["recv_scales"], stream)
    moe_expert_stub(ctx, h, bufs["recv"], bufs["recv_scales"], bufs["expert_out"], stream)
    if direct:
        moe_combine_direct(ctx, h, bufs["expert_out"], bufs["topk_w"], bufs["y"], stream)
    else:
        moe_combine(ctx, h, bufs["expert_out"], bufs["topk_w"], bufs["comb"], bufs["y"], stream)
    return h


class PreparedPath:
    """The path's library calls over fixed tensors, with every tensor checked and its
    pointer marshalled once, here, with the checks of the individual functions above.
    Each call then issues the same calls with the cached arguments: route, dispatch,
    expert stub and combine (``stages="path"``), or dispatch and combine alone
    (``stages="dispatch_combine"``, on the ids and weights already in ``bufs``), in
    the base or the direct form, or with the all-gather dispatcher when its per-rank
    copies (``gathered``, ``gathered_scales`` from ``Context.allocate_gathered``) are
    given (base combine).  The calls and their kernels are those of
    ``run_path``; only the per-call Python work goes (at 128 tokens x top-8 x 7168
    it was ~7 us of host time per step, more than the GPU's spare time).  The
    tensors must stay alive and in place while the object is used."""

    def __init__(self, ctx: Context, bufs: dict, x, logits=None, stream=None, direct: bool = False,
                 stages: str = "path", gathered=None, gathered_scales=None):
        import torch
        if stages not in ("path", "dispatch_combine"):
            raise ValueError(f"stages must be 'path' or 'dispatch_combine', not {stages!r}")
        if x is None or (stages == "path" and logits is None):
            raise ValueError("x, and for the whole path the logits, are required")
        if gathered is not None and direct:
            raise ValueError("the all-gather dispatcher has no direct form")
        T, H, k, E, Na = ctx.T, ctx.H, ctx.k, ctx.E, ctx.num_assignments
        rb, nb = ctx.row_bytes, ctx.scales_per_row
        bf16 = (torch.bfloat16, torch.int16)
        self._keep = (ctx, bufs, x, logits, stream, gathered, gathered_scales)
        self._ctx = ctx
        self.handle = MoeHandle()
        h = ctypes.byref(self.handle)
        c = ctx.handle_ptr
        ids = _ptr(bufs["topk_ids"], torch.int32, 4 * T * k, "topk_ids")
        w = _ptr(bufs["topk_w"], torch.float32, 4 * T * k, "topk_w")
        ws = _ptr(bufs["workspace"], None, ctx.workspace_bytes, "workspace")
        ws_bytes = bufs["workspace"].numel() * bufs["workspace"].element_size()
        xp = _ptr(x, bf16, 2 * T * H, "x")
        recv = _ptr(bufs["recv"], None, Na * rb, "recv_buf")
        recv_sc = _ptr(bufs["recv_scales"], torch.float32, 4 * Na * nb, "recv_scales")
        out = _ptr(bufs["expert_out"], bf16, 2 * Na * H, "expert_out")
        y = _ptr(bufs["y"], bf16, 2 * T * H, "y")
        s = _stream(stream)                     # after the tensor checks
        calls = []
        if stages == "path":
            calls.append((lib.moe_route_topk, (c, _ptr(logits, torch.float32, 4 * T * E, "logits"), ids, w, s),
                          "moe_route_topk"))
        if gathered is not None:
            g = _ptr(gathered, None, ctx.P * T * rb, "gathered")
            g_sc = _ptr(gathered_scales, torch.float32, 4 * ctx.P * T * nb, "gathered_scales")
            calls.append((lib.moe_dispatch_allgather, (c, xp, ids, w, ws, ws_bytes, g, g_sc, recv, recv_sc, h, s),
                          "moe_dispatch_allgather"))
        elif direct:
            calls.append((lib.moe_dispatch_direct, (c, xp, ids, w, ws, ws_bytes, recv, recv_sc, h, s),
                          "moe_dispatch_direct"))
        else:
            send = _ptr(bufs["send"], None, Na * rb, "send_buf")
            send_sc = _ptr(bufs["send_scales"], torch.float32, 4 * Na * nb, "send_scales")
            calls.append((lib.moe_dispatch, (c, xp, ids, w, ws, ws_bytes, send, send_sc, recv, recv_sc, h, s),
                          "moe_dispatch"))
        if stages == "path":
            calls.append((lib.moe_expert_stub, (c, h, recv, recv_sc, out, s), "moe_expert_stub"))
        if direct:
            calls.append((lib.moe_combine_direct, (c, h, out, w, y, s), "moe_combine_direct"))
        else:
            comb = _ptr(bufs["comb"], bf16, 2 * Na * H, "comb_buf")
            calls.append((lib.moe_combine, (c, h, out, w, comb, y, s), "moe_combine"))
        self._calls = tuple(calls)

    def __call__(self) -> MoeHandle:
        if not self._ctx.handle_ptr:           # the cached calls hold the ctx pointer close() freed
            raise ValueError("PreparedPath: its Context has been closed")
        for fn, args, name in self._calls:
            status = fn(*args)
            if status != MOE_OK:
                raise MoeError(status, name)
        return self.handle


def _capturing(streams) -> bool:
    """Whether the current stream, or any of ``streams``, is capturing a graph."""
    import torch
    if torch.cuda.is_current_stream_capturing():
        return True
    for st in streams:
        with torch.cuda.stream(st):
            if torch.cuda.is_current_stream_capturing():
                return True
    return False


class OrderEvent:
    """A library event for ordering two streams of one device (moe_event_*): no timing, no system-scope fence."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check(lib.moe_event_create(ctypes.byref(h)), "moe_event_create")
        self.handle = h

    def record(self, stream=None):
        _check(lib.moe_event_record(self.handle, _stream(stream)), "moe_event_record")

    def wait(self, stream=None):
        """Work enqueued on stream from now on waits for this event's latest record."""
        _check(lib.moe_stream_wait_event(_stream(stream), self.handle), "moe_stream_wait_event")

    def __del__(self):
        if getattr(self, "handle", None) is not None and lib is not None:
            lib.moe_event_destroy(self.handle)
            self.handle = None


_order_events = {}   # per device, reused by run_overlapped: a wait refers to the record enqueued before it


def _order_event(device: int, i: int) -> OrderEvent:
    import torch
    pool = _order_events.setdefault(device, [])
    while len(pool) <= i:
        with torch.cuda.device(device):      # an event belongs to the device current at its creation
            pool.append(OrderEvent())
    return pool[i]


def run_overlapped(parts, comm_stream, compute_stream):
    """Micro-batches through the split phases on two streams.

    ``parts`` is a list of (ctx, bufs, x, logits), one independent problem per
    micro-batch.  Routing, both dispatch halves and both combine halves run on
    ``comm_stream``, the expert stage on ``compute_stream``; library events
    (OrderEvent: no timing, no system-scope fence) order each micro-batch's
    stages, so the expert stage of micro-batch i can overlap the dispatch of i+1
    and the combine of i-1 ([PPLX]: send and receive halves let other work run
    in between).  With one stream for both, stream order alone orders them and no
    event is recorded.  Only launches and events: the caller orders its own
    streams around the schedule and synchronises before reading the outputs.
    Returns the handles.

    Refuses graph capture (RuntimeError, before anything is enqueued): the schedule
    neither forks from nor joins back into a capturing origin stream, which a
    multi-stream capture needs, and the library's events refuse capturing streams."""
    if _capturing((comm_stream, compute_stream)):
        raise RuntimeError("run_overlapped: a stream is capturing a graph; the two-stream schedule is not built "
                           "for capture (it neither forks from nor joins the capturing stream)")
    handles = []
    two = comm_stream.cuda_stream != compute_stream.cuda_stream
    dev = comm_stream.device.index
    for i, (ctx, bufs, x, logits) in enumerate(parts):
        moe_route_topk(ctx, logits, bufs["topk_ids"], bufs["topk_w"], comm_stream)
        h = moe_dispatch_send(ctx, x, bufs["topk_ids"], bufs["topk_w"], bufs["workspace"], bufs["send"],
                              bufs["send_scales"], comm_stream)
        moe_dispatch_recv(ctx, h, bufs["send"], bufs["send_scales"], bufs["recv"], bufs["recv_scales"], comm_stream)
        handles.append(h)
        if two:
            _order_event(dev, 2 * i).record(comm_stream)             # micro-batch i dispatched
    for i, ((ctx, bufs, _, _), h) in enumerate(zip(parts, handles)):
        if two:
            _order_event(dev, 2 * i).wait(compute_stream)
        moe_expert_stub(ctx, h, bufs["recv"], bufs["recv_scales"], bufs["expert_out"], compute_stream)
        if two:
            _order_event(dev, 2 * i + 1).record(compute_stream)      # micro-batch i's expert stage done
    for i, ((ctx, bufs, _, _), h) in enumerate(zip(parts, handles)):
        if two:
            _order_event(dev, 2 * i + 1).wait(comm_stream)
        moe_combine_send(ctx, h, bufs["expert_out"], bufs["comb"], comm_stream)
        moe_combine_recv(ctx, h, bufs["comb"], bufs["topk_w"], bufs["y"], comm_stream)
    return handles
