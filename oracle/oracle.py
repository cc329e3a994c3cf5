"""ctypes front end of the CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares nothing
with the HIP library; arrays are plain numpy.

Layouts (identical on both sides by definition, see the C file):
  ids int32[T, k], w float32[T, k]; rows uint8[N_a, row_bytes] (bf16 bit
  patterns or e4m3 codes); scales float32[N_a, H/128]; meta 16-byte records
  (int32 src_rank, int32 src_token, int16 slot, int16 local_expert,
  float32 weight); expert_out / comb uint16[N_a, H]; y uint16[T, H].
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")

META_DTYPE = np.dtype([("src_rank", "<i4"), ("src_token", "<i4"), ("slot", "<i2"),
                       ("local_expert", "<i2"), ("weight", "<f4")])
assert META_DTYPE.itemsize == 16

FP8_BLOCK = 128


class _Shape(ctypes.Structure):
    _fields_ = [("P", ctypes.c_int64), ("T", ctypes.c_int64), ("E", ctypes.c_int64),
                ("k", ctypes.c_int64), ("H", ctypes.c_int64), ("fp8", ctypes.c_int64)]


class _DispatchOut(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "n", "N", "C", "expert_off", "rank_recv_off", "send_off", "recv_off",
        "send_pos", "recv_pos", "send_rows", "send_scales", "send_meta",
        "recv_rows", "recv_scales", "recv_meta")]


def build() -> str:
    subprocess.run(["make", "-s", "-C", _HERE], check=True)
    return _LIB_PATH


_lib = None


def use_library(path: str):
    """Load the oracle from another build of moe_oracle.c (the mutation tests use it)."""
    global _lib, _LIB_PATH
    _LIB_PATH = path
    _lib = None
    return lib()


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = ctypes.CDLL(_LIB_PATH)
        _lib.oracle_bf16_from_double.restype = ctypes.c_uint16
        _lib.oracle_bf16_from_double.argtypes = [ctypes.c_double]
        _lib.oracle_e4m3_from_double.restype = ctypes.c_uint8
        _lib.oracle_e4m3_from_double.argtypes = [ctypes.c_double]
        _lib.oracle_e4m3_to_f32.restype = ctypes.c_float
        _lib.oracle_e4m3_to_f32.argtypes = [ctypes.c_uint8]
        _lib.oracle_bf16_to_f32.restype = ctypes.c_float
        _lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        _lib.oracle_meta_bytes.restype = ctypes.c_int64
        _lib.oracle_row_bytes.restype = ctypes.c_int64
        assert _lib.oracle_meta_bytes() == 16
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


class Shape:
    def __init__(self, P: int, T: int, E: int, k: int, H: int, fp8: bool):
        if P < 1 or T % P or E % P or not (1 <= k <= E):
            raise ValueError("bad shape")
        if fp8 and H % FP8_BLOCK:
            raise ValueError("FP8 dispatch needs H % 128 == 0")
        self.P, self.T, self.E, self.k, self.H, self.fp8 = P, T, E, k, H, bool(fp8)

    @classmethod
    def of(cls, w) -> "Shape":
        return cls(w.num_ranks, w.tokens, w.num_experts, w.top_k, w.hidden, w.dispatch_dtype != "bf16")

    @property
    def Na(self) -> int:
        return self.T * self.k

    @property
    def row_bytes(self) -> int:
        return self.H if self.fp8 else 2 * self.H

    def c(self) -> _Shape:
        return _Shape(self.P, self.T, self.E, self.k, self.H, int(self.fp8))


# ---------------------------------------------------------------------------
# formats
# ---------------------------------------------------------------------------

def bf16_from_double(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_bf16_from_double_array(ctypes.c_int64(v.size), _p(v), _p(out))
    return out


def e4m3_from_double(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().oracle_e4m3_from_double_array(ctypes.c_int64(v.size), _p(v), _p(out))
    return out


def e4m3_to_f32(c) -> np.ndarray:
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float32)
    lib().oracle_e4m3_to_f32_array(ctypes.c_int64(c.size), _p(c), _p(out))
    return out


def bf16_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# the path
# ---------------------------------------------------------------------------

def route(shape: Shape, logits: np.ndarray):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    assert logits.shape == (shape.T, shape.E)
    ids = np.empty((shape.T, shape.k), dtype=np.int32)
    w = np.empty((shape.T, shape.k), dtype=np.float32)
    s = shape.c()
    lib().oracle_route(ctypes.byref(s), _p(logits), _p(ids), _p(w))
    return ids, w


def quantize_row(H: int, x_row: np.ndarray):
    x_row = np.ascontiguousarray(x_row, dtype=np.uint16)
    q = np.empty(H, dtype=np.uint8)
    sc = np.empty(H // FP8_BLOCK, dtype=np.float32)
    lib().oracle_quantize_row(ctypes.c_int64(H), _p(x_row), _p(q), _p(sc))
    return q, sc


def dispatch(shape: Shape, x: np.ndarray, ids: np.ndarray, w: np.ndarray, payload: bool = True) -> dict:
    P, T, E, k, H, Na = shape.P, shape.T, shape.E, shape.k, shape.H, shape.Na
    x = np.ascontiguousarray(x, dtype=np.uint16)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    assert x.shape == (T, H) and ids.shape == (T, k) and w.shape == (T, k)
    if ids.size and (ids.min() < 0 or ids.max() >= E):
        raise ValueError("expert id out of range")
    nb = H // FP8_BLOCK
    o = {
        "n": np.empty((P, E), np.int32), "N": np.empty(E, np.int32), "C": np.empty((P, P), np.int32),
        "expert_off": np.empty(E + 1, np.int32), "rank_recv_off": np.empty(P + 1, np.int32),
        "send_off": np.empty((P, E), np.int32), "recv_off": np.empty((E, P), np.int32),
        "send_pos": np.empty((T, k), np.int32), "recv_pos": np.empty((T, k), np.int32),
        "send_meta": np.zeros(Na, META_DTYPE), "recv_meta": np.zeros(Na, META_DTYPE),
        "send_rows": None, "recv_rows": None, "send_scales": None, "recv_scales": None,
    }
    if payload:
        o["send_rows"] = np.zeros((Na, shape.row_bytes), np.uint8)
        o["recv_rows"] = np.zeros((Na, shape.row_bytes), np.uint8)
        if shape.fp8:
            o["send_scales"] = np.zeros((Na, nb), np.float32)
            o["recv_scales"] = np.zeros((Na, nb), np.float32)
    d = _DispatchOut(*[_p(o[name]) for name, _ in _DispatchOut._fields_])
    s = shape.c()
    lib().oracle_dispatch(ctypes.byref(s), _p(x), _p(ids), _p(w), ctypes.byref(d))
    return o


def stub(shape: Shape, expert_off: np.ndarray, recv_rows: np.ndarray, recv_scales: np.ndarray | None):
    out = np.empty((shape.Na, shape.H), dtype=np.uint16)
    s = shape.c()
    expert_off = np.ascontiguousarray(expert_off, dtype=np.int32)
    lib().oracle_stub(ctypes.byref(s), _p(expert_off), _p(np.ascontiguousarray(recv_rows)),
                      _p(None if recv_scales is None else np.ascontiguousarray(recv_scales)), _p(out))
    return out


def stub_row(shape: Shape, e: int, row: np.ndarray, scales: np.ndarray | None) -> np.ndarray:
    out = np.empty(shape.H, dtype=np.uint16)
    s = shape.c()
    lib().oracle_stub_row(ctypes.byref(s), ctypes.c_int64(e), _p(np.ascontiguousarray(row)),
                          _p(None if scales is None else np.ascontiguousarray(scales, dtype=np.float32)),
                          _p(out))
    return out


def combine(shape: Shape, recv_meta: np.ndarray, expert_out: np.ndarray, w: np.ndarray) -> dict:
    T, H, Na = shape.T, shape.H, shape.Na
    comb = np.zeros((Na, H), np.uint16)
    y32 = np.empty((T, H), np.float32)
    y = np.empty((T, H), np.uint16)
    y64 = np.empty((T, H), np.float64)
    s = shape.c()
    lib().oracle_combine(ctypes.byref(s), _p(np.ascontiguousarray(recv_meta)),
                         _p(np.ascontiguousarray(expert_out, dtype=np.uint16)),
                         _p(np.ascontiguousarray(w, dtype=np.float32)), _p(comb), _p(y32), _p(y), _p(y64))
    return {"comb": comb, "y32": y32, "y": y, "y64": y64}


def reduce_tokens(shape: Shape, tokens, comb: np.ndarray, w: np.ndarray) -> dict:
    """Weighted reduction of selected tokens only (for sampled checks at full size).

    ``comb`` holds the combine rows of those tokens, shaped [len(tokens), k, H]."""
    tokens = np.asarray(tokens, dtype=np.int64)
    n, k, H = len(tokens), shape.k, shape.H
    sub = Shape(1, n, shape.k, shape.k, H, False)  # reduction only reads T, k, H
    comb = np.ascontiguousarray(comb, dtype=np.uint16).reshape(n * k, H)
    wsub = np.ascontiguousarray(np.asarray(w, dtype=np.float32).reshape(-1, k)[tokens])
    y32 = np.empty((n, H), np.float32)
    y = np.empty((n, H), np.uint16)
    y64 = np.empty((n, H), np.float64)
    s = sub.c()
    for r in range(n):
        lib().oracle_reduce_token(ctypes.byref(s), ctypes.c_int64(r), _p(comb), _p(wsub), _p(y32), _p(y), _p(y64))
    return {"y32": y32, "y": y, "y64": y64}


def run(shape: Shape, x: np.ndarray, logits: np.ndarray | None = None, ids=None, w=None) -> dict:
    """The whole path on the CPU: route (unless ids/w are given), dispatch, stub, combine."""
    if ids is None:
        ids, w = route(shape, logits)
    d = dispatch(shape, x, ids, w, payload=True)
    out = stub(shape, d["expert_off"], d["recv_rows"], d["recv_scales"])
    c = combine(shape, d["recv_meta"], out, w)
    d.update(ids=ids, w=w, expert_out=out, **c)
    return d
