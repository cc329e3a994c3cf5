"""Seeded synthetic inputs for the MoE expert-parallel dispatch/combine path.

This module only draws numbers: it holds none of the method's arithmetic (no
softmax, no routing, no counting, no quantisation).  Both the HIP path and the
CPU oracle are fed from it, and nothing else is shared between them.

Generator (stated so it can be re-implemented anywhere):

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014), used counter-style: output ``i`` of the stream
  seeded with ``s`` is ``mix(s + (i + 1) * 0x9E3779B97F4A7C15)``.
* Each tensor has its own stream: ``stream_seed(seed, n)`` is output ``n`` of
  the SplitMix64 stream seeded with the workload seed.
* Uniforms ``u = ((z >> 11) + 1) * 2**-53`` lie in (0, 1].
* Normals by Box-Muller in float64 on consecutive pairs:
  ``n[2m] = r cos(2 pi u[2m+1])``, ``n[2m+1] = r sin(2 pi u[2m+1])`` with
  ``r = sqrt(-2 ln u[2m])``.
* Hidden states: float64 normal -> float32 -> bfloat16 (round to nearest even),
  returned as the raw uint16 bit patterns.
* Router logits: float64 normal (+ optional per-expert bias) -> float32.
* Skewed routing: a seeded permutation ``rank(e)`` of the experts (argsort of
  SplitMix64 keys) and the bias ``b_e = -0.4 * ln(1 + rank(e))``: a Zipf
  log-prior of exponent 1.2 applied at one third strength, which sends about
  45% of all top-8 assignments to the hottest 10% of 256 experts.

The five workloads mirror the shapes of the pages: a small 4-rank group, a
decode-sized batch on a DeepSeek-like layer (E=256, top-8, H=7168), the 2048
token / top-2 / H=7168 byte-model example of the expert-parallel page, a
Mixtral-like prefill (E=8, top-2) and a skewed DeepSeek-like prefill.
"""

from __future__ import annotations

import dataclasses

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

STREAM_X = 1
STREAM_LOGITS = 2
STREAM_PERM = 3

BF16 = "bf16"
FP8 = "fp8_e4m3"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_ranks: int  # P, logical expert-parallel ranks
    tokens: int  # T, tokens over all ranks (T / P per rank, blocked)
    num_experts: int  # E (E / P per rank, contiguous)
    top_k: int
    hidden: int  # H
    dispatch_dtype: str  # BF16 or FP8
    seed: int
    zipf: bool = False

    @property
    def tokens_per_rank(self) -> int:
        return self.tokens // self.num_ranks

    @property
    def assignments(self) -> int:
        return self.tokens * self.top_k

    def describe(self) -> str:
        return (f"{self.name}: P={self.num_ranks} T={self.tokens} E={self.num_experts} "
                f"k={self.top_k} H={self.hidden} dispatch={self.dispatch_dtype}"
                + (" zipf" if self.zipf else ""))


WORKLOADS = {
    "c1": Workload("c1-tiny-ep4", 4, 256, 8, 2, 256, BF16, 0x5EED0001),
    "c2": Workload("c2-decode-ep8-e256-top8-h7168", 8, 128, 256, 8, 7168, BF16, 0x5EED0002),
    "c3": Workload("c3-bytemodel-ep8-t2048-e64-top2-h7168-fp8", 8, 2048, 64, 2, 7168, FP8, 0x5EED0003),
    "c4": Workload("c4-prefill-ep8-t16384-e8-top2-h4096", 8, 16384, 8, 2, 4096, BF16, 0x5EED0004),
    "c5": Workload("c5-skewed-ep32-t8192-e256-top8-h7168-fp8", 32, 8192, 256, 8, 7168, FP8, 0x5EED0005,
                   zipf=True),
}


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs ``start .. start+count-1`` of the SplitMix64 stream seeded with ``seed``."""
    with np.errstate(over="ignore"):
        idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        return _mix(np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + idx * GOLDEN)


def stream_seed(seed: int, stream: int) -> int:
    return int(splitmix64(seed, stream, 1)[0])


def _i64(v: int) -> int:
    """The int64 with the same 64 bits as the unsigned value v."""
    v &= 0xFFFFFFFFFFFFFFFF
    return v - (1 << 64) if v >= (1 << 63) else v


def _splitmix64_torch(seed: int, start: int, count: int):
    """Same outputs as ``splitmix64`` as int64 bit patterns, on torch's multithreaded CPU ops
    (wrapping int64 products keep the low 64 bits; logical shifts are arithmetic shifts
    masked to the bits a logical shift keeps)."""
    import torch
    idx = torch.arange(start + 1, start + count + 1, dtype=torch.int64)
    z = idx * _i64(int(GOLDEN)) + _i64(seed)
    for sh, mul in ((30, _i64(int(_M1))), (27, _i64(int(_M2))), (31, None)):
        z = z ^ ((z >> sh) & ((1 << (64 - sh)) - 1))
        if mul is not None:
            z = z * mul
    return z


def normals(seed: int, count: int, chunk: int = 1 << 24) -> np.ndarray:
    """``count`` standard normals (float64) by Box-Muller over consecutive uniform pairs."""
    import torch
    out = np.empty(count, dtype=np.float64)
    pairs = (count + 1) // 2
    done = 0
    while done < pairs:
        m = min(chunk, pairs - done)
        z = _splitmix64_torch(seed, 2 * done, 2 * m)
        u = (((z >> 11) & ((1 << 53) - 1)).to(torch.float64) + 1.0) * (2.0 ** -53)
        u = u.view(m, 2)
        r = torch.sqrt(-2.0 * torch.log(u[:, 0]))
        th = (2.0 * np.pi) * u[:, 1]
        zz = torch.stack((r * torch.cos(th), r * torch.sin(th)), dim=1).reshape(-1).numpy()
        lo = 2 * done
        hi = min(count, lo + 2 * m)
        out[lo:hi] = zz[: hi - lo]
        done += m
    return out


def uniforms(seed: int, start: int, count: int) -> np.ndarray:
    z = splitmix64(seed, start, count)
    return ((z >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)


def float32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_bits_to_float32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def expert_bias(seed: int, num_experts: int) -> np.ndarray:
    """Zipf log-prior per expert: ``-0.4 * ln(1 + rank(e))`` with a seeded rank permutation."""
    keys = splitmix64(stream_seed(seed, STREAM_PERM), 0, num_experts)
    order = np.argsort(keys, kind="stable")
    rank = np.empty(num_experts, dtype=np.int64)
    rank[order] = np.arange(num_experts)
    return -0.4 * np.log1p(rank.astype(np.float64))


def make_hidden(seed: int, tokens: int, hidden: int) -> np.ndarray:
    """bfloat16 hidden states ``[tokens, hidden]`` ~ N(0, 1), as uint16 bit patterns."""
    import torch
    z = torch.from_numpy(normals(stream_seed(seed, STREAM_X), tokens * hidden)).to(torch.float32)
    return z.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).reshape(tokens, hidden)


def make_logits(seed: int, tokens: int, num_experts: int, zipf: bool = False) -> np.ndarray:
    """float32 router logits ``[tokens, num_experts]`` ~ N(0, 1) (+ Zipf bias if asked)."""
    z = normals(stream_seed(seed, STREAM_LOGITS), tokens * num_experts).reshape(tokens, num_experts)
    if zipf:
        z = z + expert_bias(seed, num_experts)[None, :]
    return z.astype(np.float32)


def make_inputs(w: Workload) -> dict:
    return {
        "x": make_hidden(w.seed, w.tokens, w.hidden),
        "logits": make_logits(w.seed, w.tokens, w.num_experts, w.zipf),
    }


def custom(name: str, P: int, T: int, E: int, k: int, H: int, dtype: str = BF16,
           seed: int = 1, zipf: bool = False) -> Workload:
    if T % P:
        raise ValueError("T must be a multiple of P (tokens are blocked over ranks)")
    return Workload(name, P, T, E, k, H, dtype, seed, zipf)


def micro_batch_rows(num_ranks: int, tokens_per_rank: int, parts: int, index: int) -> np.ndarray:
    """Rows of the rank-blocked token matrix that form micro-batch ``index`` of
    ``parts``: on every rank, its local tokens [index*Tp/parts, (index+1)*Tp/parts),
    so each micro-batch is again rank-blocked with Tp/parts tokens per rank."""
    assert tokens_per_rank % parts == 0 and 0 <= index < parts
    n = tokens_per_rank // parts
    local = np.arange(index * n, (index + 1) * n)
    return (np.arange(num_ranks)[:, None] * tokens_per_rank + local[None, :]).reshape(-1)
