"""Seeded synthetic inputs for the attention forward, shared by tests and bench.

This module holds no attention arithmetic: it draws normal variates, rounds
them to the storage type and names the workloads.  Both the CPU oracle and the
HIP path receive what it produces.

Every [L, D] slab of q, k or v for one (batch, head) has its own PCG64 stream
seeded by ``SeedSequence([*seed_words, tensor_id, b, h])`` (tensor ids q=0,
k=1, v=2, and do=3 for the upstream gradient of O fed to the backward), so any slab can be regenerated alone and slabs can be drawn in
parallel threads with identical results.  Values are ``standard_normal`` in
float32, optionally multiplied by a power of two per head (exact, so it
commutes with rounding), then rounded to nearest-even into the storage type.

The random q, k, v follow the numerical check of the quidproquo.cc guide
("Back to real models" section: random q, k, v with B=4, H=8, L=256, D=64)
and its length sweep (64 to 4096).
"""

from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3}
DTYPES = ("f32", "f16", "bf16")
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to ``dtype`` storage bits (nearest-even).

    Returns float32 for "f32" and uint16 bit patterns for "f16" / "bf16".
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32)
        if not np.all(np.isfinite(x)):
            raise ValueError("bf16 rounding here covers finite values only")
        bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        return ((u + bias) >> np.uint32(16)).astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_float32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 values of storage bits produced by ``round_to``."""
    if dtype == "f32":
        return np.asarray(bits, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def slab(seed_words: Sequence[int], tensor: str, b: int, h: int, L: int, D: int,
         dtype: str, mult: float = 1.0) -> np.ndarray:
    """Storage bits of one [L, D] slab of tensor ``tensor`` for (b, h)."""
    ss = np.random.SeedSequence([*seed_words, TENSOR_IDS[tensor], b, h])
    g = np.random.Generator(np.random.PCG64(ss))
    x = g.standard_normal((L, D), dtype=np.float32)
    if mult != 1.0:
        m, e = math.frexp(mult)
        if m != 0.5:
            raise ValueError("per-head multipliers must be powers of two")
        x *= np.float32(mult)
    return round_to(x, dtype)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention forward problem and the seed of its inputs."""

    name: str
    B: int
    H: int
    Lq: int
    Lk: int
    D: int
    dtype: str
    causal: bool
    seed_words: Tuple[int, ...]
    q_head_mult: Tuple[Tuple[int, float], ...] = ()

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def q_mult(self, h: int) -> float:
        return dict(self.q_head_mult).get(h, 1.0)

    def shape(self, tensor: str) -> Tuple[int, int, int, int]:
        L = self.Lq if tensor in ("q", "do") else self.Lk
        return (self.B, self.H, L, self.D)

    def flops(self) -> float:
        """4 D flops per (query, key) pair, halved for causal masking."""
        f = 4.0 * self.B * self.H * self.Lq * self.Lk * self.D
        return f / 2 if self.causal else f

    def kv_bytes(self) -> int:
        return 2 * self.B * self.H * self.Lk * self.D * ELEM_BYTES[self.dtype]


def _wl(name, B, H, Lq, Lk, D, dtype, causal, seed_words, q_head_mult=()):
    return Workload(name, B, H, Lq, Lk, D, dtype, causal, tuple(seed_words), tuple(q_head_mult))


SWEEP_LENGTHS = (64, 128, 256, 512, 1024, 2048, 4096)

#: The five workloads: the fp32 numerical check, the fp16 length sweep, the
#: causal bf16 prefill with x8 queries on heads 0-3 (row maxima jump late, so
#: the rescale path runs), the split-KV decode and the long-context prefill.
WORKLOADS: Dict[str, Workload] = {
    "check_f32": _wl("check_f32", 4, 8, 256, 256, 64, "f32", False, (1,)),
    **{f"sweep_f16_L{L}": _wl(f"sweep_f16_L{L}", 4, 8, L, L, 64, "f16", False, (2, L))
       for L in SWEEP_LENGTHS},
    "causal_bf16_8k": _wl("causal_bf16_8k", 1, 32, 8192, 8192, 128, "bf16", True, (3,),
                          tuple((h, 8.0) for h in range(4))),
    "decode_bf16_32k": _wl("decode_bf16_32k", 16, 32, 1, 32768, 128, "bf16", False, (4,)),
    "long_causal_bf16_64k": _wl("long_causal_bf16_64k", 1, 8, 65536, 65536, 128, "bf16", True, (5,)),
}


def custom(name: str, B: int, H: int, Lq: int, Lk: int, D: int, dtype: str,
           causal: bool, seed: int, q_head_mult=()) -> Workload:
    """A workload outside the named five (edge shapes in tests)."""
    return _wl(name, B, H, Lq, Lk, D, dtype, causal, (1000 + seed, Lq, Lk, D), q_head_mult)


def generate(wl: Workload, tensors: Sequence[str] = ("q", "k", "v"),
             threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Storage bits of whole [B, H, L, D] tensors, drawn slab by slab."""
    threads = threads or min(16, os.cpu_count() or 1)
    out = {}
    for t in tensors:
        B, H, L, D = wl.shape(t)
        st = np.float32 if wl.dtype == "f32" else np.uint16
        arr = np.empty((B, H, L, D), dtype=st)

        def fill(bh, t=t, arr=arr, L=L, D=D, H=H):
            b, h = divmod(bh, H)
            mult = wl.q_mult(h) if t == "q" else 1.0
            arr[b, h] = slab(wl.seed_words, t, b, h, L, D, wl.dtype, mult)

        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(B * H)))
        out[t] = arr
    return out


def slab_values(wl: Workload, tensor: str, b: int, h: int) -> np.ndarray:
    """Exact float32 values of one slab (regenerated from its seed)."""
    B, H, L, D = wl.shape(tensor)
    mult = wl.q_mult(h) if tensor == "q" else 1.0
    return to_float32(slab(wl.seed_words, tensor, b, h, L, D, wl.dtype, mult), wl.dtype)


def sample_rows(wl: Workload, h: int, n: int = 256) -> np.ndarray:
    """Sorted query rows checked per head where the full output is too big.

    Rows 0 and Lq-1 are always present; the other n-2 are drawn without
    replacement from 1..Lq-2 by ``SeedSequence([seed_words[0], 1, h])``.
    """
    L = wl.Lq
    if L <= n:
        return np.arange(L)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed_words[0], 1, h])))
    mid = g.choice(np.arange(1, L - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, L - 1], mid])).astype(np.int64)


def ragged_lengths(seed: int, B: int, Lk_max: int, lo: int = 1) -> np.ndarray:
    """Per-sequence KV-cache lengths for ragged decode: B int32 values drawn
    uniformly from [lo, Lk_max] by ``SeedSequence([seed, 3])``."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 3])))
    return rng.integers(lo, Lk_max + 1, size=B, dtype=np.int64).astype(np.int32)


def bool_mask(seed: int, shape: Sequence[int], keep: float = 0.6, empty_rows: int = 0) -> np.ndarray:
    """uint8 mask of ``shape`` ([Bm, Hm, Lq, Lk]): each entry 1 with
    probability ``keep`` (``SeedSequence([seed, 6])``); the first
    ``empty_rows`` query rows of slab (0, 0) are all zero."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 6])))
    m = (rng.random(tuple(shape)) < keep).astype(np.uint8)
    m[0, 0, :empty_rows] = 0
    return m


def additive_mask(seed: int, shape: Sequence[int], sigma: float = 2.0, neg_inf: float = 0.1) -> np.ndarray:
    """float32 mask of ``shape``: N(0, sigma^2) entries, a fraction
    ``neg_inf`` of them -inf (``SeedSequence([seed, 7])``)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    m = (rng.standard_normal(tuple(shape)) * sigma).astype(np.float32)
    m[rng.random(tuple(shape)) < neg_inf] = -np.inf
    return m



def rising_scores(seed: int, B: int, H: int, Lq: int, Lk: int, D: int,
                  span: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """float32 q, k, v ([B, H, L, D]) whose scores q_i . k_j move steadily
    along the keys: q_i = a u + e_i and k_j = t_j a u + e'_j with u a random
    unit vector per (b, h), a = sqrt(span), e, e' of standard deviation 0.1
    per component, and t_j = j / (Lk - 1) for even heads (scores rising by
    about ``span`` over a row) or 1 - j / (Lk - 1) for odd heads (the first
    keys dominate).  v is standard normal.  ``SeedSequence([seed, 8])``."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 8])))
    u = rng.standard_normal((B, H, 1, D))
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    a = math.sqrt(span)
    t = np.arange(Lk, dtype=np.float64) / max(1, Lk - 1)
    t = np.where((np.arange(H) % 2 == 0)[None, :, None], t[None, None, :], 1.0 - t[None, None, :])
    q = a * u + 0.1 * rng.standard_normal((B, H, Lq, D))
    k = t[..., None] * a * u + 0.1 * rng.standard_normal((B, H, Lk, D))
    v = rng.standard_normal((B, H, Lk, D))
    return q.astype(np.float32), k.astype(np.float32), v.astype(np.float32)
