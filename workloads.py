"""Seeded synthetic workloads for block-sparse attention.

This module holds no part of the method's arithmetic: only the workload table,
the random draws, and the bf16 round-to-nearest-even of those draws (the input
precision).  Both the HIP path and the CPU oracle read the arrays made here,
and nothing else is shared between them.

Recipe (the same for every workload; all batch = 1):
  rng = numpy.random.default_rng(seed)          # PCG64
  q = rng.standard_normal([b, h, n, d], float32)
  k = rng.standard_normal([b, h, n, d], float32)
  v = rng.standard_normal([b, h, n, d], float32)
  if key_offsets:                               # separates block scores
      off = rng.normal(0, 0.5, [b, h, n/B, d]) -> float32
      k += off repeated over the B keys of each block   (in float32)
  if dtype == bf16: round q, k, v to bf16, nearest-even
Backward workloads add an incoming gradient of the float32 output:
  dout = default_rng(seed + 1000).standard_normal([b, h, n, d], float32)
A batch of sequences of different lengths draws sequence i by the same recipe
with n = lengths[i] and seed + i (its key blocks, and offsets, start at its own
first row) and lays the batch out [heads, total, d]: each head's rows of all
sequences one after the other.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    n: int
    d: int
    dtype: str            # "fp32" or "bf16"
    seed: int
    block: int = 64
    topk: int = 0         # 0 for the static pattern
    causal: bool = False
    key_offsets: bool = False
    window: int = -1      # static pattern only
    stride: int = 0       # static pattern only
    description: str = field(default="", compare=False)

    @property
    def static(self) -> bool:
        return self.topk == 0

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    @property
    def bh(self) -> int:
        return self.batch * self.heads

    @property
    def nb(self) -> int:
        return -(-self.n // self.block)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32_n1k", 1, 1, 1024, 64, "fp32", seed=0, topk=4,
                 description="dynamic, fp32 N(0,1), h=1 N=1024 D=64 B=64 k=4, non-causal"),
        Workload("dyn_bf16_n4k", 1, 8, 4096, 64, "bf16", seed=1, topk=16, key_offsets=True,
                 description="dynamic, bf16 N(0,1) + per-block key offsets N(0,0.5^2), "
                             "h=8 N=4096 D=64 B=64 k=16, non-causal"),
        Workload("dyn_bf16_n32k", 1, 8, 32768, 64, "bf16", seed=2, topk=16, key_offsets=True,
                 description="dynamic, bf16 N(0,1) + per-block key offsets N(0,0.5^2), "
                             "h=8 N=32768 D=64 B=64 k=16, non-causal"),
        Workload("static_fp32_n8k", 1, 1, 8192, 64, "fp32", seed=3, window=32, stride=512,
                 description="static window+stride, fp32 N(0,1), h=1 N=8192 D=64, "
                             "|i-j|<=32 or j%512==0, 64x64 tiles"),
        Workload("causal_bf16_n128k", 1, 8, 131072, 128, "bf16", seed=4, topk=32, causal=True,
                 key_offsets=True,
                 description="dynamic causal, bf16 N(0,1) + per-block key offsets N(0,0.5^2), "
                             "h=8 N=131072 D=128 B=64 k=32"),
    ]
}

HEADLINE = "dyn_bf16_n32k"
SMALL = "tiny_fp32_n1k"


def bf16_round(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Round float32 to bf16, nearest-even.  Returns (float32 values, uint16 bits)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    bits = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    vals = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return vals, bits


@dataclass
class Inputs:
    """q, k, v as float32 arrays [b, h, n, d] holding the exact input values;
    for bf16 workloads also the uint16 bit patterns handed to the device."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_bits: np.ndarray | None = None
    k_bits: np.ndarray | None = None
    v_bits: np.ndarray | None = None


def generate(w: Workload | str, *, n: int | None = None, heads: int | None = None,
             batch: int | None = None, seed: int | None = None) -> Inputs:
    """Draw the inputs of a workload (optionally at another size or seed)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    b = batch if batch is not None else w.batch
    h = heads if heads is not None else w.heads
    nn = n if n is not None else w.n
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shape = (b, h, nn, w.d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if w.key_offsets:
        nb = -(-nn // w.block)
        off = rng.normal(0.0, 0.5, size=(b, h, nb, w.d)).astype(np.float32)
        k += np.repeat(off, w.block, axis=2)[:, :, :nn, :]
    if w.dtype == "bf16":
        q, qb = bf16_round(q)
        k, kb = bf16_round(k)
        v, vb = bf16_round(v)
        return Inputs(q, k, v, qb, kb, vb)
    return Inputs(q, k, v)


def grad_output(shape, seed: int) -> np.ndarray:
    """The incoming gradient dout for a backward workload: float32 N(0, 1)."""
    rng = np.random.default_rng(seed + 1000)
    return rng.standard_normal(tuple(shape), dtype=np.float32)


def generate_varlen(w: Workload | str, lengths, *, heads: int | None = None,
                    seed: int | None = None) -> tuple[Inputs, np.ndarray]:
    """A batch of sequences of the given lengths (see the module docstring).
    Returns (inputs as [1, heads, total, d] arrays, cu_seqlens int32)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    s0 = w.seed if seed is None else seed
    parts = [generate(w, n=int(n), heads=heads, batch=1, seed=s0 + i) for i, n in enumerate(lengths)]
    cat = lambda name: (None if getattr(parts[0], name) is None
                        else np.ascontiguousarray(np.concatenate([getattr(p, name) for p in parts], axis=2)))
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return Inputs(cat("q"), cat("k"), cat("v"), cat("q_bits"), cat("k_bits"), cat("v_bits")), cu
