"""Seeded synthetic rank buffers for the quantized-reduce workloads.

This module draws random numbers and converts them to the storage type; it
holds none of the method's arithmetic (no scale, code, sum or rounding rule of
the quantizer).  Both the library's tests and the CPU oracle's tests take
their inputs from here, so it imports neither of them.

Recipe (one ``numpy.random.default_rng(seed)`` per workload; ranks are drawn
one after another, r = 0..N-1, each in the order base values -> multipliers
-> outlier positions -> outlier values; draws are float64, cast to float32
with round-to-nearest-even, then to bfloat16 with round-to-nearest-even
unless the workload is float32):

  tiny        N=4,  4,096 bf16 ~ Normal(0, 1)                      block 128
  outliers    N=8,  16,777,216 bf16 ~ Normal(0, 1); n//1000 positions per
              rank (drawn without replacement) replaced by Normal(0,1)*50
                                                                   block 256
  prefill     N=8,  [8192, 5376] bf16 ~ Laplace(0, 0.5) times a per-row
              LogNormal(0, 1) multiplier                           block 256
  ring        N=4,  [2048, 3840] bf16 ~ Laplace(0, 0.5); n//2000 positions
              per rank multiplied by 100                           block 256
  smallblock  N=16, 67,108,864 fp32 ~ Normal(0, 1e-3) times a per-64-element
              LogNormal(0, 2) multiplier                           block 64

The hidden widths 5376 and 3840 are those of the public Gemma 3 27B and 12B
model configurations, the two models whose prefill the EQuARX abstract
reports; the value distributions stand in for prefill activations.
Smaller instances of a recipe (fewer elements or rows, same distribution)
serve as parity cases.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Iterator

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    seed: int
    nranks: int
    shape: tuple            # per-rank shape: (n,) or (rows, hidden)
    dtype: str              # "bf16" or "f32"
    block: int
    description: str

    @property
    def n(self) -> int:
        return int(np.prod(self.shape))

    def resized(self, *, n: int | None = None, rows: int | None = None,
                nranks: int | None = None) -> "Workload":
        """The same recipe at a smaller size (parity cases)."""
        shape = self.shape
        if n is not None:
            if len(shape) != 1:
                raise ValueError("2-D workloads resize by rows")
            shape = (int(n),)
        if rows is not None:
            if len(shape) != 2:
                raise ValueError("1-D workloads resize by n")
            shape = (int(rows), shape[1])
        return dataclasses.replace(self, shape=shape,
                                   nranks=self.nranks if nranks is None else int(nranks))


WORKLOADS = {
    "tiny": Workload("tiny", 0, 4, (4096,), "bf16", 128,
                     "N=4 x 4,096 bf16 ~ N(0,1), block 128"),
    "outliers": Workload("outliers", 1, 8, (16_777_216,), "bf16", 256,
                         "N=8 x 16,777,216 bf16 ~ N(0,1) with 0.1% N(0,1)*50 outliers, block 256"),
    "prefill": Workload("prefill", 2, 8, (8192, 5376), "bf16", 256,
                        "N=8 x [8192, 5376] bf16 ~ Laplace(0,0.5) x per-row LogNormal(0,1), block 256"),
    "ring": Workload("ring", 3, 4, (2048, 3840), "bf16", 256,
                     "N=4 x [2048, 3840] bf16 ~ Laplace(0,0.5), 0.05% outliers x100, block 256"),
    "smallblock": Workload("smallblock", 4, 16, (67_108_864,), "f32", 64,
                           "N=16 x 67,108,864 fp32 ~ N(0,1e-3) x per-block LogNormal(0,2), block 64"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even,
    done by torch's CPU conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32).reshape(-1))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _draw_rank(w: Workload, rng: np.random.Generator) -> np.ndarray:
    n = w.n
    if w.key == "tiny":
        v = rng.normal(0.0, 1.0, n)
    elif w.key == "outliers":
        v = rng.normal(0.0, 1.0, n)
        k = n // 1000
        pos = rng.choice(n, k, replace=False)
        v[pos] = rng.normal(0.0, 1.0, k) * 50.0
    elif w.key == "prefill":
        rows, hidden = w.shape
        v = rng.laplace(0.0, 0.5, (rows, hidden))
        v *= rng.lognormal(0.0, 1.0, rows)[:, None]
    elif w.key == "ring":
        v = rng.laplace(0.0, 0.5, n)
        k = n // 2000
        pos = rng.choice(n, k, replace=False)
        v[pos] *= 100.0
    elif w.key == "smallblock":
        if n % 64:
            raise ValueError("smallblock needs n % 64 == 0")
        v = rng.normal(0.0, 1e-3, n)
        v *= np.repeat(rng.lognormal(0.0, 2.0, n // 64), 64)
    else:
        raise KeyError(w.key)
    v32 = np.asarray(v, np.float64).reshape(-1).astype(np.float32)
    if w.dtype == "bf16":
        return f32_to_bf16_bits(v32)
    return v32


def iter_ranks(w: Workload) -> Iterator[np.ndarray]:
    """Rank buffers r = 0..N-1 in draw order (1-D: bf16 as uint16 patterns,
    or float32)."""
    rng = np.random.default_rng(w.seed)
    for _ in range(w.nranks):
        yield _draw_rank(w, rng)


def ranks(w: Workload) -> list[np.ndarray]:
    return list(iter_ranks(w))


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def uniform_bf16(seed: int, nranks: int, n: int, scale: float = 1.0) -> list[np.ndarray]:
    """Generic parity input: N bf16 buffers ~ Normal(0, scale)."""
    rng = np.random.default_rng(seed)
    return [f32_to_bf16_bits(rng.normal(0.0, scale, n).astype(np.float32)) for _ in range(nranks)]


def uniform_f32(seed: int, nranks: int, n: int, scale: float = 1.0) -> list[np.ndarray]:
    """Generic parity input: N fp32 buffers ~ Normal(0, scale)."""
    rng = np.random.default_rng(seed)
    return [rng.normal(0.0, scale, n).astype(np.float32) for _ in range(nranks)]


def wide_range_f32(seed: int, n: int, block: int, log2_span: int = 60) -> np.ndarray:
    """fp32 values ~ Normal(0,1) times a per-block power of two drawn from
    2**[-span, span] (exercises tiny, huge and subnormal-adjacent scales)."""
    rng = np.random.default_rng(seed)
    v = rng.normal(0.0, 1.0, n)
    nb = -(-n // block)
    e = rng.integers(-log2_span, log2_span + 1, nb)
    v *= np.repeat(np.ldexp(1.0, e), block)[:n]
    return v.astype(np.float32)


def device_rank(w: Workload, r: int, device, seed_offset: int = 0):
    """The same recipe drawn on the GPU with torch's generator (seeded with
    w.seed * 1000 + r): a different random stream from the host recipe, for
    throughput runs that need no CPU comparison.  Returns a 1-D torch tensor
    (bfloat16 or float32)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(w.seed * 1000 + r + seed_offset)
    n = w.n
    if w.key in ("tiny", "outliers"):
        v = torch.randn(n, generator=g, device=device, dtype=torch.float32)
        if w.key == "outliers":
            k = n // 1000
            pos = torch.randperm(n, generator=g, device=device)[:k]
            v[pos] = torch.randn(k, generator=g, device=device) * 50.0
    elif w.key in ("prefill", "ring"):
        u = torch.rand(n, generator=g, device=device, dtype=torch.float32) - 0.5
        v = -0.5 * torch.sign(u) * torch.log1p(-2.0 * u.abs()).clamp_min(-40.0)  # Laplace(0, 0.5)
        if w.key == "prefill":
            rows, hidden = w.shape
            mult = torch.exp(torch.randn(rows, generator=g, device=device))
            v = (v.view(rows, hidden) * mult[:, None]).reshape(-1)
        else:
            k = n // 2000
            pos = torch.randperm(n, generator=g, device=device)[:k]
            v[pos] *= 100.0
    elif w.key == "smallblock":
        v = torch.randn(n, generator=g, device=device) * 1e-3
        v = (v.view(-1, 64) * torch.exp(2.0 * torch.randn(n // 64, generator=g, device=device))[:, None]).reshape(-1)
    else:
        raise KeyError(w.key)
    return v.to(torch.bfloat16) if w.dtype == "bf16" else v
