"""Seeded synthetic inputs for the all-reduce workloads.

This module only draws random numbers; it holds none of the all-reduce's
arithmetic. Both sides of a check use it: the GPU library is fed the tensors
it makes, and the CPU oracle is fed host copies of the same tensors.

Workloads (per-rank shapes and value distributions):

* ``small``  -- 4 ranks x 4096 fp32, uniform[-1, 1), SUM (plus the 4-element
  integer example [10r, 10r+1, 10r+2, 10r+3] printed by the handbook chapter
  "集合通信原语", section 五个原语).
* ``bucket25`` -- 8 ranks, one 25 MiB DDP-style gradient bucket per rank
  (6,553,600 fp32), N(0, 1e-3^2), AVG. The 25 MB bucket is the DDP default the
  mhpq.cn article (section 5.2) names.
* ``sweep`` -- 8 ranks, 1 KiB .. 256 MiB per rank in powers of two; fp32
  uniform[-1, 1) and int32 uniform[-1000, 1000], SUM.
* ``grad7b`` -- 8 ranks, a 7e9-element fp16 gradient per rank (14 GB, the 7B
  model of the geek-doc page, section 一), N(0, 1e-3^2) with 1% of the
  elements drawn from N(0, 1) instead, generated in fp32 and rounded to fp16.
* ``bucket64`` -- 64 ranks x 67,108,864 fp32 (256 MiB), laid out as a flat
  bucket of tensors whose byte sizes are log-uniform in [4 KiB, 64 MiB];
  uniform[-1, 1) for MAX/MIN, uniform[0.99, 1.01) for PROD.

Seeds: workload k, rank r uses ``torch.Generator(device).manual_seed(1000*k + r)``.
"""
from __future__ import annotations

import math

import numpy as np
import torch

WORKLOAD_IDS = {"small": 1, "bucket25": 2, "sweep": 3, "grad7b": 4, "bucket64": 5}

# Elements generated per slice when filling very large tensors (bounds the
# fp32 temporaries to 1 GiB).
_SLICE = 1 << 28


def generator(workload: str, rank: int, device="cpu", salt: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(1000 * WORKLOAD_IDS[workload] + rank + 1_000_003 * salt)
    return g


def _fill(out: torch.Tensor, draw):
    """Fill ``out`` slice by slice with ``draw(n) -> fp32 tensor``, rounding to out's dtype."""
    flat = out.view(-1)
    for lo in range(0, flat.numel(), _SLICE):
        hi = min(lo + _SLICE, flat.numel())
        flat[lo:hi].copy_(draw(hi - lo))
    return out


def uniform(count: int, lo: float, hi: float, gen: torch.Generator, dtype=torch.float32, device="cpu", out=None):
    """uniform[lo, hi) drawn in fp32, rounded to ``dtype`` (into ``out`` if given)."""
    if out is None:
        out = torch.empty(count, dtype=dtype, device=device)
    return _fill(out, lambda n: torch.empty(n, dtype=torch.float32, device=device).uniform_(lo, hi, generator=gen))


def gaussian(count: int, std: float, gen: torch.Generator, dtype=torch.float32, device="cpu",
             outlier_frac: float = 0.0, outlier_std: float = 1.0, out=None):
    """N(0, std^2) drawn in fp32; with probability ``outlier_frac`` an element is
    drawn from N(0, outlier_std^2) instead. Rounded to ``dtype`` (into ``out`` if given)."""
    def draw(n):
        x = torch.randn(n, dtype=torch.float32, device=device, generator=gen) * std
        if outlier_frac > 0:
            pick = torch.rand(n, dtype=torch.float32, device=device, generator=gen) < outlier_frac
            big = torch.randn(n, dtype=torch.float32, device=device, generator=gen) * outlier_std
            x = torch.where(pick, big, x)
        return x
    if out is None:
        out = torch.empty(count, dtype=dtype, device=device)
    return _fill(out, draw)


def int_uniform(count: int, lo: int, hi: int, gen: torch.Generator, device="cpu"):
    """int32 uniform on the closed range [lo, hi]."""
    return torch.randint(lo, hi + 1, (count,), dtype=torch.int32, device=device, generator=gen)


def worked_example(nranks: int = 4, dtype=torch.float32, device="cpu"):
    """Rank r holds [10r, 10r+1, 10r+2, 10r+3] (the handbook's 4-rank example)."""
    return [(torch.arange(4, dtype=torch.float32) + 10 * r).to(dtype=dtype, device=device) for r in range(nranks)]


def bucket_sizes(total_elems: int, elem_bytes: int, lo_bytes: int, hi_bytes: int, seed: int):
    """Element counts of tensors packed into one flat bucket of ``total_elems``.

    Byte sizes are drawn log-uniform in [lo_bytes, hi_bytes], rounded to whole
    elements; tensors are packed until the bucket is full and the last one is
    truncated to fit."""
    rng = np.random.default_rng(seed)
    sizes = []
    left = total_elems
    while left > 0:
        b = math.exp(rng.uniform(math.log(lo_bytes), math.log(hi_bytes)))
        n = max(1, int(round(b / elem_bytes)))
        n = min(n, left)
        sizes.append(n)
        left -= n
    return sizes


# Rank inputs per workload ----------------------------------------------------

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "i32": torch.int32}


def rank_inputs(workload: str, nranks: int, count: int, dtype: str, device="cpu", op: str = "sum", salt: int = 0):
    """One tensor per rank with ``workload``'s value distribution."""
    td = TORCH_DTYPE[dtype]
    out = []
    for r in range(nranks):
        g = generator(workload, r, device, salt)
        if dtype == "i32":
            out.append(int_uniform(count, -1000, 1000, g, device))
        elif workload == "bucket25":
            out.append(gaussian(count, 1e-3, g, td, device))
        elif workload == "grad7b":
            out.append(gaussian(count, 1e-3, g, td, device, outlier_frac=0.01, outlier_std=1.0))
        elif workload == "bucket64" and op == "prod":
            out.append(uniform(count, 0.99, 1.01, g, td, device))
        else:
            out.append(uniform(count, -1.0, 1.0, g, td, device))
    return out


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """Host numpy copy; bf16 comes back as uint16 bit patterns."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()
