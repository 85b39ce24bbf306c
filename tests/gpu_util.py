"""Helpers for the GPU tests: rank buffers with guard bands, host copies, and
the comparison with the CPU oracle.

Every rank buffer is its own allocation laid out as
[64-byte guard][payload][64-byte guard]; guards hold 0xA5 bytes and are
checked after each call, so a write outside the payload fails the test.
Output buffers start filled with 0xFF bytes (NaN for floats, -1 for int32),
so an element the library never writes shows up.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import ring_all_reduce_ar_amd as ar
import synthetic

GUARD = 64
TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "i32": torch.int32}
ESIZE = {"f32": 4, "f16": 2, "bf16": 2, "i32": 4}
EPV = {"f32": 4, "f16": 8, "bf16": 8, "i32": 4}


class RankBuf:
    """One rank's payload inside a guarded byte allocation (optionally
    shifted by `offset` bytes, to make it unaligned)."""

    def __init__(self, count: int, dtype: str, device="cuda", offset: int = 0, fill: int = 0xFF):
        e = ESIZE[dtype]
        nbytes = count * e
        self.raw = torch.full((GUARD + offset + nbytes + GUARD,), 0xA5, dtype=torch.uint8, device=device)
        self.lo = GUARD + offset
        self.hi = self.lo + nbytes
        self.raw[self.lo:self.hi] = fill
        self.count = count
        self.dtype = dtype
        self.view = self.raw[self.lo:self.hi].view(TORCH[dtype])

    def ptr(self) -> int:
        return self.raw.data_ptr() + self.lo

    def sub_ptr(self, elem_offset: int) -> int:
        return self.ptr() + elem_offset * ESIZE[self.dtype]

    def guards_ok(self) -> bool:
        return bool((self.raw[:self.lo] == 0xA5).all() and (self.raw[self.hi:] == 0xA5).all())


def host(t: torch.Tensor) -> np.ndarray:
    return synthetic.to_numpy(t)


def bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).view({2: np.uint16, 4: np.uint32}[a.dtype.itemsize])


def nan_mask(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        b = bits(a)
        return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)
    if dtype in ("f32", "f16"):
        return np.isnan(a)
    return np.zeros(a.shape, dtype=bool)


def assert_same(got: np.ndarray, exp: np.ndarray, dtype: str, what: str = ""):
    """Bitwise equality; NaN positions must match (NaN payloads are not compared)."""
    assert got.shape == exp.shape, (what, got.shape, exp.shape)
    gnan, enan = nan_mask(got, dtype), nan_mask(exp, dtype)
    assert np.array_equal(gnan, enan), f"{what}: NaN positions differ"
    gb, eb = bits(got), bits(exp)
    bad = np.nonzero((gb != eb) & ~gnan)[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {got.size} elements differ; first at {bad[:5].tolist()}: "
                           f"got {got[bad[:5]]} expected {exp[bad[:5]]}")


def make_inputs(n, count, dtype, op, seed, device="cuda"):
    """Seeded inputs for a parity case (the sweep workload's distributions;
    PROD in [0.99, 1.01) so products stay finite)."""
    wl = "bucket64" if op == "prod" else "sweep"
    return synthetic.rank_inputs(wl, n, count, dtype, device=device, op=op, salt=seed)


def run_all_reduce(comm, xs, dtype, op, mode, inplace=False, offset=0, ws=None, stream=None):
    """Copy the inputs into guarded rank buffers, all-reduce, return
    (outputs as host arrays, send bufs, recv bufs)."""
    n, count = len(xs), xs[0].numel()
    send = [RankBuf(count, dtype, offset=offset) for _ in range(n)]
    for b, x in zip(send, xs):
        b.view.copy_(x)
    recv = send if inplace else [RankBuf(count, dtype, offset=offset) for _ in range(n)]
    ar.ar_all_reduce(comm, [b.ptr() for b in send], [b.ptr() for b in recv], count, dtype, op, mode, stream)
    torch.cuda.synchronize()
    for b in send + recv:
        assert b.guards_ok(), "guard band overwritten"
    return [host(b.view) for b in recv], send, recv


def oracle_threads() -> int:
    """Host threads for the oracle's threaded fold (bit-identical to its
    serial fold: tests/test_oracle_threads.py): the host's share for this
    job (OMP_NUM_THREADS), else the affinity mask, at most 16."""
    import os
    env = os.environ.get("OMP_NUM_THREADS", "")
    t = int(env) if env.isdigit() and int(env) > 0 else len(os.sched_getaffinity(0))
    return max(1, min(t, 16))


def oracle_all_reduce(xs, dtype, op):
    return oracle.fold_all_reduce_threads([host(x) for x in xs], dtype, op, oracle_threads())


def attach_workspace(comm, coll, n, count, dtype, mode):
    need = ar.ar_workspace_bytes(coll, n, count, dtype, mode)
    if need == 0:
        ar.ar_comm_set_workspace(comm, None)
        return None
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ar.ar_comm_set_workspace(comm, ws)
    return ws
