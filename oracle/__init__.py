"""CPU oracle for the ring all-reduce -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library (``ring_all_reduce_ar_amd``)
never imports, links or calls it, and the two share no code: this package is
plain C (``ring_oracle.c``, built with gcc) behind a ctypes wrapper that takes
host numpy arrays.

What it computes (see ``ring_oracle.c`` for the sources cited section by
section): the ring all-reduce of the handbook chapter "集合通信原语" (section
环形 all-reduce 与通信量) and of the geek-doc page "训练梯度同步与集合通信"
(section 三), with the reduce ops of the mhpq.cn article (section 2.1) and fp32
accumulation for fp16/bf16 (same article, section 5.3). Two independent
forms -- a literal ring simulation with per-rank byte counters and a
per-element fold -- must agree bit for bit.

Dtypes are named 'f32', 'f16', 'bf16', 'i32'. numpy has no bfloat16, so bf16
buffers are numpy uint16 arrays holding the bit patterns.
Ops are named 'sum', 'avg', 'max', 'min', 'prod'.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ring_oracle.c")
# The default library is built from the threaded timing harness, which
# includes ring_oracle.c: it holds the serial checker and the threaded forms.
_SRC_THREADS = os.path.join(_HERE, "ring_oracle_threads.c")
_LIB = os.path.join(_HERE, "liboracle_ar.so")

DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "i32": 3}
OPS = {"sum": 0, "avg": 1, "max": 2, "min": 3, "prod": 4}
NP_DTYPE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "i32": np.int32}
ELEM_SIZE = {"f32": 4, "f16": 2, "bf16": 2, "i32": 4}

GCC_CMD = ["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-o", _LIB, _SRC, "-lm"]


def build(src: str = _SRC_THREADS, out: str = _LIB) -> str:
    """Compile the oracle with gcc (always recompiles). Returns the library path.
    The default source is the threaded harness (serial checker included); a
    test may build a variant of ring_oracle.c alone, which then lacks the
    threaded entry points. Each process compiles to its own temporary file
    and renames it into place, so parallel test workers building at once do
    not race."""
    tmp = f"{out}.tmp{os.getpid():x}"
    cmd = [tmp if a == _LIB else src if a == _SRC else a for a in GCC_CMD]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class Oracle:
    """ctypes handle on one build of ``ring_oracle.c`` (the default build, or a
    variant a test compiled at another path)."""

    def __init__(self, path: str = _LIB):
        lib = ctypes.CDLL(path)
        u64, i32, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p
        pp = ctypes.POINTER(ctypes.c_void_p)
        pu64 = ctypes.POINTER(ctypes.c_uint64)
        lib.orc_ring_all_reduce.argtypes = [i32, u64, i32, i32, pp, pu64]
        lib.orc_fold_all_reduce.argtypes = [i32, u64, i32, i32, pp, pp]
        lib.orc_all_reduce_elements.argtypes = [i32, u64, i32, i32, vp, pu64, u64, vp]
        lib.orc_reduce_scatter.argtypes = [i32, u64, i32, i32, pp, pp, pu64]
        lib.orc_all_gather.argtypes = [i32, u64, i32, pp, pp, pu64]
        lib.orc_chunk_bounds.argtypes = [i32, u64, i32, pu64, pu64]
        lib.orc_all_to_all.argtypes = [i32, u64, i32, pp, pp, pu64]
        lib.orc_tree_all_reduce.argtypes = [i32, u64, i32, i32, pp, pp, pu64]
        for name in ("orc_f32_to_f16", "orc_f16_to_f32", "orc_f32_to_bf16", "orc_bf16_to_f32"):
            getattr(lib, name).argtypes = [vp, vp, u64]
            getattr(lib, name).restype = None
        self.threaded = hasattr(lib, "orc_ring_all_reduce_threads")
        if self.threaded:
            lib.orc_ring_all_reduce_threads.argtypes = [i32, u64, i32, i32, pp, pu64, i32]
            lib.orc_fold_all_reduce_threads.argtypes = [i32, u64, i32, i32, pp, pp, i32]
        self.lib = lib
        self.path = path

    def ring_all_reduce(self, bufs, dtype: str, op: str):
        """In-place all-reduce of ``bufs`` (one array per rank) by the literal ring.

        Returns the list of bytes each rank sent (storage-type bytes per send)."""
        n = len(bufs)
        count = bufs[0].size
        _check_bufs(bufs, dtype, count)
        sent = (ctypes.c_uint64 * n)()
        _rc(self.lib.orc_ring_all_reduce(n, count, DTYPES[dtype], OPS[op], _ptrs(bufs), sent), "ring_all_reduce")
        return [int(s) for s in sent]

    def ring_all_reduce_threads(self, bufs, dtype: str, op: str, nthreads: int):
        """ring_all_reduce on ``nthreads`` host threads: each half-step of the
        ring (all ranks send; all ranks combine or copy) split over
        (rank x piece) items, a barrier between half-steps. Same bytes and
        byte counts as the serial form. Returns the bytes each rank sent."""
        n = len(bufs)
        count = bufs[0].size
        _check_bufs(bufs, dtype, count)
        sent = (ctypes.c_uint64 * n)()
        _rc(self.lib.orc_ring_all_reduce_threads(n, count, DTYPES[dtype], OPS[op], _ptrs(bufs), sent, nthreads),
            "ring_all_reduce_threads")
        return [int(s) for s in sent]

    def fold_all_reduce_threads(self, inputs, dtype: str, op: str, nthreads: int, out=None):
        """fold_all_reduce on ``nthreads`` host threads over element ranges.
        ``out`` (one array per rank, may be ``inputs``) receives the result;
        new arrays are returned when it is None."""
        n = len(inputs)
        count = inputs[0].size
        _check_bufs(inputs, dtype, count)
        outs = out if out is not None else [np.empty(count, dtype=NP_DTYPE[dtype]) for _ in range(n)]
        _check_bufs(outs, dtype, count)
        _rc(self.lib.orc_fold_all_reduce_threads(n, count, DTYPES[dtype], OPS[op], _ptrs(inputs), _ptrs(outs),
                                                 nthreads), "fold_all_reduce_threads")
        return outs

    def fold_all_reduce(self, inputs, dtype: str, op: str):
        """Per-element-fold all-reduce. Returns one new output array per rank."""
        n = len(inputs)
        count = inputs[0].size
        _check_bufs(inputs, dtype, count)
        outs = [np.empty(count, dtype=NP_DTYPE[dtype]) for _ in range(n)]
        _rc(self.lib.orc_fold_all_reduce(n, count, DTYPES[dtype], OPS[op], _ptrs(inputs), _ptrs(outs)), "fold")
        return outs

    def all_reduce_elements(self, vals, idx, count: int, dtype: str, op: str):
        """All-reduced values of the elements ``idx`` of an n-rank x count input.

        ``vals`` has shape (len(idx), n): vals[j, r] = rank r's input at idx[j]."""
        vals = np.ascontiguousarray(vals, dtype=NP_DTYPE[dtype])
        idx = np.ascontiguousarray(idx, dtype=np.uint64)
        m, n = vals.shape
        out = np.empty(m, dtype=NP_DTYPE[dtype])
        _rc(self.lib.orc_all_reduce_elements(n, count, DTYPES[dtype], OPS[op], vals.ctypes.data,
                                             idx.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), m,
                                             out.ctypes.data), "all_reduce_elements")
        return out

    def reduce_scatter(self, inputs, dtype: str, op: str, with_sent: bool = False):
        """Reduce-scatter: inputs[r] has n*recvcount elements; returns outs[r] = block r."""
        n = len(inputs)
        _check_bufs(inputs, dtype, inputs[0].size)
        if inputs[0].size % n:
            raise ValueError("reduce_scatter input size must be a multiple of the rank count")
        rcount = inputs[0].size // n
        outs = [np.empty(rcount, dtype=NP_DTYPE[dtype]) for _ in range(n)]
        sent = (ctypes.c_uint64 * n)()
        _rc(self.lib.orc_reduce_scatter(n, rcount, DTYPES[dtype], OPS[op], _ptrs(inputs), _ptrs(outs), sent),
            "reduce_scatter")
        return (outs, [int(s) for s in sent]) if with_sent else outs

    def all_gather(self, inputs, dtype: str, with_sent: bool = False):
        """All-gather by the ring: returns outs[r] = the inputs concatenated in rank order."""
        n = len(inputs)
        sc = inputs[0].size
        _check_bufs(inputs, dtype, sc)
        outs = [np.empty(n * sc, dtype=NP_DTYPE[dtype]) for _ in range(n)]
        sent = (ctypes.c_uint64 * n)()
        _rc(self.lib.orc_all_gather(n, sc, DTYPES[dtype], _ptrs(inputs), _ptrs(outs), sent), "all_gather")
        return (outs, [int(s) for s in sent]) if with_sent else outs

    def tree_all_reduce(self, inputs, dtype: str, op: str, with_sent: bool = False):
        """Tree-order all-reduce (pairwise levels up to rank 0, then broadcast down)."""
        n = len(inputs)
        count = inputs[0].size
        _check_bufs(inputs, dtype, count)
        outs = [np.empty(count, dtype=NP_DTYPE[dtype]) for _ in range(n)]
        sent = (ctypes.c_uint64 * n)()
        _rc(self.lib.orc_tree_all_reduce(n, count, DTYPES[dtype], OPS[op], _ptrs(inputs), _ptrs(outs), sent), "tree")
        return (outs, [int(s) for s in sent]) if with_sent else outs

    def all_to_all(self, inputs, dtype: str, with_sent: bool = False):
        """All-to-all: inputs[r] holds n blocks; outs[p] block r = inputs[r] block p."""
        n = len(inputs)
        total = inputs[0].size
        _check_bufs(inputs, dtype, total)
        if total % n:
            raise ValueError("all_to_all input size must be a multiple of the rank count")
        outs = [np.empty(total, dtype=NP_DTYPE[dtype]) for _ in range(n)]
        sent = (ctypes.c_uint64 * n)()
        _rc(self.lib.orc_all_to_all(n, total // n, DTYPES[dtype], _ptrs(inputs), _ptrs(outs), sent), "all_to_all")
        return (outs, [int(s) for s in sent]) if with_sent else outs

    def chunk_bounds(self, n: int, count: int):
        """[(lo, hi)] for the n chunks of a count-element buffer."""
        lo, hi = ctypes.c_uint64(), ctypes.c_uint64()
        out = []
        for c in range(n):
            _rc(self.lib.orc_chunk_bounds(n, count, c, ctypes.byref(lo), ctypes.byref(hi)), "chunk_bounds")
            out.append((int(lo.value), int(hi.value)))
        return out

    def _convert(self, fn, x, src, dst):
        x = np.ascontiguousarray(x, dtype=src)
        y = np.empty(x.size, dtype=dst)
        getattr(self.lib, fn)(x.ctypes.data, y.ctypes.data, x.size)
        return y

    def f32_to_f16_bits(self, x):
        return self._convert("orc_f32_to_f16", x, np.float32, np.uint16)

    def f16_bits_to_f32(self, h):
        return self._convert("orc_f16_to_f32", h, np.uint16, np.float32)

    def f32_to_bf16_bits(self, x):
        return self._convert("orc_f32_to_bf16", x, np.float32, np.uint16)

    def bf16_bits_to_f32(self, b):
        return self._convert("orc_bf16_to_f32", b, np.uint16, np.float32)


def _ptrs(arrays):
    return (ctypes.c_void_p * len(arrays))(*[a.ctypes.data for a in arrays])


def _check_bufs(bufs, dtype, count=None):
    want = NP_DTYPE[dtype]
    for b in bufs:
        if b.dtype != want or not b.flags["C_CONTIGUOUS"]:
            raise TypeError(f"oracle expects C-contiguous {np.dtype(want)} arrays for {dtype}, got {b.dtype}")
        if count is not None and b.size != count:
            raise ValueError(f"rank buffer has {b.size} elements, expected {count}")


def _rc(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


_default = None


def get() -> Oracle:
    """The default oracle build (compiled on first use if missing or stale)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(os.path.getmtime(_SRC),
                                                                     os.path.getmtime(_SRC_THREADS)):
            build()
        _default = Oracle(_LIB)
    return _default


def ring_all_reduce(bufs, dtype, op):
    return get().ring_all_reduce(bufs, dtype, op)


def fold_all_reduce(inputs, dtype, op):
    return get().fold_all_reduce(inputs, dtype, op)


def ring_all_reduce_threads(bufs, dtype, op, nthreads):
    return get().ring_all_reduce_threads(bufs, dtype, op, nthreads)


def fold_all_reduce_threads(inputs, dtype, op, nthreads, out=None):
    return get().fold_all_reduce_threads(inputs, dtype, op, nthreads, out)


def all_reduce_elements(vals, idx, count, dtype, op):
    return get().all_reduce_elements(vals, idx, count, dtype, op)


def reduce_scatter(inputs, dtype, op, with_sent=False):
    return get().reduce_scatter(inputs, dtype, op, with_sent)


def all_gather(inputs, dtype, with_sent=False):
    return get().all_gather(inputs, dtype, with_sent)


def all_to_all(inputs, dtype, with_sent=False):
    return get().all_to_all(inputs, dtype, with_sent)


def tree_all_reduce(inputs, dtype, op, with_sent=False):
    return get().tree_all_reduce(inputs, dtype, op, with_sent)


def chunk_bounds(n, count):
    return get().chunk_bounds(n, count)
