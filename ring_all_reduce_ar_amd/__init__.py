"""Python binding of liballreduce (the C ABI in include/allreduce.h).

Argument marshalling only: every step of the all-reduce runs in the HIP
kernels of ``liballreduce.so``. The functions carry the C names and raise
``ArError`` where the C call returns a non-success code. Buffers may be
passed as torch tensors (their ``data_ptr()`` is taken) or as integer device
addresses; streams as ``torch.cuda.Stream``, an integer ``hipStream_t`` or
``None`` (torch's current stream on the comm's device).

The library is built in-tree by ``python ring_all_reduce_ar_amd/build.py``;
importing this package without it raises ImportError: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liballreduce.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python ring_all_reduce_ar_amd/build.py` first")

# One process must hold one HIP runtime. torch ships its own libamdhip64 /
# libhsa-runtime64; importing torch first loads them, and liballreduce.so's
# dependency on libamdhip64.so.7 then binds to that same runtime instead of
# loading a second one from /opt/rocm (two HSA runtimes in one process leave
# the second without a device).
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

MAX_RANKS = 64  # AR_MAX_RANKS
MAX_TENSORS = 65536  # AR_MAX_TENSORS
NOALLOC_SCRATCH_BYTES = 64 << 20  # AR_NOALLOC_SCRATCH_BYTES

# ar_result_t
AR_SUCCESS, AR_ERR_INVALID_ARGUMENT, AR_ERR_UNSUPPORTED, AR_ERR_HIP, AR_ERR_OUT_OF_MEMORY, AR_ERR_INTERNAL = range(6)
# ar_dtype_t
AR_FLOAT32, AR_FLOAT16, AR_BFLOAT16, AR_INT32 = range(4)
# ar_op_t
AR_SUM, AR_AVG, AR_MAX, AR_MIN, AR_PROD = range(5)
# ar_mode_t
AR_MODE_FUSED, AR_MODE_RING_STEPWISE, AR_MODE_RING_GRAPH, AR_MODE_TREE, AR_MODE_TREE_STEPWISE = range(5)
# ar_access_t
AR_ACCESS_AUTO, AR_ACCESS_STREAMING, AR_ACCESS_CACHED = range(3)
ACCESS_NAMES = {"auto": AR_ACCESS_AUTO, "streaming": AR_ACCESS_STREAMING, "cached": AR_ACCESS_CACHED}
# ar_collective_t
AR_COLL_ALL_REDUCE, AR_COLL_REDUCE_SCATTER, AR_COLL_ALL_GATHER, AR_COLL_ALL_TO_ALL = range(4)

DTYPE_NAMES = {"f32": AR_FLOAT32, "f16": AR_FLOAT16, "bf16": AR_BFLOAT16, "i32": AR_INT32}
OP_NAMES = {"sum": AR_SUM, "avg": AR_AVG, "max": AR_MAX, "min": AR_MIN, "prod": AR_PROD}
MODE_NAMES = {"fused": AR_MODE_FUSED, "stepwise": AR_MODE_RING_STEPWISE, "graph": AR_MODE_RING_GRAPH,
              "tree": AR_MODE_TREE, "tree_stepwise": AR_MODE_TREE_STEPWISE}

EXPORTED_SYMBOLS = (
    "ar_comm_create", "ar_comm_destroy", "ar_comm_nranks", "ar_workspace_bytes", "ar_comm_set_workspace",
    "ar_all_reduce", "ar_all_reduce_noalloc", "ar_reduce_scatter", "ar_all_gather", "ar_all_to_all", "ar_all_reduce_multi",
    "ar_comm_set_step_timing", "ar_comm_set_access", "ar_comm_set_streaming", "ar_last_step_times_ms",
    "ar_result_string", "ar_last_error",
)

_c_int, _c_size, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
_ptr_array = ctypes.POINTER(ctypes.c_void_p)

_lib.ar_comm_create.argtypes = [ctypes.POINTER(_vp), _c_int, _c_int]
_lib.ar_comm_destroy.argtypes = [_vp]
_lib.ar_comm_nranks.argtypes = [_vp]
_lib.ar_comm_nranks.restype = _c_int
_lib.ar_workspace_bytes.argtypes = [_c_int, _c_int, _c_size, _c_int, _c_int]
_lib.ar_workspace_bytes.restype = _c_size
_lib.ar_comm_set_workspace.argtypes = [_vp, _vp, _c_size]
_lib.ar_all_reduce.argtypes = [_vp, _ptr_array, _ptr_array, _c_size, _c_int, _c_int, _c_int, _vp]
_lib.ar_all_reduce_noalloc.argtypes = [_vp, _ptr_array, _ptr_array, _c_size, _c_int, _c_int, _c_int, _vp]
_lib.ar_reduce_scatter.argtypes = [_vp, _ptr_array, _ptr_array, _c_size, _c_int, _c_int, _c_int, _vp]
_lib.ar_all_gather.argtypes = [_vp, _ptr_array, _ptr_array, _c_size, _c_int, _c_int, _vp]
_lib.ar_all_to_all.argtypes = [_vp, _ptr_array, _ptr_array, _c_size, _c_int, _c_int, _vp]
_lib.ar_all_reduce_multi.argtypes = [_vp, _c_int, _ptr_array, _ptr_array, ctypes.POINTER(_c_size), _c_int, _c_int,
                                     _c_int, _vp]
_lib.ar_comm_set_step_timing.argtypes = [_vp, _c_int]
_lib.ar_comm_set_streaming.argtypes = [_vp, _c_int]
_lib.ar_comm_set_access.argtypes = [_vp, _c_int]
_lib.ar_last_step_times_ms.argtypes = [_vp, ctypes.POINTER(ctypes.c_float), _c_int, ctypes.POINTER(_c_int)]
_lib.ar_result_string.argtypes = [_c_int]
_lib.ar_result_string.restype = ctypes.c_char_p
_lib.ar_last_error.argtypes = []
_lib.ar_last_error.restype = ctypes.c_char_p
for _name in ("ar_comm_create", "ar_comm_destroy", "ar_comm_set_workspace", "ar_all_reduce", "ar_all_reduce_noalloc",
              "ar_reduce_scatter",
              "ar_all_gather", "ar_all_to_all", "ar_all_reduce_multi", "ar_comm_set_step_timing",
              "ar_comm_set_streaming", "ar_comm_set_access", "ar_last_step_times_ms"):
    getattr(_lib, _name).restype = _c_int


class ArError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        detail = (_lib.ar_last_error() or b"").decode(errors="replace")
        super().__init__(f"{where}: {ar_result_string(code)} ({code}): {detail}")


def _check(code: int, where: str):
    if code != AR_SUCCESS:
        raise ArError(code, where)


def ar_result_string(code: int) -> str:
    return _lib.ar_result_string(code).decode()


def ar_last_error() -> str:
    return (_lib.ar_last_error() or b"").decode(errors="replace")


def _enum(value, names, what):
    if isinstance(value, str):
        if value not in names:
            raise ValueError(f"unknown {what} {value!r}; expected one of {sorted(names)}")
        return names[value]
    return int(value)


def torch_dtype_code(dtype) -> int:
    import torch
    table = {torch.float32: AR_FLOAT32, torch.float16: AR_FLOAT16, torch.bfloat16: AR_BFLOAT16, torch.int32: AR_INT32}
    if dtype not in table:
        raise TypeError(f"unsupported dtype {dtype}")
    return table[dtype]


def _addr(buf) -> int:
    if isinstance(buf, int):
        return buf
    if hasattr(buf, "data_ptr"):
        if not buf.is_contiguous():
            raise ValueError("rank buffers must be contiguous")
        return buf.data_ptr()
    raise TypeError(f"expected a tensor or an int address, got {type(buf).__name__}")


_PTR_ARRAY_TYPES = {}  # length -> ctypes array type (building the type costs more than the array)


def _ptrs(bufs):
    n = len(bufs)
    t = _PTR_ARRAY_TYPES.get(n)
    if t is None:
        t = _PTR_ARRAY_TYPES[n] = ctypes.c_void_p * n
    return t(*[b if type(b) is int else _addr(b) for b in bufs])


def _ptr_pair(sendbufs, recvbufs):
    """The send and recv pointer arrays; one array serves both when the same
    list is passed for both (in place)."""
    s = _ptrs(sendbufs)
    return s, (s if recvbufs is sendbufs else _ptrs(recvbufs))


def _stream(stream, device: int):
    if stream is None:
        import torch
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Comm:
    """Owns an ``ar_comm_t``; ``handle`` is the raw pointer."""

    def __init__(self, nranks: int, device: int = 0):
        h = ctypes.c_void_p()
        _check(_lib.ar_comm_create(ctypes.byref(h), nranks, device), "ar_comm_create")
        self.handle = h
        self.nranks = nranks
        self.device = device

    def close(self):
        if self.handle:
            _lib.ar_comm_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def _h(comm):
    return comm.handle if isinstance(comm, Comm) else comm


def ar_comm_create(nranks: int, device: int = 0) -> Comm:
    return Comm(nranks, device)


def ar_comm_destroy(comm: Comm):
    comm.close()


def ar_comm_nranks(comm) -> int:
    return _lib.ar_comm_nranks(_h(comm))


def ar_workspace_bytes(coll, nranks: int, count: int, dtype, mode) -> int:
    v = _lib.ar_workspace_bytes(int(coll), nranks, count, _enum(dtype, DTYPE_NAMES, "dtype"),
                                _enum(mode, MODE_NAMES, "mode"))
    if v == ctypes.c_size_t(-1).value:
        raise ValueError("ar_workspace_bytes: invalid arguments or overflow")
    return v


def ar_comm_set_workspace(comm, buf, nbytes: int | None = None):
    """Attach a device workspace (tensor or address); ``None`` detaches."""
    if buf is None:
        _check(_lib.ar_comm_set_workspace(_h(comm), None, 0), "ar_comm_set_workspace")
        return
    if nbytes is None:
        nbytes = buf.numel() * buf.element_size()
    _check(_lib.ar_comm_set_workspace(_h(comm), _addr(buf), nbytes), "ar_comm_set_workspace")


def ar_all_reduce(comm, sendbufs, recvbufs, count: int, dtype, op, mode="fused", stream=None):
    _check(_lib.ar_all_reduce(_h(comm), *_ptr_pair(sendbufs, recvbufs), count, _enum(dtype, DTYPE_NAMES, "dtype"),
                              _enum(op, OP_NAMES, "op"), _enum(mode, MODE_NAMES, "mode"),
                              _stream(stream, comm.device if isinstance(comm, Comm) else 0)), "ar_all_reduce")


def ar_all_reduce_noalloc(comm, sendbufs, recvbufs, count: int, dtype, op, mode="fused", stream=None):
    """ar_all_reduce with its partial sums in the library's device scratch
    array instead of the comm's workspace; allocates nothing."""
    _check(_lib.ar_all_reduce_noalloc(_h(comm), *_ptr_pair(sendbufs, recvbufs), count,
                                      _enum(dtype, DTYPE_NAMES, "dtype"), _enum(op, OP_NAMES, "op"),
                                      _enum(mode, MODE_NAMES, "mode"),
                                      _stream(stream, comm.device if isinstance(comm, Comm) else 0)),
           "ar_all_reduce_noalloc")


def ar_reduce_scatter(comm, sendbufs, recvbufs, recvcount: int, dtype, op, mode="fused", stream=None):
    _check(_lib.ar_reduce_scatter(_h(comm), *_ptr_pair(sendbufs, recvbufs), recvcount,
                                  _enum(dtype, DTYPE_NAMES, "dtype"), _enum(op, OP_NAMES, "op"),
                                  _enum(mode, MODE_NAMES, "mode"),
                                  _stream(stream, comm.device if isinstance(comm, Comm) else 0)), "ar_reduce_scatter")


def ar_all_gather(comm, sendbufs, recvbufs, sendcount: int, dtype, mode="fused", stream=None):
    _check(_lib.ar_all_gather(_h(comm), *_ptr_pair(sendbufs, recvbufs), sendcount,
                              _enum(dtype, DTYPE_NAMES, "dtype"), _enum(mode, MODE_NAMES, "mode"),
                              _stream(stream, comm.device if isinstance(comm, Comm) else 0)), "ar_all_gather")


def ar_all_to_all(comm, sendbufs, recvbufs, blockcount: int, dtype, mode="fused", stream=None):
    _check(_lib.ar_all_to_all(_h(comm), *_ptr_pair(sendbufs, recvbufs), blockcount,
                              _enum(dtype, DTYPE_NAMES, "dtype"), _enum(mode, MODE_NAMES, "mode"),
                              _stream(stream, comm.device if isinstance(comm, Comm) else 0)), "ar_all_to_all")


def ar_all_reduce_multi(comm, sendbufs, recvbufs, counts, dtype, op, mode="fused", stream=None):
    """sendbufs / recvbufs: one list of per-rank buffers per tensor
    (``sendbufs[t][r]``), or a flat tensor-major list; counts[t] elements."""
    nt = len(counts)
    flat_s = [b for row in sendbufs for b in row] if nt and isinstance(sendbufs[0], (list, tuple)) else list(sendbufs)
    flat_r = [b for row in recvbufs for b in row] if nt and isinstance(recvbufs[0], (list, tuple)) else list(recvbufs)
    arr = (ctypes.c_size_t * max(nt, 1))(*counts)
    _check(_lib.ar_all_reduce_multi(_h(comm), nt, *_ptr_pair(flat_s, flat_r), arr, _enum(dtype, DTYPE_NAMES, "dtype"),
                                    _enum(op, OP_NAMES, "op"), _enum(mode, MODE_NAMES, "mode"),
                                    _stream(stream, comm.device if isinstance(comm, Comm) else 0)),
           "ar_all_reduce_multi")


def ar_comm_set_step_timing(comm, enable: bool):
    _check(_lib.ar_comm_set_step_timing(_h(comm), 1 if enable else 0), "ar_comm_set_step_timing")


def ar_comm_set_streaming(comm, enable: bool):
    _check(_lib.ar_comm_set_streaming(_h(comm), 1 if enable else 0), "ar_comm_set_streaming")


def ar_comm_set_access(comm, access):
    """access: "auto", "streaming", "cached" or an AR_ACCESS_* value."""
    _check(_lib.ar_comm_set_access(_h(comm), _enum(access, ACCESS_NAMES, "access")), "ar_comm_set_access")


def ar_last_step_times_ms(comm, cap: int = 2 * MAX_RANKS + 1):
    out = (ctypes.c_float * cap)()
    n = ctypes.c_int()
    _check(_lib.ar_last_step_times_ms(_h(comm), out, cap, ctypes.byref(n)), "ar_last_step_times_ms")
    return [out[i] for i in range(min(n.value, cap))]
