"""The C-ABI library loads and exports every function include/allreduce.h
declares; host-side argument checks that need no device (no compute calls)."""
import ctypes
import os
import re

import pytest

import ring_all_reduce_ar_amd as ar

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "allreduce.h")


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ar_[a-z_]+)\s*\(", text)))


def test_header_declares_the_abi():
    names = declared_functions()
    for need in ("ar_all_reduce", "ar_reduce_scatter", "ar_all_gather", "ar_comm_create", "ar_comm_destroy"):
        assert need in names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(ar.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(declared_functions()) == sorted(ar.EXPORTED_SYMBOLS)


def test_result_strings():
    assert ar.ar_result_string(ar.AR_SUCCESS) == "success"
    assert ar.ar_result_string(ar.AR_ERR_INVALID_ARGUMENT) == "invalid argument"
    assert ar.ar_result_string(99) == "unknown result code"


def test_workspace_sizes():
    C = ar
    assert ar.ar_workspace_bytes(C.AR_COLL_ALL_REDUCE, 8, 1000, "f16", "stepwise") == 4000
    assert ar.ar_workspace_bytes(C.AR_COLL_ALL_REDUCE, 8, 1000, "bf16", "stepwise") == 4000
    assert ar.ar_workspace_bytes(C.AR_COLL_ALL_REDUCE, 8, 1000, "f32", "stepwise") == 0
    assert ar.ar_workspace_bytes(C.AR_COLL_ALL_REDUCE, 8, 1000, "f16", "fused") == 0
    assert ar.ar_workspace_bytes(C.AR_COLL_ALL_REDUCE, 1, 1000, "f16", "stepwise") == 0
    assert ar.ar_workspace_bytes(C.AR_COLL_REDUCE_SCATTER, 8, 1000, "i32", "stepwise") == 32000
    assert ar.ar_workspace_bytes(C.AR_COLL_ALL_GATHER, 8, 1000, "f32", "stepwise") == 0
    assert ar.ar_workspace_bytes(C.AR_COLL_ALL_REDUCE, 8, 7_000_000_000, "f16", "stepwise") == 28_000_000_000
    with pytest.raises(ValueError):
        ar.ar_workspace_bytes(C.AR_COLL_ALL_REDUCE, 0, 1000, "f16", "stepwise")
    with pytest.raises(ValueError):
        ar.ar_workspace_bytes(C.AR_COLL_REDUCE_SCATTER, 64, 2**62, "f32", "stepwise")


def test_null_comm_is_rejected_without_a_device():
    lib = ar._lib
    arr = (ctypes.c_void_p * 1)(1 << 12)
    rc = lib.ar_all_reduce(None, arr, arr, 16, ar.AR_FLOAT32, ar.AR_SUM, ar.AR_MODE_FUSED, None)
    assert rc == ar.AR_ERR_INVALID_ARGUMENT
    assert "comm" in ar.ar_last_error()
    assert lib.ar_reduce_scatter(None, arr, arr, 16, 0, 0, 0, None) == ar.AR_ERR_INVALID_ARGUMENT
    assert lib.ar_all_gather(None, arr, arr, 16, 0, 0, None) == ar.AR_ERR_INVALID_ARGUMENT
    assert lib.ar_comm_set_workspace(None, None, 0) == ar.AR_ERR_INVALID_ARGUMENT
    assert lib.ar_comm_set_step_timing(None, 1) == ar.AR_ERR_INVALID_ARGUMENT
    assert lib.ar_comm_set_streaming(None, 1) == ar.AR_ERR_INVALID_ARGUMENT
    assert lib.ar_comm_destroy(None) == ar.AR_SUCCESS
    assert lib.ar_comm_nranks(None) == -1


def test_comm_create_rejects_bad_rank_counts_before_touching_hip():
    for n in (0, -1, ar.MAX_RANKS + 1):
        h = ctypes.c_void_p()
        assert ar._lib.ar_comm_create(ctypes.byref(h), n, 0) == ar.AR_ERR_INVALID_ARGUMENT
        assert not h.value
    assert ar._lib.ar_comm_create(None, 4, 0) == ar.AR_ERR_INVALID_ARGUMENT


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "8"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2 and "one GPU" in p.stderr


def test_one_hip_runtime_in_the_process():
    """Importing the binding maps exactly one libamdhip64 and one HSA runtime
    (torch's), even when nothing imported torch before it."""
    import subprocess
    import sys
    code = ("import ring_all_reduce_ar_amd\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "libs = {l.split()[-1] for l in maps if 'amdhip64' in l or 'hsa-runtime64' in l}\n"
            "print(len([x for x in libs if 'amdhip64' in x]), len([x for x in libs if 'hsa-runtime64' in x]))\n")
    p = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert p.returncode == 0, p.stderr
    assert p.stdout.split() == ["1", "1"], p.stdout


def test_binding_limits_match_the_header():
    text = open(HEADER, encoding="utf-8").read()
    defs = dict(re.findall(r"#define\s+(AR_MAX_\w+)\s+(\d+)", text))
    assert int(defs["AR_MAX_RANKS"]) == ar.MAX_RANKS
    assert int(defs["AR_MAX_TENSORS"]) == ar.MAX_TENSORS
