"""Access flavours (`ar_comm_set_access`, `ar_comm_set_streaming`): the
one-launch calls with non-temporal loads and stores at sizes where the
default would cache, and cached ones where it would stream. The results are
the same bits either way, and equal to the oracle's."""
import pytest

import gpu_util as gu
import oracle
import ring_all_reduce_ar_amd as ar
from test_gpu_multi import check as check_multi
from test_gpu_parity import _all_gather, _all_to_all, _reduce_scatter

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [3, 8, 64])
def test_streaming_all_reduce(n):
    """Fused (ring order) and tree-fused all-reduce, 16-byte and element
    paths, cached against streaming on one comm, both against the oracle."""
    cases = (("f32", "sum", (1 << 20) + 5, 0), ("bf16", "avg", 300_007, 0), ("f16", "max", 70_001, 2),
             ("i32", "prod", 4099, 0))
    with ar.Comm(n, 0) as comm:
        for dtype, op, count, offset in cases:
            xs = gu.make_inputs(n, count, dtype, op, seed=count % 97 + n)
            for mode in ("fused", "tree"):
                if mode == "fused":
                    exp = gu.oracle_all_reduce(xs, dtype, op)
                else:
                    exp = oracle.tree_all_reduce([gu.host(x) for x in xs], dtype, op)
                ar.ar_comm_set_streaming(comm, False)
                base, _, _ = gu.run_all_reduce(comm, xs, dtype, op, mode, offset=offset)
                ar.ar_comm_set_streaming(comm, True)
                got, _, _ = gu.run_all_reduce(comm, xs, dtype, op, mode, offset=offset, inplace=True)
                ar.ar_comm_set_streaming(comm, False)
                for r in range(n):
                    what = f"streaming n={n} {dtype} {op} {mode} count={count} offset={offset} rank {r}"
                    gu.assert_same(got[r], base[r], dtype, what + " vs cached")
                    gu.assert_same(got[r], exp[r], dtype, what + " vs oracle")


@pytest.mark.parametrize("n", [3, 8])
def test_streaming_exports_and_all_to_all(n):
    """Fused reduce-scatter, all-gather and all-to-all with streaming on."""
    with ar.Comm(n, 0) as comm:
        ar.ar_comm_set_streaming(comm, True)
        for dtype in ("f32", "bf16"):
            rc = 3 * 1024 + gu.EPV[dtype]
            xs = gu.make_inputs(n, n * rc, dtype, "avg", seed=5 * n)
            exp = oracle.reduce_scatter([gu.host(x) for x in xs], dtype, "avg")
            for inplace in (False, True):
                got = _reduce_scatter(comm, xs, dtype, "avg", "fused", inplace)
                for r in range(n):
                    gu.assert_same(got[r], exp[r], dtype, f"streaming RS n={n} {dtype} inplace={inplace} rank {r}")
            sc = 1000 + 3
            xs = gu.make_inputs(n, sc, dtype, "sum", seed=6 * n)
            exp = oracle.all_gather([gu.host(x) for x in xs], dtype)
            for inplace in (False, True):
                got = _all_gather(comm, xs, dtype, "fused", inplace)
                for r in range(n):
                    gu.assert_same(got[r], exp[r], dtype, f"streaming AG n={n} {dtype} inplace={inplace} rank {r}")
            xs = gu.make_inputs(n, n * (2048 + gu.EPV[dtype]), dtype, "sum", seed=7 * n)
            exp = oracle.all_to_all([gu.host(x) for x in xs], dtype)
            got = _all_to_all(comm, xs, dtype, "fused")
            for p in range(n):
                gu.assert_same(got[p], exp[p], dtype, f"streaming A2A n={n} {dtype} rank {p}")


@pytest.mark.parametrize("n", [8, 64])
def test_streaming_multi_tensor(n):
    """The multi-tensor all-reduce with streaming on: against the oracle and
    the flat call (also streaming), in place and out of place, shifted
    starts."""
    sizes = [3, 40_000 + 1, 7, 2 * 256 * 4 + 5, n * 513, 1]
    with ar.Comm(n, 0) as comm:
        ar.ar_comm_set_streaming(comm, True)
        check_multi(comm, sizes, "f32", "sum", seed=n + 40)
        check_multi(comm, sizes, "bf16", "max", seed=n + 41, inplace=True, offset=6)


@pytest.mark.parametrize("n,dtype,op,count", [(8, "f32", "avg", 5_242_883), (4, "bf16", "sum", 20_971_529),
                                              (8, "f16", "max", 8_388_611)])
def test_access_flavours_agree(n, dtype, op, count):
    """Footprints between half and all of the last-level cache, where the
    default (AR_ACCESS_AUTO) all-reduce streams through the rank-major
    kernel while AR_ACCESS_CACHED keeps cached two-tile kernels: auto,
    streaming and cached give the same bits, equal to the oracle's, in place."""
    xs = gu.make_inputs(n, count, dtype, op, seed=count % 89)
    exp = gu.oracle_all_reduce(xs, dtype, op)
    with ar.Comm(n, 0) as comm:
        for access in ("auto", "streaming", "cached"):
            ar.ar_comm_set_access(comm, access)
            got, _, _ = gu.run_all_reduce(comm, xs, dtype, op, "fused", inplace=True)
            for r in range(n):
                gu.assert_same(got[r], exp[r], dtype, f"access={access} n={n} {dtype} {op} count={count} rank {r}")


def test_access_rejects_unknown_values():
    with ar.Comm(2, 0) as comm:
        for bad in (-1, 3, 99):
            with pytest.raises(ar.ArError) as ei:
                ar.ar_comm_set_access(comm, bad)
            assert ei.value.code == ar.AR_ERR_INVALID_ARGUMENT
        ar.ar_comm_set_access(comm, "cached")
        ar.ar_comm_set_streaming(comm, True)
        ar.ar_comm_set_streaming(comm, False)
