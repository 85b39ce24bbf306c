"""Seeded random shapes through the C ABI against the oracle, bit for bit:
rank counts 1..64 (every remainder of the 8-rank batches of the
any-rank-count kernels), ragged sizes, every dtype and op, fused and
stepwise, in and out of place, and buffers shifted off 16-byte alignment."""
import numpy as np
import pytest
import torch

import gpu_util as gu
import oracle
import ring_all_reduce_ar_amd as ar

pytestmark = pytest.mark.gpu

DTYPES = ("f32", "f16", "bf16", "i32")
OPS = ("sum", "avg", "max", "min", "prod")


def _cases(seed, k):
    rng = np.random.default_rng(seed)
    for i in range(k):
        n = int(rng.integers(1, 65))
        per = int(rng.integers(1, max(2, 3_000_000 // n)))
        count = int(rng.integers(0, min(per, 200_000) + 1))
        yield (i, n, count, DTYPES[int(rng.integers(4))], OPS[int(rng.integers(5))],
               ("fused", "stepwise")[int(rng.integers(2))], bool(rng.integers(2)), int(rng.integers(0, 2)))


@pytest.mark.parametrize("case", list(_cases(2024, 60)), ids=lambda c: f"ar{c[0]}-n{c[1]}-{c[3]}-{c[4]}-{c[5]}")
def test_random_all_reduce(case):
    i, n, count, dtype, op, mode, inplace, shifted = case
    xs = gu.make_inputs(n, count, dtype, op, seed=1000 + i)
    offset = gu.ESIZE[dtype] if shifted else 0
    with ar.Comm(n, 0) as comm:
        ws = gu.attach_workspace(comm, ar.AR_COLL_ALL_REDUCE, n, count, dtype, mode)
        outs, _, _ = gu.run_all_reduce(comm, xs, dtype, op, mode, inplace=inplace, offset=offset)
        del ws
    if count == 0:
        return
    exp = gu.oracle_all_reduce(xs, dtype, op)
    for r in range(n):
        gu.assert_same(outs[r], exp[r], dtype, f"case {case} rank {r}")


@pytest.mark.parametrize("case", list(_cases(7, 30)), ids=lambda c: f"rs{c[0]}-n{c[1]}-{c[3]}-{c[4]}-{c[5]}")
def test_random_reduce_scatter(case):
    i, n, count, dtype, op, mode, inplace, _ = case
    rc = max(1, count // n)
    xs = gu.make_inputs(n, n * rc, dtype, op, seed=2000 + i)
    exp = oracle.reduce_scatter([gu.host(x) for x in xs], dtype, op)
    with ar.Comm(n, 0) as comm:
        send = [gu.RankBuf(n * rc, dtype) for _ in range(n)]
        for b, x in zip(send, xs):
            b.view.copy_(x)
        recv = [] if inplace else [gu.RankBuf(rc, dtype) for _ in range(n)]
        recv_ptrs = [send[r].sub_ptr(r * rc) for r in range(n)] if inplace else [b.ptr() for b in recv]
        ws = gu.attach_workspace(comm, ar.AR_COLL_REDUCE_SCATTER, n, rc, dtype, mode)
        ar.ar_reduce_scatter(comm, [b.ptr() for b in send], recv_ptrs, rc, dtype, op, mode)
        torch.cuda.synchronize()
        del ws
        for b in send + recv:
            assert b.guards_ok()
        for r in range(n):
            got = gu.host(send[r].view[r * rc:(r + 1) * rc]) if inplace else gu.host(recv[r].view)
            gu.assert_same(got, exp[r], dtype, f"case {case} rank {r}")


@pytest.mark.parametrize("case", list(_cases(99, 30)), ids=lambda c: f"ag{c[0]}-n{c[1]}-{c[3]}-{c[5]}")
def test_random_all_gather_and_all_to_all(case):
    i, n, count, dtype, _, mode, inplace, _ = case
    sc = max(1, count // n)
    xs = gu.make_inputs(n, sc, dtype, "sum", seed=3000 + i)
    exp = oracle.all_gather([gu.host(x) for x in xs], dtype)
    with ar.Comm(n, 0) as comm:
        recv = [gu.RankBuf(n * sc, dtype) for _ in range(n)]
        if inplace:
            for r in range(n):
                recv[r].view[r * sc:(r + 1) * sc].copy_(xs[r])
            send, send_ptrs = [], [recv[r].sub_ptr(r * sc) for r in range(n)]
        else:
            send = [gu.RankBuf(sc, dtype) for _ in range(n)]
            for b, x in zip(send, xs):
                b.view.copy_(x)
            send_ptrs = [b.ptr() for b in send]
        ar.ar_all_gather(comm, send_ptrs, [b.ptr() for b in recv], sc, dtype, mode)
        torch.cuda.synchronize()
        for b in send + recv:
            assert b.guards_ok()
        for r in range(n):
            gu.assert_same(gu.host(recv[r].view), exp[r], dtype, f"all-gather case {case} rank {r}")
        # all-to-all over the gathered buffers (n blocks of sc per rank)
        a_in = [b.view.clone() for b in recv]
        a_exp = oracle.all_to_all([gu.host(x) for x in a_in], dtype)
        a_out = [gu.RankBuf(n * sc, dtype) for _ in range(n)]
        ar.ar_all_to_all(comm, [x.data_ptr() for x in a_in], [b.ptr() for b in a_out], sc, dtype, mode)
        torch.cuda.synchronize()
        for r in range(n):
            assert a_out[r].guards_ok()
            gu.assert_same(gu.host(a_out[r].view), a_exp[r], dtype, f"all-to-all case {case} rank {r}")


def _large_cases(seed, k):
    rng = np.random.default_rng(seed)
    for i in range(k):
        n = int(rng.integers(5, 9))
        dtype = DTYPES[int(rng.integers(4))]
        nbytes = int(rng.integers(130 << 20, 600 << 20))
        count = nbytes // gu.ESIZE[dtype] - int(rng.integers(0, 9))
        yield (i, n, count, dtype, OPS[int(rng.integers(5))])


@pytest.mark.parametrize("case", list(_large_cases(31, 10)), ids=lambda c: f"big{c[0]}-n{c[1]}-{c[3]}-{c[4]}")
def test_random_large_all_reduce_sampled(case):
    """130-600 MB per rank at 5-8 ranks (the rank-major, non-temporal kernels),
    in place: sampled elements (every chunk boundary among them) against the
    oracle, all ranks identical."""
    import test_gpu_full_size as fs
    i, n, count, dtype, op = case
    with ar.Comm(n, 0) as comm:
        bufs = gu.make_inputs(n, count, dtype, op, seed=4000 + i)
        fs.check_sampled(comm, bufs, dtype, op, "fused", seed=i)
        del bufs
    fs.free()
