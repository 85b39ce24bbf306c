"""Graph-captured ring (AR_MODE_RING_GRAPH) and capture safety of the other
modes: same bits as the oracle, cached graphs replay correctly after the
buffers change, the cache evicts, a caller's own torch.cuda.graph capture of
the fused and stepwise calls replays correctly between eager work."""
import pytest
import torch

import gpu_util as gu
import oracle
import ring_all_reduce_ar_amd as ar

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i32"])
@pytest.mark.parametrize("n", [2, 3, 8, 64])
def test_graph_mode_parity(n, dtype):
    with ar.Comm(n, 0) as comm:
        for op in ("sum", "avg", "max", "prod"):
            for count in (n * (1024 + gu.EPV[dtype]), n * 1000 + 7):
                xs = gu.make_inputs(n, count, dtype, op, seed=count)
                exp = gu.oracle_all_reduce(xs, dtype, op)
                ws = gu.attach_workspace(comm, ar.AR_COLL_ALL_REDUCE, n, count, dtype, "graph")
                outs, _, _ = gu.run_all_reduce(comm, xs, dtype, op, "graph")
                for r in range(n):
                    gu.assert_same(outs[r], exp[r], dtype, f"graph n={n} {dtype} {op} count={count} rank {r}")
                ar.ar_comm_set_workspace(comm, None)
                del ws


def test_graph_cache_hit_sees_new_contents():
    """Same pointers, new contents: the cached graph computes on the new data."""
    n, count, dtype = 8, 8 * 4096, "f16"
    with ar.Comm(n, 0) as comm:
        bufs = [gu.RankBuf(count, dtype) for _ in range(n)]
        ws = gu.attach_workspace(comm, ar.AR_COLL_ALL_REDUCE, n, count, dtype, "graph")
        ptrs = [b.ptr() for b in bufs]
        for trial in range(4):
            xs = gu.make_inputs(n, count, dtype, "sum", seed=100 + trial)
            for b, x in zip(bufs, xs):
                b.view.copy_(x)
            exp = gu.oracle_all_reduce(xs, dtype, "sum")
            ar.ar_all_reduce(comm, ptrs, ptrs, count, dtype, "sum", "graph")
            torch.cuda.synchronize()
            for r in range(n):
                assert bufs[r].guards_ok()
                gu.assert_same(gu.host(bufs[r].view), exp[r], dtype, f"trial {trial} rank {r}")
        ar.ar_comm_set_workspace(comm, None)
        del ws


def test_graph_cache_eviction():
    """More distinct signatures than the cache holds: every call still correct."""
    n = 4
    with ar.Comm(n, 0) as comm:
        for k in range(20):
            count = n * (256 + 4 * k)
            xs = gu.make_inputs(n, count, "f32", "sum", seed=k)
            exp = gu.oracle_all_reduce(xs, "f32", "sum")
            outs, _, _ = gu.run_all_reduce(comm, xs, "f32", "sum", "graph")
            for r in range(n):
                gu.assert_same(outs[r], exp[r], "f32", f"eviction k={k} rank {r}")


# The refused call enqueues nothing, so the capture ends empty by design.
@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_graph_mode_refused_inside_capture():
    n, count = 4, 4 * 256
    with ar.Comm(n, 0) as comm:
        bufs = [torch.zeros(count, device="cuda") for _ in range(n)]
        ptrs = [b.data_ptr() for b in bufs]
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.capture_begin()
            try:
                with pytest.raises(ar.ArError) as ei:
                    ar.ar_all_reduce(comm, ptrs, ptrs, count, "f32", "sum", "graph", s)
                assert ei.value.code == ar.AR_ERR_INVALID_ARGUMENT
            finally:
                g.capture_end()


@pytest.mark.parametrize("mode", ["fused", "stepwise"])
def test_caller_capture_replays(mode):
    """A caller captures out-of-place all-reduces in torch.cuda.graph; every
    replay, with eager work and synchronisation between replays, matches the
    eager result and the oracle."""
    n, count, dtype = 8, 8 * 8192 + 3, "bf16"
    with ar.Comm(n, 0) as comm:
        send = [gu.RankBuf(count, dtype) for _ in range(n)]
        recv = [gu.RankBuf(count, dtype) for _ in range(n)]
        ws = gu.attach_workspace(comm, ar.AR_COLL_ALL_REDUCE, n, count, dtype, mode)
        sp, rp = [b.ptr() for b in send], [b.ptr() for b in recv]
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            ar.ar_all_reduce(comm, sp, rp, count, dtype, "avg", mode, s)
        for trial in range(4):
            xs = gu.make_inputs(n, count, dtype, "avg", seed=200 + trial)
            for b, x in zip(send, xs):
                b.view.copy_(x)
            for b in recv:
                b.view.fill_(0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            exp = gu.oracle_all_reduce(xs, dtype, "avg")
            got = [gu.host(b.view) for b in recv]
            eager = [gu.RankBuf(count, dtype) for _ in range(n)]
            ar.ar_all_reduce(comm, sp, [b.ptr() for b in eager], count, dtype, "avg", mode)
            torch.cuda.synchronize()
            for r in range(n):
                assert recv[r].guards_ok()
                gu.assert_same(got[r], exp[r], dtype, f"replay {trial} rank {r}")
                gu.assert_same(gu.host(eager[r].view), got[r], dtype, f"eager vs replay {trial} rank {r}")
        ar.ar_comm_set_workspace(comm, None)
        del ws


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i32"])
@pytest.mark.parametrize("n", [2, 5, 8])
def test_graph_mode_reduce_scatter_and_all_gather(n, dtype):
    """The graph-replayed ring for the reduce-scatter and all-gather exports:
    the first call captures, the later ones (same pointers, new contents)
    replay; each against the oracle."""
    with ar.Comm(n, 0) as comm:
        rc = 1024 + gu.EPV[dtype]
        send = [gu.RankBuf(n * rc, dtype) for _ in range(n)]
        recv = [gu.RankBuf(rc, dtype) for _ in range(n)]
        gathered = [gu.RankBuf(n * rc, dtype) for _ in range(n)]
        ws = gu.attach_workspace(comm, ar.AR_COLL_REDUCE_SCATTER, n, rc, dtype, "graph")
        for trial in range(3):
            xs = gu.make_inputs(n, n * rc, dtype, "avg", seed=trial)
            for b, x in zip(send, xs):
                b.view.copy_(x)
            ar.ar_reduce_scatter(comm, [b.ptr() for b in send], [b.ptr() for b in recv], rc, dtype, "avg", "graph")
            ar.ar_all_gather(comm, [b.ptr() for b in recv], [b.ptr() for b in gathered], rc, dtype, "graph")
            torch.cuda.synchronize()
            exp = oracle.reduce_scatter([gu.host(x) for x in xs], dtype, "avg")
            exp_ag = oracle.all_gather(exp, dtype)
            for r in range(n):
                assert recv[r].guards_ok() and gathered[r].guards_ok()
                gu.assert_same(gu.host(recv[r].view), exp[r], dtype, f"graph RS n={n} trial {trial} rank {r}")
                gu.assert_same(gu.host(gathered[r].view), exp_ag[r], dtype, f"graph AG n={n} trial {trial} rank {r}")
        ar.ar_comm_set_workspace(comm, None)
        del ws
