"""GPU library vs the CPU oracle, element by element and bit for bit, through
the C ABI: all-reduce, reduce-scatter and all-gather in both modes, every
dtype and op, in and out of place, aligned and unaligned, with chunk
lengths that span several 256-thread tiles, ragged last chunks, empty
chunks and the degenerate single-rank case."""
import numpy as np
import pytest
import torch

import gpu_util as gu
import goldens
import oracle
import ring_all_reduce_ar_amd as ar

pytestmark = pytest.mark.gpu

DTYPES = ("f32", "f16", "bf16", "i32")
OPS = ("sum", "avg", "max", "min", "prod")
MODES = ("fused", "stepwise")
NS = (1, 2, 3, 4, 5, 7, 8, 9, 16, 64)


@pytest.fixture(scope="module")
def comm_for():
    comms = {}

    def get(n):
        if n not in comms:
            comms[n] = ar.Comm(n, 0)
        return comms[n]

    yield get
    for c in comms.values():
        c.close()


def counts_for(n, dtype):
    """0, fewer elements than ranks (empty chunks), a vector-path size whose
    chunks span several tiles, the same with a ragged last chunk, and a size
    whose chunk length is not a whole number of 16-byte vectors."""
    q1 = 4096 + gu.EPV[dtype]
    out = [0, 1, n - 1, n * q1, n * q1 - 3, n * q1 + 5]
    return sorted({c for c in out if c >= 0})


def test_worked_example(comm_for):
    """The handbook's printed 4-rank example through the library, both modes."""
    g = goldens.load("collectives_4rank_example.txt")
    comm = comm_for(4)
    for dtype in DTYPES:
        for mode in MODES:
            xs = [torch.tensor(goldens.numbers(g[f"input.{r}"]), dtype=gu.TORCH[dtype], device="cuda") for r in range(4)]
            ws = gu.attach_workspace(comm, ar.AR_COLL_ALL_REDUCE, 4, 4, dtype, mode)
            outs, _, _ = gu.run_all_reduce(comm, xs, dtype, "sum", mode)
            for r in range(4):
                exp = goldens.numbers(g[f"all_reduce.{r}"])
                got = torch.from_numpy(outs[r].view(np.int16)).view(torch.bfloat16).float().tolist() \
                    if dtype == "bf16" else outs[r].astype(np.float64).tolist()
                assert got == exp, (dtype, mode, r, got)
            del ws


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("inplace", [False, True])
def test_small_config_bit_exact(comm_for, mode, inplace):
    """4 ranks x 4096 fp32 uniform[-1, 1), SUM: bit-exact with the ring."""
    import synthetic
    xs = synthetic.rank_inputs("small", 4, 4096, "f32", device="cuda")
    outs, _, _ = gu.run_all_reduce(comm_for(4), xs, "f32", "sum", mode, inplace=inplace)
    exp = gu.oracle_all_reduce(xs, "f32", "sum")
    ring = [gu.host(x) for x in xs]
    oracle.ring_all_reduce(ring, "f32", "sum")
    for r in range(4):
        gu.assert_same(outs[r], exp[r], "f32", f"rank {r}")
        gu.assert_same(outs[r], ring[r], "f32", f"rank {r} vs ring")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n", NS)
def test_all_reduce_parity(comm_for, n, dtype, mode):
    comm = comm_for(n)
    for op in OPS:
        for count in counts_for(n, dtype):
            xs = gu.make_inputs(n, count, dtype, op, seed=7 * n + count)
            exp = gu.oracle_all_reduce(xs, dtype, op) if count else None
            for inplace in (False, True):
                ws = gu.attach_workspace(comm, ar.AR_COLL_ALL_REDUCE, n, count, dtype, mode)
                outs, _, _ = gu.run_all_reduce(comm, xs, dtype, op, mode, inplace=inplace)
                del ws
                if count == 0:
                    continue
                for r in range(n):
                    gu.assert_same(outs[r], exp[r], dtype, f"n={n} {dtype} {op} {mode} count={count} "
                                                          f"inplace={inplace} rank {r}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n", (2, 3, 8, 64))
def test_all_reduce_unaligned(comm_for, n, dtype, mode):
    """Buffers shifted by one element off 16-byte alignment take the
    element-wise kernels and still match bit for bit."""
    comm = comm_for(n)
    count = n * 1000 + 3
    for op in ("sum", "avg", "max"):
        xs = gu.make_inputs(n, count, dtype, op, seed=11)
        exp = gu.oracle_all_reduce(xs, dtype, op)
        ws = gu.attach_workspace(comm, ar.AR_COLL_ALL_REDUCE, n, count, dtype, mode)
        outs, _, _ = gu.run_all_reduce(comm, xs, dtype, op, mode, offset=gu.ESIZE[dtype])
        del ws
        for r in range(n):
            gu.assert_same(outs[r], exp[r], dtype, f"unaligned n={n} {dtype} {op} {mode} rank {r}")


def _reduce_scatter(comm, xs, dtype, op, mode, inplace):
    n = len(xs)
    rc = xs[0].numel() // n
    send = [gu.RankBuf(n * rc, dtype) for _ in range(n)]
    for b, x in zip(send, xs):
        b.view.copy_(x)
    if inplace:
        recv_ptrs = [send[r].sub_ptr(r * rc) for r in range(n)]
    else:
        recv = [gu.RankBuf(rc, dtype) for _ in range(n)]
        recv_ptrs = [b.ptr() for b in recv]
    ws = gu.attach_workspace(comm, ar.AR_COLL_REDUCE_SCATTER, n, rc, dtype, mode)
    ar.ar_reduce_scatter(comm, [b.ptr() for b in send], recv_ptrs, rc, dtype, op, mode)
    torch.cuda.synchronize()
    del ws
    for b in send + ([] if inplace else recv):
        assert b.guards_ok()
    if inplace:
        return [gu.host(send[r].view[r * rc:(r + 1) * rc]) for r in range(n)]
    return [gu.host(b.view) for b in recv]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n", (1, 2, 3, 4, 8, 16, 64))
def test_reduce_scatter_parity(comm_for, n, dtype, mode):
    """Rank c receives block c of the reduction (handbook, section 五个原语)."""
    comm = comm_for(n)
    for op in OPS:
        for rc in (1, 3 * 1024 + gu.EPV[dtype], 1000 + 3):
            xs = gu.make_inputs(n, n * rc, dtype, op, seed=rc + n)
            exp = oracle.reduce_scatter([gu.host(x) for x in xs], dtype, op)
            for inplace in (False, True):
                got = _reduce_scatter(comm, xs, dtype, op, mode, inplace)
                for r in range(n):
                    gu.assert_same(got[r], exp[r], dtype, f"RS n={n} {dtype} {op} {mode} rc={rc} "
                                                         f"inplace={inplace} rank {r}")


def _all_gather(comm, xs, dtype, mode, inplace):
    n = len(xs)
    sc = xs[0].numel()
    recv = [gu.RankBuf(n * sc, dtype) for _ in range(n)]
    if inplace:
        for r in range(n):
            recv[r].view[r * sc:(r + 1) * sc].copy_(xs[r])
        send_ptrs = [recv[r].sub_ptr(r * sc) for r in range(n)]
        send = []
    else:
        send = [gu.RankBuf(sc, dtype) for _ in range(n)]
        for b, x in zip(send, xs):
            b.view.copy_(x)
        send_ptrs = [b.ptr() for b in send]
    ar.ar_all_gather(comm, send_ptrs, [b.ptr() for b in recv], sc, dtype, mode)
    torch.cuda.synchronize()
    for b in send + recv:
        assert b.guards_ok()
    return [gu.host(b.view) for b in recv]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n", (1, 2, 3, 4, 8, 16, 64))
def test_all_gather_parity(comm_for, n, dtype, mode):
    """Every rank receives the send blocks in rank order."""
    comm = comm_for(n)
    for sc in (1, 3 * 1024 + gu.EPV[dtype], 1000 + 3):
        xs = gu.make_inputs(n, sc, dtype, "sum", seed=sc)
        exp = oracle.all_gather([gu.host(x) for x in xs], dtype)
        for inplace in (False, True):
            got = _all_gather(comm, xs, dtype, mode, inplace)
            for r in range(n):
                gu.assert_same(got[r], exp[r], dtype, f"AG n={n} {dtype} {mode} sc={sc} inplace={inplace} rank {r}")


@pytest.mark.parametrize("n", (2, 4, 8, 64))
def test_rs_then_ag_equals_ar(comm_for, n):
    """Reduce-scatter then all-gather equals all-reduce, bit for bit, on the GPU."""
    comm = comm_for(n)
    for dtype in DTYPES:
        rc = 2048 + gu.EPV[dtype]
        xs = gu.make_inputs(n, n * rc, dtype, "sum", seed=5)
        ar_out, _, _ = gu.run_all_reduce(comm, xs, dtype, "sum", "fused")
        blocks = _reduce_scatter(comm, xs, dtype, "sum", "fused", False)
        gathered = _all_gather(comm, [torch.from_numpy(b.view(np.int16)).view(gu.TORCH[dtype]).cuda()
                                      if dtype == "bf16" else torch.from_numpy(b).cuda() for b in blocks],
                               dtype, "fused", False)
        for r in range(n):
            gu.assert_same(gathered[r], ar_out[r], dtype, f"RS+AG vs AR n={n} {dtype} rank {r}")


def test_deterministic_and_modes_agree(comm_for):
    """Same inputs, same bits: twice in each mode, and across modes."""
    n, count = 8, 8 * 65536
    comm = comm_for(n)
    for dtype in DTYPES:
        xs = gu.make_inputs(n, count, dtype, "sum", seed=3)
        ws = gu.attach_workspace(comm, ar.AR_COLL_ALL_REDUCE, n, count, dtype, "stepwise")
        runs = [gu.run_all_reduce(comm, xs, dtype, "sum", mode)[0][0] for mode in ("fused", "fused", "stepwise",
                                                                                  "stepwise")]
        del ws
        for other in runs[1:]:
            gu.assert_same(other, runs[0], dtype, f"determinism {dtype}")


def test_side_stream(comm_for):
    """Work enqueued on a non-default stream is ordered on that stream."""
    n, count = 4, 4 * 100000
    comm = comm_for(n)
    xs = gu.make_inputs(n, count, "f32", "sum", seed=1)
    exp = gu.oracle_all_reduce(xs, "f32", "sum")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        outs, _, _ = gu.run_all_reduce(comm, xs, "f32", "sum", "stepwise", stream=s)
    for r in range(n):
        gu.assert_same(outs[r], exp[r], "f32", f"side stream rank {r}")


def test_step_timing(comm_for):
    """Stepwise calls time 2(N-1) steps; fused calls one interval."""
    n = 8
    comm = comm_for(n)
    xs = gu.make_inputs(n, n * 100000, "f32", "sum", seed=2)
    ar.ar_comm_set_step_timing(comm, True)
    try:
        gu.run_all_reduce(comm, xs, "f32", "sum", "stepwise")
        t = ar.ar_last_step_times_ms(comm)
        assert len(t) == 2 * (n - 1) and all(v > 0 for v in t), t
        gu.run_all_reduce(comm, xs, "f32", "sum", "fused")
        t = ar.ar_last_step_times_ms(comm)
        assert len(t) == 1 and t[0] > 0
    finally:
        ar.ar_comm_set_step_timing(comm, False)
    with pytest.raises(ar.ArError):
        ar.ar_last_step_times_ms(comm)


def _all_to_all(comm, xs, dtype, mode):
    n = len(xs)
    total = xs[0].numel()
    send = [gu.RankBuf(total, dtype) for _ in range(n)]
    for b, x in zip(send, xs):
        b.view.copy_(x)
    recv = [gu.RankBuf(total, dtype) for _ in range(n)]
    ar.ar_all_to_all(comm, [b.ptr() for b in send], [b.ptr() for b in recv], total // n, dtype, mode)
    torch.cuda.synchronize()
    for b in send + recv:
        assert b.guards_ok()
    return [gu.host(b.view) for b in recv]


def test_all_to_all_worked_example(comm_for):
    """Rank p receives [p, 10+p, 20+p, 30+p] (handbook, section 五个原语)."""
    g = goldens.load("collectives_4rank_example.txt")
    for mode in ("fused", "stepwise", "graph"):
        xs = [torch.tensor(goldens.numbers(g[f"input.{r}"]), dtype=torch.float32, device="cuda") for r in range(4)]
        got = _all_to_all(comm_for(4), xs, "f32", mode)
        for p in range(4):
            assert got[p].astype(np.float64).tolist() == goldens.numbers(g[f"all_to_all.{p}"]), (mode, p, got[p])


@pytest.mark.parametrize("mode", ("fused", "stepwise", "graph"))
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n", (1, 2, 3, 4, 8, 16, 64))
def test_all_to_all_parity(comm_for, n, dtype, mode):
    comm = comm_for(n)
    for bc in (1, 2048 + gu.EPV[dtype], 1000 + 3):
        xs = gu.make_inputs(n, n * bc, dtype, "sum", seed=bc + 3 * n)
        exp = oracle.all_to_all([gu.host(x) for x in xs], dtype)
        got = _all_to_all(comm, xs, dtype, mode)
        for p in range(n):
            gu.assert_same(got[p], exp[p], dtype, f"A2A n={n} {dtype} {mode} bc={bc} rank {p}")
