"""IEEE special values through every fp path: NaN, +0 and -0, +inf and -inf,
subnormals, the largest finite values (whose sums overflow), mixed with
ordinary values. The library must match the oracle bit for bit with NaN
positions compared and NaN payloads not (the pages fix neither payloads nor
any special-value rule; the oracle's readings are: NaN-propagating MAX/MIN
with +0 > -0, IEEE arithmetic with subnormals kept, one RNE conversion to
fp16/bf16 at the end)."""
import numpy as np
import pytest
import torch

import gpu_util as gu
import oracle
import ring_all_reduce_ar_amd as ar

pytestmark = pytest.mark.gpu

SPECIALS = {
    "f32": [0.0, -0.0, np.nan, np.inf, -np.inf, 1e-40, -1e-40, 1.4e-45, 3.0e38, -3.0e38, 1.0, -1.0],
    "f16": [0.0, -0.0, np.nan, np.inf, -np.inf, 6e-8, -6e-8, 3e-5, 65504.0, -65504.0, 1.0, -1.0],
    "bf16": [0.0, -0.0, np.nan, np.inf, -np.inf, 1e-39, -1e-39, 3.0e38, -3.0e38, 1.0, -1.0],
}


def special_inputs(n, count, dtype, seed, frac):
    """Per-rank tensors: uniform[-2, 2) values, each element replaced with
    probability `frac` by one of the special values."""
    rng = np.random.default_rng(seed)
    vals = rng.uniform(-2.0, 2.0, size=(n, count))
    pick = rng.random(size=(n, count)) < frac
    table = np.array(SPECIALS[dtype], dtype=np.float64)
    vals[pick] = table[rng.integers(0, table.size, size=int(pick.sum()))]
    t = torch.from_numpy(vals.astype(np.float32)).to(gu.TORCH[dtype])
    return [t[r].contiguous().to("cuda") for r in range(n)]


@pytest.mark.parametrize("mode", ("fused", "stepwise", "graph", "tree", "tree_stepwise"))
@pytest.mark.parametrize("dtype", ("f32", "f16", "bf16"))
@pytest.mark.parametrize("n", (2, 3, 8))
def test_special_values(n, dtype, mode):
    count = n * (4096 + 8) + 5
    with ar.Comm(n, 0) as comm:
        for k, op in enumerate(("sum", "avg", "max", "min", "prod")):
            # a low rate keeps most sums finite, so the ordinary values still
            # decide many bits; a high rate exercises the special-value rules
            for frac in (0.02, 0.5):
                xs = special_inputs(n, count, dtype, seed=1000 * n + 10 * k + int(frac * 10), frac=frac)
                hosts = [gu.host(x) for x in xs]
                exp = (oracle.tree_all_reduce(hosts, dtype, op) if mode.startswith("tree")
                       else oracle.fold_all_reduce(hosts, dtype, op))
                ws = gu.attach_workspace(comm, ar.AR_COLL_ALL_REDUCE, n, count, dtype, mode)
                outs, _, _ = gu.run_all_reduce(comm, xs, dtype, op, mode)
                del ws
                for r in range(n):
                    gu.assert_same(outs[r], exp[r], dtype, f"n={n} {dtype} {op} {mode} frac={frac} rank {r}")


@pytest.mark.parametrize("streaming", (False, True))
@pytest.mark.parametrize("dtype", ("f32", "f16", "bf16"))
def test_special_values_multi_and_scatter(dtype, streaming):
    n = 8
    count = n * (4096 + 8)
    with ar.Comm(n, 0) as comm:
        ar.ar_comm_set_streaming(comm, streaming)
        for k, op in enumerate(("sum", "max", "min", "prod")):
            xs = special_inputs(n, count, dtype, seed=77 + k, frac=0.3)
            hosts = [gu.host(x) for x in xs]
            exp = oracle.fold_all_reduce(hosts, dtype, op)
            cuts = [0, 3, count // 3, count]
            sizes = [b - a for a, b in zip(cuts[:-1], cuts[1:])]
            bufs = [[gu.RankBuf(s, dtype) for _ in range(n)] for s in sizes]
            for t, a in enumerate(cuts[:-1]):
                for r in range(n):
                    bufs[t][r].view.copy_(xs[r][a:a + sizes[t]])
            ptrs = [[b.ptr() for b in row] for row in bufs]
            ar.ar_all_reduce_multi(comm, ptrs, ptrs, sizes, dtype, op)
            torch.cuda.synchronize()
            for r in range(n):
                got = np.concatenate([gu.host(bufs[t][r].view) for t in range(len(sizes))])
                gu.assert_same(got, exp[r], dtype, f"multi {dtype} {op} streaming={streaming} rank {r}")
            # reduce-scatter: rank r gets chunk r of the all-reduce
            q = count // n
            rs_exp = oracle.reduce_scatter(hosts, dtype, op)
            recv = [gu.RankBuf(q, dtype) for _ in range(n)]
            ar.ar_reduce_scatter(comm, [x.data_ptr() for x in xs], [b.ptr() for b in recv], q, dtype, op, "fused")
            torch.cuda.synchronize()
            for r in range(n):
                gu.assert_same(gu.host(recv[r].view), rs_exp[r], dtype, f"rs {dtype} {op} streaming={streaming} rank {r}")
                gu.assert_same(gu.host(recv[r].view), exp[r][r * q:(r + 1) * q], dtype, f"rs vs ar rank {r}")


@pytest.mark.parametrize("mode", ("fused", "stepwise", "tree"))
@pytest.mark.parametrize("n", (2, 3, 8))
def test_int32_wrap_and_truncation(n, mode):
    """int32 at the type's limits: SUM and PROD wrap modulo 2^32, AVG of the
    wrapped sum truncates toward zero (negative sums included), MAX/MIN see
    INT32_MIN and INT32_MAX; against the oracle, bit for bit."""
    count = n * (4096 + 4) + 3
    rng = np.random.default_rng(50 + n)
    edge = np.array([2**31 - 1, -2**31, 2**31 - 2, -2**31 + 1, 0, -1, 1, 2**30, -2**30, 7, -7], dtype=np.int64)
    with ar.Comm(n, 0) as comm:
        for op in ("sum", "avg", "max", "min", "prod"):
            vals = rng.integers(-2**31, 2**31, size=(n, count), dtype=np.int64)
            pick = rng.random((n, count)) < 0.3
            vals[pick] = edge[rng.integers(0, edge.size, size=int(pick.sum()))]
            xs = [torch.from_numpy(vals[r].astype(np.int32)).cuda() for r in range(n)]
            hosts = [gu.host(x) for x in xs]
            exp = oracle.tree_all_reduce(hosts, "i32", op) if mode == "tree" else oracle.fold_all_reduce(hosts, "i32", op)
            outs, _, _ = gu.run_all_reduce(comm, xs, "i32", op, mode)
            for r in range(n):
                gu.assert_same(outs[r], exp[r], "i32", f"n={n} i32 {op} {mode} rank {r}")


@pytest.mark.parametrize("n", (3, 8, 16))
def test_special_values_streaming(n):
    """Special values through the streaming one-launch kernels (the
    rank-major fold for ring order, the tree fold), forced at small sizes by
    ar_comm_set_streaming; bit for bit against the oracle."""
    count = n * (4096 + 8) + 5
    with ar.Comm(n, 0) as comm:
        ar.ar_comm_set_streaming(comm, True)
        for dtype in ("f32", "f16", "bf16"):
            for k, op in enumerate(("sum", "avg", "max", "min", "prod")):
                xs = special_inputs(n, count, dtype, seed=3000 + 10 * n + k, frac=0.1)
                hosts = [gu.host(x) for x in xs]
                for mode in ("fused", "tree"):
                    exp = (oracle.tree_all_reduce(hosts, dtype, op) if mode == "tree"
                           else oracle.fold_all_reduce(hosts, dtype, op))
                    outs, _, _ = gu.run_all_reduce(comm, xs, dtype, op, mode, inplace=k % 2 == 0)
                    for r in range(n):
                        gu.assert_same(outs[r], exp[r], dtype, f"streaming n={n} {dtype} {op} {mode} rank {r}")


@pytest.mark.parametrize("dtype,ops", [("f16", ("sum", "max", "avg")), ("bf16", ("prod", "min"))])
def test_special_values_tiled_ring_steps(dtype, ops):
    """Special values through the tiled 16-bit ring steps (half vectors per
    lane, fp32 partials in the workspace): 8 ranks x 16,777,003 elements in
    place (a footprint just under the last-level cache: cached steps) and out
    of place (streaming steps), then the stepwise reduce-scatter at 8 x
    2,100,008 out (streaming)."""
    from test_gpu_parity import _reduce_scatter
    n, count = 8, 16_777_003
    with ar.Comm(n, 0) as comm:
        ws = gu.attach_workspace(comm, ar.AR_COLL_ALL_REDUCE, n, count, dtype, "stepwise")
        for k, op in enumerate(ops):
            xs = special_inputs(n, count, dtype, seed=4000 + k, frac=0.05)
            exp = oracle.fold_all_reduce([gu.host(x) for x in xs], dtype, op)
            for inplace in (True, False):
                outs, send, recv = gu.run_all_reduce(comm, xs, dtype, op, "stepwise", inplace=inplace)
                del send, recv
                for r in range(n):
                    gu.assert_same(outs[r], exp[r], dtype, f"tiled steps {dtype} {op} inplace={inplace} rank {r}")
            del xs, exp, outs
        ar.ar_comm_set_workspace(comm, None)
        del ws
        rc = 2_100_008
        xs = special_inputs(n, n * rc, dtype, seed=4100, frac=0.05)
        exp = oracle.reduce_scatter([gu.host(x) for x in xs], dtype, ops[0])
        got = _reduce_scatter(comm, xs, dtype, ops[0], "stepwise", False)
        for r in range(n):
            gu.assert_same(got[r], exp[r], dtype, f"tiled RS steps {dtype} {ops[0]} rank {r}")
    del xs, exp, got
    torch.cuda.empty_cache()
