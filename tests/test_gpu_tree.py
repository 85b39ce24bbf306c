"""Tree-order variant (AR_MODE_TREE, AR_MODE_TREE_STEPWISE) against the
oracle's tree, bit for bit; against the ring within the closed-form
tolerance 4*N*eps*sum|x| (plus one output ulp for fp16/bf16); collectives
other than all-reduce refuse the tree modes."""
import numpy as np
import pytest
import torch

import gpu_util as gu
import oracle
import ring_all_reduce_ar_amd as ar
import synthetic

pytestmark = pytest.mark.gpu

DTYPES = ("f32", "f16", "bf16", "i32")
OPS = ("sum", "avg", "max", "min", "prod")


def f64(a, dtype):
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


@pytest.mark.parametrize("mode", ("tree", "tree_stepwise"))
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n", (1, 2, 3, 4, 5, 7, 8, 9, 16, 33, 64))
def test_tree_parity(n, dtype, mode):
    with ar.Comm(n, 0) as comm:
        for op in OPS:
            for count in (1, 3 * 1024 + gu.EPV[dtype], 1000 + 3):
                xs = gu.make_inputs(n, count, dtype, op, seed=31 * n + count)
                exp = oracle.tree_all_reduce([gu.host(x) for x in xs], dtype, op)
                for inplace in (False, True):
                    ws = gu.attach_workspace(comm, ar.AR_COLL_ALL_REDUCE, n, count, dtype, mode)
                    outs, _, _ = gu.run_all_reduce(comm, xs, dtype, op, mode, inplace=inplace)
                    ar.ar_comm_set_workspace(comm, None)
                    del ws
                    for r in range(n):
                        gu.assert_same(outs[r], exp[r], dtype, f"tree n={n} {dtype} {op} {mode} count={count} "
                                                              f"inplace={inplace} rank {r}")


@pytest.mark.parametrize("n,dtype,op,count,mode,inplace", [
    (8, "f32", "sum", 9_000_003, "tree", False),
    (5, "bf16", "avg", 30_000_005, "tree", True),
    (16, "f32", "max", 5_000_001, "tree", False),
    (8, "f16", "prod", 20_000_003, "tree_stepwise", False),
    (7, "f32", "min", 10_000_001, "tree_stepwise", True),
    (33, "i32", "sum", 2_000_003, "tree_stepwise", False),
])
def test_tree_streaming_full_compare(n, dtype, op, count, mode, inplace):
    """Beyond the last-level cache the tree kernels launch one workgroup per
    tile of 256 vectors (tail elements past the last whole vector): every
    element of every rank against the oracle's tree, guard bands."""
    with ar.Comm(n, 0) as comm:
        xs = gu.make_inputs(n, count, dtype, op, seed=n + count % 53)
        exp = oracle.tree_all_reduce([gu.host(x) for x in xs], dtype, op)
        ws = gu.attach_workspace(comm, ar.AR_COLL_ALL_REDUCE, n, count, dtype, mode)
        outs, _, _ = gu.run_all_reduce(comm, xs, dtype, op, mode, inplace=inplace)
        ar.ar_comm_set_workspace(comm, None)
        del ws
        for r in range(n):
            gu.assert_same(outs[r], exp[r], dtype, f"tree n={n} {dtype} {op} {mode} count={count} inplace={inplace} "
                                                  f"rank {r}")
    del xs, exp, outs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ("f32", "f16", "bf16"))
@pytest.mark.parametrize("n", (8, 64))
def test_tree_within_tolerance_of_ring(n, dtype):
    """|tree - ring| <= 4*N*eps*sum|x| (eps = 2^-23), plus one output ulp for
    fp16/bf16 on each side; AVG scales the bound by 1/N."""
    count = n * 4096
    with ar.Comm(n, 0) as comm:
        for op in ("sum", "avg"):
            xs = gu.make_inputs(n, count, dtype, op, seed=5)
            tree, _, _ = gu.run_all_reduce(comm, xs, dtype, op, "tree")
            ring, _, _ = gu.run_all_reduce(comm, xs, dtype, op, "fused")
            x64 = np.stack([f64(gu.host(x), dtype) for x in xs])
            absum = np.abs(x64).sum(axis=0) / (n if op == "avg" else 1)
            ulp = {"f32": 0.0, "f16": 2.0 ** -10, "bf16": 2.0 ** -7}[dtype]
            t, g = f64(tree[0], dtype), f64(ring[0], dtype)
            tol = 4 * n * 2.0 ** -23 * absum + ulp * np.maximum(np.abs(t), np.abs(g)) + 1e-30
            assert np.all(np.abs(t - g) <= tol), (n, dtype, op, float(np.max(np.abs(t - g) - tol)))
            differ = np.count_nonzero(gu.bits(tree[0]) != gu.bits(ring[0]))
            print(f"n={n} {dtype} {op}: {differ} of {count} elements differ from the ring")


def test_tree_sampled_at_full_size():
    """8 ranks x 7e9 fp16 (14 GB each), AVG, fused tree, in place: sampled
    elements against the oracle's tree, all ranks identical."""
    n, count = 8, 7_000_000_000
    with ar.Comm(n, 0) as comm:
        bufs = synthetic.rank_inputs("grad7b", n, count, "f16", device="cuda")
        rng = np.random.default_rng(9)
        idx = np.unique(np.concatenate([rng.integers(0, count, 20000), [0, count - 1]]))
        it = torch.from_numpy(idx).cuda()
        before = torch.stack([b[it] for b in bufs], dim=0).cpu().numpy()  # (n, m)
        exp = oracle.tree_all_reduce([np.ascontiguousarray(before[r]) for r in range(n)], "f16", "avg")[0]
        ptrs = [b.data_ptr() for b in bufs]
        ar.ar_all_reduce(comm, ptrs, ptrs, count, "f16", "avg", "tree")
        torch.cuda.synchronize()
        for r in range(n):
            gu.assert_same(bufs[r][it].cpu().numpy(), exp, "f16", f"tree full size rank {r}")
        for r in range(1, n):
            assert torch.equal(bufs[r].view(torch.uint8), bufs[0].view(torch.uint8))
    del bufs
    torch.cuda.empty_cache()


def test_tree_modes_only_for_all_reduce():
    n = 4
    with ar.Comm(n, 0) as comm:
        s = [gu.RankBuf(n * 8, "f32") for _ in range(n)]
        d = [gu.RankBuf(n * 8, "f32") for _ in range(n)]
        sp, dp = [b.ptr() for b in s], [b.ptr() for b in d]
        for fn, args in ((ar.ar_reduce_scatter, (8, "f32", "sum")), (ar.ar_all_gather, (8, "f32")),
                         (ar.ar_all_to_all, (8, "f32"))):
            for mode in ("tree", "tree_stepwise"):
                with pytest.raises(ar.ArError) as ei:
                    fn(comm, sp, dp, *args, mode)
                assert ei.value.code == ar.AR_ERR_UNSUPPORTED


def test_tree_stepwise_half_needs_workspace():
    n, count = 8, 8 * 100
    with ar.Comm(n, 0) as comm:
        need = ar.ar_workspace_bytes(ar.AR_COLL_ALL_REDUCE, n, count, "f16", "tree_stepwise")
        assert need == 4 * (n // 2) * count
        s = [gu.RankBuf(count, "f16") for _ in range(n)]
        with pytest.raises(ar.ArError) as ei:
            ar.ar_all_reduce(comm, [b.ptr() for b in s], [b.ptr() for b in s], count, "f16", "sum", "tree_stepwise")
        assert ei.value.code == ar.AR_ERR_INVALID_ARGUMENT


def test_tree_step_timing():
    """The stepwise tree takes 2*ceil(log2 N) steps."""
    with ar.Comm(8, 0) as comm:
        xs = gu.make_inputs(8, 8 * 50000, "f32", "sum", seed=1)
        ar.ar_comm_set_step_timing(comm, True)
        gu.run_all_reduce(comm, xs, "f32", "sum", "tree_stepwise")
        assert len(ar.ar_last_step_times_ms(comm)) == 6
        ar.ar_comm_set_step_timing(comm, False)
