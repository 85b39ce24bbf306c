"""Coalesced multi-tensor all-reduce (ar_all_reduce_multi): every tensor
element gets the bits of the flat-bucket all-reduce of the concatenated
tensors (the oracle's fold over the bucket, and ar_all_reduce on a packed
copy), with separate allocations per tensor and rank, empty and odd-sized
tensors, unaligned tensors, in place, many launches' worth of tensors, and
the 64-rank mixed-size bucket at full size."""
import numpy as np
import pytest
import torch

import gpu_util as gu
import oracle
import ring_all_reduce_ar_amd as ar
import synthetic

pytestmark = pytest.mark.gpu


def run_multi(comm, sizes, dtype, op, seed, inplace=False, offset=0):
    n = comm.nranks
    total = sum(sizes)
    flat = gu.make_inputs(n, total, dtype, op, seed=seed)  # the bucket each rank would hold
    send, recv = [], []
    off = 0
    for c in sizes:
        srow = [gu.RankBuf(c, dtype, offset=offset) for _ in range(n)]
        for r in range(n):
            srow[r].view.copy_(flat[r][off:off + c])
        send.append(srow)
        recv.append(srow if inplace else [gu.RankBuf(c, dtype, offset=offset) for _ in range(n)])
        off += c
    ar.ar_all_reduce_multi(comm, [[b.ptr() for b in row] for row in send], [[b.ptr() for b in row] for row in recv],
                           sizes, dtype, op)
    torch.cuda.synchronize()
    for row in send + recv:
        for b in row:
            assert b.guards_ok()
    got = [np.concatenate([gu.host(recv[t][r].view) for t in range(len(sizes))]) if sizes else None
           for r in range(n)]
    return flat, got


def check(comm, sizes, dtype, op, seed, **kw):
    n = comm.nranks
    flat, got = run_multi(comm, sizes, dtype, op, seed, **kw)
    if sum(sizes) == 0:
        return
    exp = oracle.fold_all_reduce([gu.host(x) for x in flat], dtype, op)
    bufs = [x.clone() for x in flat]
    ptrs = [b.data_ptr() for b in bufs]
    ar.ar_all_reduce(comm, ptrs, ptrs, sum(sizes), dtype, op, "fused")
    torch.cuda.synchronize()
    for r in range(n):
        gu.assert_same(got[r], exp[r], dtype, f"multi n={n} {dtype} {op} sizes={sizes[:6]}... rank {r} vs oracle")
        gu.assert_same(got[r], gu.host(bufs[r]), dtype, f"multi vs flat rank {r}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i32"])
@pytest.mark.parametrize("n", [1, 2, 3, 8, 64])
def test_multi_matches_flat_bucket(n, dtype):
    rng = np.random.default_rng(n)
    with ar.Comm(n, 0) as comm:
        for op in ("sum", "avg", "max", "prod"):
            sizes = [int(x) for x in rng.integers(0, 3000, size=7)] + [1, 0, 5000 + 3]
            check(comm, sizes, dtype, op, seed=len(sizes) + n)
            check(comm, sizes, dtype, op, seed=9, inplace=True)
            check(comm, sizes, dtype, op, seed=11, offset=gu.ESIZE[dtype])


def test_multi_many_tensors_many_launches():
    """300 tensors at 8 ranks and 40 tensors at 64 ranks take several
    kernel-argument batches each."""
    rng = np.random.default_rng(3)
    with ar.Comm(8, 0) as comm:
        check(comm, [int(x) for x in rng.integers(1, 700, size=300)], "f32", "sum", seed=1)
    with ar.Comm(64, 0) as comm:
        check(comm, [int(x) for x in rng.integers(1, 2000, size=40)], "bf16", "avg", seed=2)


def test_multi_single_tensor_spanning_all_chunks():
    with ar.Comm(8, 0) as comm:
        check(comm, [8 * 50000 + 7], "f16", "sum", seed=4)
        check(comm, [3, 8 * 50000 + 7, 5], "f16", "sum", seed=5)


def test_multi_refuses_other_modes_and_overlap():
    with ar.Comm(4, 0) as comm:
        b = [gu.RankBuf(64, "f32") for _ in range(4)]
        p = [x.ptr() for x in b]
        for mode in ("stepwise", "graph", "tree"):
            with pytest.raises(ar.ArError) as ei:
                ar.ar_all_reduce_multi(comm, [p], [p], [64], "f32", "sum", mode)
            assert ei.value.code == ar.AR_ERR_UNSUPPORTED
        with pytest.raises(ar.ArError) as ei:  # two tensors share rank 0's buffer
            ar.ar_all_reduce_multi(comm, [p, [p[0]] + p[1:]], [p, p], [64, 64], "f32", "sum")
        assert ei.value.code == ar.AR_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("op", ["max", "min", "prod"])
def test_bucket64_mixed_tensors_full_size(op):
    """64 ranks x 64M fp32 (256 MiB), laid out as tensors of log-uniform byte
    sizes in [4 KiB, 64 MiB] (views into each rank's allocation): the
    multi-tensor call equals the flat all-reduce bit for bit, and sampled
    elements equal the oracle."""
    n, count = 64, 67_108_864
    sizes = synthetic.bucket_sizes(count, 4, 4096, 64 << 20, seed=5)
    with ar.Comm(n, 0) as comm:
        bufs = synthetic.rank_inputs("bucket64", n, count, "f32", device="cuda", op=op, salt=3)
        rng = np.random.default_rng(0)
        idx = np.unique(np.concatenate([rng.integers(0, count, 20000), np.cumsum(sizes)[:-1], [0, count - 1]]))
        it = torch.from_numpy(idx).cuda()
        vals = torch.stack([b[it] for b in bufs], dim=1).cpu().numpy()
        exp = oracle.all_reduce_elements(vals, idx, count, "f32", op)
        flat = [b.clone() for b in bufs]
        offs = np.concatenate([[0], np.cumsum(sizes)[:-1]])
        rows = [[bufs[r].data_ptr() + int(o) * 4 for r in range(n)] for o in offs]
        ar.ar_all_reduce_multi(comm, rows, rows, sizes, "f32", op)
        fp = [b.data_ptr() for b in flat]
        ar.ar_all_reduce(comm, fp, fp, count, "f32", op, "fused")
        torch.cuda.synchronize()
        for r in range(n):
            assert torch.equal(bufs[r].view(torch.int32), flat[r].view(torch.int32)), f"rank {r}"
        gu.assert_same(bufs[0][it].cpu().numpy(), exp, "f32", f"bucket64 multi {op} sampled")
        print(f"{len(sizes)} tensors per rank")
    del bufs, flat
    torch.cuda.empty_cache()
