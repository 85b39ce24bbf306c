"""Parity at the workloads' full sizes, in place, as the benchmark launches
them. Where host memory or oracle time allows, every element is compared;
otherwise sampled elements (random ones plus every chunk boundary and the
ends) are computed one by one by the oracle from host copies of their
inputs taken before the call, and two properties are checked on the whole
buffers on the device: every rank holds the same result, and nothing
outside the payload changed (guard bands of the comparison tests cover that
at small sizes)."""
import numpy as np
import pytest
import torch

import gpu_util as gu
import oracle
import ring_all_reduce_ar_amd as ar
import synthetic

pytestmark = pytest.mark.gpu


def sample_indices(n, count, rng, m=20000):
    q = -(-count // n)
    idx = set(rng.integers(0, count, size=m).tolist())
    for c in range(n + 1):
        for d in (-2, -1, 0, 1, 2):
            i = c * q + d
            if 0 <= i < count:
                idx.add(i)
    idx.update({0, count - 1})
    return np.array(sorted(idx), dtype=np.int64)


def gather(bufs, idx):
    it = torch.from_numpy(idx).to(bufs[0].device)
    vals = torch.stack([b[it] for b in bufs], dim=1).contiguous()
    return synthetic.to_numpy(vals.view(-1)).reshape(vals.shape)


def window_inputs(bufs, lo, hi):
    """Every rank's elements [lo, hi) as a host array of shape (hi - lo, n)."""
    vals = torch.stack([b[lo:hi] for b in bufs], dim=1).contiguous()
    return synthetic.to_numpy(vals.view(-1)).reshape(vals.shape)


def check_sampled(comm, bufs, dtype, op, mode, seed=0, windows=()):
    """In-place all-reduce of bufs, checked at sampled elements, on every
    element of the contiguous windows [lo, hi) given, and for identical
    ranks. The oracle computes each checked element from host copies of its
    inputs taken before the call."""
    n, count = len(bufs), bufs[0].numel()
    idx = sample_indices(n, count, np.random.default_rng(seed))
    before = gather(bufs, idx)
    exp = oracle.all_reduce_elements(before, idx, count, dtype, op)
    win_exp = []
    for lo, hi in windows:
        assert 0 <= lo < hi <= count
        win_exp.append(oracle.all_reduce_elements(window_inputs(bufs, lo, hi), np.arange(lo, hi, dtype=np.uint64),
                                                  count, dtype, op))
    ptrs = [b.data_ptr() for b in bufs]
    ar.ar_all_reduce(comm, ptrs, ptrs, count, dtype, op, mode)
    torch.cuda.synchronize()
    after = gather(bufs, idx)
    for r in range(n):
        gu.assert_same(np.ascontiguousarray(after[:, r]), exp, dtype, f"{mode} {dtype} {op} rank {r} sampled")
    for (lo, hi), w in zip(windows, win_exp):
        for r in range(n):
            gu.assert_same(synthetic.to_numpy(bufs[r][lo:hi]), w, dtype,
                           f"{mode} {dtype} {op} rank {r} window [{lo}, {hi})")
    for r in range(1, n):
        assert torch.equal(bufs[r].view(torch.uint8), bufs[0].view(torch.uint8)), f"rank {r} differs from rank 0"


def headline_windows(n, count, width=1 << 24):
    """Four contiguous windows of `width` elements: the start, one straddling
    the boundary between chunks 3 and 4, one straddling element 2^32 (where
    32-bit element indices would wrap), and the end."""
    q = -(-count // n)
    mids = [n // 2 * q, 1 << 32]
    out = [(0, width)] + [(m - width // 2, m + width // 2) for m in mids if width // 2 <= m <= count - width // 2]
    out.append((count - width, count))
    return out


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", ["fused", "stepwise"])
def test_bucket25_avg_full_compare(mode):
    """8 ranks x one 25 MiB fp32 DDP bucket, N(0, 1e-3^2), AVG: every element."""
    n, count = 8, 6_553_600
    with ar.Comm(n, 0) as comm:
        xs = synthetic.rank_inputs("bucket25", n, count, "f32", device="cuda")
        exp = oracle.fold_all_reduce([gu.host(x) for x in xs], "f32", "avg")
        ptrs = [x.data_ptr() for x in xs]
        ar.ar_all_reduce(comm, ptrs, ptrs, count, "f32", "avg", mode)
        torch.cuda.synchronize()
        for r in range(n):
            gu.assert_same(gu.host(xs[r]), exp[r], "f32", f"bucket25 {mode} rank {r}")
    del xs
    free()


@pytest.mark.parametrize("dtype", ["f32", "i32"])
@pytest.mark.parametrize("mode", ["fused", "stepwise"])
def test_sweep_sizes(mode, dtype):
    """8 ranks, 1 KiB .. 256 MiB per rank in powers of two, SUM; every
    element up to 16 MiB, sampled above."""
    n = 8
    with ar.Comm(n, 0) as comm:
        for log2 in range(10, 29):
            count = (1 << log2) // 4
            xs = synthetic.rank_inputs("sweep", n, count, dtype, device="cuda", salt=log2)
            if log2 <= 24:
                exp = oracle.fold_all_reduce([gu.host(x) for x in xs], dtype, "sum")
                ptrs = [x.data_ptr() for x in xs]
                ar.ar_all_reduce(comm, ptrs, ptrs, count, dtype, "sum", mode)
                torch.cuda.synchronize()
                for r in range(n):
                    gu.assert_same(gu.host(xs[r]), exp[r], dtype, f"sweep 2^{log2} B {mode} rank {r}")
            else:
                check_sampled(comm, xs, dtype, "sum", mode, seed=log2)
            del xs
    free()


def test_headline_windows_cover_the_shape():
    w = headline_windows(8, 7_000_000_000)
    assert len(w) == 4 and all(hi - lo == 1 << 24 for lo, hi in w)
    assert w[0][0] == 0 and w[-1][1] == 7_000_000_000
    assert w[1][0] < 4 * 875_000_000 < w[1][1] and w[2][0] < 1 << 32 < w[2][1]


def test_grad7b_fp16_avg():
    """8 ranks x 7e9 fp16 (14 GB each), N(0, 1e-3^2) with 1% N(0, 1)
    outliers, AVG with fp32 accumulation, in place: fused (the benchmark's
    launch), then stepwise on fresh inputs with its 28 GB fp32 workspace.
    Sampled elements plus four contiguous windows of 2^24 elements, compared
    element by element."""
    n, count = 8, 7_000_000_000
    wins = headline_windows(n, count)
    with ar.Comm(n, 0) as comm:
        bufs = synthetic.rank_inputs("grad7b", n, count, "f16", device="cuda")
        check_sampled(comm, bufs, "f16", "avg", "fused", seed=4, windows=wins)
        for r, b in enumerate(bufs):
            synthetic.gaussian(count, 1e-3, synthetic.generator("grad7b", r, "cuda", salt=1), torch.float16,
                               "cuda", outlier_frac=0.01, out=b)
        ws = gu.attach_workspace(comm, ar.AR_COLL_ALL_REDUCE, n, count, "f16", "stepwise")
        check_sampled(comm, bufs, "f16", "avg", "stepwise", seed=5, windows=wins)
        ar.ar_comm_set_workspace(comm, None)
        del ws
    del bufs
    free()


@pytest.mark.parametrize("op", ["max", "min", "prod"])
def test_bucket64_ops(op):
    """64 ranks x 64M fp32 (256 MiB each), MAX/MIN on uniform[-1, 1), PROD on
    uniform[0.99, 1.01), fused and stepwise."""
    n, count = 64, 67_108_864
    with ar.Comm(n, 0) as comm:
        for mode, salt in (("fused", 0), ("stepwise", 1)):
            bufs = synthetic.rank_inputs("bucket64", n, count, "f32", device="cuda", op=op, salt=salt)
            check_sampled(comm, bufs, "f32", op, mode, seed=salt)
            del bufs
            free()


def test_grad7b_reduce_scatter_then_all_gather():
    """The export shapes `bench.py --collective` times at the 7B-gradient
    size: reduce-scatter of 8 x 7e9 fp16 (14 GB in per rank, 1.75 GB out),
    AVG, out of place, then all-gather of the reduced blocks back into the
    14 GB buffers. Sampled elements (random, every block boundary, the ends)
    against the oracle's all-reduce of those elements: block r of the
    reduce-scatter is chunk r of the all-reduce, and every all-gathered rank
    holds the all-reduce."""
    n, count = 8, 7_000_000_000
    rc = count // n
    with ar.Comm(n, 0) as comm:
        send = synthetic.rank_inputs("grad7b", n, count, "f16", device="cuda", salt=2)
        recv = [torch.empty(rc, dtype=torch.float16, device="cuda") for _ in range(n)]
        idx = sample_indices(n, count, np.random.default_rng(6))
        exp = oracle.all_reduce_elements(gather(send, idx), idx, count, "f16", "avg")
        ar.ar_reduce_scatter(comm, [b.data_ptr() for b in send], [b.data_ptr() for b in recv], rc, "f16", "avg",
                             "fused")
        torch.cuda.synchronize()
        it = torch.from_numpy(idx).cuda()
        got = torch.empty(idx.size, dtype=torch.float16, device="cuda")
        for r in range(n):
            sel = (it // rc) == r
            got[sel] = recv[r][it[sel] - r * rc]
        gu.assert_same(synthetic.to_numpy(got), exp, "f16", "reduce-scatter sampled")
        ar.ar_all_gather(comm, [b.data_ptr() for b in recv], [b.data_ptr() for b in send], rc, "f16", "fused")
        torch.cuda.synchronize()
        after = gather(send, idx)
        for r in range(n):
            gu.assert_same(np.ascontiguousarray(after[:, r]), exp, "f16", f"all-gather rank {r} sampled")
        for r in range(1, n):
            assert torch.equal(send[r].view(torch.int16), send[0].view(torch.int16)), f"rank {r} differs"
    del send, recv
    free()


@pytest.mark.parametrize("n,dtype,blk,mode", [(2, "f32", 20_000_004, "fused"), (4, "f16", 9_000_008, "fused"),
                                              (16, "bf16", 600_008, "fused"), (5, "f32", 3_000_004, "fused"),
                                              (8, "f32", 1_200_004, "stepwise"), (3, "f16", 8_000_008, "stepwise")])
def test_all_to_all_tiled_full_compare(n, dtype, blk, mode):
    """Beyond the last-level cache the all-to-all takes the tiled copy (four
    vectors per thread, one workgroup per tile, ragged last tiles), in one
    launch or one per ring step: every element of every rank against the
    oracle's transpose."""
    assert 2 * n * n * blk * gu.ESIZE[dtype] > 256 << 20
    xs = gu.make_inputs(n, n * blk, dtype, "sum", seed=n + blk % 97)
    exp = oracle.all_to_all([gu.host(x) for x in xs], dtype)
    with ar.Comm(n, 0) as comm:
        recv = [gu.RankBuf(n * blk, dtype) for _ in range(n)]
        ar.ar_all_to_all(comm, [x.data_ptr() for x in xs], [b.ptr() for b in recv], blk, dtype, mode)
        torch.cuda.synchronize()
        for p in range(n):
            assert recv[p].guards_ok(), f"rank {p} guard"
            gu.assert_same(gu.host(recv[p].view), exp[p], dtype, f"all-to-all {mode} n={n} {dtype} blk={blk} rank {p}")
        del recv
    del xs, exp
    free()


def test_all_to_all_256mib_fp32_full_compare():
    """All-to-all of 8 x 256 MiB fp32 (the `--collective all_to_all` sweep
    point), every element against the oracle's transpose."""
    n, count = 8, 67_108_864
    blk = count // n
    with ar.Comm(n, 0) as comm:
        send = synthetic.rank_inputs("sweep", n, count, "f32", device="cuda", salt=9)
        recv = [torch.empty(count, dtype=torch.float32, device="cuda") for _ in range(n)]
        exp = oracle.all_to_all([gu.host(b) for b in send], "f32")
        ar.ar_all_to_all(comm, [b.data_ptr() for b in send], [b.data_ptr() for b in recv], blk, "f32", "fused")
        torch.cuda.synchronize()
        for p in range(n):
            gu.assert_same(gu.host(recv[p]), exp[p], "f32", f"all-to-all rank {p}")
    del send, recv
    free()


@pytest.mark.parametrize("n,count,dtype", [(3, 89_478_485, "f32"), (5, 134_217_727, "f16"), (7, 40_000_003, "bf16"),
                                           (2, 268_435_456, "f32"), (4, 100_000_001, "i32")])
def test_odd_rank_counts_large(n, count, dtype):
    """Rank counts and sizes whose chunk length is not a multiple of the
    16-byte vector width (chunks start inside a vector), and the 2- and
    4-rank launch shapes, at 100 MiB-1 GiB per rank: fused, in place,
    sampled elements (every chunk boundary +-2 among them) against the
    oracle, all ranks identical."""
    with ar.Comm(n, 0) as comm:
        bufs = synthetic.rank_inputs("sweep", n, count, dtype, device="cuda", salt=n)
        check_sampled(comm, bufs, dtype, "sum", "fused", seed=n)
        del bufs
    free()


def _generic_case(n, dtype, extra):
    # chunk length giving each chunk row 2G + G/3 + 1 tiles of 4 KiB, G being
    # 16 workgroups per CU over the n rows (a tile count that is no multiple
    # of the kernels' super tiles), plus `extra` elements so chunks start
    # inside a vector
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    g = max(1, cus * 16 // n)
    tiles = 2 * g + g // 3 + 1
    q = tiles * 256 * gu.EPV[dtype] + extra
    return n * q - extra // 2


@pytest.mark.parametrize("n,dtype,op,extra", [(17, "f32", "sum", 1), (33, "bf16", "avg", 3), (64, "f32", "prod", 1),
                                              (64, "f16", "max", 5), (12, "i32", "sum", 0)])
def test_generic_rank_counts_full_compare(n, dtype, op, extra):
    """Rank counts above 8 take kernels whose rank count is a run-time value
    (beyond the last-level cache, as here, the rank-major one), with ragged
    chunks: every element of every rank against the oracle, out of place,
    with guard bands."""
    count = _generic_case(n, dtype, extra)
    with ar.Comm(n, 0) as comm:
        xs = gu.make_inputs(n, count, dtype, op, seed=n)
        exp = gu.oracle_all_reduce(xs, dtype, op)
        got, send, recv = gu.run_all_reduce(comm, xs, dtype, op, "fused")
        for r in range(n):
            gu.assert_same(got[r], exp[r], dtype, f"n={n} {dtype} {op} count={count} rank {r}")
        del xs, exp, got, send, recv
    free()


@pytest.mark.parametrize("n,dtype,op,count,inplace", [
    (8, "f32", "sum", 35_000_003, False),
    (5, "f16", "avg", 70_000_001, True),
    (6, "bf16", "max", 67_108_869, True),  # 10 bytes above 128 MiB per rank
    (7, "i32", "sum", 33_554_433, False),
    (8, "f16", "prod", 67_108_880, True),
])
def test_rank_major_range_full_compare(n, dtype, op, count, inplace):
    """Once the all-reduce streams (footprints above half the last-level
    cache, as all of these) it takes its rank-major kernel from 4 ranks (a
    thread folds consecutive tiles one rank at a time, one workgroup per
    super tile): every element of every rank against the oracle, with ragged
    chunks and guard bands."""
    with ar.Comm(n, 0) as comm:
        xs = gu.make_inputs(n, count, dtype, op, seed=count % 1000)
        exp = gu.oracle_all_reduce(xs, dtype, op)
        got, send, recv = gu.run_all_reduce(comm, xs, dtype, op, "fused", inplace=inplace)
        for r in range(n):
            gu.assert_same(got[r], exp[r], dtype, f"n={n} {dtype} {op} count={count} inplace={inplace} rank {r}")
        del xs, exp, got, send, recv
    free()


def _rank_major_any_case(n, dtype, extra):
    # chunk rows of G + G/3 super tiles plus one tile (G a few hundred, from
    # the CU count), a super tile being M tiles of 4 KiB (8 above 8 ranks, 4
    # up to 8, halved for 16-bit types): the launch has one workgroup per
    # super tile, the last of which holds one tile, and every chunk after the
    # first starts inside a tile; `extra` elements make chunks start inside a
    # vector
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    g = max(1, cus * (32 if n > 32 else 16) // n)
    m = (8 if n > 8 else 4) // (2 if gu.ESIZE[dtype] == 2 else 1)
    tiles = (g + g // 3) * m + 1
    q = tiles * 256 * gu.EPV[dtype] + extra
    return n * q - extra // 2


@pytest.mark.parametrize("n,dtype,op,extra,inplace", [
    (4, "f32", "sum", 1, True),
    (4, "bf16", "avg", 3, False),
    (16, "f32", "min", 2, False),
    (12, "i32", "prod", 0, True),
    (24, "f16", "sum", 5, False),
])
def test_rank_major_any_full_compare(n, dtype, op, extra, inplace):
    """The rank-major kernel for run-time rank counts (4 ranks and above 8,
    beyond the last-level cache): hundreds of super tiles per chunk row, a
    partial last super tile, ragged chunks; every element of every rank
    against the oracle, with guard bands."""
    count = _rank_major_any_case(n, dtype, extra)
    with ar.Comm(n, 0) as comm:
        xs = gu.make_inputs(n, count, dtype, op, seed=n + extra)
        exp = gu.oracle_all_reduce(xs, dtype, op)
        got, send, recv = gu.run_all_reduce(comm, xs, dtype, op, "fused", inplace=inplace)
        for r in range(n):
            gu.assert_same(got[r], exp[r], dtype, f"n={n} {dtype} {op} count={count} inplace={inplace} rank {r}")
        del xs, exp, got, send, recv
    free()


@pytest.mark.parametrize("n,dtype,op,count", [(8, "f32", "sum", 16_777_219), (6, "bf16", "max", 33_554_441)])
def test_rank_major_from_64mib_full_compare(n, dtype, op, count):
    """From 64 MiB per rank at 5-8 ranks (beyond the last-level cache) the
    all-reduce takes the fixed-rank-count rank-major kernel: every element
    of every rank, in place as the benchmark calls it, ragged chunks."""
    with ar.Comm(n, 0) as comm:
        xs = gu.make_inputs(n, count, dtype, op, seed=count % 997)
        exp = gu.oracle_all_reduce(xs, dtype, op)
        got, send, recv = gu.run_all_reduce(comm, xs, dtype, op, "fused", inplace=True)
        for r in range(n):
            gu.assert_same(got[r], exp[r], dtype, f"n={n} {dtype} {op} count={count} rank {r}")
        del xs, exp, got, send, recv
    free()


@pytest.mark.parametrize("n,dtype,op,count,inplace", [
    (2, "f32", "sum", 22_368_261, False),
    (3, "f32", "max", 33_554_435, True),
    (2, "bf16", "avg", 50_000_003, True),
    (3, "f16", "prod", 30_000_001, False),
])
def test_rank_major_two_three_ranks_full_compare(n, dtype, op, count, inplace):
    """2 and 3 ranks with a footprint above half the last-level cache: the
    all-reduce streams through its rank-major kernel (one workgroup per super
    tile) at these rank counts too. Every element of every rank against the
    oracle, ragged chunks, guard bands."""
    assert n * count * gu.ESIZE[dtype] > 128 << 20
    with ar.Comm(n, 0) as comm:
        xs = gu.make_inputs(n, count, dtype, op, seed=count % 1009)
        exp = gu.oracle_all_reduce(xs, dtype, op)
        got, send, recv = gu.run_all_reduce(comm, xs, dtype, op, "fused", inplace=inplace)
        for r in range(n):
            gu.assert_same(got[r], exp[r], dtype, f"n={n} {dtype} {op} count={count} inplace={inplace} rank {r}")
        del xs, exp, got, send, recv
    free()


@pytest.mark.parametrize("n,dtype,op,count,inplace", [(2, "f16", "sum", (1 << 29) + 5, True),
                                                    (3, "bf16", "max", (1 << 29) + 11, False)])
def test_one_tile_super_tiles_full_compare(n, dtype, op, count, inplace):
    """16-bit all-reduces of 1 GiB per rank and more at up to 8 ranks take
    super tiles of one tile: every element of every rank against the oracle,
    ragged chunks, guard bands."""
    with ar.Comm(n, 0) as comm:
        xs = gu.make_inputs(n, count, dtype, op, seed=n + 31)
        exp = gu.oracle_all_reduce(xs, dtype, op)
        got, send, recv = gu.run_all_reduce(comm, xs, dtype, op, "fused", inplace=inplace)
        for r in range(n):
            gu.assert_same(got[r], exp[r], dtype, f"n={n} {dtype} {op} count={count} inplace={inplace} rank {r}")
        del xs, exp, got, send, recv
    free()


@pytest.mark.parametrize("n,count,dtype", [(8, 1 << 30, "f32"), (8, (1 << 31) - 5, "f16"), (6, 999_999_997, "f32")])
def test_rank_major_upper_sizes_sampled(n, count, dtype):
    """The rank-major all-reduce at 2.4-4 GiB per rank, in place as the
    benchmark launches it (one workgroup per super tile, over a hundred
    thousand workgroups): sampled elements (every chunk boundary among them)
    against the oracle, all ranks identical."""
    with ar.Comm(n, 0) as comm:
        bufs = synthetic.rank_inputs("sweep", n, count, dtype, device="cuda", salt=7)
        check_sampled(comm, bufs, dtype, "sum", "fused", seed=n)
        del bufs
    free()


@pytest.mark.parametrize("n,dtype,op,rc,inplace", [
    (2, "f32", "sum", 20_000_004, True),
    (3, "bf16", "avg", 12_000_000, False),
    (4, "f16", "max", 9_000_008, False),
    (8, "f32", "sum", 4_500_004, False),
    (5, "f16", "avg", 14_000_008, True),
    (7, "bf16", "max", 9_999_992, False),
    (6, "i32", "sum", 6_000_004, True),
    (16, "f32", "sum", 1_000_004, False),
    (64, "bf16", "avg", 70_000, True),
    (12, "i32", "max", 3_000_000, False),
])
def test_reduce_scatter_rank_major_full_compare(n, dtype, op, rc, inplace):
    """Reduce-scatter from 2 ranks beyond the last-level cache takes the
    rank-major kernels (fixed rank count at 5-8, run-time otherwise; block
    lengths here are whole 16-byte vectors, as the vector kernels need):
    every element of every rank's block against the oracle's reduce-scatter,
    out of place or in place (recv[r] inside send[r] at block r), with guard
    bands."""
    xs = gu.make_inputs(n, n * rc, dtype, op, seed=rc % 1000)
    exp = oracle.reduce_scatter([gu.host(x) for x in xs], dtype, op)
    with ar.Comm(n, 0) as comm:
        send = [gu.RankBuf(n * rc, dtype) for _ in range(n)]
        for b, x in zip(send, xs):
            b.view.copy_(x)
        if inplace:
            recv_ptrs = [send[r].sub_ptr(r * rc) for r in range(n)]
            recv = []
        else:
            recv = [gu.RankBuf(rc, dtype) for _ in range(n)]
            recv_ptrs = [b.ptr() for b in recv]
        ar.ar_reduce_scatter(comm, [b.ptr() for b in send], recv_ptrs, rc, dtype, op, "fused")
        torch.cuda.synchronize()
        for b in send + recv:
            assert b.guards_ok()
        for r in range(n):
            got = gu.host(send[r].view[r * rc:(r + 1) * rc]) if inplace else gu.host(recv[r].view)
            gu.assert_same(got, exp[r], dtype, f"RS n={n} {dtype} {op} rc={rc} inplace={inplace} rank {r}")
        del send, recv
    del xs, exp
    free()


@pytest.mark.parametrize("n,dtype,sc,inplace", [(5, "f32", 134_217_732, False), (8, "f16", 268_435_464, True),
                                               (1, "f32", 40_000_004, False), (2, "f16", 40_000_008, True),
                                               (3, "bf16", 16_000_000, False), (16, "f32", 1_048_580, False)])
def test_all_gather_rank_major_full_compare(n, dtype, sc, inplace):
    """Beyond the last-level cache the all-gather takes its rank-major copy
    (four consecutive tiles per thread, stored rank by rank, one workgroup
    per tile) at every rank count, one rank (a plain copy) included.
    All-gather is concatenation in rank order (handbook "集合通信原语",
    section 五个原语), so every output block of every rank is compared bit
    for bit with its input block on the device; the tails are ragged and the
    guard bands checked."""
    xs = gu.make_inputs(n, sc, dtype, "sum", seed=n)
    with ar.Comm(n, 0) as comm:
        recv = [gu.RankBuf(n * sc, dtype) for _ in range(n)]
        if inplace:
            for r in range(n):
                recv[r].view[r * sc:(r + 1) * sc].copy_(xs[r])
            send_ptrs, send = [recv[r].sub_ptr(r * sc) for r in range(n)], []
        else:
            send = [gu.RankBuf(sc, dtype) for _ in range(n)]
            for b, x in zip(send, xs):
                b.view.copy_(x)
            send_ptrs = [b.ptr() for b in send]
        ar.ar_all_gather(comm, send_ptrs, [b.ptr() for b in recv], sc, dtype, "fused")
        torch.cuda.synchronize()
        for b in send + recv:
            assert b.guards_ok()
        iv = torch.int16 if gu.ESIZE[dtype] == 2 else torch.int32
        for r in range(n):
            for p in range(n):
                assert torch.equal(recv[r].view[p * sc:(p + 1) * sc].view(iv), xs[p].view(iv)), (r, p)
        del send, recv
    del xs
    free()


# Ring steps take their tiled form (four vectors per thread and tile, one
# workgroup per tile; half vectors per lane for fp16/bf16) once a step has at
# least 8 tiles per CU: at 256 CUs, chunks of 2048/N tiles of 4 KiB or more.
# These sizes clear that with chunks that start inside a vector; beyond the
# last-level cache the steps stream, and 8 x 16,777,003 fp16 in place (a
# footprint just under the 256 MiB cache) takes the cached half-vector step.
@pytest.mark.parametrize("n,dtype,op,count,inplace,mode", [
    (8, "f32", "sum", 9_000_005, False, "stepwise"),
    (3, "f16", "avg", 64_000_007, True, "stepwise"),
    (5, "bf16", "max", 40_000_003, False, "stepwise"),
    (8, "f16", "sum", 16_777_003, True, "stepwise"),
    (4, "i32", "prod", 9_000_001, True, "stepwise"),
    (8, "f32", "min", 9_000_005, True, "graph"),
])
def test_tiled_ring_steps_all_reduce(n, dtype, op, count, inplace, mode):
    """The ring's reduce-scatter and all-gather steps in their tiled form:
    every element of every rank against the oracle, guard bands."""
    with ar.Comm(n, 0) as comm:
        ws = gu.attach_workspace(comm, ar.AR_COLL_ALL_REDUCE, n, count, dtype, mode)
        xs = gu.make_inputs(n, count, dtype, op, seed=n * 7 + count % 13)
        exp = gu.oracle_all_reduce(xs, dtype, op)
        got, send, recv = gu.run_all_reduce(comm, xs, dtype, op, mode, inplace=inplace)
        for r in range(n):
            gu.assert_same(got[r], exp[r], dtype, f"{mode} n={n} {dtype} {op} count={count} inplace={inplace} rank {r}")
        ar.ar_comm_set_workspace(comm, None)
        del ws, xs, exp, got, send, recv
    free()


@pytest.mark.parametrize("n,dtype,op,rc,inplace", [(8, "f32", "sum", 1_100_000, False),
                                                   (4, "f16", "avg", 4_400_000, True),
                                                   (8, "bf16", "min", 2_100_008, False),
                                                   (3, "i32", "max", 2_800_004, False)])
def test_tiled_ring_steps_reduce_scatter(n, dtype, op, rc, inplace):
    """The stepwise reduce-scatter in its tiled form (partials in the
    workspace): every element of every rank's block against the oracle."""
    from test_gpu_parity import _reduce_scatter
    xs = gu.make_inputs(n, n * rc, dtype, op, seed=n + rc % 101)
    exp = oracle.reduce_scatter([gu.host(x) for x in xs], dtype, op)
    with ar.Comm(n, 0) as comm:
        got = _reduce_scatter(comm, xs, dtype, op, "stepwise", inplace)
        for r in range(n):
            gu.assert_same(got[r], exp[r], dtype, f"RS stepwise n={n} {dtype} {op} rc={rc} inplace={inplace} rank {r}")
    del xs, exp, got
    free()


@pytest.mark.parametrize("n,dtype,sc,inplace", [(8, "f16", 2_200_000, False), (3, "f32", 3_000_004, True)])
def test_tiled_ring_steps_all_gather(n, dtype, sc, inplace):
    """The stepwise all-gather's copy steps in their tiled form: every output
    block of every rank bit for bit against its input block."""
    from test_gpu_parity import _all_gather
    xs = gu.make_inputs(n, sc, dtype, "sum", seed=sc % 89)
    with ar.Comm(n, 0) as comm:
        got = _all_gather(comm, xs, dtype, "stepwise", inplace)
    iv = np.int16 if gu.ESIZE[dtype] == 2 else np.int32
    for r in range(n):
        for p in range(n):
            assert np.array_equal(got[r][p * sc:(p + 1) * sc].view(iv), gu.host(xs[p]).view(iv)), (r, p)
    del xs, got
    free()
