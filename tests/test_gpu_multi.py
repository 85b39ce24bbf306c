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
    # offset: bytes added to every buffer, or a function (tensor, rank, side)
    # -> bytes, side 0 = send, 1 = recv
    at = offset if callable(offset) else (lambda t, r, side: offset)
    for t, c in enumerate(sizes):
        srow = [gu.RankBuf(c, dtype, offset=at(t, r, 0)) for r in range(n)]
        for r in range(n):
            srow[r].view.copy_(flat[r][off:off + c])
        send.append(srow)
        recv.append(srow if inplace else [gu.RankBuf(c, dtype, offset=at(t, r, 1)) for r in range(n)])
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


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i32"])
def test_multi_shifted_and_mixed_alignment(dtype):
    """Every rank's tensor at the same offset from a 16-byte boundary (each
    offset in turn): 16-byte vectors shifted past the first elements. Ranks
    or send/recv at different offsets: the element path. Sizes below one
    vector, across chunk boundaries and over several tiles."""
    e = gu.ESIZE[dtype]
    epv = gu.EPV[dtype]
    sizes = [1, epv - 1, epv + 1, 3 * epv + 2, 2 * 256 * epv + 5, 0, 7, 4 * 256 * epv + epv - 1, 2]
    for n in (3, 8):
        with ar.Comm(n, 0) as comm:
            for k in range(epv):
                check(comm, sizes, dtype, "sum", seed=100 + k, offset=k * e)
                check(comm, sizes, dtype, "max", seed=200 + k, offset=k * e, inplace=True)
            check(comm, sizes, dtype, "sum", seed=300, offset=lambda t, r, side: ((t + r) % epv) * e)
            check(comm, sizes, dtype, "prod", seed=301, offset=lambda t, r, side: side * e)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i32"])
def test_multi_line_and_16_byte_vector_starts(dtype):
    """Rank pointers at one offset from a 128-byte line: vectors start on the
    first whole line, up to 128/e - 1 elements in (offsets chosen so that the
    first vector is 0, 1, 2, ... and 128/e - 1 elements in). Pointers that
    share their 16-byte offset but sit at different offsets from a line on
    different ranks or sides: vectors start on the first 16-byte boundary.
    Pieces of every length around a line, across chunk boundaries and over
    several tiles."""
    e = gu.ESIZE[dtype]
    epv = gu.EPV[dtype]
    line = 128 // e
    sizes = [1, line - 1, line + 1, 3 * epv + 2, 2 * 256 * epv + 5, 0, 7, 4 * 256 * epv + epv - 1, 2,
             1000 * epv + 3, 2 * line + 1]
    # a buffer's address is a 512-byte aligned allocation plus the 64-byte
    # guard plus its offset: these offsets put its first whole line 0, e, 2e,
    # ..., 128 - e bytes away
    lead = sorted({0, e, 2 * e, 16 - e, 16, 64 - e, 64, 64 + e, 112, 128 - e})
    for n in (3, 8):
        with ar.Comm(n, 0) as comm:
            for i, b in enumerate(lead):
                o = (64 - b) % 128
                check(comm, sizes, dtype, "sum", seed=400 + i, offset=o, inplace=i % 2 == 1)
            for k in (0, 1, epv - 1):
                at = (lambda k: lambda t, r, side: 16 * ((t + r + 3 * side) % 8) + k * e)(k)
                check(comm, sizes, dtype, "max", seed=500 + k, offset=at)
                at_in = (lambda k: lambda t, r, side: 16 * ((t + r) % 8) + k * e)(k)
                check(comm, sizes, dtype, "avg" if dtype != "i32" else "min", seed=600 + k, offset=at_in,
                      inplace=True)


def test_multi_many_tensors_many_launches():
    """300 tensors at 8 ranks and 40 tensors at 64 ranks take several
    kernel-argument batches each."""
    rng = np.random.default_rng(3)
    with ar.Comm(8, 0) as comm:
        check(comm, [int(x) for x in rng.integers(1, 700, size=300)], "f32", "sum", seed=1)
    with ar.Comm(64, 0) as comm:
        check(comm, [int(x) for x in rng.integers(1, 2000, size=40)], "bf16", "avg", seed=2)


@pytest.mark.parametrize("n", [17, 64])
def test_multi_generic_rank_count_both_tile_halves(n):
    """Above 8 ranks the rank count is a run-time value; a multi-tensor tile is
    two 256-vector halves folded together. Tensors large enough that each
    chunk holds pieces spanning several tiles, with ragged and shifted
    pieces, against the oracle and the flat call."""
    for dtype, op in (("f32", "sum"), ("bf16", "avg"), ("f32", "max")):
        epv = gu.EPV[dtype]
        sizes = [3, n * 3 * 256 * epv + 5, 7, n * 2 * 256 * epv - 1, n * 700 + 1]
        with ar.Comm(n, 0) as comm:
            check(comm, sizes, dtype, op, seed=n)
            check(comm, sizes, dtype, op, seed=n + 1, inplace=True)


@pytest.mark.parametrize("n", [8, 17, 64])
def test_multi_views_of_flat_buckets(n):
    """In-place tensors that are views into one flat buffer per rank, at the
    same offsets on every rank (the DDP layout): every view shares its offset
    from a 128-byte line across ranks, so its vectors start on a line. Mixed
    sizes listed out of memory order, a base shifted off 16-byte alignment,
    and one tensor in its own allocation in the same call: against the
    oracle's fold over the bucket in the listed order, with guard bands and
    untouched gaps."""
    for dtype, op, shift in (("f32", "sum", 0), ("bf16", "avg", 2), ("f16", "max", 6), ("i32", "prod", 4)):
        e = gu.ESIZE[dtype]
        sizes = [3, 40_000, 1, 123_457, 7, 65_536, n * 513]
        gap = 3  # elements between neighbouring views
        order = [4, 0, 6, 2, 5, 1, 3]  # memory order of the listed tensors
        starts = {}
        pos = 0
        for t in order:
            starts[t] = pos
            pos += sizes[t] + gap
        extra = 10_001  # this tensor gets its own allocation per rank
        total = sum(sizes) + extra
        flat_in = gu.make_inputs(n, total, dtype, op, seed=n + 5)
        bufs = [gu.RankBuf(pos + 8, dtype, offset=shift) for _ in range(n)]
        own = [gu.RankBuf(extra, dtype) for _ in range(n)]
        rows, off = [], 0
        listed = sizes[:3] + [extra] + sizes[3:]
        for t, c in enumerate(listed):
            if t == 3:
                for r in range(n):
                    own[r].view.copy_(flat_in[r][off:off + c])
                rows.append([own[r].ptr() for r in range(n)])
            else:
                k = t if t < 3 else t - 1
                for r in range(n):
                    bufs[r].view[starts[k]:starts[k] + c].copy_(flat_in[r][off:off + c])
                rows.append([bufs[r].sub_ptr(starts[k]) for r in range(n)])
            off += c
        with ar.Comm(n, 0) as comm:
            ar.ar_all_reduce_multi(comm, rows, rows, listed, dtype, op)
            torch.cuda.synchronize()
        for b in bufs + own:
            assert b.guards_ok()
        exp = oracle.fold_all_reduce([gu.host(x) for x in flat_in], dtype, op)
        for r in range(n):
            parts, off = [], 0
            for t, c in enumerate(listed):
                if t == 3:
                    parts.append(gu.host(own[r].view))
                else:
                    k = t if t < 3 else t - 1
                    parts.append(gu.host(bufs[r].view[starts[k]:starts[k] + c]))
                off += c
            gu.assert_same(np.concatenate(parts), exp[r], dtype, f"views n={n} {dtype} {op} rank {r}")
            # the gaps between views (filled with 0xFF bytes, never part of a
            # tensor) are untouched
            host = np.ascontiguousarray(gu.host(bufs[r].view))
            for k in order:
                g0 = starts[k] + sizes[k]
                assert np.all(host[g0:g0 + gap].view(np.uint8) == 0xFF), (n, dtype, r, k)


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


@pytest.mark.parametrize("dtype,op,shift", [("f32", "sum", 3), ("bf16", "avg", 0), ("f32", "max", 1),
                                            ("i32", "sum", 2)])
def test_bucket8_rank_major_multi_full_compare(dtype, op, shift):
    """8 ranks x 160 MiB of bucket: the streaming multi-tensor call takes the
    rank-major kernel (tiles of four quarters, two for 16-bit types, one
    workgroup per tile). Views of log-uniform sizes into one allocation per
    rank, its base shifted `shift` elements off a line: every element against
    the oracle's fold over the flat bucket, and bit for bit against the flat
    call."""
    n = 8
    e = gu.ESIZE[dtype]
    count = (160 << 20) // e + 12_345
    sizes = synthetic.bucket_sizes(count, e, 4096, 64 << 20, seed=9)
    assert sum(sizes) == count
    flat_in = gu.make_inputs(n, count, dtype, op, seed=77)
    bufs = [gu.RankBuf(count, dtype, offset=shift * e) for _ in range(n)]
    for r in range(n):
        bufs[r].view.copy_(flat_in[r])
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    rows = [[bufs[r].sub_ptr(int(o)) for r in range(n)] for o in offs]
    flat = [x.clone() for x in flat_in]
    with ar.Comm(n, 0) as comm:
        ar.ar_all_reduce_multi(comm, rows, rows, sizes, dtype, op)
        fp = [b.data_ptr() for b in flat]
        ar.ar_all_reduce(comm, fp, fp, count, dtype, op, "fused")
        torch.cuda.synchronize()
    exp = oracle.fold_all_reduce([gu.host(x) for x in flat_in], dtype, op)
    for r in range(n):
        assert bufs[r].guards_ok(), f"rank {r} guard"
        got = gu.host(bufs[r].view)
        gu.assert_same(got, exp[r], dtype, f"rank-major multi {dtype} {op} rank {r} vs oracle")
        gu.assert_same(got, gu.host(flat[r]), dtype, f"rank-major multi {dtype} {op} rank {r} vs flat")
    print(f"{len(sizes)} tensors per rank, {count * e / 2**20:.1f} MiB per rank")
    del flat_in, bufs, flat
    torch.cuda.empty_cache()


def test_bucket8_rank_major_multi_out_of_place():
    """The rank-major multi-tensor kernel with separate send and recv
    allocations per tensor (fp16, 8 ranks, 140 MiB per rank), tiny tensors
    among large ones: against the oracle."""
    n, dtype = 8, "f16"
    sizes = [1, 7, 70_000_000, 3, 4095, 1_500_001, 8, 1_900_000, 5]
    assert sum(sizes) * 2 > 128 << 20
    send, recv, exp = _multi_case(n, sizes, dtype, "sum", seed=78)
    with ar.Comm(n, 0) as comm:
        ar.ar_all_reduce_multi(comm, _ptrs(send), _ptrs(recv), sizes, dtype, "sum")
        torch.cuda.synchronize()
    _check_multi(recv, exp, dtype, "rank-major multi out of place")
    for row in send + recv:
        for b in row:
            assert b.guards_ok()
    del send, recv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n,dtype,op,shift,mib", [(4, "f32", "sum", 1, 40), (5, "f16", "avg", 3, 30),
                                                  (6, "bf16", "max", 0, 24), (7, "i32", "prod", 2, 20),
                                                  (8, "f16", "sum", 5, 18), (8, "f32", "min", 0, 17)])
def test_rank_major_multi_few_ranks_full_compare(n, dtype, op, shift, mib):
    """4 to 8 ranks with a footprint above half the last-level cache (the
    default streams): the multi-tensor call takes the rank-major tiles for
    run-time rank counts from 4 ranks, one workgroup per tile. Views of
    log-uniform sizes into one allocation per rank, its base `shift`
    elements off a line, in place: every element against the oracle's fold
    over the flat bucket, and bit for bit against the flat call."""
    e = gu.ESIZE[dtype]
    count = (mib << 20) // e + 777
    assert n * count * e > 128 << 20
    sizes = synthetic.bucket_sizes(count, e, 4096, 16 << 20, seed=n + mib)
    flat_in = gu.make_inputs(n, count, dtype, op, seed=n + 3 * shift)
    bufs = [gu.RankBuf(count, dtype, offset=shift * e) for _ in range(n)]
    for r in range(n):
        bufs[r].view.copy_(flat_in[r])
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    rows = [[bufs[r].sub_ptr(int(o)) for r in range(n)] for o in offs]
    flat = [x.clone() for x in flat_in]
    with ar.Comm(n, 0) as comm:
        ar.ar_all_reduce_multi(comm, rows, rows, sizes, dtype, op)
        fp = [b.data_ptr() for b in flat]
        ar.ar_all_reduce(comm, fp, fp, count, dtype, op, "fused")
        torch.cuda.synchronize()
    exp = gu.oracle_all_reduce(flat_in, dtype, op)
    for r in range(n):
        assert bufs[r].guards_ok(), f"rank {r} guard"
        got = gu.host(bufs[r].view)
        gu.assert_same(got, exp[r], dtype, f"rank-major multi n={n} {dtype} {op} rank {r} vs oracle")
        gu.assert_same(got, gu.host(flat[r]), dtype, f"rank-major multi n={n} {dtype} {op} rank {r} vs flat")
    print(f"{len(sizes)} tensors per rank")
    del flat_in, bufs, flat
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n,dtype,op,shift", [(17, "f32", "sum", 3), (17, "bf16", "avg", 0), (64, "f32", "min", 1),
                                              (64, "f16", "max", 5), (24, "i32", "prod", 2)])
def test_rank_major_any_multi_full_compare(n, dtype, op, shift):
    """Above 8 ranks beyond the last-level cache the multi-tensor call takes
    the rank-major tiles for run-time rank counts. Views of log-uniform sizes
    into one allocation per rank, its base `shift` elements off a line, in
    place: every element against the oracle's fold over the flat bucket, and
    bit for bit against the flat call."""
    e = gu.ESIZE[dtype]
    count = ((5 << 20) if n > 32 else (20 << 20)) // e + 12_345
    assert n * count * e > 256 << 20
    sizes = synthetic.bucket_sizes(count, e, 4096, 64 << 20, seed=n)
    flat_in = gu.make_inputs(n, count, dtype, op, seed=n + shift)
    bufs = [gu.RankBuf(count, dtype, offset=shift * e) for _ in range(n)]
    for r in range(n):
        bufs[r].view.copy_(flat_in[r])
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    rows = [[bufs[r].sub_ptr(int(o)) for r in range(n)] for o in offs]
    flat = [x.clone() for x in flat_in]
    with ar.Comm(n, 0) as comm:
        ar.ar_all_reduce_multi(comm, rows, rows, sizes, dtype, op)
        fp = [b.data_ptr() for b in flat]
        ar.ar_all_reduce(comm, fp, fp, count, dtype, op, "fused")
        torch.cuda.synchronize()
    exp = gu.oracle_all_reduce(flat_in, dtype, op)
    for r in range(n):
        assert bufs[r].guards_ok(), f"rank {r} guard"
        got = gu.host(bufs[r].view)
        gu.assert_same(got, exp[r], dtype, f"rank-major-any multi n={n} {dtype} {op} rank {r} vs oracle")
        gu.assert_same(got, gu.host(flat[r]), dtype, f"rank-major-any multi n={n} {dtype} {op} rank {r} vs flat")
    del flat_in, bufs, flat
    torch.cuda.empty_cache()


def test_rank_major_any_multi_out_of_place():
    """The rank-major tiles for run-time rank counts with separate send and
    recv allocations per tensor (fp16, 17 ranks, 23 MB per rank), tiny
    tensors (no whole vector) among large ones: against the oracle."""
    n, dtype = 17, "f16"
    sizes = [1, 7, 9_000_000, 3, 4095, 1_500_001, 8, 900_000, 5]
    assert 2 * n * sum(sizes) * 2 > 256 << 20
    send, recv, exp = _multi_case(n, sizes, dtype, "sum", seed=79)
    with ar.Comm(n, 0) as comm:
        ar.ar_all_reduce_multi(comm, _ptrs(send), _ptrs(recv), sizes, dtype, "sum")
        torch.cuda.synchronize()
    _check_multi(recv, exp, dtype, "rank-major-any multi out of place")
    for row in send + recv:
        for b in row:
            assert b.guards_ok()
    del send, recv
    torch.cuda.empty_cache()


def _multi_case(n, sizes, dtype, op, seed):
    """Send tensors filled from a seeded flat bucket, empty recv tensors, and
    the oracle's flat-bucket result."""
    total = sum(sizes)
    flat = gu.make_inputs(n, total, dtype, op, seed=seed)
    exp = gu.oracle_all_reduce(flat, dtype, op)
    send, recv, off = [], [], 0
    for c in sizes:
        row = [gu.RankBuf(c, dtype) for _ in range(n)]
        for r in range(n):
            row[r].view.copy_(flat[r][off:off + c])
        send.append(row)
        recv.append([gu.RankBuf(c, dtype) for _ in range(n)])
        off += c
    return send, recv, exp


def _check_multi(recv, exp, dtype, what):
    for r in range(len(exp)):
        got = np.concatenate([gu.host(row[r].view) for row in recv])
        gu.assert_same(got, exp[r], dtype, f"{what} rank {r}")


def _ptrs(rows):
    return [[b.ptr() for b in row] for row in rows]


@pytest.mark.parametrize("n", [8, 64])
def test_multi_captured_replays(n):
    """Captured in torch.cuda.graph (3 tensors per launch at 64 ranks),
    replayed four times with eager multi-tensor calls between replays: every
    replay and every eager call equals the oracle."""
    dtype, op = "bf16", "sum"
    sizes = [5000, 1, 40000, 0, 8 * 1024 + 3, 777, 30000, 12, 65536]
    send, recv, exp = _multi_case(n, sizes, dtype, op, seed=11)
    send2, recv2, exp2 = _multi_case(n, sizes[::-1], dtype, op, seed=12)
    with ar.Comm(n, 0) as comm:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            ar.ar_all_reduce_multi(comm, _ptrs(send), _ptrs(recv), sizes, dtype, op, "fused", s)
        for trial in range(4):
            for row in recv + recv2:
                for b in row:
                    b.view.fill_(0)
            torch.cuda.synchronize()
            g.replay()
            ar.ar_all_reduce_multi(comm, _ptrs(send2), _ptrs(recv2), sizes[::-1], dtype, op)
            torch.cuda.synchronize()
            _check_multi(recv, exp, dtype, f"replay {trial}")
            _check_multi(recv2, exp2, dtype, f"eager between replays {trial}")


def test_multi_many_launches_and_two_streams():
    """Many small tensors (1500 per rank: dozens of kernel-argument batches),
    calls of different sizes in a row, and two calls in flight on two
    streams at once: every result equals the oracle."""
    n, dtype, op = 8, "f32", "max"
    small = [1000, 2000]
    many = [64 + (t % 7) * 1000 for t in range(1500)]
    big = [4 << 20, 3 << 20]
    with ar.Comm(n, 0) as comm:
        cases = []
        for k, sizes in enumerate((small, many, small)):
            send, recv, exp = _multi_case(n, sizes, dtype, op, seed=30 + k)
            ar.ar_all_reduce_multi(comm, _ptrs(send), _ptrs(recv), sizes, dtype, op)
            cases.append((recv, exp, f"case {k}"))
        torch.cuda.synchronize()
        for recv, exp, what in cases:
            _check_multi(recv, exp, dtype, what)
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        sa, ra, ea = _multi_case(n, big, dtype, op, seed=40)
        sb, rb, eb = _multi_case(n, many, dtype, op, seed=41)
        torch.cuda.synchronize()
        ar.ar_all_reduce_multi(comm, _ptrs(sa), _ptrs(ra), big, dtype, op, "fused", s1)
        ar.ar_all_reduce_multi(comm, _ptrs(sb), _ptrs(rb), many, dtype, op, "fused", s2)
        torch.cuda.synchronize()
        _check_multi(ra, ea, dtype, "stream 1")
        _check_multi(rb, eb, dtype, "stream 2")


def test_multi_at_the_tensor_limit():
    """AR_MAX_TENSORS tensors per rank (views of 16-element slices of one
    allocation per rank, in place), then one more is INVALID_ARGUMENT."""
    n, per, t = 8, 16, ar.MAX_TENSORS
    count = per * t
    with ar.Comm(n, 0) as comm:
        flat = gu.make_inputs(n, count, "f32", "sum", seed=77)
        exp = oracle.fold_all_reduce([gu.host(x) for x in flat], "f32", "sum")
        rows = [[flat[r].data_ptr() + k * per * 4 for r in range(n)] for k in range(t)]
        ar.ar_all_reduce_multi(comm, rows, rows, [per] * t, "f32", "sum")
        torch.cuda.synchronize()
        for r in range(n):
            gu.assert_same(gu.host(flat[r]), exp[r], "f32", f"{t} tensors rank {r}")
        with pytest.raises(ar.ArError) as ei:
            ar.ar_all_reduce_multi(comm, rows + rows[:1], rows + rows[:1], [per] * (t + 1), "f32", "sum")
        assert ei.value.code == ar.AR_ERR_INVALID_ARGUMENT


def _views_case(n, sizes, dtype, op, seed, layout, inplace):
    """Tensors as views into one send (and one recv) allocation per rank, at
    the same offsets on every rank. layout: "gapped" (tensor order, a few
    elements between tensors), "shuffled" (memory order differs from tensor
    order, tensor 0 lowest), "base_not_first" (tensor 0 in the middle).
    Returns (flat inputs, outputs per rank in tensor order)."""
    e = gu.ESIZE[dtype]
    total = sum(sizes)
    flat = gu.make_inputs(n, total, dtype, op, seed=seed)
    order = list(range(len(sizes)))
    if layout == "shuffled":
        rest = order[1:]
        np.random.default_rng(seed).shuffle(rest)
        order = [0] + rest
    elif layout == "base_not_first":
        order = order[1:len(order) // 2 + 1] + [0] + order[len(order) // 2 + 1:]
    where, pos = {}, 0
    for t in order:
        pos += 3 + (t % 5)  # a gap of a few elements before every tensor
        where[t] = pos
        pos += sizes[t]
    span = pos + 8
    send = [gu.RankBuf(span, dtype, offset=2 * e) for _ in range(n)]
    recv = send if inplace else [gu.RankBuf(span, dtype, offset=2 * e) for _ in range(n)]
    off = 0
    for t, c in enumerate(sizes):
        for r in range(n):
            send[r].view[where[t]:where[t] + c].copy_(flat[r][off:off + c])
        off += c
    rows_s = [[send[r].sub_ptr(where[t]) for r in range(n)] for t in range(len(sizes))]
    rows_r = [[recv[r].sub_ptr(where[t]) for r in range(n)] for t in range(len(sizes))]
    return flat, send, recv, rows_s, rows_r, where


@pytest.mark.parametrize("n,dtype,op,layout,inplace,total_mib", [
    (8, "f32", "sum", "gapped", True, 1), (8, "bf16", "avg", "shuffled", False, 1),
    (3, "f16", "max", "gapped", False, 1), (64, "f32", "min", "shuffled", True, 1),
    (5, "i32", "prod", "base_not_first", True, 1), (8, "f32", "sum", "gapped", False, 48),
    (8, "f16", "avg", "shuffled", True, 40), (64, "f32", "max", "gapped", True, 6),
])
def test_multi_views_layouts(n, dtype, op, layout, inplace, total_mib):
    """Tensors as views at one offset into every rank's allocation, cached and
    streaming sizes: gaps between tensors, memory order unlike tensor order
    (the ring chunks follow tensor order), tensor 0 in the middle, out of
    place. Every element against the oracle's fold over the bucket in tensor
    order, and bit for bit against the flat call on a packed copy."""
    e = gu.ESIZE[dtype]
    rng = np.random.default_rng(n + total_mib)
    target = (total_mib << 20) // e
    sizes = []
    while sum(sizes) < target:
        sizes.append(int(rng.integers(1, max(2, target // 6))))
    sizes += [0, 7]
    flat, send, recv, rows_s, rows_r, where = _views_case(n, sizes, dtype, op, seed=n * 3 + total_mib, layout=layout,
                                                          inplace=inplace)
    with ar.Comm(n, 0) as comm:
        ar.ar_all_reduce_multi(comm, rows_s, rows_r, sizes, dtype, op)
        torch.cuda.synchronize()
        packed = [x.clone() for x in flat]
        pp = [b.data_ptr() for b in packed]
        ar.ar_all_reduce(comm, pp, pp, sum(sizes), dtype, op, "fused")
        torch.cuda.synchronize()
    exp = gu.oracle_all_reduce(flat, dtype, op)
    for r in range(n):
        assert recv[r].guards_ok() and send[r].guards_ok(), f"rank {r} guard"
        got = np.concatenate([gu.host(recv[r].view[where[t]:where[t] + c]) for t, c in enumerate(sizes)])
        gu.assert_same(got, exp[r], dtype, f"views n={n} {dtype} {op} {layout} inplace={inplace} rank {r}")
        gu.assert_same(got, gu.host(packed[r]), dtype, f"views vs flat rank {r}")
    del flat, send, recv, packed
    torch.cuda.empty_cache()
