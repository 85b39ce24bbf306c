"""ar_all_reduce_noalloc, the allocation-free all-reduce: through the C ABI,
bit for bit against ar_all_reduce (with a caller-attached workspace) on the
same inputs, two calls in a row on one comm with the second smaller, in the
modes whose fp16/bf16 partial sums need device memory and in those that need
none; the scratch limit and graph mode are refused before any device work;
and the calls leave the device's free memory unchanged."""
import pytest
import torch

import gpu_util as gu
import ring_all_reduce_ar_amd as ar
import synthetic

pytestmark = pytest.mark.gpu

LIMIT_F16 = ar.NOALLOC_SCRATCH_BYTES // 4  # fp32 partial slots: fp16/bf16 ring-stepwise elements per rank

# (nranks, dtype, op, mode, (first count, second smaller count), in place)
CASES = [
    (8, "f16", "avg", "stepwise", (3_000_011, 4099), True),
    (8, "bf16", "sum", "stepwise", (LIMIT_F16, 1001), True),
    (8, "f16", "sum", "stepwise", (1_000_000, 999_999), False),
    (64, "bf16", "avg", "stepwise", (262_147, 64), True),
    (5, "f16", "prod", "tree_stepwise", (1_000_003, 77), True),
    (3, "bf16", "max", "tree_stepwise", (65_536, 3), False),
    (8, "f32", "sum", "stepwise", (1 << 20, 333), True),
    (8, "i32", "avg", "fused", ((1 << 20) + 7, 5), True),
    (6, "f16", "min", "tree", (100_003, 17), True),
]


def _run(comm, fn, xs, outs, count, dtype, op, mode):
    fn(comm, [x.data_ptr() for x in xs], [o.data_ptr() for o in outs], count, dtype, op, mode)


@pytest.mark.parametrize("n,dtype,op,mode,counts,inplace", CASES,
                         ids=[f"{c[0]}-{c[1]}-{c[2]}-{c[3]}-{'in' if c[5] else 'out'}" for c in CASES])
def test_noalloc_matches_all_reduce(n, dtype, op, mode, counts, inplace):
    with ar.Comm(n, 0) as comm:
        for call, count in enumerate(counts):
            print(f"[noalloc] n={n} {dtype} {op} {mode} count={count} call={call}", flush=True)
            xs = synthetic.rank_inputs("sweep", n, count, dtype, device="cuda", op=op, salt=call)
            ref_in = [x.clone() for x in xs]
            ref_out = ref_in if inplace else [torch.empty_like(x) for x in xs]
            ws = None
            need = ar.ar_workspace_bytes(ar.AR_COLL_ALL_REDUCE, n, count, dtype, mode)
            if need:
                ws = torch.empty(need, dtype=torch.uint8, device="cuda")
                ar.ar_comm_set_workspace(comm, ws)
            _run(comm, ar.ar_all_reduce, ref_in, ref_out, count, dtype, op, mode)
            ar.ar_comm_set_workspace(comm, None)  # the allocation-free call must not need it
            got_in = [x.clone() for x in xs]
            got_out = got_in if inplace else [torch.empty_like(x) for x in xs]
            torch.cuda.synchronize()
            free_before = torch.cuda.mem_get_info()[0]
            _run(comm, ar.ar_all_reduce_noalloc, got_in, got_out, count, dtype, op, mode)
            torch.cuda.synchronize()
            assert torch.cuda.mem_get_info()[0] == free_before, "the allocation-free call changed free device memory"
            for r in range(n):
                gu.assert_same(gu.host(got_out[r]), gu.host(ref_out[r]), dtype,
                               f"noalloc {mode} {dtype} {op} n={n} count={count} rank {r}")
            if not inplace:
                for r in range(n):
                    assert torch.equal(got_in[r].view(torch.uint8), xs[r].view(torch.uint8)), "input changed"
            del xs, ref_in, ref_out, got_in, got_out, ws


def test_noalloc_refuses_beyond_the_scratch_and_graph_mode():
    n, count = 8, LIMIT_F16 + 1
    with ar.Comm(n, 0) as comm:
        bufs = [torch.zeros(count, dtype=torch.float16, device="cuda") for _ in range(n)]
        with pytest.raises(ar.ArError) as ei:
            ar.ar_all_reduce_noalloc(comm, bufs, bufs, count, "f16", "sum", "stepwise")
        assert ei.value.code == ar.AR_ERR_INVALID_ARGUMENT and "AR_NOALLOC_SCRATCH_BYTES" in str(ei.value)
        with pytest.raises(ar.ArError) as ei:
            ar.ar_all_reduce_noalloc(comm, bufs, bufs, 1024, "f16", "sum", "graph")
        assert ei.value.code == ar.AR_ERR_UNSUPPORTED
        # the fused mode needs no partial-sum memory at any size
        ar.ar_all_reduce_noalloc(comm, bufs, bufs, count, "f16", "sum", "fused")
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(bufs[0])) == 0


def test_noalloc_records_no_step_events():
    n, count = 4, 4096
    with ar.Comm(n, 0) as comm:
        ar.ar_comm_set_step_timing(comm, True)
        xs = synthetic.rank_inputs("small", n, count, "f16", device="cuda")
        ar.ar_all_reduce_noalloc(comm, xs, xs, count, "f16", "sum", "stepwise")
        torch.cuda.synchronize()
        with pytest.raises(ar.ArError):
            ar.ar_last_step_times_ms(comm)
