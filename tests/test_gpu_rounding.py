"""fp16 PROD rounds twice: the last multiply in fp32, then the conversion to
fp16 (mhpq.cn article, section 5.3). The inputs put the last fp32 product of
many elements exactly on an fp16 tie that rounding the exact product would
break the other way, so a kernel whose compiler merged that multiply with the
conversion (one rounding) fails here. Every ring-order path is checked bit
for bit against the oracle."""
import numpy as np
import pytest
import torch

import gpu_util as gu
import oracle
import ring_all_reduce_ar_amd as ar
import rounding_cases

pytestmark = pytest.mark.gpu


def planted(n):
    count = n * (4096 + 8) + 5
    xs, idx = rounding_cases.ring_prod_inputs(n, count, max(7, count // 256), seed=40 + n)
    return [torch.from_numpy(x).to("cuda") for x in xs], idx


@pytest.mark.parametrize("mode", ("fused", "stepwise", "graph"))
@pytest.mark.parametrize("n", (3, 5, 8, 16))
def test_f16_prod_rounds_twice(n, mode):
    xs, idx = planted(n)
    exp = gu.oracle_all_reduce(xs, "f16", "prod")
    with ar.Comm(n, 0) as comm:
        ws = gu.attach_workspace(comm, ar.AR_COLL_ALL_REDUCE, n, xs[0].numel(), "f16", mode)
        outs, _, _ = gu.run_all_reduce(comm, xs, "f16", "prod", mode)
        del ws
    for r in range(n):
        gu.assert_same(outs[r], exp[r], "f16", f"n={n} {mode} rank {r} ({idx.size} planted ties)")


@pytest.mark.parametrize("n", (3, 8))
def test_f16_prod_rounds_twice_multi(n):
    xs, idx = planted(n)
    count = xs[0].numel()
    exp = gu.oracle_all_reduce(xs, "f16", "prod")
    cuts = [0, 1000, 1003, count // 2, count]
    sizes = [b - a for a, b in zip(cuts[:-1], cuts[1:])]
    with ar.Comm(n, 0) as comm:
        bufs = [[gu.RankBuf(s, "f16") for _ in range(n)] for s in sizes]
        for t, (a, b) in enumerate(zip(cuts[:-1], cuts[1:])):
            for r in range(n):
                bufs[t][r].view.copy_(xs[r][a:b])
        ptrs = [[b.ptr() for b in row] for row in bufs]
        ar.ar_all_reduce_multi(comm, ptrs, ptrs, sizes, "f16", "prod")
        torch.cuda.synchronize()
    for r in range(n):
        got = np.concatenate([gu.host(bufs[t][r].view) for t in range(len(sizes))])
        gu.assert_same(got, exp[r], "f16", f"multi n={n} rank {r}")
