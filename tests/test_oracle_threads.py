"""The threaded forms of the oracle (the CPU baseline's timing harness) give
the serial oracle's bits and byte counts for every dtype and op, any thread
count, ragged and empty chunks, and more threads than work."""
import numpy as np
import pytest

import oracle
import pins


def _inputs(rng, n, count, dt, op):
    return pins.random_inputs(rng, n, count, dt, op)


@pytest.mark.parametrize("nthreads", [1, 2, 3, 8, 16, 33])
def test_threaded_ring_equals_serial(nthreads):
    o = oracle.get()
    assert o.threaded, "the default oracle build holds the threaded entry points"
    rng = np.random.default_rng(100 + nthreads)
    for n in (1, 2, 3, 4, 5, 8, 9, 16, 64):
        for count in sorted({0, 1, n - 1, n, 3 * n + 1, 257, 1000}):
            for dt in pins.DTYPES:
                for op in pins.OPS:
                    xs = _inputs(rng, n, count, dt, op)
                    serial = [a.copy() for a in xs]
                    s_sent = o.ring_all_reduce(serial, dt, op)
                    threaded = [a.copy() for a in xs]
                    t_sent = o.ring_all_reduce_threads(threaded, dt, op, nthreads)
                    assert t_sent == s_sent, (n, count, dt, op, nthreads)
                    for r in range(n):
                        assert pins.same_bits(threaded[r], serial[r]), (n, count, dt, op, nthreads, r)


@pytest.mark.parametrize("nthreads", [1, 4, 16, 33])
def test_threaded_fold_equals_serial(nthreads):
    o = oracle.get()
    rng = np.random.default_rng(200 + nthreads)
    for n in (1, 3, 8, 64):
        for count in (0, 1, 5, n * 7 + 3, 4099):
            for dt in pins.DTYPES:
                for op in pins.OPS:
                    xs = _inputs(rng, n, count, dt, op)
                    exp = o.fold_all_reduce(xs, dt, op)
                    got = o.fold_all_reduce_threads(xs, dt, op, nthreads)
                    for r in range(n):
                        assert pins.same_bits(got[r], exp[r]), (n, count, dt, op, nthreads)
                    inplace = [a.copy() for a in xs]
                    o.fold_all_reduce_threads(inplace, dt, op, nthreads, out=inplace)
                    for r in range(n):
                        assert pins.same_bits(inplace[r], exp[r]), (n, count, dt, op, nthreads, "in place")


def test_threaded_rejects_bad_thread_counts():
    o = oracle.get()
    xs = [np.zeros(8, dtype=np.float32) for _ in range(2)]
    for t in (0, -1, 257):
        with pytest.raises(RuntimeError):
            o.ring_all_reduce_threads(xs, "f32", "sum", t)
        with pytest.raises(RuntimeError):
            o.fold_all_reduce_threads(xs, "f32", "sum", t)
