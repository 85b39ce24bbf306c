"""Pins of the CPU oracle to things other than itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with what the pages or the mathematics fix:

* values the pages print (fixtures under tests/golden/, each citing its page);
* the pages' closed forms (bytes sent per rank, 2(N-1)/N * S);
* the pages' invariants (all ranks identical; reduce-scatter then all-gather
  equals all-reduce);
* library routines for the special cases they cover (torch.chunk for the
  partition, numpy/torch conversions for fp16/bf16, numpy max/min,
  np.concatenate for all-gather);
* brute force with Python integers for int32, and error bounds against exact
  sums and products (math.fsum, fractions) for floating point.

``test_oracle_pins.py`` runs them against the oracle; ``test_oracle_mutants.py``
plants mistakes in copies of the oracle's source and checks that some pin
fails for each.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch

import goldens
from goldens import numbers

DTYPES = ("f32", "f16", "bf16", "i32")
OPS = ("sum", "avg", "max", "min", "prod")
ELEM = {"f32": 4, "f16": 2, "bf16": 2, "i32": 4}


# --------------------------------------------------------------------------
# value helpers (library conversions only)
# --------------------------------------------------------------------------
def as_dtype(values, dtype):
    """float64/int values -> storage array (bf16 as uint16 bit patterns, via torch)."""
    v = np.asarray(values, dtype=np.float64)
    if dtype == "f32":
        return v.astype(np.float32)
    if dtype == "f16":
        return v.astype(np.float16)
    if dtype == "bf16":
        t = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return v.astype(np.int64).astype(np.int32)


def to_f64(a, dtype):
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "i32":
        return a.astype(np.int64)
    return a.astype(np.float64)


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view({2: np.uint16, 4: np.uint32}[a.dtype.itemsize])


def same_bits(a, b):
    return a.shape == b.shape and np.array_equal(bits(a), bits(b))


def random_inputs(rng, n, count, dtype, op):
    """Inputs with a wide dynamic range so that the summation order shows."""
    if dtype == "i32":
        if op in ("max", "min", "sum", "avg", "prod"):
            return [rng.integers(-2**31, 2**31, size=count, dtype=np.int64).astype(np.int32) for _ in range(n)]
    if op == "prod":
        return [as_dtype(rng.uniform(0.5, 1.5, size=count), dtype) for _ in range(n)]
    return [as_dtype(rng.uniform(-1, 1, size=count) * 10.0 ** rng.uniform(-3, 3, size=count), dtype)
            for _ in range(n)]


def torch_chunk_lens(n, count):
    """Chunk lengths torch.chunk gives (the pages' ring uses t.chunk(n)), padded
    with empty chunks when torch returns fewer than n."""
    lens = [c.numel() for c in torch.arange(count).chunk(n)] if count else []
    return lens + [0] * (n - len(lens))


def wrap32(v):
    return ((v + 2**31) % 2**32) - 2**31


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------
def pin_worked_example(o):
    """The handbook's printed 4-rank example (all_reduce, reduce_scatter,
    all_gather after reduce_scatter, RS+AG == AR), in every dtype, plus the
    average as the printed sum divided by 4."""
    g = goldens.load("collectives_4rank_example.txt")
    n = int(g["nranks"])
    x = [numbers(g[f"input.{r}"]) for r in range(n)]
    for dt in DTYPES:
        xin = [as_dtype(v, dt) for v in x]
        folded = o.fold_all_reduce(xin, dt, "sum")
        ring = [a.copy() for a in xin]
        o.ring_all_reduce(ring, dt, "sum")
        rs = o.reduce_scatter(xin, dt, "sum")
        ag = o.all_gather(rs, dt)
        avg = o.fold_all_reduce(xin, dt, "avg")
        for r in range(n):
            exp = numbers(g[f"all_reduce.{r}"])
            assert to_f64(folded[r], dt).tolist() == exp, (dt, r, folded[r])
            assert to_f64(ring[r], dt).tolist() == exp, (dt, r, ring[r])
            assert to_f64(rs[r], dt).tolist() == numbers(g[f"reduce_scatter.{r}"]), (dt, r, rs[r])
            assert to_f64(ag[r], dt).tolist() == numbers(g[f"all_gather.{r}"]), (dt, r, ag[r])
            assert same_bits(ag[r], folded[r]) == (g["rs_ag_equals_ar"] == "true")
            assert to_f64(avg[r], dt).tolist() == numbers(g["avg.0"]), (dt, r, avg[r])


def pin_bytes_sent_page(o):
    """ring_allreduce.py's printed run: 4 ranks x randn(1024) fp32, every rank
    sends 6144 bytes, and the result is allclose(atol=1e-5) to the exact sum."""
    g = goldens.load("ring_bytes_sent.txt")
    n, count = int(g["nranks"]), int(g["count"])
    xs = [torch.randn(count, generator=torch.Generator().manual_seed(r)).numpy() for r in range(n)]
    assert xs[0].nbytes == int(g["bytes_per_rank"])
    bufs = [a.copy() for a in xs]
    sent = o.ring_all_reduce(bufs, g["dtype"], "sum")
    assert sent == numbers(g["sent"]), sent
    exact = np.array([math.fsum(float(xs[r][i]) for r in range(n)) for i in range(count)])
    atol = float(g["allclose_atol"])
    for b in bufs:
        assert np.allclose(b.astype(np.float64), exact, atol=atol, rtol=1e-5)


def pin_bytes_closed_form(o):
    """Bytes sent: 2(N-1)/N * S per rank for divisible counts (geek-doc section
    四; handbook ring section); in general each rank sends every chunk but
    two, so sum over ranks = 2(N-1)S and rank r sends
    2S - |chunk r+1| e - |chunk r+2| e; reduce-scatter and all-gather each
    send (N-1)/N of their full size."""
    rng = np.random.default_rng(11)
    for dt in ("f32", "f16"):
        e = ELEM[dt]
        for n in (1, 2, 3, 4, 5, 7, 8, 9, 16):
            for count in sorted({0, 1, max(n - 1, 1), n, 3 * n, 5 * n + 1, 17, 64, 1000}):
                bufs = random_inputs(rng, n, count, dt, "sum")
                sent = o.ring_all_reduce(bufs, dt, "sum")
                S = count * e
                lens = torch_chunk_lens(n, count)
                assert sum(sent) == 2 * (n - 1) * S, (dt, n, count, sent)
                for r in range(n):
                    assert sent[r] == 2 * S - lens[(r + 1) % n] * e - lens[(r + 2) % n] * e, (dt, n, count, r)
                    if count % n == 0:
                        assert sent[r] * n == 2 * (n - 1) * S
            k = 7
            xs = random_inputs(rng, n, n * k, dt, "sum")
            _, rs_sent = o.reduce_scatter(xs, dt, "sum", with_sent=True)
            assert rs_sent == [(n - 1) * k * e] * n, (dt, n, rs_sent)
            _, ag_sent = o.all_gather([a[:k].copy() for a in xs], dt, with_sent=True)
            assert ag_sent == [(n - 1) * k * e] * n, (dt, n, ag_sent)


def pin_partition_torch_chunk(o):
    """Chunk boundaries follow torch.chunk (the page's ring calls t.chunk(n)),
    with empty trailing chunks where torch returns fewer than n."""
    for n in (1, 2, 3, 4, 5, 7, 8, 9, 16, 64):
        for count in list(range(0, 3 * n + 3)) + [1000, 4097, 65537]:
            b = o.chunk_bounds(n, count)
            lens = [hi - lo for lo, hi in b]
            assert lens == torch_chunk_lens(n, count), (n, count, lens)
            assert b[0][0] == 0 and all(b[i][1] == b[i + 1][0] for i in range(n - 1)) and b[-1][1] == count


def pin_ring_order(o):
    """fp32 sums follow the ring order c, c+1, ..., c+N-1 for chunk c (hand
    derivation from the geek-doc page's 4-GPU walk-through, section 三)."""
    g = goldens.load("ring_order_fp32.txt")
    n = int(g["nranks"])
    for case in ("big_at_0", "big_at_2"):
        xs = [as_dtype(numbers(g[f"{case}.input.{r}"]), "f32") for r in range(n)]
        for op in ("sum", "avg"):
            exp = numbers(g[f"{case}.{op}"])
            folded = o.fold_all_reduce(xs, "f32", op)
            ring = [a.copy() for a in xs]
            o.ring_all_reduce(ring, "f32", op)
            rs = o.reduce_scatter(xs, "f32", op)
            for r in range(n):
                assert folded[r].astype(np.float64).tolist() == exp, (case, op, folded[r])
                assert ring[r].astype(np.float64).tolist() == exp, (case, op, ring[r])
                assert float(rs[r][0]) == exp[r], (case, op, r, rs[r])


def pin_fp32_accumulate(o):
    """fp16/bf16 inputs are reduced in fp32 and rounded once (mhpq.cn article,
    section 5.3; hand-derived fixture)."""
    g = goldens.load("fp32_accumulate_low_precision.txt")
    n = int(g["nranks"])
    for dt in ("f16", "bf16"):
        xs = [as_dtype(numbers(g[f"{dt}.input.{r}"]), dt) for r in range(n)]
        exp = numbers(g[f"{dt}.sum"])
        folded = o.fold_all_reduce(xs, dt, "sum")
        ring = [a.copy() for a in xs]
        o.ring_all_reduce(ring, dt, "sum")
        for r in range(n):
            assert to_f64(folded[r], dt).tolist() == exp, (dt, folded[r])
            assert to_f64(ring[r], dt).tolist() == exp, (dt, ring[r])


def pin_forms_agree(o):
    """The literal ring and the per-element fold agree bit for bit, and every
    rank ends with the same result (the pages' defining invariant)."""
    rng = np.random.default_rng(5)
    for n in (1, 2, 3, 4, 5, 7, 8, 9, 16, 64):
        for count in sorted({0, 1, n + 1, max(3 * n - 1, 1), 37, 130}):
            for dt in DTYPES:
                for op in OPS:
                    xs = random_inputs(rng, n, count, dt, op)
                    folded = o.fold_all_reduce(xs, dt, op)
                    ring = [a.copy() for a in xs]
                    o.ring_all_reduce(ring, dt, op)
                    for r in range(n):
                        assert same_bits(folded[r], ring[r]), (n, count, dt, op, r)
                        assert same_bits(ring[r], ring[0]), (n, count, dt, op, r)


def pin_int_brute_force(o):
    """int32: every op against Python integers (order-free, exact), wrapped
    mod 2^32; AVG truncates toward zero."""
    rng = np.random.default_rng(3)
    for n in range(1, 10):
        for count in sorted({1, 5, n + 2, 23}):
            for op in OPS:
                xs = random_inputs(rng, n, count, "i32", op)
                vals = [[int(xs[r][i]) for r in range(n)] for i in range(count)]
                if op == "sum":
                    exp = [wrap32(sum(v)) for v in vals]
                elif op == "avg":
                    exp = []
                    for v in vals:
                        s = wrap32(sum(v))
                        q = abs(s) // n
                        exp.append(q if s >= 0 else -q)
                elif op == "prod":
                    exp = [wrap32(math.prod(v)) for v in vals]
                elif op == "max":
                    exp = [max(v) for v in vals]
                else:
                    exp = [min(v) for v in vals]
                folded = o.fold_all_reduce(xs, "i32", op)
                ring = [a.copy() for a in xs]
                o.ring_all_reduce(ring, "i32", op)
                for r in range(n):
                    assert folded[r].tolist() == exp, (n, count, op)
                    assert ring[r].tolist() == exp, (n, count, op)


def pin_fp_maxmin(o):
    """MAX/MIN are order-free: compare with numpy's maximum/minimum; signed
    zeros (+0 > -0) and NaN propagation checked case by case."""
    rng = np.random.default_rng(9)
    for dt in ("f32", "f16", "bf16"):
        for n in (1, 2, 3, 5, 8, 16):
            xs = random_inputs(rng, n, 200, dt, "max")
            x64 = np.stack([to_f64(a, dt) for a in xs])
            for op, fn in (("max", np.maximum), ("min", np.minimum)):
                out = o.fold_all_reduce(xs, dt, op)
                ring = [a.copy() for a in xs]
                o.ring_all_reduce(ring, dt, op)
                exp = fn.reduce(x64, axis=0)
                for r in range(n):
                    assert np.array_equal(to_f64(out[r], dt), exp), (dt, n, op)
                    assert np.array_equal(to_f64(ring[r], dt), exp), (dt, n, op)
        z0 = as_dtype([0.0, -0.0, 0.0, -0.0, np.nan, 1.0], dt)
        z1 = as_dtype([0.0, 0.0, -0.0, -0.0, 1.0, np.nan], dt)
        for op, sign in (("max", [False, False, False, True]), ("min", [False, True, True, True])):
            out = to_f64(o.fold_all_reduce([z0, z1], dt, op)[0], dt)
            assert np.signbit(out[:4]).tolist() == sign and np.all(out[:4] == 0), (dt, op, out)
            assert np.isnan(out[4]) and np.isnan(out[5]), (dt, op, out)


def _gamma(k, u):
    return k * u / (1 - k * u)


def pin_sum_error_bound(o):
    """SUM/AVG against the exact sum (math.fsum): recursive summation in fp32
    is within gamma_{N-1} * sum|x| (Higham, Accuracy and Stability of
    Numerical Algorithms, section 4.2), plus one rounding of the result to
    fp16/bf16 and one for the AVG divide."""
    rng = np.random.default_rng(13)
    u32 = 2.0 ** -24
    unit = {"f32": (2.0 ** -24, 2.0 ** -150), "f16": (2.0 ** -11, 2.0 ** -25), "bf16": (2.0 ** -8, 2.0 ** -134)}
    for dt in ("f32", "f16", "bf16"):
        for n in (2, 3, 4, 8, 16, 64):
            xs = random_inputs(rng, n, 300, dt, "sum")
            x64 = np.stack([to_f64(a, dt) for a in xs])
            exact = np.array([math.fsum(x64[:, i]) for i in range(x64.shape[1])])
            absum = np.abs(x64).sum(axis=0)
            g = _gamma(n - 1, u32)
            uo, tiny = unit[dt]
            for op in ("sum", "avg"):
                y = to_f64(o.fold_all_reduce(xs, dt, op)[0], dt)
                ref = exact if op == "sum" else exact / n
                scale = 1.0 if op == "sum" else 1.0 / n
                bound = g * absum * scale * (1 + 2 * u32) + (uo + u32) * np.abs(y) + tiny + 2.0 ** -52 * absum
                assert np.all(np.abs(y - ref) <= bound), (dt, n, op, np.max(np.abs(y - ref) - bound))


def pin_avg_pow2(o):
    """For N a power of two, AVG equals SUM scaled by 2^-k exactly (fp32)."""
    rng = np.random.default_rng(17)
    for n in (2, 4, 8, 16, 64):
        xs = random_inputs(rng, n, 257, "f32", "sum")
        s = o.fold_all_reduce(xs, "f32", "sum")[0]
        a = o.fold_all_reduce(xs, "f32", "avg")[0]
        assert same_bits(a, (s * np.float32(1.0 / n)).astype(np.float32)), n


def pin_avg_divide(o):
    """AVG is the finished sum divided once by N ("sum, then divide by N":
    mhpq.cn article, section 2.1; geek-doc page "训练梯度同步与集合通信",
    section 三), as one correctly rounded fp32 division, at any N. IEEE 754
    division in numpy (np.float32 / np.float32) is the library routine:
      fp32:      AVG == SUM / N, bit for bit;
      fp16/bf16: the fp32 sum of the exactly widened inputs (the oracle's
                 fp32 SUM of those fp32 values, whose order the ring-order
                 golden pins) divided by N in fp32, then rounded once to the
                 storage type by numpy (fp16) or torch (bf16), equals AVG.
    Non-powers of two are where a reciprocal multiply, x * (1/N), differs
    from x / N (power-of-two N are exact both ways)."""
    rng = np.random.default_rng(23)
    for n in (3, 5, 6, 7, 9, 63):
        for dt in ("f32", "f16", "bf16"):
            xs = random_inputs(rng, n, 2048, dt, "sum")
            avg = o.fold_all_reduce(xs, dt, "avg")[0]
            wide = [to_f64(a, dt).astype(np.float32) for a in xs]  # exact: every fp16/bf16 is an fp32
            s32 = o.fold_all_reduce(wide, "f32", "sum")[0]
            with np.errstate(over="ignore", under="ignore"):
                q = (s32 / np.float32(n)).astype(np.float32)
            if dt == "f32":
                exp = q
            elif dt == "f16":
                with np.errstate(over="ignore"):
                    exp = q.astype(np.float16)
            else:
                exp = torch.from_numpy(q.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            assert same_bits(avg, exp), (n, dt, int(np.sum(bits(avg) != bits(exp))))
            ring = [a.copy() for a in xs]
            o.ring_all_reduce(ring, dt, "avg")
            assert same_bits(ring[0], exp), (n, dt, "ring form")


def pin_prod_bound(o):
    """fp32 PROD against the exact product of the fp32 inputs (fractions): the
    relative error of N-1 rounded products is within gamma_{N-1}."""
    rng = np.random.default_rng(19)
    for n in (2, 3, 8, 64):
        xs = [as_dtype(rng.uniform(0.99, 1.01, size=50), "f32") for _ in range(n)]
        y = o.fold_all_reduce(xs, "f32", "prod")[0].astype(np.float64)
        g = _gamma(n - 1, 2.0 ** -24)
        for i in range(50):
            p = math.prod(Fraction(float(xs[r][i])) for r in range(n))
            assert abs(Fraction(float(y[i])) - p) <= Fraction(g) * abs(p), (n, i)


def pin_prod_double_rounding(o):
    """fp16 PROD is an fp32 product in ring order, rounded to fp16 once at the
    end (mhpq.cn article, section 5.3): on inputs where the last fp32 multiply
    lands on an fp16 tie, the result is numpy's fp32 product converted by
    numpy, which differs from rounding the exact product."""
    import rounding_cases
    for n in (3, 8):
        count = n * 64 + 5
        xs, idx = rounding_cases.ring_prod_inputs(n, count, 7, seed=5 + n)
        q = -(-count // n)
        c = np.arange(count) // q
        order = [(c + k) % n for k in range(n)]
        x = np.stack(xs)
        p = x[order[0], np.arange(count)].astype(np.float32)
        for k in range(1, n - 1):
            p = p * x[order[k], np.arange(count)].astype(np.float32)
        last = x[order[n - 1], np.arange(count)]
        exp = (p * last.astype(np.float32)).astype(np.float16)
        once = (p.astype(np.float64) * last.astype(np.float64)).astype(np.float16)
        assert idx.size > 0 and np.all(exp[idx] != once[idx]), "inputs do not separate one rounding from two"
        folded = o.fold_all_reduce(xs, "f16", "prod")
        ring = [a.copy() for a in xs]
        o.ring_all_reduce(ring, "f16", "prod")
        for r in range(n):
            assert same_bits(folded[r], exp), (n, r)
            assert same_bits(ring[r], exp), (n, r)


def pin_f16_conversions(o):
    """fp16 <-> fp32 conversions equal numpy's on all 2^16 patterns and on
    random fp32, on every halfway point between adjacent fp16 values and on its
    fp32 neighbours (NaN payloads are not compared)."""
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = o.f16_bits_to_f32(allh)
    ref = allh.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(f), nan)
    assert np.array_equal(f[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    rng = np.random.default_rng(23)
    finite = allh[~np.isnan(allh.view(np.float16)) & (allh & 0x7FFF != 0x7C00)].view(np.float16)
    pos = np.unique(np.abs(finite.astype(np.float64)))
    mid = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    x = np.concatenate([
        rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32).view(np.float32),
        mid, -mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(np.inf)),
        np.array([65504, 65519.99, 65520, 65536, 1e-8, 2.0 ** -25, 2.0 ** -24, np.inf, -np.inf, 0.0, -0.0],
                 dtype=np.float32)])
    h = o.f32_to_f16_bits(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16)
    nan = np.isnan(x)
    assert np.array_equal(np.isnan(h.view(np.float16)), nan)
    assert np.array_equal(h[~nan], ref.view(np.uint16)[~nan])


def pin_bf16_conversions(o):
    """bf16 <-> fp32 conversions equal torch's on all 2^16 patterns and on
    random fp32 and halfway points (NaN payloads are not compared)."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = o.bf16_bits_to_f32(allb)
    ref = torch.from_numpy(allb.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(f), nan)
    assert np.array_equal(f[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    rng = np.random.default_rng(29)
    base = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    ties = (base & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = np.concatenate([base, ties, ties + np.uint32(1), ties - np.uint32(1)]).view(np.float32)
    b = o.f32_to_bf16_bits(x)
    refb = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(np.isnan(to_f64(b, "bf16")), nan)
    assert np.array_equal(b[~nan], refb[~nan])


def pin_rs_ag_equals_ar(o):
    """Reduce-scatter followed by all-gather equals all-reduce, bit for bit
    (handbook, section 五个原语; geek-doc page, section 六)."""
    rng = np.random.default_rng(31)
    for n in (1, 2, 3, 4, 8, 16):
        for dt in DTYPES:
            for op in OPS:
                xs = random_inputs(rng, n, n * 9, dt, op)
                ar = o.fold_all_reduce(xs, dt, op)
                ag = o.all_gather(o.reduce_scatter(xs, dt, op), dt)
                for r in range(n):
                    assert same_bits(ag[r], ar[r]), (n, dt, op, r)


def pin_all_gather_concat(o):
    """All-gather output of every rank is the rank-ordered concatenation."""
    rng = np.random.default_rng(37)
    for n in (1, 2, 3, 5, 8):
        for dt in DTYPES:
            xs = random_inputs(rng, n, 13, dt, "sum")
            exp = np.concatenate(xs)
            for out in o.all_gather(xs, dt):
                assert same_bits(out, exp), (n, dt)


def pin_elements_match(o):
    """The one-element-at-a-time evaluator equals the fold on sampled indices."""
    rng = np.random.default_rng(41)
    for n in (1, 3, 8, 64):
        for dt in DTYPES:
            for op in OPS:
                count = 5 * n + 3
                xs = random_inputs(rng, n, count, dt, op)
                full = o.fold_all_reduce(xs, dt, op)[0]
                idx = rng.integers(0, count, size=20)
                vals = np.stack([xs[r][idx] for r in range(n)], axis=1)
                got = o.all_reduce_elements(vals, idx, count, dt, op)
                assert same_bits(got, full[idx]), (n, dt, op)


def pin_all_to_all(o):
    """All-to-all: the handbook's printed output (rank p gets [p, 10+p, 20+p,
    30+p]), numpy's transpose of the (rank, block) grid, applying it twice
    gives the input back, and each rank sends (n-1)/n of its data
    (handbook "集合通信原语", sections 五个原语 and 环形 all-reduce 与通信量)."""
    g = goldens.load("collectives_4rank_example.txt")
    n = int(g["nranks"])
    for dt in DTYPES:
        xs = [as_dtype(numbers(g[f"input.{r}"]), dt) for r in range(n)]
        outs, sent = o.all_to_all(xs, dt, with_sent=True)
        for p in range(n):
            assert to_f64(outs[p], dt).tolist() == numbers(g[f"all_to_all.{p}"]), (dt, p, outs[p])
        assert sent == [(n - 1) * ELEM[dt]] * n, sent
    rng = np.random.default_rng(43)
    for n in (1, 2, 3, 5, 8):
        for dt in DTYPES:
            bc = 7
            xs = random_inputs(rng, n, n * bc, dt, "sum")
            outs, sent = o.all_to_all(xs, dt, with_sent=True)
            grid = np.stack(xs).reshape(n, n, bc)
            exp = np.ascontiguousarray(grid.transpose(1, 0, 2)).reshape(n, n * bc)
            for p in range(n):
                assert same_bits(outs[p], exp[p]), (n, dt, p)
            back = o.all_to_all(outs, dt)
            for r in range(n):
                assert same_bits(back[r], xs[r]), (n, dt, r)
            assert sent == [(n - 1) * bc * ELEM[dt]] * n


def pin_tree(o):
    """Tree-order variant (geek-doc page, section 六): the printed integer
    example, the hand-derived fp32 order (tree (x0+x1)+(x2+x3) against the
    ring's chunk orders), order-free ops equal to the ring, the pairwise
    summation bound gamma_ceil(log2 N) * sum|x| (Higham, section 4.2), the
    closed-form tolerance 4*N*eps*sum|x| against the ring, and bytes sent:
    every edge carries S up and S down (2(N-1)S in all), the root sends
    ceil(log2 N)*S, odd ranks (leaves) send S."""
    g = goldens.load("collectives_4rank_example.txt")
    xs = [as_dtype(numbers(g[f"input.{r}"]), "f32") for r in range(4)]
    for r, out in enumerate(o.tree_all_reduce(xs, "f32", "sum")):
        assert out.astype(np.float64).tolist() == numbers(g[f"all_reduce.{r}"])
    t = goldens.load("tree_order_fp32.txt")
    xs = [as_dtype(numbers(t[f"input.{r}"]), "f32") for r in range(4)]
    for op in ("sum", "avg"):
        for out in o.tree_all_reduce(xs, "f32", op):
            assert out.astype(np.float64).tolist() == numbers(t[f"tree.{op}"]), (op, out)
    assert o.fold_all_reduce(xs, "f32", "sum")[0].astype(np.float64).tolist() == numbers(t["ring.sum"])
    rng = np.random.default_rng(47)
    eps = 2.0 ** -23
    for n in (1, 2, 3, 4, 5, 7, 8, 9, 16, 64):
        for dt in DTYPES:
            for op in OPS:
                xs = random_inputs(rng, n, 33, dt, op)
                tree, sent = o.tree_all_reduce(xs, dt, op, with_sent=True)
                S = 33 * ELEM[dt]
                L = (n - 1).bit_length()
                assert sum(sent) == 2 * (n - 1) * S
                assert sent[0] == L * S, (n, sent)
                assert all(sent[r] == S for r in range(1, n, 2)), (n, sent)
                for r in range(1, n):
                    assert same_bits(tree[r], tree[0]), (n, dt, op)
                ring = o.fold_all_reduce(xs, dt, op)[0]
                if dt == "i32" or op in ("max", "min"):
                    assert same_bits(tree[0], ring), (n, dt, op)
                elif op in ("sum", "avg"):
                    x64 = np.stack([to_f64(a, dt) for a in xs])
                    absum = np.abs(x64).sum(axis=0) / (n if op == "avg" else 1)
                    exact = np.array([math.fsum(x64[:, i]) for i in range(33)]) / (n if op == "avg" else 1)
                    ulp = {"f32": 0.0, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}[dt]
                    y = to_f64(tree[0], dt)
                    bound = _gamma(L, 2.0 ** -24) * absum * 1.01 + (ulp + 2.0 ** -24) * np.abs(y) + 1e-30
                    assert np.all(np.abs(y - exact) <= bound), (n, dt, op)
                    tol = 4 * n * eps * absum + 2 * ulp * np.abs(y) + 1e-30
                    assert np.all(np.abs(y - to_f64(ring, dt)) <= tol), (n, dt, op)


ALL_PINS = [
    pin_worked_example, pin_bytes_sent_page, pin_bytes_closed_form, pin_partition_torch_chunk,
    pin_ring_order, pin_fp32_accumulate, pin_forms_agree, pin_int_brute_force, pin_fp_maxmin,
    pin_sum_error_bound, pin_avg_pow2, pin_avg_divide, pin_prod_bound, pin_prod_double_rounding, pin_f16_conversions,
    pin_bf16_conversions,
    pin_rs_ag_equals_ar, pin_all_gather_concat, pin_elements_match, pin_all_to_all,
    pin_tree,
]


if __name__ == "__main__":
    # Run every pin against the oracle build named on the command line and
    # report which ones fail (used by the mutant tests).
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import oracle
    lib = oracle.Oracle(sys.argv[1])
    for pin in ALL_PINS:
        try:
            pin(lib)
            print("pass", pin.__name__, flush=True)
        except (AssertionError, RuntimeError, ValueError) as exc:
            print("CAUGHT", pin.__name__, repr(exc)[:200], flush=True)
            if "--all" not in sys.argv:
                break
