"""fp16 PROD inputs on which one rounding and two roundings disagree.

fp16 inputs are reduced in fp32 and the finished value is rounded to fp16
once (mhpq.cn article, section 5.3). For PROD the last fp32 multiply already
rounds: when that fp32 product lands exactly halfway between two fp16 values
while the exact product does not, rounding the fp32 product to fp16 (ties to
even) can go the other way from rounding the exact product. A kernel that
merges the last multiply and the conversion into one mixed-precision FMA
rounds once and gets those elements wrong by one fp16 ulp.

The search uses numpy's IEEE fp32 multiply; the exact product of an fp32
value and an fp16 value has at most 35 significant bits, so fp64 holds it
exactly. The ring folds chunk c in rank order c, c+1, ..., c+N-1 (mod N), so
a found tuple is rotated per chunk to reach the ranks in that order.
"""
from __future__ import annotations

import numpy as np


def _fold32(t: np.ndarray):
    """Sequential fp32 product over axis 1: (fp32 product of all but the last
    factor, fp32 product of all)."""
    p = t[:, 0].astype(np.float32)
    for k in range(1, t.shape[1] - 1):
        p = p * t[:, k].astype(np.float32)
    return p, p * t[:, -1].astype(np.float32)


def discriminating_tuples(n: int, want: int, seed: int) -> np.ndarray:
    """`want` rows of n fp16 factors in [0.5, 2) (in fold order) whose last
    fp32 product is an fp16 tie that ties-to-even rounds the other way from
    the exact product."""
    assert n >= 3, "a product of two fp16 values is exact in fp32"
    rng = np.random.default_rng(seed)
    found = []
    have = 0
    while have < want:
        m = 1 << 20
        # fp16 values in [0.5, 2): exponent -1 or 0, random 10-bit mantissa.
        bits = (rng.integers(14, 16, size=(m, n), dtype=np.uint16) << 10) | rng.integers(0, 1024, size=(m, n),
                                                                                        dtype=np.uint16)
        t = bits.view(np.float16)
        head, p32 = _fold32(t)
        exact = head.astype(np.float64) * t[:, -1].astype(np.float64)
        u = p32.view(np.uint32)
        # fp32 values in [2^-14, 65504] convert with 13 dropped mantissa bits;
        # a tie has exactly the top dropped bit set.
        tie = (u & 0x1FFF) == 0x1000
        up_even = ((u >> 13) & 1) == 1          # ties-to-even rounds up iff the kept LSB is odd
        up_exact = exact > p32.astype(np.float64)
        normal = (np.abs(p32) >= np.float32(2.0 ** -14)) & (np.abs(p32) < np.float32(65504.0))
        sel = normal & tie & (exact != p32.astype(np.float64)) & (up_even != up_exact)
        found.append(t[sel])
        have += int(sel.sum())
    return np.concatenate(found)[:want]


def ring_prod_inputs(n: int, count: int, every: int, seed: int):
    """Per-rank fp16 arrays of `count` elements: random factors in [0.5, 2),
    with a discriminating tuple at every `every`-th element, rotated so the
    ring's fold for that element's chunk meets its factors in order.
    Returns (arrays, indices of the planted elements)."""
    rng = np.random.default_rng(seed + 1)
    xs = rng.uniform(0.5, 2.0, size=(n, count)).astype(np.float16)
    if count == 0:
        return list(xs), np.zeros(0, dtype=np.int64)
    idx = np.arange(0, count, every, dtype=np.int64)
    tuples = discriminating_tuples(n, idx.size, seed)
    q = -(-count // n)
    chunk = idx // q
    for k in range(n):
        xs[(chunk + k) % n, idx] = tuples[:, k]
    return list(xs), idx
