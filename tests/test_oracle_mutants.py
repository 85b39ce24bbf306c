"""Plant plausible mistakes in copies of the oracle's C source (on the CPU) and
check that at least one pin catches each: a dropped term, a wrong index or
sign, a wrong rounding, a transposed or misplaced operand."""
import os
import subprocess
import sys

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ring_oracle.c")

# (name, text in the source, replacement)
MUTANTS = [
    ("rs_recv_index", "int c = mod(r - s - 1, n);", "int c = mod(r - s, n);"),
    ("rs_send_index", "int c = mod(r - s, n);\n            bounds(n, count, c, &lo, &hi);\n            acc_t* to",
     "int c = mod(r - s + 1, n);\n            bounds(n, count, c, &lo, &hi);\n            acc_t* to"),
    ("ag_recv_index", "bounds(n, count, mod(r - s, n), &lo, &hi);", "bounds(n, count, mod(r - s + 1, n), &lo, &hi);"),
    ("finished_chunk_holder", "bounds(n, count, (r + 1) % n, &lo, &hi);", "bounds(n, count, r, &lo, &hi);"),
    ("rs_export_holder", "int holder = mod(c - 1, n);", "int holder = c;"),
    ("partition_floor", "(count + (uint64_t)n - 1) / (uint64_t)n", "(count + (uint64_t)n / 2) / (uint64_t)n"),
    ("fold_starts_at_zero", "int c = (int)(i / q);", "int c = 0;"),
    ("fold_reverse_ring", "in[(c + k) % n]", "in[(c + n - k) % n]"),
    ("fold_drops_last_rank", "for (int k = 1; k < n; k++) acc = combine(dtype, op, widen(dtype, in[",
     "for (int k = 1; k < n - 1; k++) acc = combine(dtype, op, widen(dtype, in["),
    ("sum_sign", "r.f = local.f + incoming.f;", "r.f = local.f - incoming.f;"),
    ("int_sum_sign", "r.u = local.u + incoming.u;", "r.u = local.u - incoming.u;"),
    ("avg_not_divided", "a.f = a.f / (float)n;", "a.f = a.f;"),
    ("avg_multiplies_reciprocal", "a.f = a.f / (float)n;", "a.f = a.f * (1.0f / (float)(3 * n));"),
    ("avg_reciprocal_of_n", "a.f = a.f / (float)n;", "a.f = a.f * (1.0f / (float)n);"),
    ("int_avg_floor", "a.u = (uint32_t)((int32_t)a.u / (int32_t)n);",
     "a.u = (uint32_t)(int32_t)floor((double)(int32_t)a.u / (double)n);"),
    ("max_zero_sign", "return (signbit(a) && signbit(b)) ? -0.0f : 0.0f;",
     "return (signbit(a) || signbit(b)) ? -0.0f : 0.0f;"),
    ("min_is_max", "return a < b ? a : b;", "return a > b ? a : b;"),
    ("int_max_unsigned", "r.u = (uint32_t)(a > b ? a : b);", "r.u = local.u > incoming.u ? local.u : incoming.u;"),
    ("prod_is_sum", "r.f = local.f * incoming.f;", "r.f = local.f + incoming.f;"),
    ("half_truncates", "float m = rintf(ldexpf(a, 10 - e));", "float m = truncf(ldexpf(a, 10 - e));"),
    ("half_subnormal_truncates", "float m = rintf(a * 0x1p24f);", "float m = truncf(a * 0x1p24f);"),
    ("half_bias", "(uint16_t)((e + 15) << 10)", "(uint16_t)((e + 14) << 10)"),
    ("half_decode_subnormal", "mag = ldexpf((float)frac, -24);", "mag = ldexpf((float)frac, -25);"),
    ("bf16_ties_away", "float m = rintf(ldexpf(a, 7 - e));", "float m = roundf(ldexpf(a, 7 - e));"),
    ("bf16_subnormal", "float m = rintf(ldexpf(a, 133));", "float m = rintf(ldexpf(a, 132));"),
    ("bytes_in_acc_type", "if (sent) sent[r] += (hi - lo) * e;", "if (sent) sent[r] += (hi - lo) * sizeof(acc_t);"),
    ("ag_bytes_dropped", "(size_t)(hi - lo) * e);\n            sent[r] += (hi - lo) * e;",
     "(size_t)(hi - lo) * e);\n            sent[r] += 0 * (hi - lo) * e;"),
    ("f16_accumulates_in_f16", "acc = combine(dtype, op, widen(dtype, in[(c + k) % n], i), acc);",
     "acc = combine(dtype, op, widen(dtype, in[(c + k) % n], i), acc);\n"
     "            if (dtype == ORC_F16) acc.f = half_to_float(float_to_half(acc.f));"),
    ("alltoall_transposed_wrong", "memcpy((unsigned char*)out[p] + (size_t)r * blk, (const unsigned char*)in[r] + (size_t)p * blk, blk);",
     "memcpy((unsigned char*)out[p] + (size_t)p * blk, (const unsigned char*)in[r] + (size_t)r * blk, blk);"),
    ("alltoall_counts_own_block", "if (sent && p != r) sent[r] += blk;", "if (sent) sent[r] += blk;"),
    ("tree_pairs_wrong_partner", "int q = r + stride;", "int q = r + stride / 2 + (stride == 1);"),
    ("tree_no_broadcast_count", "memcpy(out[r + stride], out[r], bytes);\n            if (sent) sent[r] += bytes;",
     "memcpy(out[r + stride], out[r], bytes);"),
    ("tree_sequential_order", "for (uint64_t i = 0; i < count; i++) W[r][i] = combine(dtype, op, W[r][i], W[q][i]);",
     "for (uint64_t i = 0; i < count; i++) W[r][i] = combine(dtype, op, W[r][i], W[q][i]);\n"
     "            if (r == 0 && stride == 1) for (int k = 2; k < n; k++) for (uint64_t i = 0; i < count; i++) W[0][i] = combine(dtype, op, W[0][i], W[k][i]);\n"
     "            if (r == 0 && stride == 1) { stride = n; break; }"),
    ("allgather_block_order", "memmove((unsigned char*)out[r] + (size_t)r * blk, in[r], blk);",
     "memmove((unsigned char*)out[r] + (size_t)((r + 1) % n) * blk, in[r], blk);"),
]


def test_mutant_table_matches_source():
    src = open(SRC, encoding="utf-8").read()
    for name, old, _ in MUTANTS:
        assert src.count(old) == 1, f"mutant {name}: pattern found {src.count(old)} times"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_some_pin_catches_mutant(tmp_path, name, old, new):
    src = open(SRC, encoding="utf-8").read()
    assert src.count(old) == 1
    mutant_src = tmp_path / "ring_oracle_mutant.c"
    mutant_src.write_text(src.replace(old, new), encoding="utf-8")
    lib = oracle.build(str(mutant_src), str(tmp_path / "liboracle_mutant.so"))
    # Run the pins in a child process: a mutant may also crash (an index
    # mistake can read out of bounds), which counts as caught.
    proc = subprocess.run([sys.executable, pins.__file__, lib], capture_output=True, text=True, timeout=600)
    caught = proc.returncode != 0 or "CAUGHT" in proc.stdout
    assert caught, f"no pin catches mutant {name}: {proc.stdout[-2000:]}"
