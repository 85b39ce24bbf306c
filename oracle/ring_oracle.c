/*
 * ring_oracle.c -- plain, slow CPU oracle for the ring all-reduce.
 *
 * TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the CPU-baseline leg
 * of the benchmark load this file's library to check the GPU library against;
 * the GPU library never loads, links or calls it, and the two share no source,
 * header, table or helper.
 *
 * Sources (web pages; cited by title and section):
 *  [P1] mhpq.cn news/451051, "all-reduce 到底怎样让每张卡上的模型保持一致":
 *       s2.1 (the five reduce ops; AVG = sum then divide by N),
 *       s2.2 (deterministic result), s3.2 (reduce-scatter + all-gather ring),
 *       s5.3 (reduce fp16/bf16 gradients in fp32).
 *  [P3] geek-doc.cn, "训练梯度同步与集合通信:从参数服务器到 Ring AllReduce":
 *       section 三 (the two ring phases, the 4-GPU walk-through: chunk 0 grows
 *       as g0+g1, then +g2, then +g3; the result is the sum divided by N),
 *       section 四 (per-rank traffic 2(N-1)/N * M), section 六 (tree
 *       reduction: cards add in pairs, the results add in pairs again, after
 *       log2(N) levels the root holds the result, which is then broadcast back
 *       down the tree).
 *  [P4] anrans.github.io handbook, "集合通信原语": section 五个原语 (printed
 *       4-rank example; reduce_scatter gives rank r block r; all_gather
 *       concatenates in rank order) and section 环形 all-reduce 与通信量
 *       (ring_allreduce.py: chunk views from t.chunk(n); reduce-scatter step s
 *       sends chunk (rank - s) to the right and adds the received chunk into
 *       chunk (rank - s - 1); all-gather step s sends chunk (rank + 1 - s) and
 *       copies the received one into chunk (rank - s); bytes sent counted as
 *       numel * element_size per send); all_to_all in section 五个原语: rank
 *       r's p-th block goes to rank p, which stores it as its r-th block; each
 *       rank sends (n-1)/n of its data (its own block stays).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - partition: q = ceil(count / N); chunk c = [c*q, min((c+1)*q, count)),
 *    empty when c*q >= count (the chunk boundaries torch.chunk uses, with
 *    empty trailing chunks where torch would return fewer than N).
 *  - accumulator: fp32 for fp32/fp16/bf16 (inputs widened exactly, one
 *    round-to-nearest-even back to the storage type at the end, after the AVG
 *    divide); uint32 two's-complement wrap for int32.
 *  - AVG: one correctly rounded fp32 divide by N (int32: C division, which
 *    truncates toward zero), applied at the rank that finishes the chunk,
 *    before the all-gather.
 *  - MAX/MIN: NaN if either operand is NaN (canonical quiet NaN); otherwise
 *    the larger/smaller value, with +0 > -0. NaN payloads are not specified.
 *  - combine operand order: local (+) incoming, as the page's code adds the
 *    received buffer into its own chunk.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -fno-fast-math.
 * No FMA contraction, no flush-to-zero: x86-64 SSE arithmetic is IEEE single.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_I32 = 3 };
enum { ORC_SUM = 0, ORC_AVG = 1, ORC_MAX = 2, ORC_MIN = 3, ORC_PROD = 4 };

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_ENOMEM (-2)

/* One accumulator slot: fp32 for the floating types, uint32 for int32. */
typedef union {
    float f;
    uint32_t u;
} acc_t;

/* ------------------------------------------------------------------------ */
/* bit casts                                                                  */
/* ------------------------------------------------------------------------ */
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* ------------------------------------------------------------------------ */
/* IEEE-754 binary16 and bfloat16 conversions, written from the format       */
/* definitions (sign, biased exponent, fraction) and round-to-nearest-even.  */
/* ------------------------------------------------------------------------ */

/* binary16 -> binary32. Every half value is exactly representable. */
static float half_to_float(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) & 1u;
    uint32_t exp = (uint32_t)(h >> 10) & 0x1Fu;
    uint32_t frac = (uint32_t)h & 0x3FFu;
    float mag;
    if (exp == 0) {
        /* zero or subnormal: frac * 2^-24 */
        mag = ldexpf((float)frac, -24);
    } else if (exp == 31) {
        if (frac == 0)
            mag = INFINITY;
        else
            return u2f((sign << 31) | 0x7F800000u | (frac << 13) | 0x00400000u);
    } else {
        /* normal: (1024 + frac) * 2^(exp - 15 - 10) */
        mag = ldexpf((float)(1024u + frac), (int)exp - 25);
    }
    return sign ? -mag : mag;
}

/* binary32 -> binary16, round to nearest, ties to even. */
static uint16_t float_to_half(float x)
{
    uint32_t bits = f2u(x);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    float a = fabsf(x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7E00u);
    if (isinf(x))
        return (uint16_t)(sign | 0x7C00u);
    if (a < 0x1p-14f) {
        /* subnormal range: the result is an integer multiple of 2^-24.
         * a * 2^24 is exact (power-of-two scaling of a normal or subnormal
         * float whose result stays below 2^10); rintf rounds it to the
         * nearest integer, ties to even (the default rounding mode). A
         * result of 1024 is the smallest normal, whose bit pattern is 0x0400. */
        float m = rintf(a * 0x1p24f);
        return (uint16_t)(sign | (uint16_t)m);
    }
    int e;
    (void)frexpf(a, &e); /* a = f * 2^e with f in [0.5, 1): unbiased exponent e-1 */
    e -= 1;
    /* significand with 10 fraction bits: a / 2^(e-10) in [1024, 2048) */
    float m = rintf(ldexpf(a, 10 - e));
    if (m == 2048.0f) {
        m = 1024.0f;
        e += 1;
    }
    if (e > 15)
        return (uint16_t)(sign | 0x7C00u); /* overflow to infinity */
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)((uint32_t)m - 1024u));
}

/* bfloat16 -> binary32: the upper half of the binary32 pattern. */
static float bf16_to_float(uint16_t b) { return u2f((uint32_t)b << 16); }

/* binary32 -> bfloat16 (8 exponent bits, 7 fraction bits), ties to even. */
static uint16_t float_to_bf16(float x)
{
    uint32_t bits = f2u(x);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    float a = fabsf(x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0u);
    if (isinf(x))
        return (uint16_t)(sign | 0x7F80u);
    if (a < 0x1p-126f) {
        /* subnormal range: integer multiple of 2^-133. a * 2^133 < 2^7 is exact. */
        float m = rintf(ldexpf(a, 133));
        return (uint16_t)(sign | (uint16_t)m);
    }
    int e;
    (void)frexpf(a, &e);
    e -= 1;
    /* significand with 7 fraction bits: a / 2^(e-7) in [128, 256) */
    float m = rintf(ldexpf(a, 7 - e));
    if (m == 256.0f) {
        m = 128.0f;
        e += 1;
    }
    if (e > 127)
        return (uint16_t)(sign | 0x7F80u);
    return (uint16_t)(sign | (uint16_t)((e + 127) << 7) | (uint16_t)((uint32_t)m - 128u));
}

/* ------------------------------------------------------------------------ */
/* element access and the reduce ops                                          */
/* ------------------------------------------------------------------------ */
static size_t elem_size(int dtype)
{
    switch (dtype) {
    case ORC_F32: return 4;
    case ORC_F16: return 2;
    case ORC_BF16: return 2;
    case ORC_I32: return 4;
    default: return 0;
    }
}

/* Read element i of a storage-typed buffer into an accumulator (exact). */
static acc_t widen(int dtype, const void* buf, uint64_t i)
{
    acc_t a;
    switch (dtype) {
    case ORC_F32: a.f = ((const float*)buf)[i]; break;
    case ORC_F16: a.f = half_to_float(((const uint16_t*)buf)[i]); break;
    case ORC_BF16: a.f = bf16_to_float(((const uint16_t*)buf)[i]); break;
    default: a.u = ((const uint32_t*)buf)[i]; break;
    }
    return a;
}

/* Write an accumulator back in the storage type (round to nearest even). */
static void narrow(int dtype, acc_t a, void* buf, uint64_t i)
{
    switch (dtype) {
    case ORC_F32: ((float*)buf)[i] = a.f; break;
    case ORC_F16: ((uint16_t*)buf)[i] = float_to_half(a.f); break;
    case ORC_BF16: ((uint16_t*)buf)[i] = float_to_bf16(a.f); break;
    default: ((uint32_t*)buf)[i] = a.u; break;
    }
}

static float fp_max(float a, float b)
{
    if (isnan(a) || isnan(b))
        return u2f(0x7FC00000u);
    if (a == 0.0f && b == 0.0f) /* +0 > -0: the result is -0 only if both are -0 */
        return (signbit(a) && signbit(b)) ? -0.0f : 0.0f;
    return a > b ? a : b;
}

static float fp_min(float a, float b)
{
    if (isnan(a) || isnan(b))
        return u2f(0x7FC00000u);
    if (a == 0.0f && b == 0.0f) /* -0 < +0: the result is +0 only if both are +0 */
        return (signbit(a) || signbit(b)) ? -0.0f : 0.0f;
    return a < b ? a : b;
}

/* local (+) incoming. SUM and AVG both add here; AVG divides at the end. */
static acc_t combine(int dtype, int op, acc_t local, acc_t incoming)
{
    acc_t r;
    if (dtype == ORC_I32) {
        int32_t a = (int32_t)local.u, b = (int32_t)incoming.u;
        switch (op) {
        case ORC_SUM:
        case ORC_AVG: r.u = local.u + incoming.u; break;       /* wraps mod 2^32 */
        case ORC_PROD: r.u = local.u * incoming.u; break;      /* wraps mod 2^32 */
        case ORC_MAX: r.u = (uint32_t)(a > b ? a : b); break;
        default: r.u = (uint32_t)(a < b ? a : b); break;
        }
        return r;
    }
    switch (op) {
    case ORC_SUM:
    case ORC_AVG: r.f = local.f + incoming.f; break;
    case ORC_PROD: r.f = local.f * incoming.f; break;
    case ORC_MAX: r.f = fp_max(local.f, incoming.f); break;
    default: r.f = fp_min(local.f, incoming.f); break;
    }
    return r;
}

/* AVG: divide the finished sum by N once. */
static acc_t finalize(int dtype, int op, int n, acc_t a)
{
    if (op != ORC_AVG)
        return a;
    if (dtype == ORC_I32)
        a.u = (uint32_t)((int32_t)a.u / (int32_t)n); /* C division truncates toward zero */
    else
        a.f = a.f / (float)n; /* one correctly rounded binary32 divide */
    return a;
}

/* ------------------------------------------------------------------------ */
/* partition                                                                  */
/* ------------------------------------------------------------------------ */
static uint64_t chunk_len(int n, uint64_t count) { return count == 0 ? 0 : (count + (uint64_t)n - 1) / (uint64_t)n; }

static void bounds(int n, uint64_t count, int c, uint64_t* lo, uint64_t* hi)
{
    uint64_t q = chunk_len(n, count);
    uint64_t a = (uint64_t)c * q, b = (uint64_t)(c + 1) * q;
    *lo = a < count ? a : count;
    *hi = b < count ? b : count;
}

static int mod(int a, int n) { int m = a % n; return m < 0 ? m + n : m; }

static int valid(int n, int dtype, int op)
{
    return n >= 1 && n <= 4096 && elem_size(dtype) != 0 && op >= ORC_SUM && op <= ORC_PROD;
}

/* ------------------------------------------------------------------------ */
/* the literal ring                                                           */
/* ------------------------------------------------------------------------ */

/*
 * Reduce-scatter phase of the ring on per-rank accumulator copies W[r].
 * Each of the N-1 steps has two halves, as a real exchange would: first every
 * rank copies the chunk it sends into its right neighbour's message buffer,
 * then every rank combines the message it received into its own chunk.
 * Step s: rank r sends chunk (r - s) mod N and combines into chunk
 * (r - s - 1) mod N. After the last step rank r holds the complete
 * reduction of chunk (r + 1) mod N.
 */
static int ring_reduce_scatter_phase(int n, uint64_t count, int dtype, int op, acc_t** W, uint64_t* sent)
{
    uint64_t q = chunk_len(n, count);
    size_t e = elem_size(dtype);
    acc_t** msg = (acc_t**)calloc((size_t)n, sizeof(acc_t*));
    if (!msg)
        return ORC_ENOMEM;
    for (int r = 0; r < n; r++) {
        msg[r] = (acc_t*)malloc((size_t)(q ? q : 1) * sizeof(acc_t));
        if (!msg[r]) {
            for (int k = 0; k < r; k++) free(msg[k]);
            free(msg);
            return ORC_ENOMEM;
        }
    }
    for (int s = 0; s < n - 1; s++) {
        for (int r = 0; r < n; r++) { /* send */
            uint64_t lo, hi;
            int c = mod(r - s, n);
            bounds(n, count, c, &lo, &hi);
            acc_t* to = msg[(r + 1) % n];
            for (uint64_t i = lo; i < hi; i++) to[i - lo] = W[r][i];
            if (sent) sent[r] += (hi - lo) * e;
        }
        for (int r = 0; r < n; r++) { /* receive and combine: local (+) incoming */
            uint64_t lo, hi;
            int c = mod(r - s - 1, n);
            bounds(n, count, c, &lo, &hi);
            for (uint64_t i = lo; i < hi; i++) W[r][i] = combine(dtype, op, W[r][i], msg[r][i - lo]);
        }
    }
    for (int r = 0; r < n; r++) free(msg[r]);
    free(msg);
    return ORC_OK;
}

static void free_ranks(int n, acc_t** W)
{
    if (!W) return;
    for (int r = 0; r < n; r++) free(W[r]);
    free(W);
}

/* Per-rank accumulator copies of the inputs (each element widened exactly). */
static acc_t** widen_ranks(int n, uint64_t count, int dtype, const void* const* in)
{
    acc_t** W = (acc_t**)calloc((size_t)n, sizeof(acc_t*));
    if (!W) return NULL;
    for (int r = 0; r < n; r++) {
        W[r] = (acc_t*)malloc((size_t)(count ? count : 1) * sizeof(acc_t));
        if (!W[r]) { free_ranks(n, W); return NULL; }
        for (uint64_t i = 0; i < count; i++) W[r][i] = widen(dtype, in[r], i);
    }
    return W;
}

/*
 * All-reduce by the literal ring, in place on host buffers bufs[0..n-1]
 * (count elements each). sent[r] receives the bytes rank r sent, counted in
 * the storage type (numel * element_size per send). Returns 0 or < 0.
 */
int orc_ring_all_reduce(int n, uint64_t count, int dtype, int op, void* const* bufs, uint64_t* sent)
{
    if (!valid(n, dtype, op) || !bufs || !sent)
        return ORC_EINVAL;
    for (int r = 0; r < n; r++) {
        sent[r] = 0;
        if (!bufs[r] && count) return ORC_EINVAL;
    }
    if (count == 0)
        return ORC_OK;
    size_t e = elem_size(dtype);
    acc_t** W = widen_ranks(n, count, dtype, (const void* const*)bufs);
    if (!W) return ORC_ENOMEM;
    int rc = ring_reduce_scatter_phase(n, count, dtype, op, W, sent);
    if (rc != ORC_OK) { free_ranks(n, W); return rc; }

    /* The holder of each finished chunk applies AVG and rounds to the storage type. */
    for (int r = 0; r < n; r++) {
        uint64_t lo, hi;
        bounds(n, count, (r + 1) % n, &lo, &hi);
        for (uint64_t i = lo; i < hi; i++) narrow(dtype, finalize(dtype, op, n, W[r][i]), bufs[r], i);
    }
    free_ranks(n, W);

    /* All-gather: N-1 steps of forwarding finished chunks in the storage type.
     * Step s: rank r sends chunk (r + 1 - s) mod N and copies the received
     * chunk into chunk (r - s) mod N. */
    uint64_t q = chunk_len(n, count);
    unsigned char** msg = (unsigned char**)calloc((size_t)n, sizeof(unsigned char*));
    if (!msg) return ORC_ENOMEM;
    for (int r = 0; r < n; r++) {
        msg[r] = (unsigned char*)malloc((size_t)q * e);
        if (!msg[r]) { for (int k = 0; k < r; k++) free(msg[k]); free(msg); return ORC_ENOMEM; }
    }
    for (int s = 0; s < n - 1; s++) {
        for (int r = 0; r < n; r++) {
            uint64_t lo, hi;
            bounds(n, count, mod(r + 1 - s, n), &lo, &hi);
            memcpy(msg[(r + 1) % n], (unsigned char*)bufs[r] + lo * e, (size_t)(hi - lo) * e);
            sent[r] += (hi - lo) * e;
        }
        for (int r = 0; r < n; r++) {
            uint64_t lo, hi;
            bounds(n, count, mod(r - s, n), &lo, &hi);
            memcpy((unsigned char*)bufs[r] + lo * e, msg[r], (size_t)(hi - lo) * e);
        }
    }
    for (int r = 0; r < n; r++) free(msg[r]);
    free(msg);
    return ORC_OK;
}

/*
 * The same all-reduce as a per-element fold: element i of chunk c is
 * acc = x_c[i]; acc = x_{c+k}[i] (+) acc for k = 1..N-1 (ranks mod N);
 * then AVG and rounding; then the value goes to every output. This is the
 * order in which a chunk's partial sum travels round the ring. in and out
 * may be the same buffers (every input of element i is read before any
 * output of element i is written).
 */
int orc_fold_all_reduce(int n, uint64_t count, int dtype, int op, const void* const* in, void* const* out)
{
    if (!valid(n, dtype, op) || !in || !out)
        return ORC_EINVAL;
    uint64_t q = chunk_len(n, count);
    for (uint64_t i = 0; i < count; i++) {
        int c = (int)(i / q);
        acc_t acc = widen(dtype, in[c], i);
        for (int k = 1; k < n; k++) acc = combine(dtype, op, widen(dtype, in[(c + k) % n], i), acc);
        acc = finalize(dtype, op, n, acc);
        for (int r = 0; r < n; r++) narrow(dtype, acc, out[r], i);
    }
    return ORC_OK;
}

/*
 * Selected elements of an all-reduce of n ranks x count elements, one at a
 * time (for checks at sizes too large to copy to the host whole).
 * vals[j*n + r] is rank r's input at element idx[j] (storage type);
 * out[j] receives the all-reduced value of element idx[j].
 */
int orc_all_reduce_elements(int n, uint64_t count, int dtype, int op, const void* vals, const uint64_t* idx,
                            uint64_t m, void* out)
{
    if (!valid(n, dtype, op) || (m && (!vals || !idx || !out)))
        return ORC_EINVAL;
    uint64_t q = chunk_len(n, count);
    for (uint64_t j = 0; j < m; j++) {
        if (idx[j] >= count) return ORC_EINVAL;
        int c = (int)(idx[j] / q);
        uint64_t base = j * (uint64_t)n;
        acc_t acc = widen(dtype, vals, base + (uint64_t)c);
        for (int k = 1; k < n; k++) acc = combine(dtype, op, widen(dtype, vals, base + (uint64_t)((c + k) % n)), acc);
        narrow(dtype, finalize(dtype, op, n, acc), out, j);
    }
    return ORC_OK;
}

/*
 * Reduce-scatter: in[r] holds n*recvcount elements; out[c] receives the
 * reduced block c (rank r gets block r). Computed by the ring's
 * reduce-scatter phase; block c is finished at rank (c - 1) mod n.
 * sent[r] (may be NULL) receives rank r's bytes sent.
 */
int orc_reduce_scatter(int n, uint64_t recvcount, int dtype, int op, const void* const* in, void* const* out,
                       uint64_t* sent)
{
    if (!valid(n, dtype, op) || !in || !out)
        return ORC_EINVAL;
    if (sent) for (int r = 0; r < n; r++) sent[r] = 0;
    uint64_t count = recvcount * (uint64_t)n;
    if (count == 0)
        return ORC_OK;
    acc_t** W = widen_ranks(n, count, dtype, in);
    if (!W) return ORC_ENOMEM;
    int rc = ring_reduce_scatter_phase(n, count, dtype, op, W, sent);
    if (rc == ORC_OK) {
        for (int c = 0; c < n; c++) {
            int holder = mod(c - 1, n);
            for (uint64_t j = 0; j < recvcount; j++)
                narrow(dtype, finalize(dtype, op, n, W[holder][(uint64_t)c * recvcount + j]), out[c], j);
        }
    }
    free_ranks(n, W);
    return rc;
}

/*
 * All-gather by the ring: in[r] holds sendcount elements; out[r] receives
 * the n blocks in rank order. Rank r first places its own block; step s
 * (s = 0..n-2) forwards block (r - s) mod n to the right neighbour, which
 * stores it at block position (r - s) mod n. in[r] may equal
 * out[r] + r*sendcount elements. sent[r] (may be NULL) receives bytes sent.
 */
int orc_all_gather(int n, uint64_t sendcount, int dtype, const void* const* in, void* const* out, uint64_t* sent)
{
    if (!valid(n, dtype, ORC_SUM) || !in || !out)
        return ORC_EINVAL;
    size_t e = elem_size(dtype);
    size_t blk = (size_t)sendcount * e;
    if (sent) for (int r = 0; r < n; r++) sent[r] = 0;
    if (sendcount == 0)
        return ORC_OK;
    for (int r = 0; r < n; r++) memmove((unsigned char*)out[r] + (size_t)r * blk, in[r], blk);
    unsigned char** msg = (unsigned char**)calloc((size_t)n, sizeof(unsigned char*));
    if (!msg) return ORC_ENOMEM;
    for (int r = 0; r < n; r++) {
        msg[r] = (unsigned char*)malloc(blk);
        if (!msg[r]) { for (int k = 0; k < r; k++) free(msg[k]); free(msg); return ORC_ENOMEM; }
    }
    for (int s = 0; s < n - 1; s++) {
        for (int r = 0; r < n; r++) {
            int b = mod(r - s, n);
            memcpy(msg[(r + 1) % n], (unsigned char*)out[r] + (size_t)b * blk, blk);
            if (sent) sent[r] += blk;
        }
        for (int r = 0; r < n; r++) {
            int b = mod(r - s - 1, n);
            memcpy((unsigned char*)out[r] + (size_t)b * blk, msg[r], blk);
        }
    }
    for (int r = 0; r < n; r++) free(msg[r]);
    free(msg);
    return ORC_OK;
}

/*
 * Tree all-reduce, the literal form: level l = 0, 1, ... pairs rank r (r a
 * multiple of 2^(l+1)) with rank r + 2^l when that rank exists; the partner
 * sends its partial and r combines local (+) incoming. After the last level
 * rank 0 holds the reduction; it applies AVG and rounds to the storage type,
 * and the levels are walked back down, each parent sending the result to its
 * child. sent[r] (may be NULL) counts storage-type bytes per send. in and out
 * may be the same buffers.
 */
int orc_tree_all_reduce(int n, uint64_t count, int dtype, int op, const void* const* in, void* const* out,
                        uint64_t* sent)
{
    if (!valid(n, dtype, op) || !in || !out)
        return ORC_EINVAL;
    size_t e = elem_size(dtype);
    size_t bytes = (size_t)count * e;
    if (sent) for (int r = 0; r < n; r++) sent[r] = 0;
    if (count == 0)
        return ORC_OK;
    acc_t** W = widen_ranks(n, count, dtype, in);
    if (!W) return ORC_ENOMEM;
    int top = 1; /* 2^levels >= n */
    while (top < n) top *= 2;
    for (int stride = 1; stride < n; stride *= 2) {
        for (int r = 0; r + stride < n; r += 2 * stride) {
            int q = r + stride;
            for (uint64_t i = 0; i < count; i++) W[r][i] = combine(dtype, op, W[r][i], W[q][i]);
            if (sent) sent[q] += bytes;
        }
    }
    for (uint64_t i = 0; i < count; i++) narrow(dtype, finalize(dtype, op, n, W[0][i]), out[0], i);
    free_ranks(n, W);
    for (int stride = top / 2; stride >= 1; stride /= 2) {
        for (int r = 0; r + stride < n; r += 2 * stride) {
            memcpy(out[r + stride], out[r], bytes);
            if (sent) sent[r] += bytes;
        }
    }
    return ORC_OK;
}

/*
 * All-to-all: in[r] holds n blocks of blockcount elements; block p of rank r
 * is sent to rank p, which stores it as block r of out[p]. Rank r's own
 * block is a local copy and is not counted in sent[r]. in and out must not
 * overlap.
 */
int orc_all_to_all(int n, uint64_t blockcount, int dtype, const void* const* in, void* const* out, uint64_t* sent)
{
    if (!valid(n, dtype, ORC_SUM) || !in || !out)
        return ORC_EINVAL;
    size_t blk = (size_t)blockcount * elem_size(dtype);
    for (int r = 0; r < n; r++) {
        if (sent) sent[r] = 0;
        for (int p = 0; p < n; p++) {
            memcpy((unsigned char*)out[p] + (size_t)r * blk, (const unsigned char*)in[r] + (size_t)p * blk, blk);
            if (sent && p != r) sent[r] += blk;
        }
    }
    return ORC_OK;
}

/* Chunk c's element range [lo, hi) for n ranks over count elements. */
int orc_chunk_bounds(int n, uint64_t count, int c, uint64_t* lo, uint64_t* hi)
{
    if (n < 1 || c < 0 || c >= n || !lo || !hi)
        return ORC_EINVAL;
    bounds(n, count, c, lo, hi);
    return ORC_OK;
}

/* Array conversions, exposed so tests can pin them to library routines. */
void orc_f32_to_f16(const float* x, uint16_t* y, uint64_t m) { for (uint64_t i = 0; i < m; i++) y[i] = float_to_half(x[i]); }
void orc_f16_to_f32(const uint16_t* x, float* y, uint64_t m) { for (uint64_t i = 0; i < m; i++) y[i] = half_to_float(x[i]); }
void orc_f32_to_bf16(const float* x, uint16_t* y, uint64_t m) { for (uint64_t i = 0; i < m; i++) y[i] = float_to_bf16(x[i]); }
void orc_bf16_to_f32(const uint16_t* x, float* y, uint64_t m) { for (uint64_t i = 0; i < m; i++) y[i] = bf16_to_float(x[i]); }
