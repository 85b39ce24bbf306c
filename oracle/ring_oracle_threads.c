/*
 * ring_oracle_threads.c -- the oracle's ring all-reduce and per-element fold
 * on T host threads, for timing the CPU baseline beside the GPU.
 *
 * TEST INFRASTRUCTURE ONLY (as ring_oracle.c, whose element formats, reduce
 * ops, AVG finalize and partition it includes and reuses). The serial
 * functions of ring_oracle.c remain the checker; a CPU test requires these
 * threaded forms to give the same bits and the same byte counts.
 *
 * What runs concurrently [handbook "集合通信原语", section 环形 all-reduce 与通信量:
 * every rank takes each ring step at the same time, each sending one chunk
 * to its right neighbour and receiving one from its left]: each half-step
 * (every rank sends; every rank combines or copies what it received) is cut
 * into work items (rank r, piece j of the chunk rank r handles in that step),
 * spread over the threads, with a barrier after each half-step. Within a
 * half-step the items touch disjoint elements, so the result does not depend
 * on T. A send is one message: its bytes are counted once, by piece 0.
 *
 * The per-element fold splits [0, count) into T contiguous ranges.
 *
 * Build: gcc ... -pthread ring_oracle_threads.c (this file includes
 * ring_oracle.c, so the library holds both the serial and the threaded
 * entry points).
 */
#include <pthread.h>

#include "ring_oracle.c"

#define ORC_MAX_THREADS 256

/* Piece j of J of the range [lo, hi): [plo, phi). */
static void piece(uint64_t lo, uint64_t hi, int j, int J, uint64_t* plo, uint64_t* phi)
{
    uint64_t len = hi - lo;
    *plo = lo + len * (uint64_t)j / (uint64_t)J;
    *phi = lo + len * (uint64_t)(j + 1) / (uint64_t)J;
}

typedef struct {
    int n, dtype, op, J, T;
    uint64_t count;
    size_t e;
    void* const* bufs;
    acc_t** W;          /* per-rank fp32/uint32 working copies */
    acc_t** msg_acc;    /* per-rank receive buffers (reduce-scatter) */
    unsigned char** msg_raw; /* per-rank receive buffers (all-gather) */
    uint64_t* sent;
    pthread_barrier_t bar;
} ring_job;

typedef struct {
    ring_job* job;
    int t;
} ring_worker;

static void* ring_worker_main(void* arg)
{
    ring_worker* w = (ring_worker*)arg;
    ring_job* jb = w->job;
    const int n = jb->n, J = jb->J, T = jb->T;
    const int items = n * J;
    const uint64_t count = jb->count;
    const size_t e = jb->e;

    /* widen every rank's input into its working copy */
    for (int it = w->t; it < items; it += T) {
        int r = it / J, j = it % J;
        uint64_t lo, hi;
        piece(0, count, j, J, &lo, &hi);
        for (uint64_t i = lo; i < hi; i++) jb->W[r][i] = widen(jb->dtype, jb->bufs[r], i);
    }
    pthread_barrier_wait(&jb->bar);

    /* reduce-scatter: at step s rank r sends chunk r-s and folds the chunk
     * r-s-1 it receives from its left neighbour into its own copy */
    for (int s = 0; s < n - 1; s++) {
        for (int it = w->t; it < items; it += T) {
            int r = it / J, j = it % J;
            uint64_t lo, hi, plo, phi;
            bounds(n, count, mod(r - s, n), &lo, &hi);
            piece(lo, hi, j, J, &plo, &phi);
            acc_t* dst = jb->msg_acc[(r + 1) % n];
            for (uint64_t i = plo; i < phi; i++) dst[i - lo] = jb->W[r][i];
            if (j == 0) jb->sent[r] += (hi - lo) * e;
        }
        pthread_barrier_wait(&jb->bar);
        for (int it = w->t; it < items; it += T) {
            int r = it / J, j = it % J;
            uint64_t lo, hi, plo, phi;
            bounds(n, count, mod(r - 1 - s, n), &lo, &hi);
            piece(lo, hi, j, J, &plo, &phi);
            const acc_t* src = jb->msg_acc[r];
            for (uint64_t i = plo; i < phi; i++) jb->W[r][i] = combine(jb->dtype, jb->op, jb->W[r][i], src[i - lo]);
        }
        pthread_barrier_wait(&jb->bar);
    }

    /* the holder of chunk r+1 (rank r) applies AVG and rounds it into its buffer */
    for (int it = w->t; it < items; it += T) {
        int r = it / J, j = it % J;
        uint64_t lo, hi, plo, phi;
        bounds(n, count, (r + 1) % n, &lo, &hi);
        piece(lo, hi, j, J, &plo, &phi);
        for (uint64_t i = plo; i < phi; i++)
            narrow(jb->dtype, finalize(jb->dtype, jb->op, n, jb->W[r][i]), jb->bufs[r], i);
    }
    pthread_barrier_wait(&jb->bar);

    /* all-gather: at step s rank r forwards chunk r+1-s and stores the chunk
     * r-s it receives */
    for (int s = 0; s < n - 1; s++) {
        for (int it = w->t; it < items; it += T) {
            int r = it / J, j = it % J;
            uint64_t lo, hi, plo, phi;
            bounds(n, count, mod(r + 1 - s, n), &lo, &hi);
            piece(lo, hi, j, J, &plo, &phi);
            memcpy(jb->msg_raw[(r + 1) % n] + (plo - lo) * e, (unsigned char*)jb->bufs[r] + plo * e,
                   (size_t)(phi - plo) * e);
            if (j == 0) jb->sent[r] += (hi - lo) * e;
        }
        pthread_barrier_wait(&jb->bar);
        for (int it = w->t; it < items; it += T) {
            int r = it / J, j = it % J;
            uint64_t lo, hi, plo, phi;
            bounds(n, count, mod(r - s, n), &lo, &hi);
            piece(lo, hi, j, J, &plo, &phi);
            memcpy((unsigned char*)jb->bufs[r] + plo * e, jb->msg_raw[r] + (plo - lo) * e, (size_t)(phi - plo) * e);
        }
        pthread_barrier_wait(&jb->bar);
    }
    return NULL;
}

/* Workers wait at a start gate until every thread exists, so a failed
 * pthread_create can still release the ones already started (they return
 * without touching the job's barrier). */
typedef struct {
    pthread_mutex_t mu;
    pthread_cond_t cv;
    int state; /* 0: wait, 1: run, -1: abandon */
} start_gate;

typedef struct {
    start_gate* gate;
    void* (*fn)(void*);
    void* arg;
} gated_call;

static void* gated_main(void* p)
{
    gated_call* g = (gated_call*)p;
    pthread_mutex_lock(&g->gate->mu);
    while (g->gate->state == 0) pthread_cond_wait(&g->gate->cv, &g->gate->mu);
    int run = g->gate->state > 0;
    pthread_mutex_unlock(&g->gate->mu);
    if (run) g->fn(g->arg);
    return NULL;
}

static void open_gate(start_gate* gate, int state)
{
    pthread_mutex_lock(&gate->mu);
    gate->state = state;
    pthread_cond_broadcast(&gate->cv);
    pthread_mutex_unlock(&gate->mu);
}

/* Runs fn on T workers (workers[t] at t * worker_size bytes); the caller
 * is worker 0. */
static int run_threads(int T, void* (*fn)(void*), void* workers, size_t worker_size)
{
    pthread_t tid[ORC_MAX_THREADS];
    gated_call calls[ORC_MAX_THREADS];
    start_gate gate;
    pthread_mutex_init(&gate.mu, NULL);
    pthread_cond_init(&gate.cv, NULL);
    gate.state = 0;
    int started = 0;
    for (int t = 1; t < T; t++) {
        calls[t].gate = &gate;
        calls[t].fn = fn;
        calls[t].arg = (char*)workers + (size_t)t * worker_size;
        if (pthread_create(&tid[t], NULL, gated_main, &calls[t]) != 0)
            break;
        started = t;
    }
    int ok = started == T - 1;
    open_gate(&gate, ok ? 1 : -1);
    if (ok)
        fn(workers);
    for (int t = 1; t <= started; t++) pthread_join(tid[t], NULL);
    pthread_cond_destroy(&gate.cv);
    pthread_mutex_destroy(&gate.mu);
    return ok ? ORC_OK : ORC_ENOMEM;
}

/*
 * orc_ring_all_reduce with T threads: same arguments, same bytes out and the
 * same sent[] counts. T in 1..ORC_MAX_THREADS.
 */
int orc_ring_all_reduce_threads(int n, uint64_t count, int dtype, int op, void* const* bufs, uint64_t* sent,
                                int nthreads)
{
    if (!valid(n, dtype, op) || !bufs || !sent || nthreads < 1 || nthreads > ORC_MAX_THREADS)
        return ORC_EINVAL;
    for (int r = 0; r < n; r++) {
        sent[r] = 0;
        if (!bufs[r] && count) return ORC_EINVAL;
    }
    if (count == 0)
        return ORC_OK;
    ring_job jb;
    memset(&jb, 0, sizeof jb);
    jb.n = n;
    jb.dtype = dtype;
    jb.op = op;
    jb.T = nthreads;
    /* at least two items per thread per half-step */
    jb.J = (2 * nthreads + n - 1) / n;
    jb.count = count;
    jb.e = elem_size(dtype);
    jb.bufs = bufs;
    jb.sent = sent;
    uint64_t q = chunk_len(n, count);
    int rc = ORC_ENOMEM;
    jb.W = (acc_t**)calloc((size_t)n, sizeof(acc_t*));
    jb.msg_acc = (acc_t**)calloc((size_t)n, sizeof(acc_t*));
    jb.msg_raw = (unsigned char**)calloc((size_t)n, sizeof(unsigned char*));
    ring_worker* workers = (ring_worker*)calloc((size_t)nthreads, sizeof(ring_worker));
    if (!jb.W || !jb.msg_acc || !jb.msg_raw || !workers)
        goto out;
    for (int r = 0; r < n; r++) {
        jb.W[r] = (acc_t*)malloc((size_t)count * sizeof(acc_t));
        jb.msg_acc[r] = (acc_t*)malloc((size_t)q * sizeof(acc_t));
        jb.msg_raw[r] = (unsigned char*)malloc((size_t)q * jb.e);
        if (!jb.W[r] || !jb.msg_acc[r] || !jb.msg_raw[r])
            goto out;
    }
    if (pthread_barrier_init(&jb.bar, NULL, (unsigned)nthreads) != 0)
        goto out;
    for (int t = 0; t < nthreads; t++) {
        workers[t].job = &jb;
        workers[t].t = t;
    }
    rc = run_threads(nthreads, ring_worker_main, workers, sizeof(ring_worker));
    pthread_barrier_destroy(&jb.bar);
out:
    for (int r = 0; r < n; r++) {
        if (jb.W) free(jb.W[r]);
        if (jb.msg_acc) free(jb.msg_acc[r]);
        if (jb.msg_raw) free(jb.msg_raw[r]);
    }
    free(jb.W);
    free(jb.msg_acc);
    free(jb.msg_raw);
    free(workers);
    return rc;
}

typedef struct {
    int n, dtype, op, T, t;
    uint64_t count;
    const void* const* in;
    void* const* out;
} fold_worker;

static void* fold_worker_main(void* arg)
{
    fold_worker* w = (fold_worker*)arg;
    const int n = w->n;
    uint64_t q = chunk_len(n, w->count), lo, hi;
    piece(0, w->count, w->t, w->T, &lo, &hi);
    for (uint64_t i = lo; i < hi; i++) {
        int c = (int)(i / q); /* element i belongs to chunk c; its fold starts at rank c */
        acc_t acc = widen(w->dtype, w->in[c], i);
        for (int k = 1; k < n; k++) acc = combine(w->dtype, w->op, widen(w->dtype, w->in[(c + k) % n], i), acc);
        acc = finalize(w->dtype, w->op, n, acc);
        for (int r = 0; r < n; r++) narrow(w->dtype, acc, w->out[r], i);
    }
    return NULL;
}

/*
 * orc_fold_all_reduce with T threads over contiguous element ranges. in and
 * out may be the same buffers (each element's inputs are read before its
 * outputs are written, and the ranges are disjoint).
 */
int orc_fold_all_reduce_threads(int n, uint64_t count, int dtype, int op, const void* const* in, void* const* out,
                                int nthreads)
{
    if (!valid(n, dtype, op) || !in || !out || nthreads < 1 || nthreads > ORC_MAX_THREADS)
        return ORC_EINVAL;
    if (count == 0)
        return ORC_OK;
    fold_worker* workers = (fold_worker*)calloc((size_t)nthreads, sizeof(fold_worker));
    if (!workers)
        return ORC_ENOMEM;
    for (int t = 0; t < nthreads; t++) {
        fold_worker* w = &workers[t];
        w->n = n;
        w->dtype = dtype;
        w->op = op;
        w->T = nthreads;
        w->t = t;
        w->count = count;
        w->in = in;
        w->out = out;
    }
    int rc = run_threads(nthreads, fold_worker_main, workers, sizeof(fold_worker));
    free(workers);
    return rc;
}
