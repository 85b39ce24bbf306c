/*
 * allreduce.h -- C ABI of liballreduce, a ring all-reduce engine for one
 * AMD Instinct MI355X (gfx950) on which N "virtual ranks" are N separate
 * device buffers.
 *
 * Sources (web pages, cited by title and section):
 *  [P1] mhpq.cn news/451051, article on how all-reduce keeps every card's
 *       model identical: s2.1 (all-reduce semantics; SUM, AVG = sum then
 *       divide by N, MAX, MIN, PROD), s2.2 (every rank takes part with
 *       matching shapes; deterministic result), s3.2 (ring = reduce-scatter
 *       then all-gather), s5.3 (reduce fp16/bf16 gradients in fp32).
 *  [P2] xxqk.cn news/376101, article on AllReduce bottlenecks: s4.3 (do not
 *       mix dtypes inside one reduction).
 *  [P3] geek-doc.cn, "训练梯度同步与集合通信:从参数服务器到 Ring AllReduce":
 *       section 三 (the two ring phases of N-1 steps each), section 四
 *       (2(N-1)/N * M bytes per rank; alpha-beta model), section 六
 *       (reduce-scatter and all-gather used on their own, as in ZeRO/FSDP).
 *  [P4] anrans.github.io handbook, "集合通信原语": section 五个原语
 *       (all_reduce, reduce_scatter_tensor gives rank r block r,
 *       all_gather_into_tensor concatenates in rank order), section
 *       环形 all-reduce 与通信量 (the ring's index schedule), section α-β 模型
 *       (one-shot direct-read all-reduce for small messages).
 *
 * The pages' interface is one call per process and rank. Here one call
 * carries every rank's buffer: sendbufs[r] / recvbufs[r] are rank r's
 * device buffers, r = 0..nranks-1, so no rank can miss the call.
 *
 * Conventions for every entry point:
 *  - Pointers in sendbufs[] / recvbufs[] are device pointers on the comm's
 *    device; the arrays themselves are host memory, read only during the
 *    call. The caller owns all device memory, the workspace and the stream,
 *    and keeps them alive until the enqueued work has completed.
 *  - Calls are stream-ordered and asynchronous: they return once the work is
 *    enqueued on `stream` (NULL = the device's null stream).
 *  - Errors are returned, never raised: no call aborts or exits. A failing
 *    call enqueues nothing, except AR_ERR_HIP, which reports a launch error
 *    after earlier steps may have been enqueued. ar_last_error() gives a
 *    thread-local message for the last failure.
 *  - count == 0 (or recvcount/sendcount == 0) is a successful no-op.
 *  - Results are deterministic: the same inputs give the same bits on every
 *    call, and the ring modes (fused, stepwise, graph) give the same bits.
 *  - A comm holds mutable state (workspace, timing events, graph cache): calls
 *    on one comm must not run concurrently from several host threads. Calls
 *    on different comms may.
 */
#ifndef LIBALLREDUCE_ALLREDUCE_H
#define LIBALLREDUCE_ALLREDUCE_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AR_MAX_RANKS 64
#define AR_MAX_TENSORS 65536
/* Bytes of the library-owned device scratch array that ar_all_reduce_noalloc
 * uses on each GPU (64 MiB). */
#define AR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

typedef struct ar_comm* ar_comm_t;

typedef enum {
    AR_SUCCESS = 0,
    AR_ERR_INVALID_ARGUMENT = 1, /* bad pointer, enum, size, alias or workspace */
    AR_ERR_UNSUPPORTED = 2,      /* a valid request the library does not serve */
    AR_ERR_HIP = 3,              /* a HIP runtime call or kernel launch failed */
    AR_ERR_OUT_OF_MEMORY = 4,    /* host allocation for the comm failed */
    AR_ERR_INTERNAL = 5
} ar_result_t;

/* Storage types. fp16 and bf16 are reduced in fp32 and rounded once, to
 * nearest even, at the end [P1 s5.3]; int32 wraps modulo 2^32. One dtype
 * per call [P2 s4.3]. */
typedef enum { AR_FLOAT32 = 0, AR_FLOAT16 = 1, AR_BFLOAT16 = 2, AR_INT32 = 3 } ar_dtype_t;

/* Reduce ops [P1 s2.1]. AVG is the sum divided once by nranks (fp: one
 * correctly rounded fp32 divide; int32: truncation toward zero). MAX/MIN
 * return NaN when either operand is NaN and order +0 above -0. */
typedef enum { AR_SUM = 0, AR_AVG = 1, AR_MAX = 2, AR_MIN = 3, AR_PROD = 4 } ar_op_t;

/* AR_MODE_FUSED: one launch that reads every rank's element once and writes
 * the result to every output -- the direct-read ("one-shot") pattern [P4
 * section α-β 模型] -- folding the ranks in ring order, so its bits equal the
 * ring's.
 * AR_MODE_RING_STEPWISE: the ring itself, one launch per ring step:
 * N-1 reduce-scatter steps then N-1 all-gather steps [P3 section 三;
 * P4 section 环形 all-reduce 与通信量].
 * AR_MODE_RING_GRAPH: the same ring steps, captured once into a HIP graph
 * per call signature (collective, buffer pointers, count, dtype, op,
 * workspace) and replayed as one graph launch afterwards, which removes the
 * per-step launch cost that the alpha term of the alpha-beta model charges
 * [P3 section 四; P4 section α-β 模型: graph-captured custom all-reduce].
 * A comm keeps up to 16 graphs (least recently used evicted). The pointers
 * in a cached graph are fixed: a later call with the same pointers and sizes
 * replays it whatever the buffers now hold. Must not be used while `stream`
 * is itself being captured (INVALID_ARGUMENT): capture AR_MODE_RING_STEPWISE
 * or AR_MODE_FUSED instead -- both are capture-safe (no synchronous calls,
 * no memsets, no allocation). Same bits as the other modes. */
/* AR_MODE_TREE and AR_MODE_TREE_STEPWISE (all-reduce only; other
 * collectives return UNSUPPORTED): the tree variant [P3 section 六]. Ranks
 * combine in pairs, the pair results combine in pairs again, and after
 * ceil(log2 N) levels rank 0 holds the reduction, which is broadcast back
 * down: level l pairs rank r (a multiple of 2^(l+1)) with r + 2^l. Every
 * element is folded in that order (no chunks), so for fp SUM/AVG/PROD the
 * bits differ from the ring's; the difference is bounded by
 * 4*N*eps*sum|x_i| (eps = 2^-23, plus one output ulp for fp16/bf16).
 * AR_MODE_TREE: one launch, each element's tree evaluated in registers.
 * AR_MODE_TREE_STEPWISE: 2*ceil(log2 N) launches (the pages' step count);
 * fp16/bf16 partials need ar_workspace_bytes(...) of fp32 workspace. */
typedef enum {
    AR_MODE_FUSED = 0,
    AR_MODE_RING_STEPWISE = 1,
    AR_MODE_RING_GRAPH = 2,
    AR_MODE_TREE = 3,
    AR_MODE_TREE_STEPWISE = 4
} ar_mode_t;

/* Access flavour of the one-launch calls; see ar_comm_set_access. */
typedef enum {
    AR_ACCESS_AUTO = 0,
    AR_ACCESS_STREAMING = 1,
    AR_ACCESS_CACHED = 2
} ar_access_t;

typedef enum {
    AR_COLL_ALL_REDUCE = 0,
    AR_COLL_REDUCE_SCATTER = 1,
    AR_COLL_ALL_GATHER = 2,
    AR_COLL_ALL_TO_ALL = 3
} ar_collective_t;

/* Create a communicator for `nranks` (1..AR_MAX_RANKS) virtual ranks on HIP
 * device `hip_device`. On success *comm owns host state and a few HIP
 * events; release it with ar_comm_destroy. Errors: INVALID_ARGUMENT for a
 * NULL comm pointer or nranks out of range, HIP if the device cannot be
 * queried, OUT_OF_MEMORY. */
ar_result_t ar_comm_create(ar_comm_t* comm, int nranks, int hip_device);

/* Destroy a communicator (NULL is a no-op). Work already enqueued that uses
 * it must have completed. */
ar_result_t ar_comm_destroy(ar_comm_t comm);

/* Number of ranks the communicator was created with, or -1 for NULL. */
int ar_comm_nranks(ar_comm_t comm);

/* Device workspace (bytes) a call needs; 0 when none. `count` is the
 * collective's own count argument (count, recvcount or sendcount).
 * The ring modes (stepwise and graph) need it: all-reduce of fp16/bf16
 * keeps fp32 partial sums, 4*count bytes; reduce-scatter keeps the partials
 * of all nranks blocks, 4*nranks*recvcount bytes. AR_MODE_TREE_STEPWISE
 * with fp16/bf16 keeps floor(N/2) fp32 partial buffers:
 * 4*floor(N/2)*roundup(count, 4) bytes. Everything else: 0. Returns (size_t)-1 for
 * invalid arguments or if the size overflows. */
size_t ar_workspace_bytes(ar_collective_t coll, int nranks, size_t count, ar_dtype_t dtype, ar_mode_t mode);

/* Attach a caller-owned device workspace (16-byte aligned, `bytes` long) to
 * the communicator; NULL/0 detaches it. The library never allocates device
 * memory itself. Calls that share a workspace must be ordered on one
 * stream. Errors: INVALID_ARGUMENT for a NULL comm, a misaligned pointer,
 * or bytes > 0 with a NULL pointer. */
ar_result_t ar_comm_set_workspace(ar_comm_t comm, void* dev_ptr, size_t bytes);

/* All-reduce [P1 s2.1; P3 section 三; P4 section 五个原语]: after the call
 * recvbufs[r][i] = op over ranks of sendbufs[r][i], i < count, identical for
 * every r. Chunk c of the ring is elements [c*q, min((c+1)*q, count)) with
 * q = ceil(count/nranks), and chunk c is folded in rank order
 * c, c+1, ..., c+nranks-1 (mod nranks): acc = x_c; acc = x_{c+k} (+) acc.
 * sendbufs[r] and recvbufs[r] each hold `count` elements of `dtype`.
 * In place is allowed (sendbufs[r] == recvbufs[r]); any other overlap
 * between any two of the 2*nranks buffers (or the workspace) is
 * INVALID_ARGUMENT. Ring-mode fp16/bf16 needs a workspace of
 * ar_workspace_bytes(...) bytes, else INVALID_ARGUMENT. Pointers must be
 * aligned to the element size (else INVALID_ARGUMENT). With every pointer
 * 16-byte aligned the fused kernel moves 16-byte vectors (chunk ends that
 * fall inside a vector are done element by element); the stepwise steps
 * also need q to be a multiple of 16/sizeof(dtype). Other layouts take
 * element-wise kernels. The results are the same bits either way. */
ar_result_t ar_all_reduce(ar_comm_t comm, const void* const sendbufs[], void* const recvbufs[], size_t count,
                          ar_dtype_t dtype, ar_op_t op, ar_mode_t mode, hipStream_t stream);

/* Allocation-free all-reduce, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments, results (bit for bit) and errors as
 * ar_all_reduce, with these differences:
 *  - the fp32 partial sums of the ring-stepwise and tree-stepwise fp16/bf16
 *    paths live in a library-owned device array of AR_NOALLOC_SCRATCH_BYTES
 *    on each GPU (set up by ar_comm_create, held until the process ends);
 *    the comm's workspace is not used. A call that would need more, i.e.
 *    ar_workspace_bytes(AR_COLL_ALL_REDUCE, ...) > AR_NOALLOC_SCRATCH_BYTES
 *    (ring-stepwise fp16/bf16 beyond 16,777,216 elements per rank), is
 *    INVALID_ARGUMENT;
 *  - AR_MODE_RING_GRAPH is UNSUPPORTED (instantiating a graph allocates);
 *  - step timing (ar_comm_set_step_timing) records nothing for this call.
 * The call allocates nothing: no hipMalloc, hipFree, event or graph. The
 * caller still owns the send and recv buffers and the stream.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (nothing in it needs to start at zero: each step writes a slot
 * before any later step reads it). Calls on one GPU that may overlap in time
 * (unordered streams, several host threads) race on the array: the caller
 * must order them. INVALID_ARGUMENT also if ar_comm_create could not look
 * up the array's address on the comm's device (ar_last_error says why). */
ar_result_t ar_all_reduce_noalloc(ar_comm_t comm, const void* const sendbufs[], void* const recvbufs[], size_t count,
                                  ar_dtype_t dtype, ar_op_t op, ar_mode_t mode, hipStream_t stream);

/* Reduce-scatter [P3 section 六; P4 section 五个原语]: sendbufs[r] holds
 * nranks*recvcount elements; recvbufs[c] (recvcount elements) receives
 * block c of the reduction, block c being folded in the same ring order as
 * in ar_all_reduce, so reduce-scatter followed by all-gather equals
 * all-reduce bit for bit. In place: recvbufs[r] == sendbufs[r] +
 * r*recvcount elements. The ring modes need a workspace of
 * ar_workspace_bytes(...) bytes. Errors as ar_all_reduce. */
ar_result_t ar_reduce_scatter(ar_comm_t comm, const void* const sendbufs[], void* const recvbufs[],
                              size_t recvcount, ar_dtype_t dtype, ar_op_t op, ar_mode_t mode, hipStream_t stream);

/* All-gather [P3 section 六; P4 section 五个原语]: sendbufs[r] holds
 * sendcount elements; every recvbufs[r] (nranks*sendcount elements)
 * receives the nranks send blocks in rank order. In place:
 * sendbufs[r] == recvbufs[r] + r*sendcount elements. Errors as
 * ar_all_reduce (no workspace is needed). */
ar_result_t ar_all_gather(ar_comm_t comm, const void* const sendbufs[], void* const recvbufs[], size_t sendcount,
                          ar_dtype_t dtype, ar_mode_t mode, hipStream_t stream);

/* All-to-all, the "transpose" primitive [P4 section 五个原语 (all_to_all_single:
 * rank r's p-th block goes to rank p); P3 section 六]: sendbufs[r] holds
 * nranks blocks of blockcount elements; block r of recvbufs[p] receives
 * block p of sendbufs[r], for every r and p. Each rank sends (n-1)/n of its
 * data. AR_MODE_FUSED moves every block in one launch; the ring modes take n
 * steps, step s moving block (r + s) mod n of every rank r (step 0 is each
 * rank's own block). No workspace. Send and recv buffers must not overlap at
 * all (there is no in-place form); errors otherwise as ar_all_reduce. */
ar_result_t ar_all_to_all(ar_comm_t comm, const void* const sendbufs[], void* const recvbufs[], size_t blockcount,
                          ar_dtype_t dtype, ar_mode_t mode, hipStream_t stream);

/* Coalesced multi-tensor all-reduce: many gradient tensors reduced in one
 * call without packing them into a bucket first -- the pages' gradient
 * bucketing and small-tensor fusion [P1 s5.1-s5.2 (DDP buckets, default
 * 25 MB); P2 s5.3 (merge same-shape gradients into one call); P3 section 四
 * (fuse small tensors so the per-step latency is paid once)].
 * Tensor t of rank r is sendbufs[t*nranks + r] / recvbufs[t*nranks + r]
 * with counts[t] elements (t < ntensors <= AR_MAX_TENSORS; empty tensors
 * allowed). The tensors of a rank form one virtual flat bucket, in tensor
 * order; the ring's chunks are taken over that bucket, so every element gets
 * exactly the bits ar_all_reduce gives on the packed bucket. Each tensor may
 * be in place (send == recv); any other overlap is INVALID_ARGUMENT.
 * AR_MODE_FUSED only (other modes: UNSUPPORTED). Launches: one per batch of
 * tensors whose rank pointers fit the kernel arguments (about 3.8 KB; a
 * tensor in place on every rank takes n pointers, otherwise 2n: e.g. about
 * 40 in-place tensors per launch at 8 ranks, 6 at 64). Tensors whose rank
 * pointers all sit at the same offset from a 16-byte boundary are read and
 * written in 16-byte vectors; others element by element. When the pointers
 * also share their offset from a 128-byte line (views at one offset into
 * per-rank buckets), the vectors start on the tensor's first whole line,
 * which keeps every wave's access to whole lines. No workspace. */
ar_result_t ar_all_reduce_multi(ar_comm_t comm, int ntensors, const void* const sendbufs[], void* const recvbufs[],
                                const size_t counts[], ar_dtype_t dtype, ar_op_t op, ar_mode_t mode,
                                hipStream_t stream);

/* Per-step timing of stepwise calls (the alpha-beta model's per-step cost,
 * [P3 section 四; P4 section α-β 模型]). When enabled, each stepwise call
 * records a HIP event before its first step and after every step; fused
 * and graph-mode calls record one interval. Recording adds a little
 * per-step overhead and is not meant for the caller's own graph capture. */
ar_result_t ar_comm_set_step_timing(ar_comm_t comm, int enable);

/* Access flavour of the one-launch calls (fused and tree all-reduce, fused
 * reduce-scatter, all-gather and all-to-all, multi-tensor all-reduce): with
 * non-temporal ("streaming") loads and stores, which pass data through the
 * caches without keeping it, or with ordinary cached ones, which let a call
 * on buffers still in the 256 MB last-level cache run from it.
 *  AR_ACCESS_AUTO (the default): non-temporal when the call's distinct bytes
 *    exceed half the last-level cache for the all-reduce (a footprint that
 *    large is unlikely to be resident in full, and cold calls gain more than
 *    warm ones lose: 8 ranks x 25 MiB fp32, 73 against 86 us cold, 71
 *    against 62 us warm) and the whole cache for the other collectives;
 *  AR_ACCESS_STREAMING: non-temporal at every size, for buffers known to
 *    come from HBM;
 *  AR_ACCESS_CACHED: cached whenever the footprint fits in the cache, for
 *    buffers a kernel has just written (e.g. a gradient bucket right after
 *    the backward pass).
 * Launch shapes follow the flavour chosen; results are the same bits either
 * way. The ring-stepwise and graph modes always use cached access except the
 * all-to-all steps beyond the cache. The setting is per comm and takes
 * effect from the next call. NULL comm or an unknown value:
 * INVALID_ARGUMENT. */
ar_result_t ar_comm_set_access(ar_comm_t comm, ar_access_t access);

/* ar_comm_set_access(comm, enable ? AR_ACCESS_STREAMING : AR_ACCESS_AUTO). */
ar_result_t ar_comm_set_streaming(ar_comm_t comm, int enable);

/* Step durations (ms) of the last timed call on this comm: waits for that
 * call's last event, writes min(cap, steps) values to out and the step
 * count to *nsteps. INVALID_ARGUMENT if timing was off or nothing was
 * timed yet. */
ar_result_t ar_last_step_times_ms(ar_comm_t comm, float* out, int cap, int* nsteps);

/* Static description of a result code. */
const char* ar_result_string(ar_result_t result);

/* Thread-local detail of the last failed call on this thread ("" if none). */
const char* ar_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBALLREDUCE_ALLREDUCE_H */
