// api.cpp -- the C ABI of liballreduce (include/allreduce.h): argument
// checks, the ring plan (chunk partition and step schedule), mode dispatch,
// per-step event timing and thread-local error text. Every check runs before
// the first HIP call, so a rejected call touches no device state.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <new>
#include <string>
#include <vector>

#include "allreduce.h"
#include "kernels.h"

#define AR_EXPORT extern "C" __attribute__((visibility("default")))

struct ar_comm {
    int nranks = 0;
    int device = 0;
    int num_cus = 256;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    bool debug = false;
    bool step_timing = false;
    ar_access_t access = AR_ACCESS_AUTO;  // access flavour of the one-launch calls (ar_comm_set_access)
    std::vector<hipEvent_t> events;  // step boundaries of the last timed call
    int last_steps = -1;
    // AR_MODE_RING_GRAPH: instantiated graphs keyed by call signature.
    struct GraphEntry {
        std::vector<uintptr_t> key;
        hipGraphExec_t exec;
        uint64_t last_use;
    };
    static constexpr size_t kMaxGraphs = 16;
    std::vector<GraphEntry> graphs;
    uint64_t use_clock = 0;
    hipStream_t capture_stream = nullptr;
    // ar_all_reduce_noalloc: this device's AR_NOALLOC_SCRATCH_BYTES array,
    // looked up at creation (or why the lookup failed).
    void* scratch = nullptr;
    std::string scratch_err;
};

namespace {

thread_local std::string g_last_error;

ar_result_t fail(ar_result_t code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

ar_result_t hip_fail(hipError_t e, const char* what)
{
    return fail(AR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t elem_size(ar_dtype_t d)
{
    switch (d) {
    case AR_FLOAT32: return 4;
    case AR_FLOAT16: return 2;
    case AR_BFLOAT16: return 2;
    case AR_INT32: return 4;
    }
    return 0;
}

bool valid_dtype(int d) { return d >= AR_FLOAT32 && d <= AR_INT32; }
bool valid_op(int o) { return o >= AR_SUM && o <= AR_PROD; }
bool valid_mode(int m) { return m >= AR_MODE_FUSED && m <= AR_MODE_TREE_STEPWISE; }
bool tree_mode(int m) { return m == AR_MODE_TREE || m == AR_MODE_TREE_STEPWISE; }

const char* dtype_name(ar_dtype_t d)
{
    static const char* names[] = {"fp32", "fp16", "bf16", "int32"};
    return valid_dtype(d) ? names[d] : "?";
}

// a * b without overflow, else false.
bool mul_ok(size_t a, size_t b, size_t* out)
{
    if (a != 0 && b > SIZE_MAX / a) return false;
    *out = a * b;
    return true;
}

uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Restores the caller's current device on scope exit.
struct DeviceGuard {
    int prev = -1;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int dev)
    {
        err = hipGetDevice(&prev);
        if (err == hipSuccess && prev != dev) err = hipSetDevice(dev);
        else if (err == hipSuccess) prev = -1;
    }
    ~DeviceGuard()
    {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

struct Interval {
    uintptr_t lo, hi;
    const char* what;
    int rank;
};

// Sorts `iv` by start. An interval overlaps an earlier one exactly when it
// starts before the largest end seen so far (empty intervals overlap
// nothing); on the first such pair returns true with *a the later interval
// and *b the earlier one.
bool find_overlap(std::vector<Interval>& iv, size_t* a, size_t* b)
{
    std::sort(iv.begin(), iv.end(), [](const Interval& x, const Interval& y) { return x.lo < y.lo; });
    size_t last = SIZE_MAX;  // the interval with the largest end so far
    for (size_t i = 0; i < iv.size(); ++i) {
        if (iv[i].hi == iv[i].lo) continue;
        if (last != SIZE_MAX && iv[i].lo < iv[last].hi) {
            *a = i;
            *b = last;
            return true;
        }
        if (last == SIZE_MAX || iv[i].hi > iv[last].hi) last = i;
    }
    return false;
}

// The 2n rank buffers (plus the workspace) must not overlap, except that a
// rank's send buffer may sit at `inplace_off` bytes into its recv buffer
// (all-reduce: 0; all-gather: r*sendbytes) or its recv buffer at
// `inplace_off` bytes into its send buffer (reduce-scatter: r*recvbytes).
ar_result_t check_buffers(int n, const void* const send[], void* const recv[], size_t send_bytes, size_t recv_bytes,
                          int coll, size_t elem, const void* ws, size_t ws_need)
{
    std::vector<Interval> iv;
    iv.reserve(2 * n + 1);
    for (int r = 0; r < n; ++r) {
        if (!send[r]) return fail(AR_ERR_INVALID_ARGUMENT, "sendbufs[%d] is NULL", r);
        if (!recv[r]) return fail(AR_ERR_INVALID_ARGUMENT, "recvbufs[%d] is NULL", r);
        if (reinterpret_cast<uintptr_t>(send[r]) % elem || reinterpret_cast<uintptr_t>(recv[r]) % elem)
            return fail(AR_ERR_INVALID_ARGUMENT, "rank %d buffer is not aligned to the %zu-byte element size", r, elem);
        const uintptr_t s = reinterpret_cast<uintptr_t>(send[r]);
        const uintptr_t d = reinterpret_cast<uintptr_t>(recv[r]);
        if (s > UINTPTR_MAX - send_bytes || d > UINTPTR_MAX - recv_bytes)
            return fail(AR_ERR_INVALID_ARGUMENT, "rank %d buffer wraps the address space", r);
        bool inplace = false;
        if (coll == AR_COLL_ALL_REDUCE) inplace = (s == d);
        else if (coll == AR_COLL_REDUCE_SCATTER) inplace = (d == s + static_cast<uintptr_t>(r) * recv_bytes);
        else if (coll == AR_COLL_ALL_GATHER) inplace = (s == d + static_cast<uintptr_t>(r) * send_bytes);
        if (inplace) {
            iv.push_back({std::min(s, d), std::max(s + send_bytes, d + recv_bytes), "in-place buffer", r});
        } else {
            iv.push_back({s, s + send_bytes, "sendbufs", r});
            iv.push_back({d, d + recv_bytes, "recvbufs", r});
        }
    }
    if (ws_need) iv.push_back({reinterpret_cast<uintptr_t>(ws), reinterpret_cast<uintptr_t>(ws) + ws_need, "workspace", -1});
    size_t a, b;
    if (find_overlap(iv, &a, &b))
        return fail(AR_ERR_INVALID_ARGUMENT, "%s[%d] overlaps %s[%d] (only the documented in-place layout may alias)",
                    iv[a].what, iv[a].rank, iv[b].what, iv[b].rank);
    return AR_SUCCESS;
}

// Workgroups per chunk row: enough to cover the chunk, capped so that the
// whole grid is `per_cu` workgroups per CU (grid-stride loops take the rest).
int grid_for(const ar_comm* comm, uint64_t units_per_row, int rows, int per_cu = 8)
{
    const uint64_t want = std::max<uint64_t>(1, ceil_div(units_per_row, ar::kBlock));
    const uint64_t cap = std::max<uint64_t>(1, static_cast<uint64_t>(comm->num_cus) * per_cu / std::max(1, rows));
    return static_cast<int>(std::min(want, cap));
}

// The last-level cache of MI355X (Infinity Cache): a fused call whose
// distinct bytes fit in it uses cached loads/stores, else non-temporal ones.
constexpr uint64_t kLastLevelCacheBytes = uint64_t(256) << 20;

bool use_nt(uint64_t footprint_bytes) { return footprint_bytes > kLastLevelCacheBytes; }

// Above this footprint the fused all-reduce streams by default. A footprint
// of more than half the cache is unlikely to be resident in full, and cold
// calls gain more from non-temporal access than warm ones lose: 8 ranks,
// fp32, cold (every call from HBM) / warm (repeated on one buffer set), in
// microseconds, cached two-tile against non-temporal rank-major kernels:
// 16 MiB per rank 59.4 / 41.0 against 48.7 / 48.1 (at the threshold, stays
// cached); 20 MiB 71.6 / 50.0 against 61.1 / 60.0; 25 MiB 87.0 / 62.1
// against 75.2 / 73.6. Streaming wins there unless the data is warm more
// than about half the time; at 16 ranks x 8 MiB it loses cold too (56.7
// against 60.6), which the threshold keeps cached.
constexpr uint64_t kAllReduceStreamBytes = kLastLevelCacheBytes / 2;

// The access flavour of a one-launch call (ar_comm_set_access): AUTO streams
// (non-temporal loads and stores) above `auto_bytes` of footprint
// (kAllReduceStreamBytes for the all-reduce, the whole cache for the other
// collectives), STREAMING always, CACHED above the whole cache only. The
// launch shapes follow the flavour chosen.
bool call_nt(const ar_comm* comm, uint64_t footprint_bytes, uint64_t auto_bytes)
{
    switch (comm->access) {
    case AR_ACCESS_STREAMING: return true;
    case AR_ACCESS_CACHED: return footprint_bytes > kLastLevelCacheBytes;
    default: return footprint_bytes > auto_bytes;
    }
}

// Distinct bytes of the rank buffers: in-place ranks count once.
uint64_t footprint(int n, const void* const send[], void* const recv[], uint64_t send_bytes, uint64_t recv_bytes)
{
    uint64_t f = 0;
    for (int r = 0; r < n; ++r) {
        const uintptr_t s = reinterpret_cast<uintptr_t>(send[r]), d = reinterpret_cast<uintptr_t>(recv[r]);
        const bool nested = (d >= s && d + recv_bytes <= s + send_bytes) || (s >= d && s + send_bytes <= d + recv_bytes);
        f += nested ? std::max(send_bytes, recv_bytes) : send_bytes + recv_bytes;
    }
    return f;
}

// The rank-major all-reduce kernel (16-byte vectors, non-temporal access)
// whenever the call streams, from 2 ranks. Measured against the kernels used
// before on the same buffers (fp32 unless noted): at 8 ranks +15% cold at
// 20-32 MiB per rank, +10% at 64 and 128 MiB, +5% at 256 MiB, +7.5% at
// 1 GiB, +3.6% at 4 GiB, +3% at 14 GB fp16 (with one super tile per
// workgroup, rank_major_grid); at 4 ranks +16% cold at 40 MiB and +6.6% at
// 256 MiB; at 2 ranks +3% at 128 MiB, +10% at 1 GiB; at 3 ranks +16% at
// 256 MiB; above 8 ranks see fused_rank_major_any.
bool use_rank_major(int nranks, bool vec, bool nt) { return vec && nt && nranks >= 2; }

// Tiles per super tile of the rank-major all-reduce: rank_major_any_tiles,
// or one for 16-bit types at up to 8 ranks from kOneTileBytes per rank.
int allreduce_tiles(int nranks, size_t elem, size_t bytes_per_rank)
{
    if (elem == 2 && nranks <= 8 && bytes_per_rank >= ar::kOneTileBytes) return 1;
    return ar::rank_major_any_tiles(nranks, static_cast<int>(elem));
}

// The same for the reduce-scatter layout: kScatterTiles for the
// fixed-rank-count body at 5..8 ranks, else rank_major_any_tiles.
int scatter_tiles(int nranks, size_t elem)
{
    return nranks >= 5 && nranks <= 8 ? ar::kScatterTiles : ar::rank_major_any_tiles(nranks, static_cast<int>(elem));
}

// Workgroups per chunk row for the rank-major all-reduce: one per super tile
// (`m` tiles of kBlock 16-byte vectors), so no workgroup
// strides through its row. The hardware dispatches workgroups in order, so
// the resident ones work through one chunk row after another, each on its
// own contiguous super tile. Against a grid-stride grid of 16 workgroups
// per CU on the same buffers: 8 x 256 MiB 0.755 / 0.793 ms, 8 x 1 GiB 3.00 /
// 3.22 ms, 8 x 4 GiB 12.64 / 13.10 ms, 8 x 7e9 fp16 36.9 / 38.0 ms (there
// against the two-tile kernel). The count is an upper bound on every row's
// super tiles (a chunk's first tile may start before it); extra workgroups
// find no super tile and exit. The kernels stride by the grid, so a row of
// more than kMaxGridX super tiles (chunks beyond 64 GiB) stays correct.
constexpr uint64_t kMaxGridX = (uint64_t(1) << 32) / ar::kBlock - 1;  // work-items per dimension fit 32 bits

int rank_major_grid(uint64_t q, size_t elem, int m)
{
    const uint64_t tiles = ceil_div(ceil_div(q, 16 / elem), static_cast<uint64_t>(ar::kBlock)) + 1;
    return static_cast<int>(std::clamp<uint64_t>(ceil_div(tiles, static_cast<uint64_t>(m)), 1, kMaxGridX));
}

// The same for the reduce-scatter layout, whose tiles count from the chunk
// start (block c of the output).
int rank_major_scatter_grid(uint64_t q, size_t elem, int m)
{
    const uint64_t tiles = ceil_div(ceil_div(q, 16 / elem), static_cast<uint64_t>(ar::kBlock));
    return static_cast<int>(std::clamp<uint64_t>(ceil_div(tiles, static_cast<uint64_t>(m)), 1, kMaxGridX));
}

// The ring's steps, tiled (kStepTiles vectors per thread and tile, one
// workgroup per tile) when a step has at least 8 such workgroups per CU, else
// one vector (or unit) per thread over 8 workgroups per CU. `vecs`: whole
// 16-byte vectors per chunk; `units`: the untiled kernel's work items per
// chunk. Tiled steps stream (non-temporal) when the call's footprint exceeds
// the last-level cache. Against the untiled steps on the same buffers (stepwise mode):
// fp32 8 x 256 MiB 1.744 -> 1.491 ms (non-temporal; 1.644 cached), 4 x
// 256 MiB 0.746 -> 0.647 ms, 2 x 512 MiB 0.532 -> 0.430 ms, 16 x 128 MiB
// 1.749 -> 1.643 ms, the graph mode 8 x 256 MiB 1.732 -> 1.499 ms;
// reduce-scatter 8 x 256 MiB in 1.035 -> 0.927 ms; all-gather 8 x 32 MiB in
// 0.771 -> 0.691 ms. The 16-bit steps, whose partials are fp32 in the
// workspace, tile by half vectors (rs_step_halves), so that a wave's partial
// loads cover whole lines and the partials stream as well: against
// whole-vector tiles with cached partials (streaming partials there cost
// 15-20%), fp16 8 x 256 MiB 2.117 -> 2.046 ms, 8 x 7e9 120.3 -> 116.4 ms
// (MAX; AVG 118.8 -> 115.9), the reduce-scatter 8 x 16.8M out 1.520 -> 1.446
// ms, 8 x 875M out 84.7 -> 81.7 ms; half vectors with cached partials 2.153,
// 120.2, 1.558, 83.1 ms.
struct StepShape {
    int tiles;  // 0 or ar::kStepTiles
    bool nt;
    int grid_x;
};
StepShape step_shape(const ar_comm* comm, bool vec, uint64_t vecs, uint64_t units, int nranks,
                     uint64_t footprint_bytes)
{
    const uint64_t tiles = ceil_div(vecs + 1, static_cast<uint64_t>(ar::kStepTiles) * ar::kBlock);
    if (!vec || tiles * static_cast<uint64_t>(nranks) < static_cast<uint64_t>(comm->num_cus) * 8)
        return {0, false, grid_for(comm, units, nranks)};
    return {ar::kStepTiles, use_nt(footprint_bytes), static_cast<int>(std::clamp<uint64_t>(tiles, 1, kMaxGridX))};
}

// Workgroups per row for the tiled copies (all-gather, all-to-all): one per
// tile of kRankMajorTiles x kBlock 16-byte vectors.
int copy_tile_grid(uint64_t vectors)
{
    const uint64_t m = static_cast<uint64_t>(ar::kRankMajorTiles) * ar::kBlock;
    return static_cast<int>(std::clamp<uint64_t>(ceil_div(vectors, m), 1, kMaxGridX));
}

// The multi-tensor call's rank-major tiles whenever the call streams, from 4
// ranks, as the flat all-reduce.
bool use_rank_major_multi(int nranks, bool nt) { return nt && nranks >= 4; }

// Workgroups per CU for the fused all-reduce, from sweeps of 2..16 per CU in
// one process on MI355X (fp32 SUM, 64 MiB..1 GiB per rank, N = 2..64; fp16
// at 14 GB per rank):
//  - N <= 4: 2 per CU beat 8 by 4-10 points once the data exceeds the
//    last-level cache; cache-resident calls are within 2 points of each other
//    and take 8;
//  - 5 <= N <= 32: up to 128 MiB per rank, 16 per CU (8 ranks x 25 MiB, a
//    DDP bucket, with cache rotation: 60.2% against 56.5% at 4); above, 4
//    per CU is best or within 1 point (8 x 14 GB fp16: 75.0% against 74.1%
//    at 8);
//  - N > 32: 16 per CU up to 128 MiB per rank, 12 above.
int fused_per_cu(size_t bytes_per_rank, int nranks, bool cached)
{
    const bool small = bytes_per_rank <= (size_t(128) << 20);
    if (nranks <= 4) return cached ? 8 : 2;
    if (nranks <= 32) return small ? 16 : 4;
    return small ? 16 : 12;
}

// Records the start of a call and the end of each step when timing is on.
struct StepTimer {
    ar_comm* comm;
    hipStream_t stream;
    int steps = 0;
    StepTimer(ar_comm* c, hipStream_t s) : comm(c), stream(s) {}
    hipError_t ensure(int nsteps)
    {
        while (static_cast<int>(comm->events.size()) < nsteps + 1) {
            hipEvent_t e;
            hipError_t err = hipEventCreate(&e);
            if (err != hipSuccess) return err;
            comm->events.push_back(e);
        }
        return hipSuccess;
    }
    hipError_t begin(int nsteps)
    {
        if (!comm->step_timing) return hipSuccess;
        comm->last_steps = -1;
        hipError_t err = ensure(nsteps);
        if (err != hipSuccess) return err;
        return hipEventRecord(comm->events[0], stream);
    }
    hipError_t step()
    {
        if (!comm->step_timing) return hipSuccess;
        ++steps;
        return hipEventRecord(comm->events[steps], stream);
    }
    void end()
    {
        if (comm->step_timing) comm->last_steps = steps;
    }
};

ar_result_t check_common(ar_comm_t comm, const void* const* send, void* const* recv, int dtype, int mode)
{
    if (!comm) return fail(AR_ERR_INVALID_ARGUMENT, "comm is NULL");
    if (!send) return fail(AR_ERR_INVALID_ARGUMENT, "sendbufs array is NULL");
    if (!recv) return fail(AR_ERR_INVALID_ARGUMENT, "recvbufs array is NULL");
    if (!valid_dtype(dtype)) return fail(AR_ERR_INVALID_ARGUMENT, "invalid dtype %d", dtype);
    if (!valid_mode(mode)) return fail(AR_ERR_INVALID_ARGUMENT, "invalid mode %d", mode);
    return AR_SUCCESS;
}

// The device memory a call keeps its partial sums in: the comm's attached
// workspace, or the library's scratch array for ar_all_reduce_noalloc.
struct Workspace {
    void* ptr;
    size_t bytes;
    bool scratch;
};

Workspace comm_workspace(const ar_comm* comm) { return {comm->ws, comm->ws ? comm->ws_bytes : 0, false}; }

ar_result_t need_workspace(const Workspace& ws, size_t need)
{
    if (need == 0) return AR_SUCCESS;
    if (ws.scratch && need > ws.bytes)
        return fail(AR_ERR_INVALID_ARGUMENT,
                    "this call needs %zu bytes of partial sums; the allocation-free call has %zu "
                    "(AR_NOALLOC_SCRATCH_BYTES)", need, ws.bytes);
    if (!ws.ptr || ws.bytes < need)
        return fail(AR_ERR_INVALID_ARGUMENT,
                    "this call needs a device workspace of %zu bytes (attached: %zu); see ar_workspace_bytes", need,
                    ws.bytes);
    return AR_SUCCESS;
}

template <class Args>
void fill_ptrs(Args& a, int n, const void* const send[], void* const recv[])
{
    for (int r = 0; r < n; ++r) {
        a.send[r] = send[r];
        a.recv[r] = recv[r];
    }
}

bool all_aligned16(int n, const void* const send[], void* const recv[])
{
    for (int r = 0; r < n; ++r)
        if (!aligned16(send[r]) || !aligned16(recv[r])) return false;
    return true;
}

}  // namespace

// ---------------------------------------------------------------------------
// communicator
// ---------------------------------------------------------------------------
AR_EXPORT ar_result_t ar_comm_create(ar_comm_t* comm, int nranks, int hip_device)
{
    if (!comm) return fail(AR_ERR_INVALID_ARGUMENT, "comm pointer is NULL");
    *comm = nullptr;
    if (nranks < 1 || nranks > AR_MAX_RANKS)
        return fail(AR_ERR_INVALID_ARGUMENT, "nranks %d is outside 1..%d", nranks, AR_MAX_RANKS);
    if (hip_device < 0) return fail(AR_ERR_INVALID_ARGUMENT, "hip_device %d is negative", hip_device);
    int ndev = 0;
    hipError_t e = hipGetDeviceCount(&ndev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
    if (hip_device >= ndev) return fail(AR_ERR_INVALID_ARGUMENT, "hip_device %d but %d devices", hip_device, ndev);
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, hip_device);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(multiprocessor count)");
    ar_comm* c = new (std::nothrow) ar_comm();
    if (!c) return fail(AR_ERR_OUT_OF_MEMORY, "cannot allocate the communicator");
    c->nranks = nranks;
    c->device = hip_device;
    c->num_cus = cus > 0 ? cus : 256;
    const char* dbg = std::getenv("AR_DEBUG");
    c->debug = dbg && *dbg && std::strcmp(dbg, "0") != 0;
    {
        // Set-up of ar_all_reduce_noalloc: this device's scratch array
        // address, looked up with the device current. A failure only
        // disables that entry point, which reports it.
        DeviceGuard g(hip_device);
        hipError_t se = g.err;
        if (se == hipSuccess) se = ar::scratch_address(hip_device, &c->scratch);
        if (se != hipSuccess) {
            c->scratch = nullptr;
            c->scratch_err = hipGetErrorString(se);
        }
    }
    *comm = c;
    return AR_SUCCESS;
}

AR_EXPORT ar_result_t ar_comm_destroy(ar_comm_t comm)
{
    if (!comm) return AR_SUCCESS;
    for (hipEvent_t e : comm->events) (void)hipEventDestroy(e);
    for (auto& g : comm->graphs) (void)hipGraphExecDestroy(g.exec);
    if (comm->capture_stream) (void)hipStreamDestroy(comm->capture_stream);
    delete comm;
    return AR_SUCCESS;
}

AR_EXPORT int ar_comm_nranks(ar_comm_t comm) { return comm ? comm->nranks : -1; }

AR_EXPORT size_t ar_workspace_bytes(ar_collective_t coll, int nranks, size_t count, ar_dtype_t dtype, ar_mode_t mode)
{
    if (nranks < 1 || nranks > AR_MAX_RANKS || !valid_dtype(dtype) || !valid_mode(mode)) return static_cast<size_t>(-1);
    if (coll < AR_COLL_ALL_REDUCE || coll > AR_COLL_ALL_TO_ALL) return static_cast<size_t>(-1);
    if (nranks == 1) return 0;
    const bool half = dtype == AR_FLOAT16 || dtype == AR_BFLOAT16;
    size_t out = 0;
    if (mode == AR_MODE_TREE_STEPWISE) {
        if (coll != AR_COLL_ALL_REDUCE || !half) return 0;
        if (count > SIZE_MAX - 3) return static_cast<size_t>(-1);
        size_t slots = 0;
        if (!mul_ok((count + 3) / 4 * 4, static_cast<size_t>(nranks / 2), &slots) || !mul_ok(slots, 4, &out))
            return static_cast<size_t>(-1);
        return out;
    }
    if (mode != AR_MODE_RING_STEPWISE && mode != AR_MODE_RING_GRAPH) return 0;
    if (coll == AR_COLL_ALL_REDUCE) {
        if (!half) return 0;
        return mul_ok(count, 4, &out) ? out : static_cast<size_t>(-1);
    }
    if (coll == AR_COLL_REDUCE_SCATTER) {
        size_t total = 0;
        if (!mul_ok(count, static_cast<size_t>(nranks), &total) || !mul_ok(total, 4, &out))
            return static_cast<size_t>(-1);
        return out;
    }
    return 0;
}

AR_EXPORT ar_result_t ar_comm_set_workspace(ar_comm_t comm, void* dev_ptr, size_t bytes)
{
    if (!comm) return fail(AR_ERR_INVALID_ARGUMENT, "comm is NULL");
    if (bytes > 0 && !dev_ptr) return fail(AR_ERR_INVALID_ARGUMENT, "workspace of %zu bytes at NULL", bytes);
    if (dev_ptr && !aligned16(dev_ptr)) return fail(AR_ERR_INVALID_ARGUMENT, "workspace is not 16-byte aligned");
    comm->ws = bytes ? dev_ptr : nullptr;
    comm->ws_bytes = dev_ptr ? bytes : 0;
    return AR_SUCCESS;
}

AR_EXPORT ar_result_t ar_comm_set_step_timing(ar_comm_t comm, int enable)
{
    if (!comm) return fail(AR_ERR_INVALID_ARGUMENT, "comm is NULL");
    comm->step_timing = enable != 0;
    comm->last_steps = -1;
    return AR_SUCCESS;
}

AR_EXPORT ar_result_t ar_comm_set_access(ar_comm_t comm, ar_access_t access)
{
    if (!comm) return fail(AR_ERR_INVALID_ARGUMENT, "comm is NULL");
    if (access < AR_ACCESS_AUTO || access > AR_ACCESS_CACHED)
        return fail(AR_ERR_INVALID_ARGUMENT, "invalid access flavour %d", static_cast<int>(access));
    comm->access = access;
    return AR_SUCCESS;
}

AR_EXPORT ar_result_t ar_comm_set_streaming(ar_comm_t comm, int enable)
{
    return ar_comm_set_access(comm, enable ? AR_ACCESS_STREAMING : AR_ACCESS_AUTO);
}

AR_EXPORT ar_result_t ar_last_step_times_ms(ar_comm_t comm, float* out, int cap, int* nsteps)
{
    if (!comm) return fail(AR_ERR_INVALID_ARGUMENT, "comm is NULL");
    if (!nsteps || (cap > 0 && !out)) return fail(AR_ERR_INVALID_ARGUMENT, "NULL output pointer");
    if (!comm->step_timing || comm->last_steps < 0)
        return fail(AR_ERR_INVALID_ARGUMENT, "no timed call on this comm (enable ar_comm_set_step_timing first)");
    DeviceGuard g(comm->device);
    if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
    const int k = comm->last_steps;
    *nsteps = k;
    if (k == 0) return AR_SUCCESS;
    hipError_t e = hipEventSynchronize(comm->events[k]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    for (int i = 0; i < k && i < cap; ++i) {
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, comm->events[i], comm->events[i + 1]);
        if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
        out[i] = ms;
    }
    return AR_SUCCESS;
}

// ---------------------------------------------------------------------------
// collectives
// ---------------------------------------------------------------------------
namespace {

// Enqueues one call's launches on a stream; `t` (may be null) records step events.
using Enqueue = std::function<hipError_t(hipStream_t, StepTimer*)>;

hipError_t tick(StepTimer* t) { return t ? t->step() : hipSuccess; }

// Eager: enqueue the launches directly on the caller's stream. `timing`
// false records no step events whatever the comm's setting (the
// allocation-free call creates no events).
ar_result_t run_eager(ar_comm* comm, hipStream_t stream, int nsteps, const Enqueue& fn, bool timing = true)
{
    if (!timing || !comm->step_timing) {
        hipError_t e = fn(stream, nullptr);
        return e != hipSuccess ? hip_fail(e, "kernel launch") : AR_SUCCESS;
    }
    StepTimer timer(comm, stream);
    hipError_t e = timer.begin(nsteps);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    e = fn(stream, &timer);
    if (e != hipSuccess) return hip_fail(e, "kernel launch");
    timer.end();
    return AR_SUCCESS;
}

// Graph mode: the call's launches are captured once into a hipGraph per key
// (collective, buffers, sizes, dtype, op, workspace) and the instantiated
// graph is replayed with one launch on later calls.
ar_result_t run_graph(ar_comm* comm, std::vector<uintptr_t>&& key, hipStream_t stream, const Enqueue& fn)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    if (cs != hipStreamCaptureStatusNone)
        return fail(AR_ERR_INVALID_ARGUMENT,
                    "AR_MODE_RING_GRAPH cannot be used while the stream is being captured; use AR_MODE_RING_STEPWISE "
                    "inside a capture");
    ar_comm::GraphEntry* hit = nullptr;
    for (auto& g : comm->graphs)
        if (g.key == key) hit = &g;
    if (!hit) {
        if (!comm->capture_stream) {
            e = hipStreamCreateWithFlags(&comm->capture_stream, hipStreamNonBlocking);
            if (e != hipSuccess) return hip_fail(e, "hipStreamCreateWithFlags");
        }
        e = hipStreamBeginCapture(comm->capture_stream, hipStreamCaptureModeThreadLocal);
        if (e != hipSuccess) return hip_fail(e, "hipStreamBeginCapture");
        const hipError_t le = fn(comm->capture_stream, nullptr);
        hipGraph_t graph = nullptr;
        e = hipStreamEndCapture(comm->capture_stream, &graph);
        if (le != hipSuccess || e != hipSuccess) {
            if (graph) (void)hipGraphDestroy(graph);
            return hip_fail(le != hipSuccess ? le : e, "graph capture");
        }
        hipGraphExec_t exec = nullptr;
        e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
        (void)hipGraphDestroy(graph);
        if (e != hipSuccess) return hip_fail(e, "hipGraphInstantiate");
        if (comm->graphs.size() >= ar_comm::kMaxGraphs) {
            auto oldest = std::min_element(comm->graphs.begin(), comm->graphs.end(),
                                           [](const auto& a, const auto& b) { return a.last_use < b.last_use; });
            (void)hipGraphExecDestroy(oldest->exec);
            comm->graphs.erase(oldest);
        }
        comm->graphs.push_back({std::move(key), exec, 0});
        hit = &comm->graphs.back();
    }
    hit->last_use = ++comm->use_clock;
    StepTimer timer(comm, stream);
    e = timer.begin(1);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    e = hipGraphLaunch(hit->exec, stream);
    if (e != hipSuccess) return hip_fail(e, "hipGraphLaunch");
    e = timer.step();
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    timer.end();
    return AR_SUCCESS;
}

std::vector<uintptr_t> graph_key(int coll, int n, const void* const send[], void* const recv[], size_t count, int dtype,
                                 int op, const void* ws)
{
    std::vector<uintptr_t> k{static_cast<uintptr_t>(coll), static_cast<uintptr_t>(n), count,
                             static_cast<uintptr_t>(dtype), static_cast<uintptr_t>(op),
                             reinterpret_cast<uintptr_t>(ws)};
    for (int r = 0; r < n; ++r) {
        k.push_back(reinterpret_cast<uintptr_t>(send[r]));
        k.push_back(reinterpret_cast<uintptr_t>(recv[r]));
    }
    return k;
}

bool ring_mode(ar_mode_t mode) { return mode == AR_MODE_RING_STEPWISE || mode == AR_MODE_RING_GRAPH; }

}  // namespace

namespace {

// The tree variant: a fused single pass in tree order, or 2*ceil(log2 n)
// level launches (reduce up to rank 0, broadcast back down).
ar_result_t tree_all_reduce(ar_comm* comm, const void* const sendbufs[], void* const recvbufs[], size_t count,
                            ar_dtype_t dtype, ar_op_t op, ar_mode_t mode, hipStream_t stream, const Workspace& wsp)
{
    const bool timing = !wsp.scratch;
    const int n = comm->nranks;
    const size_t e = elem_size(dtype);
    const uint64_t epv = 16 / e;
    const bool aligned = all_aligned16(n, sendbufs, recvbufs);
    DeviceGuard g(comm->device);
    if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
    if (comm->debug)
        std::fprintf(stderr, "[allreduce] all_reduce tree n=%d count=%zu dtype=%s op=%d mode=%d vec=%d\n", n, count,
                     dtype_name(dtype), static_cast<int>(op), static_cast<int>(mode), aligned ? 1 : 0);
    if (mode == AR_MODE_TREE) {
        ar::ReduceArgs a{};
        fill_ptrs(a, n, sendbufs, recvbufs);
        a.count = count;
        a.q = count;
        a.n = n;
        // One row over the whole buffer. Streaming (16-byte vectors): one
        // workgroup per 256-vector tile, in order (against 8-16 per CU on the
        // same buffers: 8 x 256 MiB fp32 0.823 -> 0.727 ms, 8 x 1 GiB fp16
        // 3.62 -> 3.00 ms, 16 x 128 MiB 0.796 -> 0.762 ms, 5 x 256 MiB 0.517 ->
        // 0.481 ms). Cached: 16 workgroups per CU up to 128 MiB per rank or
        // at 32+ ranks, 8 above (measured ±2-3% at 8 ranks).
        const int per_cu = (count * e <= (size_t(128) << 20) || n >= 32) ? 16 : 8;
        const bool nt = call_nt(comm, footprint(n, sendbufs, recvbufs, count * e, count * e), kLastLevelCacheBytes);
        const int gx = aligned && nt ? static_cast<int>(std::clamp<uint64_t>(
                                           ceil_div(ceil_div(count, epv), static_cast<uint64_t>(ar::kBlock)), 1, kMaxGridX))
                                     : grid_for(comm, aligned ? ceil_div(count, epv) : count, 1, per_cu);
        return run_eager(comm, stream, 1, [&](hipStream_t s, StepTimer* t) {
            hipError_t err = ar::launch_tree_fused(a, dtype, op, aligned, nt, gx, s);
            return err != hipSuccess ? err : tick(t);
        }, timing);
    }
    int levels = 0;
    while ((1 << levels) < n) ++levels;
    ar::TreeArgs ta{};
    fill_ptrs(ta, n, sendbufs, recvbufs);
    ta.ws = (dtype == AR_FLOAT16 || dtype == AR_BFLOAT16) ? wsp.ptr : nullptr;
    ta.ws_stride = (count + 3) / 4 * 4;
    ta.count = count;
    ta.n = n;
    // The levels' grid: beyond the last-level cache one workgroup per
    // 256-vector tile of a pair row (8 x 256 MiB fp32 1.805 -> 1.511 ms, fp16
    // 2.443 -> 2.109 ms, 16 x 128 MiB 1.960 -> 1.610 ms against 8 per CU),
    // else 8 workgroups per CU over the pairs.
    const bool lvl_exact = aligned && use_nt(footprint(n, sendbufs, recvbufs, count * e, count * e));
    const int gx = lvl_exact ? static_cast<int>(std::clamp<uint64_t>(
                                   ceil_div(ceil_div(count, epv), static_cast<uint64_t>(ar::kBlock)), 1, kMaxGridX))
                             : grid_for(comm, aligned ? ceil_div(count, epv) : count, std::max(1, n / 2));
    const bool bvec = aligned;
    Enqueue fn = [=](hipStream_t s, StepTimer* t) mutable {
        for (int l = 0; l < levels; ++l) {
            ta.stride = 1 << l;
            ta.last = l == levels - 1;
            hipError_t err = ar::launch_tree_reduce_level(ta, dtype, op, aligned, gx, s);
            if (err == hipSuccess) err = tick(t);
            if (err != hipSuccess) return err;
        }
        for (int l = levels - 1; l >= 0; --l) {
            ta.stride = 1 << l;
            hipError_t err = ar::launch_tree_bcast_level(ta, e, bvec, gx, s);
            if (err == hipSuccess) err = tick(t);
            if (err != hipSuccess) return err;
        }
        return hipSuccess;
    };
    return run_eager(comm, stream, 2 * levels, fn, timing);
}

}  // namespace

namespace {

// The all-reduce behind ar_all_reduce and ar_all_reduce_noalloc; `wsp` holds
// the partial sums of the stepwise fp16/bf16 paths. The scratch array
// (wsp.scratch) records no step events. Arguments are checked by the caller
// for comm, arrays, dtype and mode.
ar_result_t all_reduce_impl(ar_comm_t comm, const void* const sendbufs[], void* const recvbufs[], size_t count,
                            ar_dtype_t dtype, ar_op_t op, ar_mode_t mode, hipStream_t stream, const Workspace& wsp)
{
    ar_result_t rc = AR_SUCCESS;
    const bool timing = !wsp.scratch;
    if (!valid_op(op)) return fail(AR_ERR_INVALID_ARGUMENT, "invalid op %d", static_cast<int>(op));
    const int n = comm->nranks;
    const size_t e = elem_size(dtype);
    size_t bytes = 0;
    if (!mul_ok(count, e, &bytes)) return fail(AR_ERR_INVALID_ARGUMENT, "count %zu overflows", count);
    if (count == 0) return AR_SUCCESS;
    const bool stepwise = ring_mode(mode) && n > 1;
    const size_t ws_need = ar_workspace_bytes(AR_COLL_ALL_REDUCE, n, count, dtype, mode);
    if (ws_need == static_cast<size_t>(-1)) return fail(AR_ERR_INVALID_ARGUMENT, "workspace size overflows");
    rc = need_workspace(wsp, ws_need);
    if (rc != AR_SUCCESS) return rc;
    rc = check_buffers(n, sendbufs, recvbufs, bytes, bytes, AR_COLL_ALL_REDUCE, e, wsp.ptr, ws_need);
    if (rc != AR_SUCCESS) return rc;
    if (tree_mode(mode) && n > 1)
        return tree_all_reduce(comm, sendbufs, recvbufs, count, dtype, op, mode, stream, wsp);

    // Ring plan: q = ceil(count / n); chunk c = [c*q, min((c+1)*q, count)).
    const uint64_t q = ceil_div(count, static_cast<uint64_t>(n));
    const uint64_t epv = 16 / e;
    // 16-byte vectors whenever every pointer is aligned; chunks that start
    // or end inside a vector get element-wise heads and tails.
    const bool vec = all_aligned16(n, sendbufs, recvbufs);
    DeviceGuard g(comm->device);
    if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
    if (comm->debug)
        std::fprintf(stderr, "[allreduce] all_reduce n=%d count=%zu dtype=%s op=%d mode=%d q=%llu vec=%d\n", n, count,
                     dtype_name(dtype), static_cast<int>(op), static_cast<int>(mode),
                     static_cast<unsigned long long>(q), vec ? 1 : 0);

    if (!stepwise) {
        ar::ReduceArgs a{};
        fill_ptrs(a, n, sendbufs, recvbufs);
        a.count = count;
        a.q = q;
        a.n = n;
        const bool nt = call_nt(comm, footprint(n, sendbufs, recvbufs, bytes, bytes), kAllReduceStreamBytes);
        const int rm_tiles = use_rank_major(n, vec, nt) ? allreduce_tiles(n, e, bytes) : 0;
        const int gx = rm_tiles ? rank_major_grid(q, e, rm_tiles)
                                  : grid_for(comm, vec ? ceil_div(q, epv) : q, n, fused_per_cu(bytes, n, !nt));
        return run_eager(comm, stream, 1, [&](hipStream_t s, StepTimer* t) {
            hipError_t err = ar::launch_fused_reduce(a, dtype, op, false, vec, nt, rm_tiles, gx, s);
            return err != hipSuccess ? err : tick(t);
        }, timing);
    }

    // Reduce-scatter: n-1 steps. fp32/int32 partials travel in the recv
    // buffers (as the ring adds into its own chunk views); fp16/bf16 partials
    // stay in fp32 in the workspace, one slot per element.
    ar::StepArgs sa{};
    fill_ptrs(sa, n, sendbufs, recvbufs);
    sa.ws = (dtype == AR_FLOAT16 || dtype == AR_BFLOAT16) ? wsp.ptr : nullptr;
    sa.count = count;
    sa.q = q;
    sa.n = n;
    sa.scatter = 0;
    const uint64_t foot = footprint(n, sendbufs, recvbufs, bytes, bytes);
    const StepShape rs_shape = step_shape(comm, vec, ceil_div(q, epv), vec ? ceil_div(q, epv) : q, n, foot);
    // All-gather: n-1 copy steps; step s moves chunk (r - s) mod n from rank r-1 to rank r.
    ar::CopyArgs ca{};
    for (int r = 0; r < n; ++r) ca.recv[r] = recvbufs[r];
    ca.total = bytes;
    ca.qb = q * e;
    ca.n = n;
    ca.shift = 0;
    const bool cvec = vec;
    const StepShape ag_shape =
        step_shape(comm, cvec, ceil_div(ca.qb, 16), cvec ? ceil_div(ca.qb, 16) : ceil_div(ca.qb, 2), n, foot);
    Enqueue fn = [=](hipStream_t s, StepTimer* t) mutable {
        for (int st = 0; st < n - 1; ++st) {
            sa.s = st;
            sa.first = st == 0;
            sa.last = st == n - 2;
            hipError_t err = ar::launch_rs_step(sa, dtype, op, vec, rs_shape.tiles, rs_shape.nt, rs_shape.grid_x, s);
            if (err == hipSuccess) err = tick(t);
            if (err != hipSuccess) return err;
        }
        for (int st = 0; st < n - 1; ++st) {
            ca.s = st;
            hipError_t err = ar::launch_copy_step(ca, cvec, ag_shape.tiles, ag_shape.nt, ag_shape.grid_x, s);
            if (err == hipSuccess) err = tick(t);
            if (err != hipSuccess) return err;
        }
        return hipSuccess;
    };
    if (mode == AR_MODE_RING_GRAPH)
        return run_graph(comm, graph_key(AR_COLL_ALL_REDUCE, n, sendbufs, recvbufs, count, dtype, op, sa.ws), stream, fn);
    return run_eager(comm, stream, 2 * (n - 1), fn, timing);
}

}  // namespace

AR_EXPORT ar_result_t ar_all_reduce(ar_comm_t comm, const void* const sendbufs[], void* const recvbufs[], size_t count,
                                    ar_dtype_t dtype, ar_op_t op, ar_mode_t mode, hipStream_t stream)
{
    ar_result_t rc = check_common(comm, sendbufs, recvbufs, dtype, mode);
    if (rc != AR_SUCCESS) return rc;
    return all_reduce_impl(comm, sendbufs, recvbufs, count, dtype, op, mode, stream, comm_workspace(comm));
}

AR_EXPORT ar_result_t ar_all_reduce_noalloc(ar_comm_t comm, const void* const sendbufs[], void* const recvbufs[],
                                            size_t count, ar_dtype_t dtype, ar_op_t op, ar_mode_t mode,
                                            hipStream_t stream)
{
    ar_result_t rc = check_common(comm, sendbufs, recvbufs, dtype, mode);
    if (rc != AR_SUCCESS) return rc;
    if (mode == AR_MODE_RING_GRAPH)
        return fail(AR_ERR_UNSUPPORTED, "AR_MODE_RING_GRAPH instantiates a graph, which allocates; the "
                                        "allocation-free call takes the other modes");
    if (!comm->scratch)
        return fail(AR_ERR_INVALID_ARGUMENT, "the scratch array's address on device %d is unknown: %s",
                    comm->device, comm->scratch_err.c_str());
    return all_reduce_impl(comm, sendbufs, recvbufs, count, dtype, op, mode, stream,
                           Workspace{comm->scratch, AR_NOALLOC_SCRATCH_BYTES, true});
}

AR_EXPORT ar_result_t ar_reduce_scatter(ar_comm_t comm, const void* const sendbufs[], void* const recvbufs[],
                                        size_t recvcount, ar_dtype_t dtype, ar_op_t op, ar_mode_t mode,
                                        hipStream_t stream)
{
    ar_result_t rc = check_common(comm, sendbufs, recvbufs, dtype, mode);
    if (rc != AR_SUCCESS) return rc;
    if (tree_mode(mode))
        return fail(AR_ERR_UNSUPPORTED, "the tree modes are defined for all-reduce only");
    if (!valid_op(op)) return fail(AR_ERR_INVALID_ARGUMENT, "invalid op %d", static_cast<int>(op));
    const int n = comm->nranks;
    const size_t e = elem_size(dtype);
    size_t rbytes = 0, total = 0, sbytes = 0;
    if (!mul_ok(recvcount, e, &rbytes) || !mul_ok(recvcount, static_cast<size_t>(n), &total) || !mul_ok(total, e, &sbytes))
        return fail(AR_ERR_INVALID_ARGUMENT, "recvcount %zu overflows", recvcount);
    if (recvcount == 0) return AR_SUCCESS;
    const bool stepwise = ring_mode(mode) && n > 1;
    const size_t ws_need = stepwise ? ar_workspace_bytes(AR_COLL_REDUCE_SCATTER, n, recvcount, dtype, mode) : 0;
    if (ws_need == static_cast<size_t>(-1)) return fail(AR_ERR_INVALID_ARGUMENT, "workspace size overflows");
    rc = need_workspace(comm_workspace(comm), ws_need);
    if (rc != AR_SUCCESS) return rc;
    rc = check_buffers(n, sendbufs, recvbufs, sbytes, rbytes, AR_COLL_REDUCE_SCATTER, e, comm->ws, ws_need);
    if (rc != AR_SUCCESS) return rc;

    const uint64_t q = recvcount;  // block c of the reduction is chunk c of the ring
    const uint64_t epv = 16 / e;
    const bool vec = all_aligned16(n, sendbufs, recvbufs) && q % epv == 0;
    DeviceGuard g(comm->device);
    if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
    if (comm->debug)
        std::fprintf(stderr, "[allreduce] reduce_scatter n=%d recvcount=%zu dtype=%s op=%d mode=%d vec=%d\n", n,
                     recvcount, dtype_name(dtype), static_cast<int>(op), static_cast<int>(mode), vec ? 1 : 0);

    if (!stepwise) {
        // 4 workgroups per CU at 1-2 ranks (2 ranks x 1 GiB: 76.4% against
        // 72.0% at 8), 8 above (best or within 1.5 points at 8 ranks)
        ar::ReduceArgs a{};
        fill_ptrs(a, n, sendbufs, recvbufs);
        a.count = total;
        a.q = q;
        a.n = n;
        const bool nt = call_nt(comm, footprint(n, sendbufs, recvbufs, sbytes, rbytes), kLastLevelCacheBytes);
        // Rank-major kernels beyond the last-level cache from 2 ranks, one
        // workgroup per super tile: the fixed-rank-count body at 5..8 ranks
        // (+9 points at 256 MiB, +3.7 at 1 GiB, +1.5 at 14 GB against the
        // two-tile kernels on the same buffers with 8-16 workgroups per CU;
        // the exact grid then took 8 x 7e9 fp16 from 21.86 to 20.85 ms and
        // 8 x 64 MiB fp32 from 0.407 to 0.397 ms; the run-time body there
        // measured 1-2% slower at 8 ranks, 1% faster at 5-6; one tile per
        // super tile there against four: 8 x 7e9 fp16 20.65 -> 20.17 ms,
        // 8 x 256 MiB fp32 0.411 -> 0.401 ms), the run-time one at 2..4 ranks
        // (+8.7% at 4 x 64 MiB, +2.6% at 2 x 512 MiB of input against the
        // two-tile kernel) and above 8.
        const bool rank_major = vec && nt && n >= 2;
        const int rm_tiles = rank_major ? scatter_tiles(n, e) : 0;
        const int gx_f = rank_major ? rank_major_scatter_grid(q, e, rm_tiles)
                                    : grid_for(comm, vec ? ceil_div(q, epv) : q, n, n <= 2 ? 4 : 8);
        return run_eager(comm, stream, 1, [&](hipStream_t s, StepTimer* t) {
            hipError_t err = ar::launch_fused_reduce(a, dtype, op, true, vec, nt, rm_tiles, gx_f, s);
            return err != hipSuccess ? err : tick(t);
        });
    }
    // The ring's reduce-scatter phase with partials in the workspace; the
    // last step writes finished chunk c to recvbufs[c].
    ar::StepArgs sa{};
    fill_ptrs(sa, n, sendbufs, recvbufs);
    sa.ws = comm->ws;
    sa.count = total;
    sa.q = q;
    sa.n = n;
    sa.scatter = 1;
    const StepShape shape = step_shape(comm, vec, ceil_div(q, epv), vec ? ceil_div(q, epv) : q, n,
                                       footprint(n, sendbufs, recvbufs, sbytes, rbytes));
    Enqueue fn = [=](hipStream_t s, StepTimer* t) mutable {
        for (int st = 0; st < n - 1; ++st) {
            sa.s = st;
            sa.first = st == 0;
            sa.last = st == n - 2;
            hipError_t err = ar::launch_rs_step(sa, dtype, op, vec, shape.tiles, shape.nt, shape.grid_x, s);
            if (err == hipSuccess) err = tick(t);
            if (err != hipSuccess) return err;
        }
        return hipSuccess;
    };
    if (mode == AR_MODE_RING_GRAPH)
        return run_graph(comm, graph_key(AR_COLL_REDUCE_SCATTER, n, sendbufs, recvbufs, recvcount, dtype, op, sa.ws),
                         stream, fn);
    return run_eager(comm, stream, n - 1, fn);
}

AR_EXPORT ar_result_t ar_all_gather(ar_comm_t comm, const void* const sendbufs[], void* const recvbufs[],
                                    size_t sendcount, ar_dtype_t dtype, ar_mode_t mode, hipStream_t stream)
{
    ar_result_t rc = check_common(comm, sendbufs, recvbufs, dtype, mode);
    if (rc != AR_SUCCESS) return rc;
    if (tree_mode(mode))
        return fail(AR_ERR_UNSUPPORTED, "the tree modes are defined for all-reduce only");
    const int n = comm->nranks;
    const size_t e = elem_size(dtype);
    size_t blk = 0, rbytes = 0;
    if (!mul_ok(sendcount, e, &blk) || !mul_ok(blk, static_cast<size_t>(n), &rbytes))
        return fail(AR_ERR_INVALID_ARGUMENT, "sendcount %zu overflows", sendcount);
    if (sendcount == 0) return AR_SUCCESS;
    rc = check_buffers(n, sendbufs, recvbufs, blk, rbytes, AR_COLL_ALL_GATHER, e, nullptr, 0);
    if (rc != AR_SUCCESS) return rc;
    const bool stepwise = ring_mode(mode) && n > 1;
    const bool vec = all_aligned16(n, sendbufs, recvbufs) && blk % 16 == 0;
    DeviceGuard g(comm->device);
    if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
    if (comm->debug)
        std::fprintf(stderr, "[allreduce] all_gather n=%d sendcount=%zu dtype=%s mode=%d vec=%d\n", n, sendcount,
                     dtype_name(dtype), static_cast<int>(mode), vec ? 1 : 0);
    const StepShape shape = step_shape(comm, vec, ceil_div(blk, 16), vec ? ceil_div(blk, 16) : ceil_div(blk, 2), n,
                                       footprint(n, sendbufs, recvbufs, blk, rbytes));

    if (!stepwise) {
        ar::CopyArgs a{};
        fill_ptrs(a, n, sendbufs, recvbufs);
        a.total = blk;
        a.n = n;
        const bool nt = call_nt(comm, footprint(n, sendbufs, recvbufs, blk, rbytes), kLastLevelCacheBytes);
        // Streaming: the rank-major copy (kRankMajorTiles vectors per thread
        // loaded once, stored to every rank), one workgroup per tile; against
        // the grid-stride copies used before on the same buffers, fp32: 1 rank
        // x 1 GiB (a plain copy) 0.357 -> 0.341 ms, 8 x 32 MiB in 0.435 ->
        // 0.363 ms, 8 x 128 MiB 1.71 -> 1.48 ms, 2 x 512 MiB 0.597 -> 0.558 ms,
        // 8 x 1.75 GB fp16 22.06 -> 21.93 ms, 16 x 8 MiB level. Cached: one
        // vector per thread per step, 4 workgroups per CU for a single rank
        // (a plain copy: 73.5% of peak at 1 GiB against 66.0% at 8), 3 at 2
        // ranks, 8 above.
        const bool rank_major = vec && nt;
        const int gx_f = rank_major ? copy_tile_grid(blk / 16)
                                    : grid_for(comm, vec ? ceil_div(blk, 16) : ceil_div(blk, 2), n,
                                               n == 1 ? 4 : n == 2 ? 3 : 8);
        return run_eager(comm, stream, 1, [&](hipStream_t s, StepTimer* t) {
            hipError_t err = ar::launch_fused_gather(a, vec, nt, rank_major, gx_f, s);
            return err != hipSuccess ? err : tick(t);
        });
    }
    // Each rank first places its own block (unless in place), then n-1 ring
    // steps: at step s rank r receives block (r - s - 1) mod n from rank r-1.
    ar::CopyArgs la{};
    int m = 0;
    bool lvec = vec;
    for (int r = 0; r < n; ++r) {
        const char* dst = static_cast<const char*>(recvbufs[r]) + static_cast<size_t>(r) * blk;
        if (dst == sendbufs[r]) continue;
        la.send[m] = sendbufs[r];
        la.recv[m] = const_cast<char*>(dst);
        ++m;
    }
    la.n = m;
    la.total = blk;
    la.dst_stride = 0;
    const int gx_local = grid_for(comm, lvec ? ceil_div(blk, 16) : ceil_div(blk, 2), std::max(m, 1));
    ar::CopyArgs ca{};
    for (int r = 0; r < n; ++r) ca.recv[r] = recvbufs[r];
    ca.total = rbytes;
    ca.qb = blk;
    ca.n = n;
    ca.shift = 1;
    Enqueue fn = [=](hipStream_t s, StepTimer* t) mutable {
        hipError_t err = m > 0 ? ar::launch_local_copy(la, lvec, gx_local, s) : hipSuccess;
        if (err == hipSuccess) err = tick(t);
        if (err != hipSuccess) return err;
        for (int st = 0; st < n - 1; ++st) {
            ca.s = st;
            err = ar::launch_copy_step(ca, vec, shape.tiles, shape.nt, shape.grid_x, s);
            if (err == hipSuccess) err = tick(t);
            if (err != hipSuccess) return err;
        }
        return hipSuccess;
    };
    if (mode == AR_MODE_RING_GRAPH)
        return run_graph(comm, graph_key(AR_COLL_ALL_GATHER, n, sendbufs, recvbufs, sendcount, dtype, 0, nullptr),
                         stream, fn);
    return run_eager(comm, stream, n, fn);
}

AR_EXPORT ar_result_t ar_all_to_all(ar_comm_t comm, const void* const sendbufs[], void* const recvbufs[],
                                    size_t blockcount, ar_dtype_t dtype, ar_mode_t mode, hipStream_t stream)
{
    ar_result_t rc = check_common(comm, sendbufs, recvbufs, dtype, mode);
    if (rc != AR_SUCCESS) return rc;
    if (tree_mode(mode))
        return fail(AR_ERR_UNSUPPORTED, "the tree modes are defined for all-reduce only");
    const int n = comm->nranks;
    const size_t e = elem_size(dtype);
    size_t blk = 0, total = 0;
    if (!mul_ok(blockcount, e, &blk) || !mul_ok(blk, static_cast<size_t>(n), &total))
        return fail(AR_ERR_INVALID_ARGUMENT, "blockcount %zu overflows", blockcount);
    if (blockcount == 0) return AR_SUCCESS;
    rc = check_buffers(n, sendbufs, recvbufs, total, total, AR_COLL_ALL_TO_ALL, e, nullptr, 0);
    if (rc != AR_SUCCESS) return rc;
    const bool stepwise = ring_mode(mode);
    const bool vec = all_aligned16(n, sendbufs, recvbufs) && blk % 16 == 0;
    DeviceGuard g(comm->device);
    if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
    if (comm->debug)
        std::fprintf(stderr, "[allreduce] all_to_all n=%d blockcount=%zu dtype=%s mode=%d vec=%d\n", n, blockcount,
                     dtype_name(dtype), static_cast<int>(mode), vec ? 1 : 0);
    ar::A2AArgs a{};
    fill_ptrs(a, n, sendbufs, recvbufs);
    a.blk = blk;
    a.n = n;
    const uint64_t units = vec ? ceil_div(blk, 16) : ceil_div(blk, 2);
    const bool nt = use_nt(2 * static_cast<uint64_t>(n) * total);
    if (!stepwise) {
        a.step = -1;
        // Streaming: the tiled copy, one workgroup per tile, so block pairs
        // are copied one after another (against 4 workgroups per CU on the
        // same buffers, fp32: 8 x 256 MiB 0.776 -> 0.711 ms, 8 x 32 MiB 93.4
        // -> 88.0 us, 4 x 512 MiB 0.774 -> 0.720 ms, 16 x 64 MiB 0.387 ->
        // 0.392 ms). Cached: 4 workgroups per CU, each moving one block pair
        // (8 ranks x 256 MiB: 69.3% against 62.2% at 8).
        const bool nt1 = call_nt(comm, 2 * static_cast<uint64_t>(n) * total, kLastLevelCacheBytes);
        const bool tiled = vec && nt1;
        const int gx = tiled ? copy_tile_grid(blk / 16) : grid_for(comm, units, n * n, 4);
        return run_eager(comm, stream, 1, [&](hipStream_t s, StepTimer* t) {
            hipError_t err = ar::launch_all_to_all(a, vec, nt1, tiled, gx, s);
            return err != hipSuccess ? err : tick(t);
        });
    }
    // Each step moves N block pairs; streaming steps with at least 8 tiles
    // per CU take the tiled copy, one workgroup per tile.
    const int tiles = vec ? copy_tile_grid(blk / 16) : 0;
    const bool tiled = vec && nt && static_cast<uint64_t>(tiles) * n >= static_cast<uint64_t>(comm->num_cus) * 8;
    const int gx = tiled ? tiles : grid_for(comm, units, n);
    Enqueue fn = [=](hipStream_t s, StepTimer* t) mutable {
        for (int st = 0; st < n; ++st) {
            a.step = st;
            hipError_t err = ar::launch_all_to_all(a, vec, nt, tiled, gx, s);
            if (err == hipSuccess) err = tick(t);
            if (err != hipSuccess) return err;
        }
        return hipSuccess;
    };
    if (mode == AR_MODE_RING_GRAPH)
        return run_graph(comm, graph_key(AR_COLL_ALL_TO_ALL, n, sendbufs, recvbufs, blockcount, dtype, 0, nullptr),
                         stream, fn);
    return run_eager(comm, stream, n, fn);
}

// Coalesced multi-tensor all-reduce: tensor t of rank r is
// sendbufs[t*n + r] / recvbufs[t*n + r] with counts[t] elements. The tensors
// of a rank are one virtual flat bucket in tensor order, partitioned into
// ring chunks as one buffer.
AR_EXPORT ar_result_t ar_all_reduce_multi(ar_comm_t comm, int ntensors, const void* const sendbufs[],
                                          void* const recvbufs[], const size_t counts[], ar_dtype_t dtype, ar_op_t op,
                                          ar_mode_t mode, hipStream_t stream)
{
    if (!comm) return fail(AR_ERR_INVALID_ARGUMENT, "comm is NULL");
    if (ntensors < 0 || ntensors > AR_MAX_TENSORS)
        return fail(AR_ERR_INVALID_ARGUMENT, "ntensors %d is outside 0..%d", ntensors, AR_MAX_TENSORS);
    if (ntensors > 0 && (!sendbufs || !recvbufs || !counts))
        return fail(AR_ERR_INVALID_ARGUMENT, "NULL sendbufs, recvbufs or counts array");
    if (!valid_dtype(dtype)) return fail(AR_ERR_INVALID_ARGUMENT, "invalid dtype %d", static_cast<int>(dtype));
    if (!valid_op(op)) return fail(AR_ERR_INVALID_ARGUMENT, "invalid op %d", static_cast<int>(op));
    if (!valid_mode(mode)) return fail(AR_ERR_INVALID_ARGUMENT, "invalid mode %d", static_cast<int>(mode));
    if (mode != AR_MODE_FUSED)
        return fail(AR_ERR_UNSUPPORTED, "the multi-tensor all-reduce runs in AR_MODE_FUSED only");
    const int n = comm->nranks;
    const size_t e = elem_size(dtype);
    uint64_t total = 0;
    std::vector<Interval> iv;
    for (int t = 0; t < ntensors; ++t) {
        size_t bytes = 0;
        if (!mul_ok(counts[t], e, &bytes) || total + counts[t] < total)
            return fail(AR_ERR_INVALID_ARGUMENT, "counts[%d] = %zu overflows", t, counts[t]);
        total += counts[t];
        if (counts[t] == 0) continue;
        for (int r = 0; r < n; ++r) {
            const void* sp = sendbufs[static_cast<size_t>(t) * n + r];
            const void* dp = recvbufs[static_cast<size_t>(t) * n + r];
            if (!sp || !dp) return fail(AR_ERR_INVALID_ARGUMENT, "tensor %d rank %d buffer is NULL", t, r);
            const uintptr_t s = reinterpret_cast<uintptr_t>(sp), d = reinterpret_cast<uintptr_t>(dp);
            if (s % e || d % e)
                return fail(AR_ERR_INVALID_ARGUMENT, "tensor %d rank %d buffer is not aligned to %zu bytes", t, r, e);
            if (s > UINTPTR_MAX - bytes || d > UINTPTR_MAX - bytes)
                return fail(AR_ERR_INVALID_ARGUMENT, "tensor %d rank %d buffer wraps the address space", t, r);
            if (s == d) {
                iv.push_back({s, s + bytes, "in-place tensor", t});
            } else {
                iv.push_back({s, s + bytes, "send tensor", t});
                iv.push_back({d, d + bytes, "recv tensor", t});
            }
        }
    }
    if (total == 0) return AR_SUCCESS;
    size_t oa, ob;
    if (find_overlap(iv, &oa, &ob))
        return fail(AR_ERR_INVALID_ARGUMENT, "%s %d overlaps %s %d (only send == recv may alias)", iv[oa].what,
                    iv[oa].rank, iv[ob].what, iv[ob].rank);

    DeviceGuard g(comm->device);
    if (g.err != hipSuccess) return hip_fail(g.err, "hipSetDevice");
    const uint64_t q = ceil_div(total, static_cast<uint64_t>(n));
    const uint64_t E = 16 / e;

    // Every non-empty tensor's rank pointers (n send then n recv; only n when
    // every rank's tensor is in place) and its pieces (the parts that fall in
    // one ring chunk each), in tensor order.
    struct TensorPlan {
        std::vector<const void*> ptrs;
        std::vector<ar::MultiPiece> pieces;
    };
    std::vector<TensorPlan> plan;
    uint64_t off = 0;
    for (int t = 0; t < ntensors; ++t) {
        const uint64_t cnt = counts[t];
        if (cnt == 0) continue;
        TensorPlan tp;
        // 16-byte vectors need every rank's send and recv pointer at the same
        // offset from a 16-byte boundary; a0 elements precede the first one.
        // When the pointers also share their offset from a 128-byte line
        // (views at one offset into line-aligned per-rank buckets), the
        // vectors start on the first whole line instead, so that a wave's
        // 1 KiB access covers eight lines, not nine.
        const uintptr_t mis = reinterpret_cast<uintptr_t>(sendbufs[static_cast<size_t>(t) * n]) % 128;
        bool vec = true, line = true, inplace = true;
        for (int r = 0; r < n; ++r) {
            const uintptr_t sp = reinterpret_cast<uintptr_t>(sendbufs[static_cast<size_t>(t) * n + r]);
            const uintptr_t dp = reinterpret_cast<uintptr_t>(recvbufs[static_cast<size_t>(t) * n + r]);
            vec = vec && sp % 16 == mis % 16 && dp % 16 == mis % 16;
            line = line && sp % 128 == mis && dp % 128 == mis;
            inplace = inplace && sp == dp;
        }
        const uint64_t a0 = (line ? (128 - mis) % 128 : (16 - mis % 16) % 16) / e;
        for (int r = 0; r < n; ++r) tp.ptrs.push_back(sendbufs[static_cast<size_t>(t) * n + r]);
        if (!inplace)
            for (int r = 0; r < n; ++r) tp.ptrs.push_back(recvbufs[static_cast<size_t>(t) * n + r]);
        for (uint64_t c = off / q; c * q < off + cnt; ++c) {
            const uint64_t lo = std::max(off, c * q), hi = std::min(off + cnt, (c + 1) * q);
            ar::MultiPiece pc{};
            pc.j0 = lo - off;
            pc.len = hi - lo;
            pc.chunk = static_cast<uint8_t>(c);
            pc.flags = static_cast<uint8_t>((vec ? ar::kPieceVec | (a0 << ar::kPieceShiftBit) : 0) |
                                            (inplace ? ar::kPieceInPlace : 0));
            tp.pieces.push_back(pc);
        }
        plan.push_back(std::move(tp));
        off += cnt;
    }

    uint64_t touched = 0;
    for (const Interval& x : iv) touched += x.hi - x.lo;
    const bool nt = call_nt(comm, touched, kAllReduceStreamBytes);
    // The rank-major kernel (use_rank_major_multi) cuts vector pieces into
    // tiles of rank_major_any_tiles quarters, as the flat kernel's super
    // tiles.
    const bool rank_major = use_rank_major_multi(n, nt);
    const uint64_t tile_vecs =
        rank_major ? static_cast<uint64_t>(ar::rank_major_any_tiles(n, static_cast<int>(e))) * ar::kBlock
                   : static_cast<uint64_t>(ar::kMultiVecTile);

    // Lays out tensors [t0, t1) of the plan as one table (pointer blocks,
    // then pieces with their first tiles) and returns its header.
    auto layout = [&](size_t t0, size_t t1, unsigned char* out, ar::MultiHeader* h) -> bool {
        size_t nptrs = 0;
        for (size_t t = t0; t < t1; ++t) nptrs += plan[t].ptrs.size();
        h->n = n;
        h->pieces_offset = static_cast<uint32_t>(nptrs * sizeof(void*));
        uint64_t tiles = 0;
        int np = 0;
        size_t p0 = 0;
        for (size_t t = t0; t < t1; ++t) {
            std::memcpy(out + p0 * sizeof(void*), plan[t].ptrs.data(), plan[t].ptrs.size() * sizeof(void*));
            for (ar::MultiPiece pc : plan[t].pieces) {
                pc.tile0 = static_cast<uint32_t>(tiles);
                pc.ptrs = static_cast<uint16_t>(p0);
                uint64_t piece_tiles;
                if (pc.flags & ar::kPieceVec) {
                    uint64_t vb, ve;
                    ar::piece_vectors(pc.j0, pc.j0 + pc.len, (pc.flags >> ar::kPieceShiftBit) & ar::kPieceShiftMask, E,
                                      &vb, &ve);
                    piece_tiles = std::max<uint64_t>(1, ceil_div(ve - vb, tile_vecs));
                } else {
                    piece_tiles = ceil_div(pc.len, ar::kBlock);
                }
                tiles += piece_tiles;
                std::memcpy(out + h->pieces_offset + static_cast<size_t>(np) * sizeof(pc), &pc, sizeof(pc));
                ++np;
            }
            p0 += plan[t].ptrs.size();
        }
        h->npieces = np;
        h->ntiles = static_cast<uint32_t>(tiles);
        return tiles <= UINT32_MAX;
    };
    auto table_bytes = [&](size_t t0, size_t t1) {
        size_t bytes = 0;
        for (size_t t = t0; t < t1; ++t)
            bytes += plan[t].ptrs.size() * sizeof(void*) + plan[t].pieces.size() * sizeof(ar::MultiPiece);
        return bytes;
    };

    // The two-tile kernel: at most 16 workgroups per CU (the 29-tensor
    // 256 MiB bucket ran at 7.09 ms at 64 ranks against 7.51 at 8 per CU, and
    // 0.913 against 0.929 ms at 8 ranks). The rank-major kernel: one
    // workgroup per tile, taken in order, as the flat call's super tiles.
    // Against the kernels used before on the same buffers (grid-stride, 16-32
    // per CU, tiles interleaved over N segments; a fixed-rank-count tile at 8
    // ranks; the two-tile kernel below 8 ranks and below 128 MiB per rank at
    // 8), fp32 MAX as 29 tensors: 64 x 256 MiB 6.82 -> 6.57 ms, 8 x
    // 256 MiB 0.802 -> 0.753 ms, 4 x 256 MiB 0.398 -> 0.366 ms; as 10
    // tensors 8 x 64 MiB 0.205 -> 0.183 ms, 8 x 25 MiB 80.7 -> 74.2 us.
    const int cap = comm->num_cus * 16;

    // The tables go in the kernel arguments, one launch per batch of tensors
    // that fits. (A table in device memory, written once and read by a single
    // launch, measured slower: 10.3 vs 8.1 ms for the 64-rank bucket.)
    std::vector<ar::MultiArgs> batches;
    for (size_t t0 = 0; t0 < plan.size();) {
        size_t t1 = t0 + 1;
        if (table_bytes(t0, t1) > ar::kMultiBlobBytes)
            return fail(AR_ERR_INTERNAL, "tensor %zu does not fit the kernel arguments", t0);
        while (t1 < plan.size() && table_bytes(t0, t1 + 1) <= ar::kMultiBlobBytes) ++t1;
        ar::MultiArgs a{};
        if (!layout(t0, t1, a.blob, &a.h))
            return fail(AR_ERR_INVALID_ARGUMENT, "the bucket needs more than 2^32 tiles");
        batches.push_back(a);
        t0 = t1;
    }
    if (comm->debug)
        std::fprintf(stderr, "[allreduce] all_reduce_multi n=%d tensors=%zu dtype=%s op=%d batches=%zu rank_major=%d\n",
                     n, plan.size(), dtype_name(dtype), static_cast<int>(op), batches.size(), rank_major ? 1 : 0);
    return run_eager(comm, stream, static_cast<int>(batches.size()), [&](hipStream_t s, StepTimer* t) {
        for (const auto& a : batches) {
            const uint64_t gx = rank_major ? std::min<uint64_t>(a.h.ntiles, kMaxGridX)
                                           : std::min<uint64_t>(a.h.ntiles, cap);
            hipError_t e2 = ar::launch_multi_reduce(a, dtype, op, nt, rank_major, static_cast<int>(gx), s);
            if (e2 == hipSuccess) e2 = tick(t);
            if (e2 != hipSuccess) return e2;
        }
        return hipSuccess;
    });
}

AR_EXPORT const char* ar_result_string(ar_result_t result)
{
    switch (result) {
    case AR_SUCCESS: return "success";
    case AR_ERR_INVALID_ARGUMENT: return "invalid argument";
    case AR_ERR_UNSUPPORTED: return "unsupported";
    case AR_ERR_HIP: return "HIP runtime error";
    case AR_ERR_OUT_OF_MEMORY: return "out of memory";
    case AR_ERR_INTERNAL: return "internal error";
    }
    return "unknown result code";
}

AR_EXPORT const char* ar_last_error(void) { return g_last_error.c_str(); }
