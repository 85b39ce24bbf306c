// kernels_impl.h -- device code of the ring all-reduce for CDNA4 (gfx950):
// element formats, reduce ops, the kernels, and per-dtype dispatch templates.
// Each dtype is instantiated in its own translation units (dtype_*.hip,
// tree_*.hip) so the build compiles them in parallel; kernels.hip holds the
// dtype switch and the dtype-free copy kernels.
//
// The reduction is elementwise and HBM-bound: one combine per element and
// rank against 2*sizeof(T) bytes moved, far below any matrix-core ridge, so
// there is no MFMA here. What matters is moving bytes: 16-byte (dwordx4)
// loads and non-temporal stores, one wavefront-uniform chunk per workgroup
// row so the rank order of the fold is a scalar (SGPR) choice, and enough
// loads in flight per CU.
//
// Ring order [geek-doc "训练梯度同步与集合通信", section 三; handbook
// "集合通信原语", section 环形 all-reduce 与通信量]: chunk c of the buffer is
// reduced by the ring as acc = x_c, then acc = x_{c+k} (+) acc for
// k = 1..n-1 (ranks mod n). Every kernel below folds in exactly that order,
// so the fused and stepwise modes give the same bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace ar {
namespace detail {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Rank buffers are global memory. Pointers that come from kernel arguments
// are known to be global; pointers read from a device-memory table are not,
// and would be accessed with flat instructions. gptr states it.
template <class T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* gptr(const void* p)
{
    return (const __attribute__((address_space(1))) T*)(p);
}
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gptr(void* p)
{
    return (__attribute__((address_space(1))) T*)(p);
}

// ---------------------------------------------------------------------------
// element formats
// ---------------------------------------------------------------------------
__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

__device__ __forceinline__ float half_to_f32(uint32_t h)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// v_cvt_f16_f32: round to nearest even (the default mode), subnormals kept.
// The value is pinned in a register first: otherwise the compiler may merge
// the fp32 multiply that produced it with this conversion into one
// mixed-precision FMA (v_fma_mix*), which rounds once where the fp32 product
// followed by the conversion rounds twice.
__device__ __forceinline__ uint32_t f32_to_half(float f)
{
    asm("" : "+v"(f));
    if (__builtin_isnan(f)) return ((as_u(f) >> 16) & 0x8000u) | 0x7E00u;
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return as_f(b << 16); }

// bfloat16 keeps the top 16 bits of the fp32 pattern; adding 0x7FFF plus the
// lowest kept bit rounds the dropped 16 bits to nearest, ties to even (a
// carry into the exponent is the correct rounding up, up to infinity).
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = as_u(f);
    if (__builtin_isnan(f)) return ((u >> 16) & 0x8000u) | 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

struct F32 {
    using Acc = float;
    static constexpr int kEpv = 4;  // elements per 16-byte vector
    static __device__ __forceinline__ Acc ld(const void* p, uint64_t i) { return gptr<float>(p)[i]; }
    static __device__ __forceinline__ void st(void* p, uint64_t i, Acc v) { gptr<float>(p)[i] = v; }
    static __device__ __forceinline__ void unpack(u32x4 v, Acc* a)
    {
        a[0] = as_f(v.x); a[1] = as_f(v.y); a[2] = as_f(v.z); a[3] = as_f(v.w);
    }
    static __device__ __forceinline__ u32x4 pack(const Acc* a)
    {
        return u32x4{as_u(a[0]), as_u(a[1]), as_u(a[2]), as_u(a[3])};
    }
};

struct I32 {
    using Acc = uint32_t;  // two's-complement wrap
    static constexpr int kEpv = 4;
    static __device__ __forceinline__ Acc ld(const void* p, uint64_t i) { return gptr<uint32_t>(p)[i]; }
    static __device__ __forceinline__ void st(void* p, uint64_t i, Acc v) { gptr<uint32_t>(p)[i] = v; }
    static __device__ __forceinline__ void unpack(u32x4 v, Acc* a) { a[0] = v.x; a[1] = v.y; a[2] = v.z; a[3] = v.w; }
    static __device__ __forceinline__ u32x4 pack(const Acc* a) { return u32x4{a[0], a[1], a[2], a[3]}; }
};

struct F16 {
    using Acc = float;
    static constexpr int kEpv = 8;
    static __device__ __forceinline__ Acc ld(const void* p, uint64_t i)
    {
        return half_to_f32(gptr<uint16_t>(p)[i]);
    }
    static __device__ __forceinline__ void st(void* p, uint64_t i, Acc v)
    {
        gptr<uint16_t>(p)[i] = static_cast<uint16_t>(f32_to_half(v));
    }
    static __device__ __forceinline__ void unpack(u32x4 v, Acc* a)
    {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a[2 * j] = half_to_f32(w[j] & 0xFFFFu);
            a[2 * j + 1] = half_to_f32(w[j] >> 16);
        }
    }
    static __device__ __forceinline__ u32x4 pack(const Acc* a)
    {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = f32_to_half(a[2 * j]) | (f32_to_half(a[2 * j + 1]) << 16);
        return u32x4{w[0], w[1], w[2], w[3]};
    }
    // half a vector: four elements in 8 bytes, in the order unpack uses
    static __device__ __forceinline__ void unpack4(u32x2 v, Acc* a)
    {
        a[0] = half_to_f32(v.x & 0xFFFFu);
        a[1] = half_to_f32(v.x >> 16);
        a[2] = half_to_f32(v.y & 0xFFFFu);
        a[3] = half_to_f32(v.y >> 16);
    }
    static __device__ __forceinline__ u32x2 pack4(const Acc* a)
    {
        return u32x2{f32_to_half(a[0]) | (f32_to_half(a[1]) << 16), f32_to_half(a[2]) | (f32_to_half(a[3]) << 16)};
    }
};

struct BF16 {
    using Acc = float;
    static constexpr int kEpv = 8;
    static __device__ __forceinline__ Acc ld(const void* p, uint64_t i)
    {
        return bf16_to_f32(gptr<uint16_t>(p)[i]);
    }
    static __device__ __forceinline__ void st(void* p, uint64_t i, Acc v)
    {
        gptr<uint16_t>(p)[i] = static_cast<uint16_t>(f32_to_bf16(v));
    }
    static __device__ __forceinline__ void unpack(u32x4 v, Acc* a)
    {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a[2 * j] = as_f(w[j] << 16);
            a[2 * j + 1] = as_f(w[j] & 0xFFFF0000u);
        }
    }
    static __device__ __forceinline__ u32x4 pack(const Acc* a)
    {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = f32_to_bf16(a[2 * j]) | (f32_to_bf16(a[2 * j + 1]) << 16);
        return u32x4{w[0], w[1], w[2], w[3]};
    }
    static __device__ __forceinline__ void unpack4(u32x2 v, Acc* a)
    {
        a[0] = as_f(v.x << 16);
        a[1] = as_f(v.x & 0xFFFF0000u);
        a[2] = as_f(v.y << 16);
        a[3] = as_f(v.y & 0xFFFF0000u);
    }
    static __device__ __forceinline__ u32x2 pack4(const Acc* a)
    {
        return u32x2{f32_to_bf16(a[0]) | (f32_to_bf16(a[1]) << 16), f32_to_bf16(a[2]) | (f32_to_bf16(a[3]) << 16)};
    }
};

// ---------------------------------------------------------------------------
// reduce ops: local (+) incoming [mhpq.cn all-reduce article, section 2.1]
// ---------------------------------------------------------------------------
// MAX/MIN: NaN if either operand is NaN, and +0 > -0, so both are
// commutative and associative. That is IEEE 754-2019 maximum/minimum, which
// gfx950 executes in one instruction (v_maximum3_f32 / v_minimum3_f32).
// A NaN result may carry an input's payload; only its NaN-ness is specified.
__device__ __forceinline__ float fp_max(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float fp_min(float a, float b) { return __builtin_elementwise_minimum(a, b); }

template <int OP>
__device__ __forceinline__ float combine(float local, float in)
{
    if constexpr (OP == AR_SUM || OP == AR_AVG) return local + in;
    else if constexpr (OP == AR_PROD) return local * in;
    else if constexpr (OP == AR_MAX) return fp_max(local, in);
    else return fp_min(local, in);
}

template <int OP>
__device__ __forceinline__ uint32_t combine(uint32_t local, uint32_t in)
{
    if constexpr (OP == AR_SUM || OP == AR_AVG) return local + in;
    else if constexpr (OP == AR_PROD) return local * in;
    else if constexpr (OP == AR_MAX) return static_cast<int32_t>(local) > static_cast<int32_t>(in) ? local : in;
    else return static_cast<int32_t>(local) < static_cast<int32_t>(in) ? local : in;
}

// AVG: the finished sum divided once by n (correctly rounded fp32 divide;
// int32 truncates toward zero).
template <int OP>
__device__ __forceinline__ float finalize(float a, int n)
{
    if constexpr (OP == AR_AVG) return a / static_cast<float>(n);
    else return a;
}

template <int OP>
__device__ __forceinline__ uint32_t finalize(uint32_t a, int n)
{
    if constexpr (OP == AR_AVG) return static_cast<uint32_t>(static_cast<int32_t>(a) / n);
    else return a;
}

// ---------------------------------------------------------------------------
// memory access
// ---------------------------------------------------------------------------
// Streaming loads/stores: each input is read once and each output written
// once, so both bypass cache retention (nt).
__device__ __forceinline__ u32x4 ld16_nt(const void* base, uint64_t v)
{
    return __builtin_nontemporal_load(gptr<u32x4>(base) + v);
}
__device__ __forceinline__ void st16_nt(void* base, uint64_t v, u32x4 x)
{
    __builtin_nontemporal_store(x, gptr<u32x4>(base) + v);
}
__device__ __forceinline__ u32x4 ld16(const void* base, uint64_t v) { return gptr<u32x4>(base)[v]; }
__device__ __forceinline__ void st16(void* base, uint64_t v, u32x4 x) { gptr<u32x4>(base)[v] = x; }

// The fused kernels pick the access flavour per call: when everything the
// call touches fits in the last-level cache (the 256 MB Infinity Cache of
// MI355X), ordinary loads and stores let repeated calls run from the cache
// (measured 1.6x faster for 8 x 25 MiB in place); for larger footprints
// non-temporal access streams through without evicting (equal or better).
template <bool NT>
__device__ __forceinline__ u32x4 ldv(const void* base, uint64_t v)
{
    if constexpr (NT) return ld16_nt(base, v);
    else return ld16(base, v);
}
// The same at a byte offset (a multiple of 16 past a 16-byte boundary).
template <bool NT>
__device__ __forceinline__ u32x4 ldv_at(const void* base, uint64_t byte_off)
{
    return ldv<NT>(static_cast<const char*>(base) + byte_off, 0);
}

template <bool NT>
__device__ __forceinline__ void stv(void* base, uint64_t v, u32x4 x)
{
    if constexpr (NT) st16_nt(base, v, x);
    else st16(base, v, x);
}
template <bool NT>
__device__ __forceinline__ void stv_at(void* base, uint64_t byte_off, u32x4 x)
{
    stv<NT>(static_cast<char*>(base) + byte_off, 0, x);
}

// 8-byte units (half a vector of a 16-bit type).
template <bool NT>
__device__ __forceinline__ u32x2 ldh(const void* base, uint64_t h)
{
    if constexpr (NT) return __builtin_nontemporal_load(gptr<u32x2>(base) + h);
    else return gptr<u32x2>(base)[h];
}
template <bool NT>
__device__ __forceinline__ void sth(void* base, uint64_t h, u32x2 x)
{
    if constexpr (NT) __builtin_nontemporal_store(x, gptr<u32x2>(base) + h);
    else gptr<u32x2>(base)[h] = x;
}

__device__ __forceinline__ int wrap_rank(int r, int n) { return r >= n ? r - n : r; }

__device__ __forceinline__ void chunk_range(uint64_t q, uint64_t count, int c, uint64_t& lo, uint64_t& hi)
{
    lo = min(static_cast<uint64_t>(c) * q, count);
    hi = min(lo + q, count);
}

// ---------------------------------------------------------------------------
// fused single-pass reduction
// ---------------------------------------------------------------------------
// Element i of chunk c, all ranks, in ring order.
template <class F, int OP>
__device__ __forceinline__ typename F::Acc fold_elem(const void* const* send, int c, int n, uint64_t i)
{
    typename F::Acc acc = F::ld(send[c], i);
    for (int k = 1; k < n; ++k) acc = combine<OP>(F::ld(send[wrap_rank(c + k, n)], i), acc);
    return acc;
}

// Two 16-byte vectors of every rank, at byte offsets off[0] and off[1] past
// the rank pointers (ok[u] says which exist), folded in ring order from rank
// c and finalized into out[0] and out[1], for a rank count n known only at
// run time. The ranks go in batches of 8; each batch issues its loads for
// both vectors (16 in flight per thread) before combining them in order
// (measured 3-5% faster than one vector at a time at 16-64 ranks).
template <class F, int OP, bool NT>
__device__ __forceinline__ void fold_pair_any(const void* const* send, int c, int n, const uint64_t (&off)[2],
                                              const bool (&ok)[2], u32x4 (&out)[2])
{
    using Acc = typename F::Acc;
    constexpr int E = F::kEpv;
    Acc acc[2][E];
#pragma unroll
    for (int u = 0; u < 2; ++u)
        if (ok[u]) F::unpack(ldv_at<NT>(send[c], off[u]), acc[u]);
    for (int k = 1; k < n; k += 8) {
        const int b = min(8, n - k);
        u32x4 x[2][8];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (ok[u] && j < b) x[u][j] = ldv_at<NT>(send[wrap_rank(c + k + j, n)], off[u]);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (ok[u] && j < b) {
                    Acc t[E];
                    F::unpack(x[u][j], t);
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[u][e] = combine<OP>(t[e], acc[u][e]);
                }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
        if (ok[u]) {
#pragma unroll
            for (int j = 0; j < E; ++j) acc[u][j] = finalize<OP>(acc[u][j], n);
            out[u] = F::pack(acc[u]);
        }
}

// Per-row rotation of the fused sweep, in tiles (odd, not a power of two).
constexpr uint64_t kRowSkewTiles = 37;

// The NR vectors of one element group, loaded in fold order (the chunk's
// first rank first): combined in that order, finalized, packed.
template <class F, int OP, int NR>
__device__ __forceinline__ u32x4 fold_loaded(const u32x4 (&x)[NR])
{
    using Acc = typename F::Acc;
    constexpr int E = F::kEpv;
    Acc acc[E];
    F::unpack(x[0], acc);
#pragma unroll
    for (int k = 1; k < NR; ++k) {
        Acc t[E];
        F::unpack(x[k], t);
#pragma unroll
        for (int j = 0; j < E; ++j) acc[j] = combine<OP>(t[j], acc[j]);
    }
#pragma unroll
    for (int j = 0; j < E; ++j) acc[j] = finalize<OP>(acc[j], NR);
    return F::pack(acc);
}

// Body of the fused kernel for NR ranks known at compile time: tiles t and
// t + G (G = gridDim.x) per iteration, rotated by `rot`, with all 2*NR loads
// issued before either fold (twice the reads in flight per thread; measured
// +2-6% for the reduce-scatter, +0.3-1 points for the all-reduce). Tile t
// covers vectors [org + t kBlock, org + (t+1) kBlock), clipped to the
// chunk's [v0, v1). SCATTER writes chunk c to recv[c] at v - v0, else every
// rank at v.
template <class F, int OP, int NR, bool SCATTER, bool NT>
__device__ __forceinline__ void fused_x2(const ReduceArgs& a, int c, uint64_t org, uint64_t v0, uint64_t v1,
                                         uint64_t ntiles, uint64_t rot)
{
    const uint64_t G = gridDim.x;
    const void* sp[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) sp[k] = a.send[wrap_rank(c + k, NR)];
    for (uint64_t t = blockIdx.x; t < ntiles; t += 2 * G) {
        uint64_t vv[2];
        bool ok[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint64_t tu = t + u * G;
            const uint64_t tr = tu + rot < ntiles ? tu + rot : tu + rot - ntiles;
            vv[u] = org + tr * kBlock + threadIdx.x;
            ok[u] = tu < ntiles && vv[u] >= v0 && vv[u] < v1;
        }
        u32x4 x[2][NR];
#pragma unroll
        for (int u = 0; u < 2; ++u)
            if (ok[u]) {
#pragma unroll
                for (int k = 0; k < NR; ++k) x[u][k] = ldv_at<NT>(sp[k], vv[u] * 16);
            }
#pragma unroll
        for (int u = 0; u < 2; ++u)
            if (ok[u]) {
                const u32x4 out = fold_loaded<F, OP, NR>(x[u]);
                if constexpr (SCATTER) {
                    stv<NT>(a.recv[c], vv[u] - v0, out);
                } else {
#pragma unroll
                    for (int r = 0; r < NR; ++r) stv<NT>(a.recv[r], vv[u], out);
                }
            }
    }
}


// Rank-major body of the fused reduction (NR ranks known at compile time): a
// thread takes M consecutive tiles per grid-stride step and folds them one
// rank at a time in ring order, so each stage reads M vectors from one rank
// buffer (a workgroup streams M * 4 KiB contiguous from it). The next rank's
// loads are issued before the current rank's combine, but the copy of the
// next rank's registers into the current ones makes each stage wait for its
// loads, so a wave has one stage (M loads) in flight at a time; the other
// waves of the CU (96 VGPRs: five per SIMD) cover the latency. A variant
// with a real prefetch distance of 1-3 stages held 120-130 VGPRs and ran
// 2-6% slower at 8 ranks x 64 MiB-1 GiB. Then the M results go to every rank
// (all-reduce) or to the chunk's output block (SCATTER). Each element's fold
// is the ring order of the two-tile body. The reduce-scatter takes it at 5-8
// ranks: +9 points at 256 MiB in per rank, +3.7 at 1 GiB, +1.5 at 14 GB
// against the two-tile body on the same buffers (at 8 workgroups per CU).
// The all-reduce takes the pipelined run-time body below at every rank
// count, which measured faster than this one at 8 ranks once launched with
// one workgroup per super tile.
template <class F, int OP, int NR, bool NT, int M, bool SCATTER = false>
__device__ __forceinline__ void fused_rank_major(const ReduceArgs& a, int c, uint64_t org, uint64_t v0, uint64_t v1,
                                                 uint64_t ntiles, uint64_t rot)
{
    using Acc = typename F::Acc;
    constexpr int E = F::kEpv;
    const uint64_t G = gridDim.x;
    const uint64_t nsup = (ntiles + M - 1) / M;
    const uint64_t srot = nsup ? (rot / M) % nsup : 0;
    const void* sp[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) sp[k] = a.send[wrap_rank(c + k, NR)];
    for (uint64_t st = blockIdx.x; st < nsup; st += G) {
        const uint64_t sr = st + srot < nsup ? st + srot : st + srot - nsup;
        uint64_t vv[M];
        bool ok[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const uint64_t tile = sr * M + m;
            vv[m] = org + tile * kBlock + threadIdx.x;
            ok[m] = tile < ntiles && vv[m] >= v0 && vv[m] < v1;
        }
        Acc acc[M][E];
        u32x4 xc[M], xn[M];
#pragma unroll
        for (int m = 0; m < M; ++m)
            if (ok[m]) xc[m] = ldv_at<NT>(sp[0], vv[m] * 16);
#pragma unroll
        for (int k = 1; k <= NR; ++k) {
            // xc holds rank k-1 in fold order; load rank k before combining it
            if (k < NR) {
#pragma unroll
                for (int m = 0; m < M; ++m)
                    if (ok[m]) xn[m] = ldv_at<NT>(sp[k], vv[m] * 16);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < M; ++m)
                if (ok[m]) {
                    if (k == 1) {
                        F::unpack(xc[m], acc[m]);
                    } else {
                        Acc t[E];
                        F::unpack(xc[m], t);
#pragma unroll
                        for (int j = 0; j < E; ++j) acc[m][j] = combine<OP>(t[j], acc[m][j]);
                    }
                }
            __builtin_amdgcn_sched_barrier(0);
            if (k < NR) {
#pragma unroll
                for (int m = 0; m < M; ++m) xc[m] = xn[m];
            }
        }
#pragma unroll
        for (int m = 0; m < M; ++m)
            if (ok[m]) {
#pragma unroll
                for (int j = 0; j < E; ++j) acc[m][j] = finalize<OP>(acc[m][j], NR);
                xc[m] = F::pack(acc[m]);
                if constexpr (SCATTER) stv<NT>(a.recv[c], vv[m] - v0, xc[m]);
            }
        if constexpr (!SCATTER) {
            // rank by rank: the M results go to one buffer back to back
            // (+0.6 to +1.3 points at 8 x 1 GiB against tile by tile)
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int m = 0; m < M; ++m)
                    if (ok[m]) stv<NT>(a.recv[r], vv[m], xc[m]);
        }
    }
}

// The M vectors of one rank folded into the accumulators (ring order:
// incoming (+) the partial so far, as the two-tile body does).
template <class F, int OP, int M>
__device__ __forceinline__ void fold_stage(const u32x4 (&x)[M], typename F::Acc (&acc)[M][F::kEpv])
{
    using Acc = typename F::Acc;
    constexpr int E = F::kEpv;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        Acc t[E];
        F::unpack(x[m], t);
#pragma unroll
        for (int j = 0; j < E; ++j) acc[m][j] = combine<OP>(t[j], acc[m][j]);
    }
}

template <int M, bool NT>
__device__ __forceinline__ void load_stage(u32x4 (&x)[M], const void* p, const uint64_t (&off)[M])
{
#pragma unroll
    for (int m = 0; m < M; ++m) x[m] = ldv_at<NT>(p, off[m]);
}

// Rank-major body for a rank count known only at run time: the super tile
// (M consecutive tiles) is folded one rank at a time in ring order, as in
// fused_rank_major, with two register sets that alternate between ranks, so
// one rank's M loads stay in flight while the previous rank is combined
// (the combine waits only for its own, older loads). The loads are
// unconditional: lanes past the chunk read its first vector and drop it,
// which keeps control flow out of the load-combine sequence (a guarded load
// there makes every combine wait for all loads). The next rank's pointer is
// fetched one stage ahead. Scheduling barriers pin the order. Measured
// against the batched fold (fold_pair_any) on the same buffers, fp32:
// +4 to +6% at 64 ranks x 256 MiB, +0.5 to +6% at 9-48 ranks x 256 MiB,
// +9% at 16 ranks x 64 MiB; at 4 ranks x 256 MiB +6.6% over the two-tile
// body.
// The fold of fused_rank_major_any: M vectors per rank at byte offsets off
// (every one readable) from the n ranks send[c], send[c+1], ... (mod n),
// into acc, ring order.
template <class F, int OP, bool NT, int M>
__device__ __forceinline__ void fold_rank_major_any(const void* const* send, int c, int n, const uint64_t (&off)[M],
                                                    typename F::Acc (&acc)[M][F::kEpv])
{
    u32x4 xa[M], xb[M];
    int r = c;
    const void* p = send[r];
    load_stage<M, NT>(xa, p, off);
    r = r + 1 == n ? 0 : r + 1;
    p = send[r];
    if (n > 1) {
        load_stage<M, NT>(xb, p, off);
        r = r + 1 == n ? 0 : r + 1;
        p = send[r];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < M; ++m) F::unpack(xa[m], acc[m]);
    __builtin_amdgcn_sched_barrier(0);
    int k = 1;  // xb holds fold position k (rank c + k)
    for (; k + 2 < n; k += 2) {
        load_stage<M, NT>(xa, p, off);
        r = r + 1 == n ? 0 : r + 1;
        p = send[r];
        __builtin_amdgcn_sched_barrier(0);
        fold_stage<F, OP, M>(xb, acc);
        __builtin_amdgcn_sched_barrier(0);
        load_stage<M, NT>(xb, p, off);
        r = r + 1 == n ? 0 : r + 1;
        p = send[r];
        __builtin_amdgcn_sched_barrier(0);
        fold_stage<F, OP, M>(xa, acc);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (k < n) {
        if (k + 1 < n) {
            load_stage<M, NT>(xa, p, off);
            __builtin_amdgcn_sched_barrier(0);
            fold_stage<F, OP, M>(xb, acc);
            __builtin_amdgcn_sched_barrier(0);
            fold_stage<F, OP, M>(xa, acc);
        } else {
            fold_stage<F, OP, M>(xb, acc);
        }
    }
}

template <class F, int OP, bool NT, int M, bool SCATTER>
__device__ __forceinline__ void fused_rank_major_any(const ReduceArgs& a, int c, uint64_t org, uint64_t v0,
                                                     uint64_t v1, uint64_t ntiles, uint64_t rot)
{
    using Acc = typename F::Acc;
    constexpr int E = F::kEpv;
    const int n = a.n;
    const uint64_t G = gridDim.x;
    const uint64_t nsup = (ntiles + M - 1) / M;
    const uint64_t srot = nsup ? (rot / M) % nsup : 0;
    for (uint64_t st = blockIdx.x; st < nsup; st += G) {
        const uint64_t sr = st + srot < nsup ? st + srot : st + srot - nsup;
        uint64_t vv[M], off[M];
        bool ok[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const uint64_t tile = sr * M + m;
            vv[m] = org + tile * kBlock + threadIdx.x;
            ok[m] = tile < ntiles && vv[m] >= v0 && vv[m] < v1;
            off[m] = (ok[m] ? vv[m] : v0) * 16;
        }
        Acc acc[M][E];
        fold_rank_major_any<F, OP, NT, M>(a.send, c, n, off, acc);
        u32x4 xa[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
#pragma unroll
            for (int j = 0; j < E; ++j) acc[m][j] = finalize<OP>(acc[m][j], n);
            xa[m] = F::pack(acc[m]);
        }
        if constexpr (SCATTER) {
#pragma unroll
            for (int m = 0; m < M; ++m)
                if (ok[m]) stv<NT>(a.recv[c], vv[m] - v0, xa[m]);
        } else {
            // rank by rank: M * 4 KiB back to back into each output buffer
            for (int rr = 0; rr < n; ++rr)
#pragma unroll
                for (int m = 0; m < M; ++m)
                    if (ok[m]) stv_at<NT>(a.recv[rr], off[m], xa[m]);
        }
    }
}

// RM > 0 selects a rank-major body with RM tiles per super tile: for NR
// ranks known at compile time (fused_rank_major) or, with NR = 0, at run
// time (fused_rank_major_any). Each is its own kernel, so its registers do
// not lower the occupancy of the two-tile one.
template <class F, int OP, int NR, bool SCATTER, bool NT, int RM = 0>
__global__ __launch_bounds__(kBlock) void fused_reduce_vec(const ReduceArgs a)
{
    using Acc = typename F::Acc;
    constexpr int E = F::kEpv;
    const int n = NR > 0 ? NR : a.n;
    const int c = blockIdx.y;
    uint64_t lo, hi;
    chunk_range(a.q, a.count, c, lo, hi);
    // The chunk's whole 16-byte vectors: every rank pointer is 16-byte
    // aligned, so vector v holds elements [vE, vE + E) of every buffer. A
    // chunk that starts or ends inside a vector (q not a multiple of E) has
    // fewer than E head and tail elements, done one by one below. The
    // reduce-scatter layout (SCATTER) needs q % E == 0, which the host checks.
    const uint64_t v0 = (lo + E - 1) / E;
    const uint64_t v1 = hi / E;
    const uint64_t nv = v1 > v0 ? v1 - v0 : 0;
    // Tiles of kBlock vectors, grid-strided per chunk row. All-reduce tiles
    // are the buffer's aligned 4 KiB blocks, so a wave's 1 KiB never
    // straddles an extra cache line (the chunk's first and last tiles may be
    // partial); the reduce-scatter layout counts tiles from the chunk start,
    // where its output block begins. Row c starts its sweep rotated by
    // c * kRowSkewTiles tiles: when chunk and rank buffers sit at
    // power-of-two distances, rows that move in lock step would otherwise hit
    // the same HBM banks at the same time (measured +1% with separate rank
    // allocations, +4% with rank buffers at 256 MiB strides in one
    // allocation). Each element's fold is unchanged.
    const uint64_t org = SCATTER ? v0 : v0 / kBlock * kBlock;
    const uint64_t ntiles = nv ? (v1 - 1 - org) / kBlock + 1 : 0;
    const uint64_t rot = ntiles ? (static_cast<uint64_t>(c) * kRowSkewTiles) % ntiles : 0;
    if constexpr (RM > 0 && NR > 0) {
        fused_rank_major<F, OP, NR, NT, RM, SCATTER>(a, c, org, v0, v1, ntiles, rot);
    } else if constexpr (RM > 0) {
        fused_rank_major_any<F, OP, NT, RM, SCATTER>(a, c, org, v0, v1, ntiles, rot);
    } else if constexpr (NR > 0) {
        fused_x2<F, OP, NR, SCATTER, NT>(a, c, org, v0, v1, ntiles, rot);
    } else {
        // tiles t and t + G per iteration, as fused_x2 does
        const uint64_t G = gridDim.x;
        for (uint64_t t = blockIdx.x; t < ntiles; t += 2 * G) {
            uint64_t vv[2], off[2];
            bool ok[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint64_t tu = t + u * G;
                const uint64_t tr = tu + rot < ntiles ? tu + rot : tu + rot - ntiles;
                vv[u] = org + tr * kBlock + threadIdx.x;
                off[u] = vv[u] * 16;
                ok[u] = tu < ntiles && vv[u] >= v0 && vv[u] < v1;
            }
            u32x4 out[2];
            fold_pair_any<F, OP, NT>(a.send, c, n, off, ok, out);
#pragma unroll
            for (int u = 0; u < 2; ++u)
                if (ok[u]) {
                    if constexpr (SCATTER) {
                        stv<NT>(a.recv[c], vv[u] - v0, out[u]);
                    } else {
                        for (int r = 0; r < n; ++r) stv<NT>(a.recv[r], vv[u], out[u]);
                    }
                }
        }
    }
    // Head [lo, v0 E) and tail [v1 E, hi): fewer than E elements each.
    if (blockIdx.x == 0) {
        const uint64_t head_end = v0 * E < hi ? v0 * E : hi;
        const uint64_t nhead = head_end - lo;
        const uint64_t tail_start = v1 * E > head_end ? v1 * E : head_end;
        const uint64_t ntail = hi - tail_start;
        if (threadIdx.x < nhead + ntail) {
            const uint64_t i = threadIdx.x < nhead ? lo + threadIdx.x : tail_start + (threadIdx.x - nhead);
            const Acc x = finalize<OP>(fold_elem<F, OP>(a.send, c, n, i), n);
            if constexpr (SCATTER) {
                F::st(a.recv[c], i - lo, x);
            } else {
                for (int r = 0; r < n; ++r) F::st(a.recv[r], i, x);
            }
        }
    }
}

// Element-wise variant for buffers that are not 16-byte aligned or chunks that
// do not start on a vector boundary.
template <class F, int OP, bool SCATTER>
__global__ __launch_bounds__(kBlock) void fused_reduce_scalar(const ReduceArgs a)
{
    const int n = a.n;
    const int c = blockIdx.y;
    uint64_t lo, hi;
    chunk_range(a.q, a.count, c, lo, hi);
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    for (uint64_t i = lo + static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x; i < hi; i += stride) {
        const typename F::Acc x = finalize<OP>(fold_elem<F, OP>(a.send, c, n, i), n);
        if constexpr (SCATTER) {
            F::st(a.recv[c], i - lo, x);
        } else {
            for (int r = 0; r < n; ++r) F::st(a.recv[r], i, x);
        }
    }
}

// ---------------------------------------------------------------------------
// fused all-gather: block p of send[p] -> recv[r] + p*blk for every r
// ---------------------------------------------------------------------------
// RM: each thread copies kRankMajorTiles consecutive 4 KiB tiles per
// grid-stride step and stores them rank by rank, so a workgroup writes 16 KiB
// back to back into one output buffer (measured +1 to +7.4 points at 512 MiB
// to 1.75 GB of input per rank at 8 ranks, 1-4 points slower at 64-256 MiB).
template <bool VEC, bool NT, bool RM = false>
__global__ __launch_bounds__(kBlock) void fused_gather(const CopyArgs a)
{
    const int p = blockIdx.y;
    const uint64_t blk = a.total;
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    const uint64_t t0 = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if constexpr (RM) {
        static_assert(VEC, "the rank-major copy takes 16-byte vectors");
        constexpr int M = kRankMajorTiles;
        const uint64_t nv = blk / 16, o = p * blk / 16;
        const uint64_t nsup = (nv + M * kBlock - 1) / (M * kBlock);
        for (uint64_t st = blockIdx.x; st < nsup; st += gridDim.x) {
            u32x4 x[M];
            uint64_t vv[M];
            bool ok[M];
#pragma unroll
            for (int m = 0; m < M; ++m) {
                vv[m] = (st * M + m) * kBlock + threadIdx.x;
                ok[m] = vv[m] < nv;
                x[m] = ldv<NT>(a.send[p], ok[m] ? vv[m] : 0);  // lanes past the block reload vector 0
            }
            for (int r = 0; r < a.n; ++r)
#pragma unroll
                for (int m = 0; m < M; ++m)
                    if (ok[m]) stv<NT>(a.recv[r], o + vv[m], x[m]);
        }
    } else if constexpr (VEC) {
        const uint64_t nv = blk / 16, o = p * blk / 16;
        for (uint64_t v = t0; v < nv; v += stride) {
            const u32x4 x = ldv<NT>(a.send[p], v);
            for (int r = 0; r < a.n; ++r) stv<NT>(a.recv[r], o + v, x);
        }
    } else {
        const uint64_t nh = blk / 2, o = p * blk / 2;
        const uint16_t* src = static_cast<const uint16_t*>(a.send[p]);
        for (uint64_t h = t0; h < nh; h += stride) {
            const uint16_t x = src[h];
            for (int r = 0; r < a.n; ++r) static_cast<uint16_t*>(a.recv[r])[o + h] = x;
        }
    }
}

// ---------------------------------------------------------------------------
// ring-stepwise mode
// ---------------------------------------------------------------------------
// Accumulator slots in the workspace are 32-bit patterns. The conversions
// take their operand by value: bit-casting a vector element in place (w.y)
// is compiled as a read of the vector's first element.
__device__ __forceinline__ void from_bits(uint32_t u, float& out) { out = as_f(u); }
__device__ __forceinline__ void from_bits(uint32_t u, uint32_t& out) { out = u; }
__device__ __forceinline__ uint32_t to_bits(float v) { return as_u(v); }
__device__ __forceinline__ uint32_t to_bits(uint32_t v) { return v; }

template <class F>
__device__ __forceinline__ void ws_load(const void* ws, uint64_t i, typename F::Acc* acc)
{
    constexpr int E = F::kEpv;
#pragma unroll
    for (int j = 0; j < E / 4; ++j) {
        const u32x4 w = ld16(ws, i / 4 + j);
        from_bits(w.x, acc[4 * j + 0]);
        from_bits(w.y, acc[4 * j + 1]);
        from_bits(w.z, acc[4 * j + 2]);
        from_bits(w.w, acc[4 * j + 3]);
    }
}

template <class F>
__device__ __forceinline__ void ws_store(void* ws, uint64_t i, const typename F::Acc* acc)
{
    constexpr int E = F::kEpv;
#pragma unroll
    for (int j = 0; j < E / 4; ++j) {
        const u32x4 w{to_bits(acc[4 * j + 0]), to_bits(acc[4 * j + 1]), to_bits(acc[4 * j + 2]),
                      to_bits(acc[4 * j + 3])};
        st16(ws, i / 4 + j, w);
    }
}

// One element of a reduce-scatter step at rank r (chunk c, left neighbour).
template <class F, int OP>
__device__ __forceinline__ void rs_elem(const StepArgs& a, int r, int left, int c, uint64_t lo, uint64_t i)
{
    using Acc = typename F::Acc;
    const Acc local = F::ld(a.send[r], i);
    Acc in;
    if (a.first) in = F::ld(a.send[left], i);
    else if (a.ws) from_bits(static_cast<const uint32_t*>(a.ws)[i], in);
    else in = F::ld(a.recv[left], i);
    Acc v = combine<OP>(local, in);
    if (a.last) {
        v = finalize<OP>(v, a.n);
        if (a.scatter) F::st(a.recv[c], i - lo, v);
        else F::st(a.recv[r], i, v);
    } else if (a.ws) {
        static_cast<uint32_t*>(a.ws)[i] = to_bits(v);
    } else {
        F::st(a.recv[r], i, v);
    }
}

// Reduce-scatter step s [handbook "集合通信原语", section 环形 all-reduce 与通信量]:
// every rank r combines chunk (r - s - 1) mod n of its own input with the
// partial arriving from rank r-1. grid = (blocks, n ranks). The chunks a step
// writes (rank r, chunk c) and reads from the left (rank r-1, chunk c) are
// disjoint from what rank r-1 writes in the same step (its chunk c-1), so no
// staging buffer is needed.
// The tiled form of a reduce-scatter step's whole vectors: a thread takes M
// vectors a kBlock apart per tile, issues all their loads (local, incoming)
// before combining, and the host launches one workgroup per tile, so the
// resident workgroups move through each rank's chunk in order.
template <class F, int OP, bool NT, int M>
__device__ __forceinline__ void rs_step_tiles(const StepArgs& a, int r, int left, int c, uint64_t v0, uint64_t nv)
{
    using Acc = typename F::Acc;
    constexpr int E = F::kEpv;
    constexpr int W = E / 4;  // 16-byte workspace vectors per element vector (fp32 partials)
    const int n = a.n;
    const uint64_t ntiles = (nv + M * kBlock - 1) / (M * kBlock);
    for (uint64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        uint64_t vi[M];
        bool ok[M];
        u32x4 xl[M], xi[M][W];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const uint64_t v = (t * M + m) * kBlock + threadIdx.x;
            ok[m] = v < nv;
            vi[m] = v0 + (ok[m] ? v : 0);  // lanes past the chunk reload its first vector
            xl[m] = ldv<NT>(a.send[r], vi[m]);
        }
        const bool from_ws = !a.first && a.ws;
        if (a.first) {
#pragma unroll
            for (int m = 0; m < M; ++m) xi[m][0] = ldv<NT>(a.send[left], vi[m]);
        } else if (from_ws) {
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int j = 0; j < W; ++j) xi[m][j] = ldv<NT>(a.ws, vi[m] * W + j);
        } else {
#pragma unroll
            for (int m = 0; m < M; ++m) xi[m][0] = ldv<NT>(a.recv[left], vi[m]);
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            if (!ok[m]) continue;
            Acc loc[E], in[E];
            F::unpack(xl[m], loc);
            if (from_ws) {
#pragma unroll
                for (int j = 0; j < W; ++j) {
                    from_bits(xi[m][j].x, in[4 * j + 0]);
                    from_bits(xi[m][j].y, in[4 * j + 1]);
                    from_bits(xi[m][j].z, in[4 * j + 2]);
                    from_bits(xi[m][j].w, in[4 * j + 3]);
                }
            } else {
                F::unpack(xi[m][0], in);
            }
#pragma unroll
            for (int j = 0; j < E; ++j) loc[j] = combine<OP>(loc[j], in[j]);
            if (a.last) {
#pragma unroll
                for (int j = 0; j < E; ++j) loc[j] = finalize<OP>(loc[j], n);
                if (a.scatter) stv<NT>(a.recv[c], vi[m] - v0, F::pack(loc));
                else stv<NT>(a.recv[r], vi[m], F::pack(loc));
            } else if (a.ws) {
#pragma unroll
                for (int j = 0; j < W; ++j) {
                    const u32x4 w{to_bits(loc[4 * j + 0]), to_bits(loc[4 * j + 1]), to_bits(loc[4 * j + 2]),
                                  to_bits(loc[4 * j + 3])};
                    stv<NT>(a.ws, vi[m] * W + j, w);
                }
            } else {
                stv<NT>(a.recv[r], vi[m], F::pack(loc));
            }
        }
    }
}

// The tiled step for the 16-bit types, whose partials between steps are fp32
// in the workspace (16 bytes per 8 bytes of data; workspace vector 2v + h
// holds elements 4h..4h+3 of data vector v). The threads take half vectors:
// 2M per thread and tile, lane l of a wave half l of each run of 64, so each
// load and store instruction of a wave covers one contiguous run (512 bytes of
// data, 1 KiB of partials). With a whole data vector per lane, each of its two
// partial loads would cover every other 16 bytes of 2 KiB. Each element's
// arithmetic is that of rs_step_tiles.
template <class F, int OP, bool NT, int M>
__device__ __forceinline__ void rs_step_halves(const StepArgs& a, int r, int left, int c, uint64_t v0, uint64_t nv)
{
    using Acc = typename F::Acc;
    constexpr int H = 2 * M;
    const int n = a.n;
    const uint64_t h0 = 2 * v0, nh = 2 * nv;
    const uint64_t ntiles = (nh + H * kBlock - 1) / (H * kBlock);
    const bool from_ws = !a.first && a.ws;
    for (uint64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        uint64_t hv[H];
        bool ok[H];
        u32x2 xl[H], xi[H];
        u32x4 xw[H];
#pragma unroll
        for (int m = 0; m < H; ++m) {
            const uint64_t h = (t * H + m) * kBlock + threadIdx.x;
            ok[m] = h < nh;
            hv[m] = h0 + (ok[m] ? h : 0);  // lanes past the chunk reload its first half vector
            xl[m] = ldh<NT>(a.send[r], hv[m]);
        }
        if (from_ws) {
#pragma unroll
            for (int m = 0; m < H; ++m) xw[m] = ldv<NT>(a.ws, hv[m]);
        } else {
            const void* src = a.first ? a.send[left] : a.recv[left];
#pragma unroll
            for (int m = 0; m < H; ++m) xi[m] = ldh<NT>(src, hv[m]);
        }
#pragma unroll
        for (int m = 0; m < H; ++m) {
            if (!ok[m]) continue;
            Acc loc[4], in[4];
            F::unpack4(xl[m], loc);
            if (from_ws) {
                from_bits(xw[m].x, in[0]);
                from_bits(xw[m].y, in[1]);
                from_bits(xw[m].z, in[2]);
                from_bits(xw[m].w, in[3]);
            } else {
                F::unpack4(xi[m], in);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) loc[j] = combine<OP>(loc[j], in[j]);
            if (a.last) {
#pragma unroll
                for (int j = 0; j < 4; ++j) loc[j] = finalize<OP>(loc[j], n);
                if (a.scatter) sth<NT>(a.recv[c], hv[m] - h0, F::pack4(loc));
                else sth<NT>(a.recv[r], hv[m], F::pack4(loc));
            } else if (a.ws) {
                stv<NT>(a.ws, hv[m], u32x4{to_bits(loc[0]), to_bits(loc[1]), to_bits(loc[2]), to_bits(loc[3])});
            } else {
                sth<NT>(a.recv[r], hv[m], F::pack4(loc));
            }
        }
    }
}

// M = 0: one vector per thread per grid-stride step; M > 0: rs_step_tiles
// (rs_step_halves for the 16-bit types; 16-byte vectors only), NT selecting
// non-temporal access.
template <class F, int OP, bool VEC, bool NT = false, int M = 0>
__global__ __launch_bounds__(kBlock) void rs_step(const StepArgs a)
{
    using Acc = typename F::Acc;
    constexpr int E = F::kEpv;
    const int n = a.n;
    const int r = blockIdx.y;
    const int left = r == 0 ? n - 1 : r - 1;
    int c = (r - a.s - 1) % n;
    if (c < 0) c += n;
    uint64_t lo, hi;
    chunk_range(a.q, a.count, c, lo, hi);
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    const uint64_t t0 = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if constexpr (VEC) {
        // The chunk's whole 16-byte vectors (rank pointers and the workspace
        // are 16-byte aligned); the < E elements before the first and after
        // the last are done one by one. The reduce-scatter layout (scatter)
        // needs q % E == 0, which the host checks.
        const uint64_t v0 = (lo + E - 1) / E, v1 = hi / E;
        const uint64_t nv = v1 > v0 ? v1 - v0 : 0;
        if constexpr (M > 0 && F::kEpv == 8) rs_step_halves<F, OP, NT, M>(a, r, left, c, v0, nv);
        else if constexpr (M > 0) rs_step_tiles<F, OP, NT, M>(a, r, left, c, v0, nv);
        for (uint64_t v = t0; M == 0 && v < nv; v += stride) {
            const uint64_t vi = v0 + v;
            Acc loc[E], in[E];
            F::unpack(ld16(a.send[r], vi), loc);
            if (a.first) F::unpack(ld16(a.send[left], vi), in);
            else if (a.ws) ws_load<F>(a.ws, vi * E, in);
            else F::unpack(ld16(a.recv[left], vi), in);
#pragma unroll
            for (int j = 0; j < E; ++j) loc[j] = combine<OP>(loc[j], in[j]);
            if (a.last) {
#pragma unroll
                for (int j = 0; j < E; ++j) loc[j] = finalize<OP>(loc[j], n);
                if (a.scatter) st16(a.recv[c], v, F::pack(loc));
                else st16(a.recv[r], vi, F::pack(loc));
            } else if (a.ws) {
                ws_store<F>(a.ws, vi * E, loc);
            } else {
                st16(a.recv[r], vi, F::pack(loc));
            }
        }
        if (blockIdx.x == 0) {
            const uint64_t head_end = v0 * E < hi ? v0 * E : hi;
            const uint64_t nhead = head_end - lo;
            const uint64_t tail_start = v1 * E > head_end ? v1 * E : head_end;
            const uint64_t ntail = hi - tail_start;
            if (threadIdx.x < nhead + ntail)
                rs_elem<F, OP>(a, r, left, c, lo,
                               threadIdx.x < nhead ? lo + threadIdx.x : tail_start + (threadIdx.x - nhead));
        }
    } else {
        for (uint64_t i = lo + t0; i < hi; i += stride) rs_elem<F, OP>(a, r, left, c, lo, i);
    }
}

// Copy step s of a ring: rank r copies chunk (r - s - shift) mod n from rank
// r-1 (all-gather phase [handbook, section 环形 all-reduce 与通信量]).
// M = 0: one vector per thread per grid-stride step; M > 0 (16-byte vectors
// only): M vectors a kBlock apart per thread and tile, loads before stores,
// one workgroup per tile; NT selects non-temporal access.
template <bool VEC, bool NT = false, int M = 0>
__global__ __launch_bounds__(kBlock) void copy_step(const CopyArgs a)
{
    const int n = a.n;
    const int r = blockIdx.y;
    const int left = r == 0 ? n - 1 : r - 1;
    int c = (r - a.s - a.shift) % n;
    if (c < 0) c += n;
    uint64_t lo, hi;
    chunk_range(a.qb, a.total, c, lo, hi);
    const char* src = static_cast<const char*>(a.recv[left]);
    char* dst = static_cast<char*>(a.recv[r]);
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    const uint64_t t0 = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if constexpr (VEC) {
        // whole 16-byte vectors of the chunk, then the < 16 bytes before and
        // after them in 2-byte units (chunk ends are multiples of the element
        // size, at least 2)
        const uint64_t v0 = (lo + 15) / 16, v1 = hi / 16;
        const uint64_t nv = v1 > v0 ? v1 - v0 : 0;
        if constexpr (M > 0) {
            const uint64_t ntiles = (nv + M * kBlock - 1) / (M * kBlock);
            for (uint64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
                u32x4 x[M];
                uint64_t vv[M];
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    vv[m] = (t * M + m) * kBlock + threadIdx.x;
                    x[m] = ldv<NT>(src, v0 + (vv[m] < nv ? vv[m] : 0));  // lanes past the chunk reload its first vector
                }
#pragma unroll
                for (int m = 0; m < M; ++m)
                    if (vv[m] < nv) stv<NT>(dst, v0 + vv[m], x[m]);
            }
        } else {
            for (uint64_t v = t0; v < nv; v += stride) st16(dst, v0 + v, ld16(src, v0 + v));
        }
        if (blockIdx.x != 0) return;
        const uint64_t head_end = v0 * 16 < hi ? v0 * 16 : hi;
        const uint64_t tail_start = v1 * 16 > head_end ? v1 * 16 : head_end;
        for (uint64_t b = lo + 2 * threadIdx.x; b < head_end; b += 2 * kBlock)
            *reinterpret_cast<uint16_t*>(dst + b) = *reinterpret_cast<const uint16_t*>(src + b);
        for (uint64_t b = tail_start + 2 * threadIdx.x; b < hi; b += 2 * kBlock)
            *reinterpret_cast<uint16_t*>(dst + b) = *reinterpret_cast<const uint16_t*>(src + b);
    } else {
        for (uint64_t b = lo + 2 * t0; b < hi; b += 2 * stride)
            *reinterpret_cast<uint16_t*>(dst + b) = *reinterpret_cast<const uint16_t*>(src + b);
    }
}

// send[r] -> recv[r] + r*dst_stride, `total` bytes per rank.
template <bool VEC>
__global__ __launch_bounds__(kBlock) void local_copy(const CopyArgs a)
{
    const int r = blockIdx.y;
    const char* src = static_cast<const char*>(a.send[r]);
    char* dst = static_cast<char*>(a.recv[r]) + static_cast<uint64_t>(r) * a.dst_stride;
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    const uint64_t t0 = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x;
    uint64_t done = 0;
    if constexpr (VEC) {
        const uint64_t nv = a.total / 16;
        for (uint64_t v = t0; v < nv; v += stride) st16(dst, v, ld16(src, v));
        done = nv * 16;
        if (blockIdx.x != 0) return;
        for (uint64_t b = done + 2 * threadIdx.x; b < a.total; b += 2 * kBlock)
            *reinterpret_cast<uint16_t*>(dst + b) = *reinterpret_cast<const uint16_t*>(src + b);
    } else {
        for (uint64_t b = 2 * t0; b < a.total; b += 2 * stride)
            *reinterpret_cast<uint16_t*>(dst + b) = *reinterpret_cast<const uint16_t*>(src + b);
    }
}

// ---------------------------------------------------------------------------
// tree variant [geek-doc "训练梯度同步与集合通信", section 六]: ranks combine
// in pairs, pair results combine in pairs again, the root ends with the
// reduction, which goes back down the tree. For element i the fold is the
// binomial tree over ranks 0..n-1: T(lo, hi) = T(lo, lo+P) (+) T(lo+P, hi),
// P the largest power of two below hi-lo. One thread evaluates it with a
// binary counter: slot[b] holds the partial of an aligned block of 2^b ranks;
// adding rank r carries through the slots whose bit is set in r (the lower
// ranks' block is the left operand), and the slots left at the end (the set
// bits of n) fold from the smallest block upward.
// ---------------------------------------------------------------------------
constexpr int kTreeSlots = 7;  // 2^6 = AR_MAX_RANKS

template <class F, int OP, int NR, bool NT>
__device__ __forceinline__ void tree_fold_vec(const ReduceArgs& a, int n, uint64_t vi, typename F::Acc* out)
{
    using Acc = typename F::Acc;
    constexpr int E = F::kEpv;
    constexpr int RMAX = NR > 0 ? NR : AR_MAX_RANKS;
    Acc slot[kTreeSlots][E];
#pragma unroll
    for (int rb = 0; rb < RMAX; rb += 8) {
        if (NR > 0 || rb < n) {
            u32x4 x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (rb + j < RMAX) x[j] = ldv<NT>(a.send[min(rb + j, n - 1)], vi);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int r = rb + j;  // compile-time after unrolling
                if (r < RMAX && (NR > 0 || r < n)) {
                    Acc carry[E];
                    F::unpack(x[j], carry);
                    int b = 0;
#pragma unroll
                    for (; b < kTreeSlots - 1; ++b) {
                        if (!((r >> b) & 1)) break;
#pragma unroll
                        for (int e = 0; e < E; ++e) carry[e] = combine<OP>(slot[b][e], carry[e]);
                    }
#pragma unroll
                    for (int e = 0; e < E; ++e) slot[b][e] = carry[e];
                }
            }
        }
    }
    bool have = false;
#pragma unroll
    for (int b = 0; b < kTreeSlots; ++b) {
        if ((n >> b) & 1) {
#pragma unroll
            for (int e = 0; e < E; ++e) out[e] = have ? combine<OP>(slot[b][e], out[e]) : slot[b][e];
            have = true;
        }
    }
}

template <class F, int OP>
__device__ __forceinline__ typename F::Acc tree_fold_elem(const ReduceArgs& a, int n, uint64_t i)
{
    using Acc = typename F::Acc;
    Acc slot[kTreeSlots];
#pragma unroll
    for (int r = 0; r < AR_MAX_RANKS; ++r) {
        if (r < n) {
            Acc carry = F::ld(a.send[r], i);
            int b = 0;
#pragma unroll
            for (; b < kTreeSlots - 1; ++b) {
                if (!((r >> b) & 1)) break;
                carry = combine<OP>(slot[b], carry);
            }
            slot[b] = carry;
        }
    }
    Acc out{};
    bool have = false;
#pragma unroll
    for (int b = 0; b < kTreeSlots; ++b) {
        if ((n >> b) & 1) {
            out = have ? combine<OP>(slot[b], out) : slot[b];
            have = true;
        }
    }
    return out;
}

// Fused tree all-reduce: 1-D grid-stride over 16-byte vectors of the whole
// buffer; every element takes the same tree order.
template <class F, int OP, int NR, bool NT>
__global__ __launch_bounds__(kBlock) void tree_fused_vec(const ReduceArgs a)
{
    using Acc = typename F::Acc;
    constexpr int E = F::kEpv;
    const int n = NR > 0 ? NR : a.n;
    const uint64_t nv = a.count / E;
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    for (uint64_t v = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x; v < nv; v += stride) {
        Acc acc[E];
        tree_fold_vec<F, OP, NR, NT>(a, n, v, acc);
#pragma unroll
        for (int j = 0; j < E; ++j) acc[j] = finalize<OP>(acc[j], n);
        const u32x4 out = F::pack(acc);
        for (int r = 0; r < n; ++r) stv<NT>(a.recv[r], v, out);
    }
    if (blockIdx.x == 0) {
        const uint64_t i = nv * E + threadIdx.x;
        if (i < a.count) {
            const Acc x = finalize<OP>(tree_fold_elem<F, OP>(a, n, i), n);
            for (int r = 0; r < n; ++r) F::st(a.recv[r], i, x);
        }
    }
}

template <class F, int OP>
__global__ __launch_bounds__(kBlock) void tree_fused_scalar(const ReduceArgs a)
{
    const int n = a.n;
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x; i < a.count; i += stride) {
        const typename F::Acc x = finalize<OP>(tree_fold_elem<F, OP>(a, n, i), n);
        for (int r = 0; r < n; ++r) F::st(a.recv[r], i, x);
    }
}

// Partial of rank x in the stepwise tree: recv[x] for fp32/int32 (storage =
// accumulator), fp32 workspace slot x/2 for fp16/bf16.
template <class F>
__device__ __forceinline__ typename F::Acc tree_partial_ld(const TreeArgs& a, int x, uint64_t i)
{
    typename F::Acc v;
    if (a.ws) from_bits(static_cast<const uint32_t*>(a.ws)[static_cast<uint64_t>(x / 2) * a.ws_stride + i], v);
    else v = F::ld(a.recv[x], i);
    return v;
}

template <class F>
__device__ __forceinline__ void tree_partial_st(const TreeArgs& a, int x, uint64_t i, typename F::Acc v)
{
    if (a.ws) static_cast<uint32_t*>(a.ws)[static_cast<uint64_t>(x / 2) * a.ws_stride + i] = to_bits(v);
    else F::st(a.recv[x], i, v);
}

template <class F, int OP>
__device__ __forceinline__ void tree_reduce_elem(const TreeArgs& a, int r, int q, uint64_t i)
{
    using Acc = typename F::Acc;
    // A rank holds a partial once it has received at level 0, i.e. when it
    // is even and has a right neighbour; r always has, q only if q+1 < n.
    const Acc local = a.stride == 1 ? F::ld(a.send[r], i) : tree_partial_ld<F>(a, r, i);
    const Acc in = (a.stride == 1 || q + 1 >= a.n) ? F::ld(a.send[q], i) : tree_partial_ld<F>(a, q, i);
    Acc v = combine<OP>(local, in);
    if (a.last) F::st(a.recv[0], i, finalize<OP>(v, a.n));
    else tree_partial_st<F>(a, r, i, v);
}

template <class F, int OP, bool VEC>
__global__ __launch_bounds__(kBlock) void tree_reduce_level(const TreeArgs a)
{
    using Acc = typename F::Acc;
    constexpr int E = F::kEpv;
    const int r = blockIdx.y * 2 * a.stride;
    const int q = r + a.stride;
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    const uint64_t t0 = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if constexpr (VEC) {
        const uint64_t nv = a.count / E;
        const bool local_partial = a.stride != 1, in_partial = a.stride != 1 && q + 1 < a.n;
        for (uint64_t v = t0; v < nv; v += stride) {
            Acc loc[E], in[E];
            if (!local_partial) F::unpack(ld16(a.send[r], v), loc);
            else if (a.ws) ws_load<F>(static_cast<const uint32_t*>(a.ws) + static_cast<uint64_t>(r / 2) * a.ws_stride, v * E, loc);
            else F::unpack(ld16(a.recv[r], v), loc);
            if (!in_partial) F::unpack(ld16(a.send[q], v), in);
            else if (a.ws) ws_load<F>(static_cast<const uint32_t*>(a.ws) + static_cast<uint64_t>(q / 2) * a.ws_stride, v * E, in);
            else F::unpack(ld16(a.recv[q], v), in);
#pragma unroll
            for (int j = 0; j < E; ++j) loc[j] = combine<OP>(loc[j], in[j]);
            if (a.last) {
#pragma unroll
                for (int j = 0; j < E; ++j) loc[j] = finalize<OP>(loc[j], a.n);
                st16(a.recv[0], v, F::pack(loc));
            } else if (a.ws) {
                ws_store<F>(static_cast<uint32_t*>(a.ws) + static_cast<uint64_t>(r / 2) * a.ws_stride, v * E, loc);
            } else {
                st16(a.recv[r], v, F::pack(loc));
            }
        }
        if (blockIdx.x == 0 && nv * E + threadIdx.x < a.count) tree_reduce_elem<F, OP>(a, r, q, nv * E + threadIdx.x);
    } else {
        for (uint64_t i = t0; i < a.count; i += stride) tree_reduce_elem<F, OP>(a, r, q, i);
    }
}

// Broadcast level: recv[q] = recv[r], count*elem bytes.
template <bool VEC>
__global__ __launch_bounds__(kBlock) void tree_bcast_level(const TreeArgs a, uint64_t bytes)
{
    const int r = blockIdx.y * 2 * a.stride;
    const int q = r + a.stride;
    const char* src = static_cast<const char*>(a.recv[r]);
    char* dst = static_cast<char*>(a.recv[q]);
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    const uint64_t t0 = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x;
    uint64_t done = 0;
    if constexpr (VEC) {
        const uint64_t nv = bytes / 16;
        for (uint64_t v = t0; v < nv; v += stride) st16_nt(dst, v, ld16(src, v));
        done = nv * 16;
        if (blockIdx.x != 0) return;
        for (uint64_t b = done + 2 * threadIdx.x; b < bytes; b += 2 * kBlock)
            *reinterpret_cast<uint16_t*>(dst + b) = *reinterpret_cast<const uint16_t*>(src + b);
    } else {
        for (uint64_t b = 2 * t0; b < bytes; b += 2 * stride)
            *reinterpret_cast<uint16_t*>(dst + b) = *reinterpret_cast<const uint16_t*>(src + b);
    }
}

// ---------------------------------------------------------------------------
// coalesced multi-tensor all-reduce: the tensors of each rank form one
// virtual flat bucket (concatenated in order), chunked as one buffer, so the
// bits equal a flat-bucket all-reduce, without packing copies
// ---------------------------------------------------------------------------
// The table (pointer blocks and pieces, in the kernel arguments) does not
// change while a kernel runs: it is read through the constant address space.
typedef __attribute__((address_space(4))) const unsigned char cbyte;
typedef __attribute__((address_space(4))) const MultiPiece cpiece;
typedef __attribute__((address_space(4))) const uintptr_t cuptr;

__device__ __forceinline__ MultiPiece load_piece(cpiece* p)
{
    MultiPiece r;
    r.j0 = p->j0;
    r.len = p->len;
    r.tile0 = p->tile0;
    r.ptrs = p->ptrs;
    r.chunk = p->chunk;
    r.flags = p->flags;
    return r;
}

__device__ __forceinline__ int multi_find_piece(cpiece* pieces, int npieces, uint32_t tile)
{
    int lo = 0, hi = npieces - 1;  // last piece whose first tile is <= tile
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pieces[mid].tile0 <= tile) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// One workgroup per tile (kBlock vectors, or kBlock elements for scalar
// pieces); a tile lies inside one piece, so the chunk (ring order) and the
// tensor (pointers) are uniform across the workgroup. A workgroup's tiles
// only increase, so after a binary search for its first tile it finds the
// next piece by scanning forward. NR > 0 fixes the rank count at compile time.
// RM > 0 (with NR = 0) selects the rank-major vector tile of RM
// kBlock-vector quarters (rank_major_any_tiles), folded one rank at a time by
// fold_rank_major_any as in the flat rank-major body.
template <class F, int OP, int NR, bool NT, int RM = 0>
__device__ __forceinline__ void multi_body(const MultiHeader& h, const unsigned char* table)
{
    using Acc = typename F::Acc;
    constexpr int E = F::kEpv;
    const int n = NR > 0 ? NR : h.n;
    // A grid smaller than the tile count splits the tiles into S equal
    // segments (S = rank count, like the flat kernel's chunk rows) and each
    // segment gets every S-th workgroup, which strides through it: the
    // workgroups in flight spread over the whole batch instead of one window
    // of it, and every segment has the same work. A grid of one workgroup per
    // tile takes the tiles in order (S = 1), as the flat rank-major kernels
    // take their super tiles.
    const uint32_t G = gridDim.x;
    const uint32_t S = G >= h.ntiles ? 1u : min(static_cast<uint32_t>(h.n), G);
    const uint32_t seg = blockIdx.x % S;
    const uint32_t step = G / S + (seg < G % S ? 1u : 0u);
    const uint32_t L = (h.ntiles + S - 1) / S;
    const uint32_t t_end = min(h.ntiles, (seg + 1) * L);
    const uint32_t t_first = seg * L + blockIdx.x / S;
    if (t_first >= t_end) return;
    cbyte* ctable = (cbyte*)(table);
    cpiece* pieces = (cpiece*)(ctable + h.pieces_offset);
    // The current piece and the first tile of the next one, reloaded only
    // when a tile crosses into another piece.
    int pidx = multi_find_piece(pieces, h.npieces, t_first);
    MultiPiece pc = load_piece(pieces + pidx);
    uint32_t next0 = pidx + 1 < h.npieces ? pieces[pidx + 1].tile0 : UINT32_MAX;
    for (uint32_t tile = t_first; tile < t_end; tile += step) {
        if (tile >= next0) {
            do {
                ++pidx;
                next0 = pidx + 1 < h.npieces ? pieces[pidx + 1].tile0 : UINT32_MAX;
            } while (tile >= next0);
            pc = load_piece(pieces + pidx);
        }
        // The table is read-only here; its recv pointers are device
        // addresses the kernel writes through.
        cuptr* block = (cuptr*)(ctable) + pc.ptrs;
        const void* const* send = (const void* const*)(block);
        void* const* recv = (void* const*)((pc.flags & kPieceInPlace) ? block : block + n);
        const int c = pc.chunk;
        const uint32_t ti = tile - pc.tile0;
        const uint64_t j_end = pc.j0 + pc.len;
        if (pc.flags & kPieceVec) {
            // vector k holds elements [a0 + kE, a0 + (k+1)E): its address is
            // base + a0 * sizeof(element) + 16k, aligned on every rank
            const uint64_t a0 = (pc.flags >> kPieceShiftBit) & kPieceShiftMask;
            const uint64_t boff = a0 * (16 / E);
            uint64_t vb, ve;
            piece_vectors(pc.j0, j_end, a0, E, &vb, &ve);
            if constexpr (RM > 0) {
                constexpr int M = RM;
                const uint64_t v = vb + static_cast<uint64_t>(ti) * (M * kBlock) + threadIdx.x;
                if (ve > vb) {
                    // lanes past the piece read its first vector and drop it
                    uint64_t off[M];
                    bool ok[M];
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        ok[m] = v + m * kBlock < ve;
                        off[m] = (ok[m] ? v + m * kBlock : vb) * 16 + boff;
                    }
                    Acc acc[M][E];
                    fold_rank_major_any<F, OP, NT, M>(send, c, n, off, acc);
                    u32x4 out[M];
#pragma unroll
                    for (int m = 0; m < M; ++m) {
#pragma unroll
                        for (int j = 0; j < E; ++j) acc[m][j] = finalize<OP>(acc[m][j], n);
                        out[m] = F::pack(acc[m]);
                    }
                    for (int r = 0; r < n; ++r)
#pragma unroll
                        for (int m = 0; m < M; ++m)
                            if (ok[m]) stv_at<NT>(recv[r], off[m], out[m]);
                }
            } else {
                // the tile's two halves: vectors v and v + kBlock of this thread
                const uint64_t v = vb + static_cast<uint64_t>(ti) * kMultiVecTile + threadIdx.x;
                const bool ok[2] = {v < ve, v + kBlock < ve};
                if constexpr (NR > 0) {
                    // all 2*NR loads in flight before either fold
                    const void* sp[NR];
#pragma unroll
                    for (int k = 0; k < NR; ++k) sp[k] = send[wrap_rank(c + k, NR)];
                    u32x4 x[2][NR];
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        if (ok[u]) {
#pragma unroll
                            for (int k = 0; k < NR; ++k) x[u][k] = ldv_at<NT>(sp[k], (v + u * kBlock) * 16 + boff);
                        }
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        if (ok[u]) {
                            const u32x4 out = fold_loaded<F, OP, NR>(x[u]);
#pragma unroll
                            for (int r = 0; r < NR; ++r) stv_at<NT>(recv[r], (v + u * kBlock) * 16 + boff, out);
                        }
                } else {
                    const uint64_t off[2] = {v * 16 + boff, (v + kBlock) * 16 + boff};
                    u32x4 out[2];
                    fold_pair_any<F, OP, NT>(send, c, n, off, ok, out);
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        if (ok[u])
                            for (int r = 0; r < n; ++r) stv_at<NT>(recv[r], off[u], out[u]);
                }
            }
            if (ti == 0) {
                // elements before the first whole vector (fewer than a line's)
                // and after the last (fewer than a vector's)
                const uint64_t vstart = a0 + vb * E, vend = a0 + ve * E;
                const uint64_t head_end = vstart < j_end ? (vstart > pc.j0 ? vstart : pc.j0) : j_end;
                const uint64_t nhead = head_end - pc.j0;
                // (a piece with no whole vector is all head: vend may lie
                // past j_end then)
                const uint64_t tail_lo = vend > head_end ? vend : head_end;
                const uint64_t tail_start = tail_lo < j_end ? tail_lo : j_end;
                const uint64_t ntail = j_end - tail_start;
                if (threadIdx.x < nhead + ntail) {
                    const uint64_t i = threadIdx.x < nhead ? pc.j0 + threadIdx.x : tail_start + (threadIdx.x - nhead);
                    const Acc x = finalize<OP>(fold_elem<F, OP>(send, c, n, i), n);
                    for (int r = 0; r < n; ++r) F::st(recv[r], i, x);
                }
            }
        } else {
            const uint64_t i = pc.j0 + static_cast<uint64_t>(ti) * kBlock + threadIdx.x;
            if (i < j_end) {
                const Acc x = finalize<OP>(fold_elem<F, OP>(send, c, n, i), n);
                for (int r = 0; r < n; ++r) F::st(recv[r], i, x);
            }
        }
    }
}

template <class F, int OP, int NR, bool NT, int RM = 0>
__global__ __launch_bounds__(kBlock) void multi_reduce(const MultiArgs a)
{
    multi_body<F, OP, NR, NT, RM>(a.h, a.blob);
}

// ---------------------------------------------------------------------------
// all-to-all [handbook "集合通信原语", section 五个原语]: rank r's block p
// becomes rank p's block r
// ---------------------------------------------------------------------------
// TILED (16-byte vectors, non-temporal): a thread copies kRankMajorTiles
// vectors a kBlock apart per step, all loads before the stores, and the host
// launches one workgroup per such tile, so the resident workgroups stream
// one block pair after another.
template <bool VEC, bool NT, bool TILED = false>
__global__ __launch_bounds__(kBlock) void a2a_copy(const A2AArgs a)
{
    const int y = blockIdx.y;
    int r, p;
    if (a.step < 0) {
        r = y / a.n;
        p = y - r * a.n;
    } else {
        r = y;
        p = wrap_rank(y + a.step, a.n);
    }
    const char* src = static_cast<const char*>(a.send[r]) + static_cast<uint64_t>(p) * a.blk;
    char* dst = static_cast<char*>(a.recv[p]) + static_cast<uint64_t>(r) * a.blk;
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    const uint64_t t0 = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if constexpr (TILED) {
        static_assert(VEC, "the tiled copy takes 16-byte vectors");
        constexpr int M = kRankMajorTiles;
        const uint64_t nv = a.blk / 16;
        const uint64_t ntiles = (nv + M * kBlock - 1) / (M * kBlock);
        for (uint64_t st = blockIdx.x; st < ntiles; st += gridDim.x) {
            u32x4 x[M];
            uint64_t vv[M];
#pragma unroll
            for (int m = 0; m < M; ++m) {
                vv[m] = (st * M + m) * kBlock + threadIdx.x;
                x[m] = ldv<NT>(src, vv[m] < nv ? vv[m] : 0);  // lanes past the block reload vector 0
            }
#pragma unroll
            for (int m = 0; m < M; ++m)
                if (vv[m] < nv) stv<NT>(dst, vv[m], x[m]);
        }
    } else if constexpr (VEC) {
        const uint64_t nv = a.blk / 16;
        for (uint64_t v = t0; v < nv; v += stride) stv<NT>(dst, v, ldv<NT>(src, v));
    } else {
        for (uint64_t b = 2 * t0; b < a.blk; b += 2 * stride)
            *reinterpret_cast<uint16_t*>(dst + b) = *reinterpret_cast<const uint16_t*>(src + b);
    }
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
template <class F, int OP, bool SC, bool NT>
hipError_t fused_nr(const ReduceArgs& a, dim3 grid, hipStream_t s)
{
    const dim3 block(kBlock);
    switch (a.n) {
    case 2: hipLaunchKernelGGL((fused_reduce_vec<F, OP, 2, SC, NT>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((fused_reduce_vec<F, OP, 3, SC, NT>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((fused_reduce_vec<F, OP, 4, SC, NT>), grid, block, 0, s, a); break;
    case 5: hipLaunchKernelGGL((fused_reduce_vec<F, OP, 5, SC, NT>), grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL((fused_reduce_vec<F, OP, 6, SC, NT>), grid, block, 0, s, a); break;
    case 7: hipLaunchKernelGGL((fused_reduce_vec<F, OP, 7, SC, NT>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((fused_reduce_vec<F, OP, 8, SC, NT>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((fused_reduce_vec<F, OP, 0, SC, NT>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

// The rank-major kernels: 16-byte vectors, non-temporal access. The
// all-reduce takes the run-time rank-count body at every rank count (at 5..8
// ranks it ran level with the fixed-rank-count body from 128 MiB per rank
// and 2-7% faster at 20-64 MiB); the reduce-scatter layout takes the
// fixed-rank-count body at 5..8 ranks, the run-time one above.
template <class F, int OP, bool SC>
hipError_t fused_nr_rank_major(const ReduceArgs& a, int tiles, dim3 grid, hipStream_t s)
{
    const dim3 block(kBlock);
    constexpr int M = kScatterTiles;
    constexpr int MA = rank_major_any_tiles(kRankMajorAnyMany, 16 / F::kEpv);
    constexpr int MF = rank_major_any_tiles(kRankMajorAnyMany - 1, 16 / F::kEpv);
    if (a.n > 8) {
        if (tiles != MA) return hipErrorInvalidValue;
        hipLaunchKernelGGL((fused_reduce_vec<F, OP, 0, SC, true, MA>), grid, block, 0, s, a);
        return hipGetLastError();
    }
    if constexpr (SC) {
        if (a.n >= 5) {
            if (tiles != M) return hipErrorInvalidValue;
            switch (a.n) {
            case 5: hipLaunchKernelGGL((fused_reduce_vec<F, OP, 5, SC, true, M>), grid, block, 0, s, a); break;
            case 6: hipLaunchKernelGGL((fused_reduce_vec<F, OP, 6, SC, true, M>), grid, block, 0, s, a); break;
            case 7: hipLaunchKernelGGL((fused_reduce_vec<F, OP, 7, SC, true, M>), grid, block, 0, s, a); break;
            default: hipLaunchKernelGGL((fused_reduce_vec<F, OP, 8, SC, true, M>), grid, block, 0, s, a); break;
            }
            return hipGetLastError();
        }
    }
    if (tiles == MF) {
        hipLaunchKernelGGL((fused_reduce_vec<F, OP, 0, SC, true, MF>), grid, block, 0, s, a);
        return hipGetLastError();
    }
    if constexpr (F::kEpv == 8 && !SC) {
        // 16-bit all-reduce, one tile per super tile (large buffers)
        if (tiles == 1) {
            hipLaunchKernelGGL((fused_reduce_vec<F, OP, 0, SC, true, 1>), grid, block, 0, s, a);
            return hipGetLastError();
        }
    }
    return hipErrorInvalidValue;
}

template <class F, int OP, bool SC>
hipError_t fused_n(const ReduceArgs& a, bool vec, bool nt, int rank_major_tiles, dim3 grid, hipStream_t s)
{
    if (rank_major_tiles > 0) {
        if (!vec || !nt) return hipErrorInvalidValue;
        return fused_nr_rank_major<F, OP, SC>(a, rank_major_tiles, grid, s);
    }
    if (!vec) {
        hipLaunchKernelGGL((fused_reduce_scalar<F, OP, SC>), grid, dim3(kBlock), 0, s, a);
        return hipGetLastError();
    }
    return nt ? fused_nr<F, OP, SC, true>(a, grid, s) : fused_nr<F, OP, SC, false>(a, grid, s);
}

template <class F, bool SC>
hipError_t fused_op(const ReduceArgs& a, ar_op_t op, bool vec, bool nt, int rank_major_tiles, dim3 grid,
                    hipStream_t s)
{
    switch (op) {
    case AR_SUM: return fused_n<F, AR_SUM, SC>(a, vec, nt, rank_major_tiles, grid, s);
    case AR_AVG: return fused_n<F, AR_AVG, SC>(a, vec, nt, rank_major_tiles, grid, s);
    case AR_MAX: return fused_n<F, AR_MAX, SC>(a, vec, nt, rank_major_tiles, grid, s);
    case AR_MIN: return fused_n<F, AR_MIN, SC>(a, vec, nt, rank_major_tiles, grid, s);
    case AR_PROD: return fused_n<F, AR_PROD, SC>(a, vec, nt, rank_major_tiles, grid, s);
    }
    return hipErrorInvalidValue;
}

template <class F, int OP>
hipError_t rs_vec(const StepArgs& a, bool vec, int tiles, bool nt, dim3 grid, hipStream_t s)
{
    if (tiles > 0) {
        if (!vec || tiles != kStepTiles) return hipErrorInvalidValue;
        if (nt) hipLaunchKernelGGL((rs_step<F, OP, true, true, kStepTiles>), grid, dim3(kBlock), 0, s, a);
        else hipLaunchKernelGGL((rs_step<F, OP, true, false, kStepTiles>), grid, dim3(kBlock), 0, s, a);
    } else if (vec) {
        hipLaunchKernelGGL((rs_step<F, OP, true>), grid, dim3(kBlock), 0, s, a);
    } else {
        hipLaunchKernelGGL((rs_step<F, OP, false>), grid, dim3(kBlock), 0, s, a);
    }
    return hipGetLastError();
}

template <class F>
hipError_t rs_op(const StepArgs& a, ar_op_t op, bool vec, int tiles, bool nt, dim3 grid, hipStream_t s)
{
    switch (op) {
    case AR_SUM: return rs_vec<F, AR_SUM>(a, vec, tiles, nt, grid, s);
    case AR_AVG: return rs_vec<F, AR_AVG>(a, vec, tiles, nt, grid, s);
    case AR_MAX: return rs_vec<F, AR_MAX>(a, vec, tiles, nt, grid, s);
    case AR_MIN: return rs_vec<F, AR_MIN>(a, vec, tiles, nt, grid, s);
    case AR_PROD: return rs_vec<F, AR_PROD>(a, vec, tiles, nt, grid, s);
    }
    return hipErrorInvalidValue;
}

// The tree variant uses the any-N kernel only (its 64-way unrolled rank loop
// is costly to compile, and the variant is not the hot path).
template <class F, int OP, bool NT>
hipError_t tree_nr(const ReduceArgs& a, dim3 grid, hipStream_t s)
{
    hipLaunchKernelGGL((tree_fused_vec<F, OP, 0, NT>), grid, dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

template <class F, int OP>
hipError_t tree_n(const ReduceArgs& a, bool vec, bool nt, dim3 grid, hipStream_t s)
{
    if (!vec) {
        hipLaunchKernelGGL((tree_fused_scalar<F, OP>), grid, dim3(kBlock), 0, s, a);
        return hipGetLastError();
    }
    return nt ? tree_nr<F, OP, true>(a, grid, s) : tree_nr<F, OP, false>(a, grid, s);
}

template <class F>
hipError_t tree_op(const ReduceArgs& a, ar_op_t op, bool vec, bool nt, dim3 grid, hipStream_t s)
{
    switch (op) {
    case AR_SUM: return tree_n<F, AR_SUM>(a, vec, nt, grid, s);
    case AR_AVG: return tree_n<F, AR_AVG>(a, vec, nt, grid, s);
    case AR_MAX: return tree_n<F, AR_MAX>(a, vec, nt, grid, s);
    case AR_MIN: return tree_n<F, AR_MIN>(a, vec, nt, grid, s);
    case AR_PROD: return tree_n<F, AR_PROD>(a, vec, nt, grid, s);
    }
    return hipErrorInvalidValue;
}

template <class F, int OP>
hipError_t tree_level_vec(const TreeArgs& a, bool vec, dim3 grid, hipStream_t s)
{
    if (vec) hipLaunchKernelGGL((tree_reduce_level<F, OP, true>), grid, dim3(kBlock), 0, s, a);
    else hipLaunchKernelGGL((tree_reduce_level<F, OP, false>), grid, dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

template <class F>
hipError_t tree_level_op(const TreeArgs& a, ar_op_t op, bool vec, dim3 grid, hipStream_t s)
{
    switch (op) {
    case AR_SUM: return tree_level_vec<F, AR_SUM>(a, vec, grid, s);
    case AR_AVG: return tree_level_vec<F, AR_AVG>(a, vec, grid, s);
    case AR_MAX: return tree_level_vec<F, AR_MAX>(a, vec, grid, s);
    case AR_MIN: return tree_level_vec<F, AR_MIN>(a, vec, grid, s);
    case AR_PROD: return tree_level_vec<F, AR_PROD>(a, vec, grid, s);
    }
    return hipErrorInvalidValue;
}

template <class F, int OP, bool NT>
hipError_t multi_nr(const MultiArgs& a, bool rank_major, int grid_x, hipStream_t s)
{
    const dim3 grid(grid_x), block(kBlock);
    if (rank_major) {
        // the rank-major kernel (run-time rank count, tiles of
        // rank_major_any_tiles quarters), with non-temporal access from 4
        // ranks
        if (!NT || a.h.n < 4) return hipErrorInvalidValue;
        if constexpr (NT) {
            constexpr int MA = rank_major_any_tiles(kRankMajorAnyMany, 16 / F::kEpv);
            constexpr int MF = rank_major_any_tiles(kRankMajorAnyMany - 1, 16 / F::kEpv);
            if (a.h.n > 8) hipLaunchKernelGGL((multi_reduce<F, OP, 0, NT, MA>), grid, block, 0, s, a);
            else hipLaunchKernelGGL((multi_reduce<F, OP, 0, NT, MF>), grid, block, 0, s, a);
        }
    } else if (a.h.n == 8) {
        hipLaunchKernelGGL((multi_reduce<F, OP, 8, NT>), grid, block, 0, s, a);
    } else {
        hipLaunchKernelGGL((multi_reduce<F, OP, 0, NT>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

template <class F, bool NT>
hipError_t multi_nt(const MultiArgs& a, ar_op_t op, bool rank_major, int grid_x, hipStream_t s)
{
    switch (op) {
    case AR_SUM: return multi_nr<F, AR_SUM, NT>(a, rank_major, grid_x, s);
    case AR_AVG: return multi_nr<F, AR_AVG, NT>(a, rank_major, grid_x, s);
    case AR_MAX: return multi_nr<F, AR_MAX, NT>(a, rank_major, grid_x, s);
    case AR_MIN: return multi_nr<F, AR_MIN, NT>(a, rank_major, grid_x, s);
    case AR_PROD: return multi_nr<F, AR_PROD, NT>(a, rank_major, grid_x, s);
    }
    return hipErrorInvalidValue;
}

template <class F>
hipError_t multi_op(const MultiArgs& a, ar_op_t op, bool nt, bool rank_major, int grid_x, hipStream_t s)
{
    return nt ? multi_nt<F, true>(a, op, rank_major, grid_x, s) : multi_nt<F, false>(a, op, rank_major, grid_x, s);
}

// Per-dtype entry points, each instantiated once: the ring kernels (fused,
// stepwise reduce-scatter, multi-tensor) in dtype_<name>.hip and the tree
// kernels in tree_<name>.hip, so the build compiles them in parallel.
#define AR_RING_INSTANTIATIONS(F, EXTERN)                                                                       \
    EXTERN template hipError_t fused_op<F, true>(const ReduceArgs&, ar_op_t, bool, bool, int, dim3, hipStream_t);  \
    EXTERN template hipError_t fused_op<F, false>(const ReduceArgs&, ar_op_t, bool, bool, int, dim3, hipStream_t); \
    EXTERN template hipError_t rs_op<F>(const StepArgs&, ar_op_t, bool, int, bool, dim3, hipStream_t);            \
    EXTERN template hipError_t multi_op<F>(const MultiArgs&, ar_op_t, bool, bool, int, hipStream_t);
#define AR_TREE_INSTANTIATIONS(F, EXTERN)                                                           \
    EXTERN template hipError_t tree_op<F>(const ReduceArgs&, ar_op_t, bool, bool, dim3, hipStream_t); \
    EXTERN template hipError_t tree_level_op<F>(const TreeArgs&, ar_op_t, bool, dim3, hipStream_t);

#ifndef AR_INSTANTIATE_RING
AR_RING_INSTANTIATIONS(F32, extern)
AR_RING_INSTANTIATIONS(F16, extern)
AR_RING_INSTANTIATIONS(BF16, extern)
AR_RING_INSTANTIATIONS(I32, extern)
#endif
#ifndef AR_INSTANTIATE_TREE
AR_TREE_INSTANTIATIONS(F32, extern)
AR_TREE_INSTANTIATIONS(F16, extern)
AR_TREE_INSTANTIATIONS(BF16, extern)
AR_TREE_INSTANTIATIONS(I32, extern)
#endif

}  // namespace detail
}  // namespace ar
