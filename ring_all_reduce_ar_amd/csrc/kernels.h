// kernels.h -- internal interface between the C ABI (api.cpp) and the HIP
// kernels (kernels.hip). Not installed; the public ABI is include/allreduce.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "allreduce.h"

namespace ar {

// Threads per workgroup for every kernel: four 64-wide wavefronts.
constexpr int kBlock = 256;

// Rank buffers and sizes of one reduction (all-reduce or reduce-scatter).
//   count: elements per rank in the send buffers
//   q:     chunk length; chunk c = [c*q, min((c+1)*q, count))
struct ReduceArgs {
    const void* send[AR_MAX_RANKS];
    void* recv[AR_MAX_RANKS];
    uint64_t count;
    uint64_t q;
    int n;
};

// One ring reduce-scatter step. Chunk (r - s - 1) mod n is combined at rank r:
// local (send[r]) (+) incoming (send[left] on the first step, else the
// partial kept in recv[left] or in the fp32/uint32 workspace ws).
struct StepArgs {
    const void* send[AR_MAX_RANKS];
    void* recv[AR_MAX_RANKS];
    void* ws;          // accumulator workspace (count slots of 4 bytes) or null
    uint64_t count;
    uint64_t q;
    int n;
    int s;             // step index, 0..n-2
    int first;         // s == 0
    int last;          // s == n-2: finalize (AVG, rounding) and write the result
    int scatter;       // reduce-scatter layout: finished chunk c goes to recv[c]
};

// Byte copies between rank buffers. Copy step s of a ring: chunk
// (r - s - shift) mod n of recv[left] goes to the same place in recv[r].
// Chunk c spans bytes [c*qb, min((c+1)*qb, total)). For a local copy
// (shift < 0): send[r] -> recv[r] + r*dst_stride bytes, `total` bytes each.
struct CopyArgs {
    const void* send[AR_MAX_RANKS];
    void* recv[AR_MAX_RANKS];
    uint64_t total;    // bytes per rank buffer covered by the chunks
    uint64_t qb;       // chunk length in bytes
    uint64_t dst_stride;
    int n;
    int s;
    int shift;
};

// One level of the tree variant. Reduce level (stride s = 2^l): for every
// pair (r, q = r + s) with r a multiple of 2s, r combines local (+)
// incoming; partials live in recv (fp32/int32) or in fp32 workspace slot r/2
// (fp16/bf16). Broadcast level: recv[q] = recv[r]. Grid row j is pair j.
struct TreeArgs {
    const void* send[AR_MAX_RANKS];
    void* recv[AR_MAX_RANKS];
    void* ws;
    uint64_t ws_stride;  // elements per workspace slot: count rounded up to a multiple of 4
    uint64_t count;
    int n;
    int stride;
    int last;  // the root's final level: finalize (AVG, rounding) into recv[0]
};

hipError_t launch_tree_fused(const ReduceArgs& a, ar_dtype_t dtype, ar_op_t op, bool vec, bool nt, int grid_x,
                             hipStream_t stream);
hipError_t launch_tree_reduce_level(const TreeArgs& a, ar_dtype_t dtype, ar_op_t op, bool vec, int grid_x,
                                    hipStream_t stream);
hipError_t launch_tree_bcast_level(const TreeArgs& a, size_t elem, bool vec, int grid_x, hipStream_t stream);

// Coalesced multi-tensor all-reduce. The table holds, from offset 0, each
// tensor's rank pointers (n send then n recv, or just n when every rank's
// tensor is in place), and from `pieces_offset` the pieces: a piece is the
// part of one tensor that falls in one ring chunk. Tiles (kBlock vectors, or
// kBlock elements when the tensor's pointers are not all 16-byte aligned)
// are numbered across pieces.
constexpr uint8_t kPieceVec = 1;      // 16-byte vectors in the body, elements at the ends
constexpr uint8_t kPieceInPlace = 2;  // recv pointers are the send pointers
constexpr int kPieceShiftBit = 2;     // bits 2..7: a0, the tensor's first element of its aligned run
constexpr unsigned kPieceShiftMask = 63;
// 16-byte vectors per 128-byte cache line.
constexpr uint64_t kLineVectors = 8;

// The 16-byte vectors of a piece [j0, j_end) of a tensor whose element a0 is
// the first one on a 128-byte line when every rank's pointers share one
// offset from a line, else the first one on a 16-byte boundary (the same a0
// for every rank's pointers): vector k holds elements [a0 + kE, a0 + (k+1)E),
// and the piece's whole vectors are [vb, ve), vb a multiple of a line's
// vectors so that the piece's tiles start on a line when a0 does. Shared by
// the planner and the kernel, which must agree on the tile count.
__host__ __device__ inline void piece_vectors(uint64_t j0, uint64_t j_end, uint64_t a0, uint64_t E, uint64_t* vb,
                                              uint64_t* ve)
{
    const uint64_t L = kLineVectors * E;
    *vb = j0 <= a0 ? 0 : (j0 - a0 + L - 1) / L * kLineVectors;
    *ve = j_end <= a0 ? 0 : (j_end - a0) / E;
    if (*ve < *vb) *ve = *vb;
}
struct MultiPiece {
    uint64_t j0;     // first element of the piece inside its tensor
    uint64_t len;    // elements
    uint32_t tile0;  // first tile of the piece
    uint16_t ptrs;   // index of the tensor's first pointer in the table
    uint8_t chunk;   // ring chunk (the fold starts at rank `chunk`)
    uint8_t flags;   // kPieceVec | kPieceInPlace | a0 << kPieceShiftBit
};
static_assert(sizeof(MultiPiece) == 24, "MultiPiece layout");
constexpr int kMultiBlobBytes = 3840;
// Vector pieces are cut into tiles of two kBlock-vector halves (a thread
// takes one vector in each), or of rank_major_any_tiles for the rank-major
// kernel; element pieces into tiles of kBlock elements.
constexpr int kMultiVecTile = 2 * kBlock;

// Tiles a thread of the tiled copies (all-gather, all-to-all) takes together.
constexpr int kRankMajorTiles = 4;
// Tiles per super tile of the fixed-rank-count rank-major reduce-scatter
// (5..8 ranks).
constexpr int kScatterTiles = 1;

// Tiles (of kBlock 16-byte vectors) per super tile of the rank-major kernels
// for run-time rank counts: 8 above 8 ranks and 4 up to 8 for 4-byte types
// (64 and 16 KiB per rank and stage; measured best of 2, 4, 8 and 16 at
// 4-64 ranks), half that for 2-byte types, whose eight fp32 accumulators
// per vector would otherwise push the kernel past 128 VGPRs. Shared by the
// kernels and the multi-tensor planner, which cuts pieces into such tiles.
constexpr int kRankMajorAnyMany = 9;  // a rank count above 8
__host__ __device__ constexpr int rank_major_any_tiles(int nranks, int elem_bytes)
{
    return (nranks > 8 ? 8 : 4) / (elem_bytes == 2 ? 2 : 1);
}
struct MultiHeader {
    int n;
    int npieces;
    uint32_t ntiles;
    uint32_t pieces_offset;  // bytes into the table
};
// The table travels in the kernel arguments: one launch per batch of
// tensors whose pointer blocks and pieces fit.
struct MultiArgs {
    MultiHeader h;
    alignas(16) unsigned char blob[kMultiBlobBytes];
};

// `rank_major` selects the rank-major kernel (needs nt and at least 4 ranks;
// the table's vector tiles are then rank_major_any_tiles(n, elem) * kBlock
// vectors wide).
hipError_t launch_multi_reduce(const MultiArgs& a, ar_dtype_t dtype, ar_op_t op, bool nt, bool rank_major, int grid_x,
                               hipStream_t stream);

// All-to-all block copies: row y copies block p of send[r] to block r of
// recv[p], `blk` bytes. step < 0: all n*n (r, p) pairs, row y = r*n + p;
// step s >= 0: the n pairs (r, (r + s) mod n), row y = r.
struct A2AArgs {
    const void* send[AR_MAX_RANKS];
    void* recv[AR_MAX_RANKS];
    uint64_t blk;
    int n;
    int step;
};

// `tiled` selects the tiled copy (needs vec and nt): kRankMajorTiles vectors
// per thread and step, best with one workgroup per tile.
hipError_t launch_all_to_all(const A2AArgs& a, bool vec, bool nt, bool tiled, int grid_x, hipStream_t stream);

// A super tile of one tile for 16-bit types at up to 8 ranks from this many
// bytes per rank, instead of rank_major_any_tiles. Against two tiles on the
// same buffers, fp16 at 8 ranks: +4.4% at 14 GB, +2.5% at 1 GiB, +1.5% at
// 4 GiB, -1.2% at 256 MiB, -4.3% at 64 MiB; the benchmark's first allocation
// of 8 x 14 GB: 38.0 -> 35.9 ms.
constexpr uint64_t kOneTileBytes = uint64_t(1) << 30;

// Fused single-pass reduction; `vec` selects the 16-byte kernels (the caller
// has checked that every rank pointer is 16-byte aligned, and for the
// reduce-scatter layout also q % (16/elem) == 0); `nt` selects non-temporal
// loads and stores (footprints beyond the last-level cache) over cached ones;
// `rank_major_tiles` > 0 selects the rank-major kernels (needs vec and nt)
// with that many tiles per super tile: kScatterTiles for the reduce-scatter
// layout at 5..8 ranks, else rank_major_any_tiles, or 1 for a 16-bit
// all-reduce at up to 8 ranks (other values are rejected). Any grid is correct (the
// kernels stride by it); the rank-major ones run best with one workgroup per
// super tile.
hipError_t launch_fused_reduce(const ReduceArgs& a, ar_dtype_t dtype, ar_op_t op, bool scatter, bool vec, bool nt,
                               int rank_major_tiles, int grid_x, hipStream_t stream);

// Fused all-gather: block p of send[p] (blk bytes) to recv[r] + p*blk for all r.
// `rank_major` selects the rank-major copy (needs vec and nt).
hipError_t launch_fused_gather(const CopyArgs& a, bool vec, bool nt, bool rank_major, int grid_x, hipStream_t stream);

// Vectors a thread takes per tile in the tiled ring steps.
constexpr int kStepTiles = 4;

// One ring step. `tiles` = 0: one vector (or element) per thread per
// grid-stride step; `tiles` = kStepTiles (needs vec): the tiled form, best
// with one workgroup per tile; `nt` selects non-temporal access for it.
hipError_t launch_rs_step(const StepArgs& a, ar_dtype_t dtype, ar_op_t op, bool vec, int tiles, bool nt, int grid_x,
                          hipStream_t stream);

hipError_t launch_copy_step(const CopyArgs& a, bool vec, int tiles, bool nt, int grid_x, hipStream_t stream);

// send[r] -> recv[r] + r*dst_stride, total bytes, for every rank.
hipError_t launch_local_copy(const CopyArgs& a, bool vec, int grid_x, hipStream_t stream);

// The device address of this library's AR_NOALLOC_SCRATCH_BYTES scratch
// array on `device`, which must be the current device; looked up once per
// device and cached (noalloc.hip).
hipError_t scratch_address(int device, void** out);

}  // namespace ar
