// kernels.hip -- the launch functions of kernels.h: the switch over dtypes
// (whose kernels are instantiated in dtype_*.hip) and the dtype-free copy
// kernels (all-gather, all-to-all, ring copy steps, tree broadcast).
#include "kernels_impl.h"

namespace ar {
using namespace detail;

namespace {
template <bool SC>
hipError_t fused_dtype(const ReduceArgs& a, ar_dtype_t dtype, ar_op_t op, bool vec, bool nt, int rank_major_tiles,
                       dim3 grid, hipStream_t s)
{
    switch (dtype) {
    case AR_FLOAT32: return fused_op<F32, SC>(a, op, vec, nt, rank_major_tiles, grid, s);
    case AR_FLOAT16: return fused_op<F16, SC>(a, op, vec, nt, rank_major_tiles, grid, s);
    case AR_BFLOAT16: return fused_op<BF16, SC>(a, op, vec, nt, rank_major_tiles, grid, s);
    case AR_INT32: return fused_op<I32, SC>(a, op, vec, nt, rank_major_tiles, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int tree_pairs(int n, int stride) { return n > stride ? (n - stride - 1) / (2 * stride) + 1 : 0; }

hipError_t launch_tree_fused(const ReduceArgs& a, ar_dtype_t dtype, ar_op_t op, bool vec, bool nt, int grid_x,
                             hipStream_t stream)
{
    const dim3 grid(grid_x);
    switch (dtype) {
    case AR_FLOAT32: return tree_op<F32>(a, op, vec, nt, grid, stream);
    case AR_FLOAT16: return tree_op<F16>(a, op, vec, nt, grid, stream);
    case AR_BFLOAT16: return tree_op<BF16>(a, op, vec, nt, grid, stream);
    case AR_INT32: return tree_op<I32>(a, op, vec, nt, grid, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_tree_reduce_level(const TreeArgs& a, ar_dtype_t dtype, ar_op_t op, bool vec, int grid_x,
                                    hipStream_t stream)
{
    const dim3 grid(grid_x, tree_pairs(a.n, a.stride));
    switch (dtype) {
    case AR_FLOAT32: return tree_level_op<F32>(a, op, vec, grid, stream);
    case AR_FLOAT16: return tree_level_op<F16>(a, op, vec, grid, stream);
    case AR_BFLOAT16: return tree_level_op<BF16>(a, op, vec, grid, stream);
    case AR_INT32: return tree_level_op<I32>(a, op, vec, grid, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_tree_bcast_level(const TreeArgs& a, size_t elem, bool vec, int grid_x, hipStream_t stream)
{
    const dim3 grid(grid_x, tree_pairs(a.n, a.stride));
    const uint64_t bytes = a.count * elem;
    if (vec) hipLaunchKernelGGL((tree_bcast_level<true>), grid, dim3(kBlock), 0, stream, a, bytes);
    else hipLaunchKernelGGL((tree_bcast_level<false>), grid, dim3(kBlock), 0, stream, a, bytes);
    return hipGetLastError();
}



hipError_t launch_multi_reduce(const MultiArgs& a, ar_dtype_t dtype, ar_op_t op, bool nt, bool rank_major, int grid_x,
                               hipStream_t stream)
{
    switch (dtype) {
    case AR_FLOAT32: return multi_op<F32>(a, op, nt, rank_major, grid_x, stream);
    case AR_FLOAT16: return multi_op<F16>(a, op, nt, rank_major, grid_x, stream);
    case AR_BFLOAT16: return multi_op<BF16>(a, op, nt, rank_major, grid_x, stream);
    case AR_INT32: return multi_op<I32>(a, op, nt, rank_major, grid_x, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fused_reduce(const ReduceArgs& a, ar_dtype_t dtype, ar_op_t op, bool scatter, bool vec, bool nt,
                               int rank_major_tiles, int grid_x, hipStream_t stream)
{
    const dim3 grid(grid_x, a.n);
    return scatter ? fused_dtype<true>(a, dtype, op, vec, nt, rank_major_tiles, grid, stream)
                   : fused_dtype<false>(a, dtype, op, vec, nt, rank_major_tiles, grid, stream);
}

hipError_t launch_fused_gather(const CopyArgs& a, bool vec, bool nt, bool rank_major, int grid_x, hipStream_t stream)
{
    const dim3 grid(grid_x, a.n);
    if (rank_major) {
        if (!vec || !nt) return hipErrorInvalidValue;
        hipLaunchKernelGGL((fused_gather<true, true, true>), grid, dim3(kBlock), 0, stream, a);
        return hipGetLastError();
    }
    if (!vec) hipLaunchKernelGGL((fused_gather<false, true>), grid, dim3(kBlock), 0, stream, a);
    else if (nt) hipLaunchKernelGGL((fused_gather<true, true>), grid, dim3(kBlock), 0, stream, a);
    else hipLaunchKernelGGL((fused_gather<true, false>), grid, dim3(kBlock), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_rs_step(const StepArgs& a, ar_dtype_t dtype, ar_op_t op, bool vec, int tiles, bool nt, int grid_x,
                          hipStream_t stream)
{
    const dim3 grid(grid_x, a.n);
    switch (dtype) {
    case AR_FLOAT32: return rs_op<F32>(a, op, vec, tiles, nt, grid, stream);
    case AR_FLOAT16: return rs_op<F16>(a, op, vec, tiles, nt, grid, stream);
    case AR_BFLOAT16: return rs_op<BF16>(a, op, vec, tiles, nt, grid, stream);
    case AR_INT32: return rs_op<I32>(a, op, vec, tiles, nt, grid, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_copy_step(const CopyArgs& a, bool vec, int tiles, bool nt, int grid_x, hipStream_t stream)
{
    const dim3 grid(grid_x, a.n);
    if (tiles > 0) {
        if (!vec || tiles != kStepTiles) return hipErrorInvalidValue;
        if (nt) hipLaunchKernelGGL((copy_step<true, true, kStepTiles>), grid, dim3(kBlock), 0, stream, a);
        else hipLaunchKernelGGL((copy_step<true, false, kStepTiles>), grid, dim3(kBlock), 0, stream, a);
    } else if (vec) {
        hipLaunchKernelGGL((copy_step<true>), grid, dim3(kBlock), 0, stream, a);
    } else {
        hipLaunchKernelGGL((copy_step<false>), grid, dim3(kBlock), 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_all_to_all(const A2AArgs& a, bool vec, bool nt, bool tiled, int grid_x, hipStream_t stream)
{
    const dim3 grid(grid_x, a.step < 0 ? a.n * a.n : a.n);
    if (tiled) {
        if (!vec || !nt) return hipErrorInvalidValue;
        hipLaunchKernelGGL((a2a_copy<true, true, true>), grid, dim3(kBlock), 0, stream, a);
        return hipGetLastError();
    }
    if (!vec) hipLaunchKernelGGL((a2a_copy<false, true>), grid, dim3(kBlock), 0, stream, a);
    else if (nt) hipLaunchKernelGGL((a2a_copy<true, true>), grid, dim3(kBlock), 0, stream, a);
    else hipLaunchKernelGGL((a2a_copy<true, false>), grid, dim3(kBlock), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_local_copy(const CopyArgs& a, bool vec, int grid_x, hipStream_t stream)
{
    const dim3 grid(grid_x, a.n);
    if (vec) hipLaunchKernelGGL((local_copy<true>), grid, dim3(kBlock), 0, stream, a);
    else hipLaunchKernelGGL((local_copy<false>), grid, dim3(kBlock), 0, stream, a);
    return hipGetLastError();
}

}  // namespace ar
