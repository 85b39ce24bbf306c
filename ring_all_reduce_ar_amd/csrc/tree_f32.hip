// tree_f32.hip -- instantiates the F32 tree kernels (see kernels_impl.h).
#define AR_INSTANTIATE_TREE
#include "kernels_impl.h"

namespace ar {
namespace detail {
AR_TREE_INSTANTIATIONS(F32, )
}  // namespace detail
}  // namespace ar
