// tree_bf16.hip -- instantiates the BF16 tree kernels (see kernels_impl.h).
#define AR_INSTANTIATE_TREE
#include "kernels_impl.h"

namespace ar {
namespace detail {
AR_TREE_INSTANTIATIONS(BF16, )
}  // namespace detail
}  // namespace ar
