// dtype_bf16.hip -- instantiates the BF16 ring kernels (see kernels_impl.h).
#define AR_INSTANTIATE_RING
#include "kernels_impl.h"

namespace ar {
namespace detail {
AR_RING_INSTANTIATIONS(BF16, )
}  // namespace detail
}  // namespace ar
