// dtype_i32.hip -- instantiates the I32 ring kernels (see kernels_impl.h).
#define AR_INSTANTIATE_RING
#include "kernels_impl.h"

namespace ar {
namespace detail {
AR_RING_INSTANTIATIONS(I32, )
}  // namespace detail
}  // namespace ar
