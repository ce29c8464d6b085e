// Decode GEMV kernels of one weight format (kKq4); see gemv_kernel.hpp.
#include "gemv_kernel.hpp"

namespace w4a16 {

template hipError_t launch_gemv_fmt<kKq4>(const void *, bool, const void *, const void *, const void *, void *,
                                         int, int, int, int, const float *, const GemvPlan &, hipStream_t);

}  // namespace w4a16
