// Tiled matrix-core kernels of one weight format (kKq4); see prefill_kernel.hpp.
#include "prefill_kernel.hpp"

namespace w4a16 {

template hipError_t launch_prefill_fmt<kKq4>(const void *, bool, const void *, const void *, const void *, void *,
                                            int, int, int, int, const GemmPlan &, void *, hipStream_t);

}  // namespace w4a16
