// Small-batch matrix-core kernels of one weight format (kKq4); see gemm_kernel.hpp.
#include "gemm_kernel.hpp"

namespace w4a16 {

template hipError_t launch_skinny_fmt<kKq4>(const void *, bool, const void *, const void *, const void *, void *,
                                           int, int, int, int, const GemmPlan &, hipStream_t);
template hipError_t launch_skinny_group_fmt<kKq4>(const GroupTable &, bool, int, int, int, const GemmPlan &,
                                                 hipStream_t);

}  // namespace w4a16
