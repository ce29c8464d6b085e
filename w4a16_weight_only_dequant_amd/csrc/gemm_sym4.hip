// Small-batch matrix-core kernels of one weight format (kSym4); see gemm_kernel.hpp.
#include "gemm_kernel.hpp"

namespace w4a16 {

template hipError_t launch_skinny_fmt<kSym4>(const void *, bool, const void *, const void *, const void *, void *,
                                            int, int, int, int, const GemmPlan &, hipStream_t);
template hipError_t launch_skinny_group_fmt<kSym4>(const GroupTable &, bool, int, int, int, const GemmPlan &,
                                                  hipStream_t);

}  // namespace w4a16
