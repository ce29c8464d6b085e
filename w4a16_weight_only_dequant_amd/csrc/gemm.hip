// Matrix-core (MFMA) path of the W4A16 linear layer.
#include "w4a16_internal.hpp"

namespace w4a16 {

GemmPlan gemm_plan(int64_t M, int64_t N, int64_t K, int32_t group) {
    (void)M; (void)N; (void)K; (void)group;
    GemmPlan p{};
    p.k_splits = 1;
    return p;
}

hipError_t launch_gemm(const void *, bool, const void *, const void *, const void *, void *, int,
                       int, int, int, const GemmPlan &, void *, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace w4a16
