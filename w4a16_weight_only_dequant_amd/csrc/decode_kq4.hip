// Decode kernels of one weight format (kKq4); see decode_kernel.hpp.
#include "decode_kernel.hpp"

namespace w4a16 {

template hipError_t launch_decode_fmt<kKq4>(const void *, bool, const void *, const void *, const void *, void *,
                                            int, int, int, int, const float *, const DecodePlan &, void *,
                                            hipStream_t);
template hipError_t launch_decode_group_fmt<kKq4>(const GroupTable &, bool, int, int, int, const DecodePlan *, void *,
                                                  hipStream_t);

}  // namespace w4a16
