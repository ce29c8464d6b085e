// Small-batch matrix-core path, host side: launch plan and the dispatch over
// the weight formats. The kernel is in gemm_kernel.hpp; each weight format is
// compiled in its own translation unit (this one: the 4-bit zero-point
// format; gemm_sym4.hip, gemm_sym8.hip).
#include "gemm_kernel.hpp"

namespace w4a16 {

GemmPlan gemm_plan(int64_t M, int64_t N, int64_t K, int32_t group, int kind) {
    const int forced_waves = tuning_knob("W4A16_SKINNY_WAVES", 0);
    const int forced_r = tuning_knob("W4A16_SKINNY_R", 0);
    const int skinny_max = tuning_knob("W4A16_SKINNY_MAX_M", kSkinnyMaxM);
    GemmPlan p{};
    if (kind == 0 || (kind < 0 && M <= skinny_max)) {
        p.kind = 0;
        const int64_t columns = ceil_div(K / kChunk, kColChunks);
        // waves splitting K: eight (two per SIMD) up to M = 16, where each
        // workgroup has little else in flight (measured: M = 8, K = 28672:
        // 80 -> 61 us; M = 2..16, K = 5120: 3-7 % faster), four above
        int64_t w = M <= 16 ? 8 : 4;
        if (columns > w * 64) w = ceil_div(columns, 64);
        if (w > columns) w = columns;
        if (forced_waves > 0) w = forced_waves;
        // row blocks per workgroup: more share each activation fragment, fewer
        // make more workgroups; measured best: four for wide matrices (>= 768
        // blocks; at group 32 four spill), two from 320 blocks, else one
        const int64_t nblocks = ceil_div(N, kRowBlock);
        int rpw = (nblocks >= 768 && group >= 64) ? 4 : (nblocks >= 320 ? 2 : 1);
        if (forced_r == 1 || forced_r == 2 || forced_r == 4) rpw = forced_r;
        if (w > kSkinnyMaxWaves) w = kSkinnyMaxWaves;
        if (w < 1) w = 1;
        p.waves = (int)w;
        p.rows_per_wg = rpw;
        return p;
    }
    p.kind = 1;
    p.tile = prefill_tile(M, N);
    prefill_stream_k(M, N, K, device_cu_count(), p);
    return p;
}

hipError_t launch_gemm(const void *x, bool bf16, const void *qweight, const void *scales, const void *zeros,
                       void *y, int M, int N, int K, int group, int fmt, const GemmPlan &plan, void *workspace,
                       hipStream_t stream) {
    if (plan.kind != 0)
        return launch_prefill(x, bf16, qweight, scales, zeros, y, M, N, K, group, fmt, plan, workspace, stream);
    switch (fmt) {
        case kSym4: return launch_skinny_fmt<kSym4>(x, bf16, qweight, scales, zeros, y, M, N, K, group, plan, stream);
        case kSym8: return launch_skinny_fmt<kSym8>(x, bf16, qweight, scales, zeros, y, M, N, K, group, plan, stream);
        case kKq4: return launch_skinny_fmt<kKq4>(x, bf16, qweight, scales, zeros, y, M, N, K, group, plan, stream);
        default: return launch_skinny_fmt<kAsym4>(x, bf16, qweight, scales, zeros, y, M, N, K, group, plan, stream);
    }
}

hipError_t launch_gemm_group(const GroupTable &tab, bool bf16, int M, int K, int group, int fmt, const GemmPlan &plan,
                             hipStream_t stream) {
    switch (fmt) {
        case kSym4: return launch_skinny_group_fmt<kSym4>(tab, bf16, M, K, group, plan, stream);
        case kSym8: return launch_skinny_group_fmt<kSym8>(tab, bf16, M, K, group, plan, stream);
        case kKq4: return launch_skinny_group_fmt<kKq4>(tab, bf16, M, K, group, plan, stream);
        default: return launch_skinny_group_fmt<kAsym4>(tab, bf16, M, K, group, plan, stream);
    }
}

template hipError_t launch_skinny_fmt<kAsym4>(const void *, bool, const void *, const void *, const void *, void *,
                                              int, int, int, int, const GemmPlan &, hipStream_t);
template hipError_t launch_skinny_group_fmt<kAsym4>(const GroupTable &, bool, int, int, int, const GemmPlan &,
                                                    hipStream_t);

}  // namespace w4a16
