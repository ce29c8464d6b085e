// Tiled matrix-core path (large M), host side: the tile choice and the
// dispatch over the weight formats. The kernel is in prefill_kernel.hpp; each
// weight format is compiled in its own translation unit (this one: the 4-bit
// zero-point format; prefill_sym4.hip, prefill_sym8.hip).
#include "prefill_kernel.hpp"

namespace w4a16 {

int prefill_tile(int64_t M, int64_t N) {
    static const int forced = [] {
        const char *v = getenv("W4A16_PREFILL_TILE");
        return v ? atoi(v) : -1;
    }();
    if (forced >= 0 && forced <= kTile256x256w8) return forced;
    // time ~ rounds of workgroups over the 256 CUs x time of one tile; the
    // relative tile times (0.62, 0.67, 1.0 for 64, 128, 256 rows) were
    // measured at K = 5120
    // (the 256-row tile runs with eight waves, two per SIMD: 4-7% faster than
    // four at K = 5120, M = 2048)
    static const int kinds[3] = {kTile64x256, kTile128x256, kTile256x256w8};
    static const int rows[3] = {64, 128, 256};
    static const double tile_time[3] = {0.62, 0.67, 1.0};
    const int64_t n_tiles = ceil_div(N, 256);
    int best = kTile256x256w8;
    double best_cost = 1e300;
    for (int t = 0; t < 3; ++t) {
        const int64_t tiles = ceil_div(M, rows[t]) * n_tiles;
        const double cost = (double)ceil_div(tiles, 256) * tile_time[t];
        if (cost < best_cost - 1e-9) {
            best_cost = cost;
            best = kinds[t];
        }
    }
    return best;
}

hipError_t launch_prefill(const void *x, bool bf16, const void *qweight, const void *scales, const void *zeros,
                          void *y, int M, int N, int K, int group, int fmt, const GemmPlan &plan, hipStream_t stream) {
    switch (fmt) {
        case kSym4: return launch_prefill_fmt<kSym4>(x, bf16, qweight, scales, zeros, y, M, N, K, group, plan, stream);
        case kSym8: return launch_prefill_fmt<kSym8>(x, bf16, qweight, scales, zeros, y, M, N, K, group, plan, stream);
        case kKq4: return launch_prefill_fmt<kKq4>(x, bf16, qweight, scales, zeros, y, M, N, K, group, plan, stream);
        default: return launch_prefill_fmt<kAsym4>(x, bf16, qweight, scales, zeros, y, M, N, K, group, plan, stream);
    }
}

template hipError_t launch_prefill_fmt<kAsym4>(const void *, bool, const void *, const void *, const void *, void *,
                                               int, int, int, int, const GemmPlan &, hipStream_t);

}  // namespace w4a16
