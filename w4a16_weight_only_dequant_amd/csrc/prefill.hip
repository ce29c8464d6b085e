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

// Stream-K: with T columns per tile and `tiles` tiles on `cus` compute units,
// whole-tile scheduling takes ceil(tiles / cus) rounds where tiles / cus would
// do. When the last round is at most half full, the tiles of the last two
// rounds are split by columns over exactly `cus` workgroups (each then gets
// at least one tile's worth, so a tile is shared by at most two of them); the
// earlier rounds stay whole tiles. Every piece of a split tile costs about
// what a whole tile's start and end cost (measured ~10 us at K = 5120), so a
// fuller last round gains nothing (432 tiles of 256 x 256 on 256 CUs:
// 283 us either way; 264 tiles: 266 -> 185 us). Needs at least 4 columns per
// tile, so that a split tile still has a head and a tail of some length.
void prefill_stream_k(int64_t M, int64_t N, int64_t K, int cus, GemmPlan &plan) {
    static const int enabled = [] {
        const char *v = getenv("W4A16_PREFILL_SK");
        return v ? atoi(v) : 1;
    }();
    plan.dp_tiles = 0;
    plan.sk_wgs = 0;
    const int64_t tiles = ceil_div(M, tile_rows(plan.tile)) * ceil_div(N, kTileCols);
    const int64_t T = ceil_div(K / kChunk, kColChunks);
    if (!enabled || cus < 8 || T < 4 || tiles <= cus) return;
    const int64_t rounds = ceil_div(tiles, cus);
    const int64_t last = tiles - (rounds - 1) * cus;   // tiles of the last round
    if (2 * last > cus) return;
    plan.dp_tiles = (int)((rounds - 2) * cus);
    plan.sk_wgs = cus;
}

unsigned long long next_sk_token() {
    static std::atomic<unsigned long long> counter{0};
    return counter.fetch_add(1, std::memory_order_relaxed) + 1;
}

size_t prefill_workspace_bytes(const GemmPlan &plan) {
    if (plan.kind != 1 || plan.sk_wgs == 0) return 0;
    const size_t part = (size_t)plan.sk_wgs * tile_rows(plan.tile) * kTileCols * sizeof(float);
    return part + align_up((size_t)plan.sk_wgs * 8, 256);
}

hipError_t launch_prefill(const void *x, bool bf16, const void *qweight, const void *scales, const void *zeros,
                          void *y, int M, int N, int K, int group, int fmt, const GemmPlan &plan, void *workspace,
                          hipStream_t stream) {
    void *ws = workspace;
    switch (fmt) {
        case kSym4: return launch_prefill_fmt<kSym4>(x, bf16, qweight, scales, zeros, y, M, N, K, group, plan, ws, stream);
        case kSym8: return launch_prefill_fmt<kSym8>(x, bf16, qweight, scales, zeros, y, M, N, K, group, plan, ws, stream);
        case kKq4: return launch_prefill_fmt<kKq4>(x, bf16, qweight, scales, zeros, y, M, N, K, group, plan, ws, stream);
        default: return launch_prefill_fmt<kAsym4>(x, bf16, qweight, scales, zeros, y, M, N, K, group, plan, ws, stream);
    }
}

template hipError_t launch_prefill_fmt<kAsym4>(const void *, bool, const void *, const void *, const void *, void *,
                                               int, int, int, int, const GemmPlan &, void *, hipStream_t);

}  // namespace w4a16
