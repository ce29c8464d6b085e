// Tiled matrix-core path (large M), host side: the tile choice and the
// dispatch over the weight formats. The kernel is in prefill_kernel.hpp; each
// weight format is compiled in its own translation unit (this one: the 4-bit
// zero-point format; prefill_sym4.hip, prefill_sym8.hip).
#include <algorithm>
#include <chrono>
#include <random>

#include "prefill_kernel.hpp"

namespace w4a16 {

int prefill_tile(int64_t M, int64_t N) {
    const int forced = tuning_knob("W4A16_PREFILL_TILE", -1);
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
// 283 us either way; 264 tiles: 266 -> 185 us). Measured on MI355X it pays
// from 16 columns per tile (K >= 2048: M = 2048, N = 8448 at K = 2048 102
// against 117 us, at K = 1024 77 against 65 us) and while the whole-tile rounds
// are few (at most four: seven rounds at M = 4096, N = 24832, K = 2048: 457
// against 433 us).
//
// K split for a grid too small for the device: with at most half as many
// tiles as compute units (mid-size batches: M = 64, N = 15360 is 60 tiles of
// 64 x 256), every tile walks all of K on one compute unit while the others
// idle. Its columns are then split over S workgroups (S = CUs / tiles, at
// most 16, each range at least 4 columns; S recomputed so that no range is
// empty); each leaves an fp32 partial tile and the last to arrive adds the S
// partials in split order (the kernel's split epilogue). Tiles of 4 waves
// only (64 and 128 rows). Between those two the plan takes the one with less
// work per workgroup, rows x columns, over its rounds (equal: 128 rows).
// Measured on MI355X, N = 15360, K = 5120, bf16: M = 64, 64-row tiles split 4
// ways 37 us (128-row 52); M = 128, 128-row tiles split 4 ways 49 us (64-row
// split 2 ways 54.5); M = 192 and 256, 128-row tiles split 2 ways 70 / 68 us
// (64-row whole tiles 78 / 77); a second workgroup per compute unit (twice
// the splits) was slower everywhere (61 us at M = 64).
struct TileSplit {
    int64_t tiles, splits, cols;
};
static TileSplit split_of(int tile, int64_t M, int64_t N, int64_t T, int cus) {
    TileSplit s{ceil_div(M, tile_rows(tile)) * ceil_div(N, kTileCols), 1, T};
    if (cus < 8 || 2 * s.tiles > cus) return s;
    int64_t S = std::min<int64_t>({(int64_t)cus / s.tiles, T / 4, (int64_t)kMaxTileSplits});
    if (S < 2) return s;
    const int64_t cols = ceil_div(T, S);
    S = ceil_div(T, cols);
    if (S < 2) return s;
    s.splits = S;
    s.cols = cols;
    return s;
}
static void prefill_split_k(int64_t M, int64_t N, int64_t K, int cus, GemmPlan &plan) {
    plan.splits = 1;
    plan.split_cols = 0;
    plan.split_tiles = 0;
    if (tuning_knob("W4A16_PREFILL_SPLIT", 1) != 1) return;
    if (plan.tile != kTile64x256 && plan.tile != kTile128x256) return;
    const int64_t T = ceil_div(K / kChunk, kColChunks);
    const TileSplit s64 = split_of(kTile64x256, M, N, T, cus), s128 = split_of(kTile128x256, M, N, T, cus);
    if (s64.splits == 1 && s128.splits == 1) return;
    auto work = [&](const TileSplit &s, int rows) {
        return (double)rows * (double)s.cols * (double)ceil_div(s.tiles * s.splits, cus > 0 ? cus : 1);
    };
    const bool use128 = work(s128, 128) <= work(s64, 64);
    const TileSplit &s = use128 ? s128 : s64;
    plan.tile = use128 ? kTile128x256 : kTile64x256;
    if (s.splits < 2) return;
    plan.splits = (int)s.splits;
    plan.split_cols = (int)s.cols;
    plan.split_tiles = (int)s.tiles;
}

void prefill_stream_k(int64_t M, int64_t N, int64_t K, int cus, GemmPlan &plan) {
    const int enabled = tuning_knob("W4A16_PREFILL_SK", 1);
    plan.dp_tiles = 0;
    plan.sk_wgs = 0;
    prefill_split_k(M, N, K, cus, plan);
    if (plan.splits > 1) return;
    const int64_t tiles = ceil_div(M, tile_rows(plan.tile)) * ceil_div(N, kTileCols);
    const int64_t T = ceil_div(K / kChunk, kColChunks);
    if (!enabled || cus < 8 || T < 16 || tiles <= cus) return;
    const int64_t rounds = ceil_div(tiles, cus);
    if (rounds > 4) return;
    const int64_t last = tiles - (rounds - 1) * cus;   // tiles of the last round
    if (2 * last > cus) return;
    plan.dp_tiles = (int)((rounds - 2) * cus);
    plan.sk_wgs = cus;
}

// splitmix64's output function (Steele, Lea and Flood, "Fast splittable
// pseudorandom number generators", 2014): a bijection of 64-bit words, so
// distinct counter values give distinct tokens.
static unsigned long long mix64(unsigned long long z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static unsigned long long token_seed() {
    std::random_device rd;
    unsigned long long s = ((unsigned long long)rd() << 32) ^ rd();
    s ^= (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count();
    return s;
}

unsigned long long next_sk_token() {
    static const unsigned long long seed = token_seed();
    static std::atomic<unsigned long long> counter{0};
    const unsigned long long c = counter.fetch_add(1, std::memory_order_relaxed);
    const unsigned long long t = mix64(seed + c * 0x9E3779B97F4A7C15ull);
    return t != 0 ? t : 0x9E3779B97F4A7C15ull;   // 0 marks an empty flag
}

size_t prefill_workspace_bytes(const GemmPlan &plan) {
    if (plan.kind != 1) return 0;
    if (plan.splits > 1)   // partial tiles [tiles][splits][rows x 256] fp32, then a counter per tile
        return (size_t)plan.split_tiles * plan.splits * tile_rows(plan.tile) * kTileCols * sizeof(float) +
               align_up((size_t)plan.split_tiles * 8, 256);
    if (plan.sk_wgs == 0) return 0;
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
