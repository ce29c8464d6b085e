// Internal declarations shared by the kernels and the C ABI of the gfx950
// W4A16 library. Not installed; the public interface is include/w4a16.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <atomic>

namespace w4a16 {

// Packed device layout. Rows come in blocks of 16 (the last block may hold
// fewer, rows_b = min(16, N - 16 b)); K comes in chunks of 32 weights
// (C = K / 32) grouped in columns of 4 chunks (the last column may hold fewer,
// nc = min(4, C - 4 t)). A chunk of one row is 4 dwords of 8 nibbles; dword d
// holds k = 32 c + 8 d + i (i = 0..7) in nibble i/2 + 4 (i%2), even k in the
// low half-word. Inside column t of block b the dwords are ordered
// [d][row][chunk], so for a full column the 16 bytes at d*256 + r*16 are
// dword d of the column's 4 chunks of row r, and the whole column (16 rows)
// is one contiguous KiB: a wave loads it with one 16-byte load per lane, and
// each lane then holds one 8-weight k-slice of four consecutive chunks, which
// is exactly the B operand of four 16x16x32 MFMAs (one chunk each).
constexpr int kRowBlock = 16;
constexpr int kChunk = 32;
constexpr int kColChunks = 4;

// Metadata (layout 3): row-major, so that one row's metadata along K is
// contiguous. G8 = K / group rounded up to a multiple of 8. Scales [N][G8]
// fp16; zero-points [N][G8 / 8] words of eight 4-bit values (group g of a row
// in bits 4 (g % 8) of the row's word g / 8); K-quant super-block records
// [N][K / 256] of 16 bytes. Padded slots hold 0.
__host__ __device__ inline int meta_slots(int K, int group) { return ((K / group) + 7) & ~7; }

__host__ __device__ inline int64_t dword_offset(int n, int c, int d, int N, int K) {
    const int b = n / kRowBlock, r = n % kRowBlock;
    const int rows_b = (N - b * kRowBlock) < kRowBlock ? (N - b * kRowBlock) : kRowBlock;
    const int C = K / kChunk;
    const int t = c / kColChunks, j = c % kColChunks;
    const int nc = (C - t * kColChunks) < kColChunks ? (C - t * kColChunks) : kColChunks;
    return (int64_t)b * kRowBlock * (K / 8) + (int64_t)t * rows_b * 16 + (int64_t)d * rows_b * nc +
           (int64_t)r * nc + j;
}

// Development-only overrides of the launch plans (tiles, waves, splits):
// read from the environment only in a build compiled with
// -DW4A16_TUNING_KNOBS; the shipped library's dispatch is fixed and the
// fallback is returned.
int tuning_knob(const char *name, int fallback);

// Weight formats (the values of w4a16_format in the public header).
enum { kAsym4 = 0, kSym4 = 1, kSym8 = 2, kKq4 = 3 };

// The dynamic-LDS limit of one kernel (hipFuncAttributeMaxDynamicSharedMemorySize)
// is per kernel and per device. Each launcher keeps one record per kernel;
// raise_dyn_lds sets the attribute on the current device only when a launch
// needs more than was set there before (values only grow, under one lock), so
// steady-state launches make no attribute call and concurrent callers never
// lower a limit another one relies on.
constexpr int kAttrDevices = 64;
struct DynLdsAttr {
    std::atomic<int> set[kAttrDevices];
};
hipError_t raise_dyn_lds(const void *kern, size_t bytes, DynLdsAttr &attr);

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Host-side plan for one decode launch (M <= kDecodeMaxM): `splits`
// workgroups per 16-row block, each over `cols` 128-weight columns of K with
// `waves` waves of `ncol` columns; `mt` activation rows held. ok is false
// when the shape is outside the kernel's range (see decode_plan). N: the rows
// of the launch (all problems of a grouped launch).
constexpr int kDecodeMaxM = 8;
struct DecodePlan {
    int mt, ncol, waves;
    int splits, cols;
    size_t lds;   // dynamic LDS bytes of one workgroup
    bool bcast;   // single launches: the variant with activations in registers (decode_bcast_kernel)
    bool ok;
};
DecodePlan decode_plan(int64_t M, int64_t N, int64_t K, int32_t group, int fmt, bool awq);
// Static LDS of the decode kernel a plan launches (beside plan.lds)
size_t decode_static_lds(const DecodePlan &plan);
// Workspace of a decode launch over N rows: none without a split; else the
// blocks' arrival counters (padded to 256 bytes) and fp32 partials.
size_t decode_workspace_bytes(const DecodePlan &plan, int64_t M, int64_t N);

// Plan for the matrix-core kernels: kind 0 streams the weights through
// registers for M <= kSkinnyMaxM (16-row MFMA tiles of activations, one per
// workgroup), kind 1 is the LDS-tiled GEMM for everything larger.
// measured crossover to the tiled kernel with its K split (N = 15360, K = 5120,
// bf16: M = 32 28.9 against 38.6 us, M = 48 41.1 against 38.5 us)
constexpr int kSkinnyMaxM = 32;
enum { kTile64x256 = 0, kTile128x256 = 1, kTile256x256 = 2, kTile256x256w8 = 3 };
struct GemmPlan {
    int kind;          // 0 = skinny, 1 = tiled
    int waves;         // skinny: waves per workgroup (split K)
    int rows_per_wg;   // skinny: 16-row blocks per workgroup (1, 2, 4)
    int tile;          // tiled: one of kTile*
    int dp_tiles;      // tiled, stream-K: tiles computed whole, one workgroup each
    int sk_wgs;        // tiled, stream-K: workgroups sharing the other tiles' columns (0: none)
    int splits;        // tiled, K split: workgroups per tile (1: none), each `split_cols` columns of K,
    int split_cols;    //   over `split_tiles` tiles
    int split_tiles;
    int sk_expire_test;   // 1: consumers wait for a token no producer writes (exercises the expiry path)
};

// kind: -1 the dispatch's choice (small-batch up to kSkinnyMaxM rows), 0 or 1
// that kind whatever M is
GemmPlan gemm_plan(int64_t M, int64_t N, int64_t K, int32_t group, int kind = -1);
// Compute units of the current device (cached per device; 0 if unknown).
int device_cu_count();
// Tile rows / columns of a tiled kind.
inline int tile_rows(int tile) { return tile == kTile64x256 ? 64 : (tile == kTile128x256 ? 128 : 256); }
constexpr int kTileCols = 256;
constexpr int kMaxTileSplits = 16;   // K split: workgroups per tile at most
// Stream-K split of the tiled GEMM for this shape on `cus` compute units
// (fills plan.dp_tiles / plan.sk_wgs), or its K split when the tiles fill at
// most half the compute units (plan.splits / split_cols / split_tiles), and
// the workspace that needs: stream-K, one fp32 partial tile per stream-K
// workgroup, then one 8-byte flag each; K split, one fp32 partial tile per
// (tile, split), then one 8-byte arrival counter per tile.
void prefill_stream_k(int64_t M, int64_t N, int64_t K, int cus, GemmPlan &plan);
size_t prefill_workspace_bytes(const GemmPlan &plan);
// Stream-K hand-over token: distinct for every launch in this process and
// never 0; a 64-bit mix of a random per-process seed and a counter, so that
// neither flags left by other launches nor whatever the workspace held before
// (small integers, indices) match it except by a 2^-64 chance. A replayed
// graph reuses its token; the consumers clear every flag they used, so a
// complete launch leaves all flags at 0.
unsigned long long next_sk_token();
// Process-wide error word in pinned, device-visible host memory (its address
// on the current device; nullptr before w4a16_init ran on it). A stream-K
// consumer whose bounded wait runs out writes its tile as NaN and sets the
// word; the next compute call takes it and returns W4A16_ERR_HIP.
unsigned int *kernel_error_word();

// Problems of one grouped launch (kernel argument, passed by value).
constexpr int kMaxGroup = 8;
struct GroupTable {
    const void *x[kMaxGroup];
    const void *qweight[kMaxGroup];
    const void *scales[kMaxGroup];
    const void *zeros[kMaxGroup];
    void *y[kMaxGroup];
    int N[kMaxGroup];
    int first[kMaxGroup + 1];   // first workgroup of each problem (set by the launcher)
    int count;
};
// Launchers. `group` is 32, 64, 128 or 256; `fmt` one of kAsym4, kSym4,
// kSym8, kKq4 (zeros is read by kAsym4 only; kKq4 takes group 256 and its
// 16-byte super-block records in `scales`).
hipError_t launch_gemm_group(const GroupTable &tab, bool bf16, int M, int K, int group, int fmt,
                             const GemmPlan &plan, hipStream_t stream);

hipError_t launch_pack(const float *w, int N, int K, int group, int fmt, void *qweight,
                       void *scales, void *zeros, hipStream_t stream);
hipError_t launch_unpack(const void *qweight, const void *scales, const void *zeros,
                         int N, int K, int group, int fmt, uint8_t *codes, uint16_t *scales_out,
                         uint8_t *zeros_out, hipStream_t stream);
// Quality report: five fp64 sums per (row block, slice of K) into `partial`,
// then one workgroup folds them in a fixed order into out[8].
size_t quant_error_partial_bytes(int N, int K);
hipError_t launch_quant_error(const float *w, const void *qweight, const void *scales, const void *zeros,
                              int N, int K, int group, int fmt, double *out, double *partial,
                              hipStream_t stream);
// x_out[m][k] = rne16(x[m][k] * act_mul[k]).
hipError_t launch_scale_activations(const void *x, bool bf16, const float *act_mul, void *x_out, int64_t M,
                                    int K, hipStream_t stream);
// act_mul: NULL, or fp32 activation multipliers [K] (AWQ's run-time scaling);
// workspace: decode_workspace_bytes(plan, M, N) bytes (NULL when that is 0)
hipError_t launch_decode(const void *x, bool bf16, const void *qweight, const void *scales,
                         const void *zeros, void *y, int M, int N, int K, int group, int fmt,
                         const float *act_mul, const DecodePlan &plan, void *workspace, hipStream_t stream);
// plans[p]: the plan of a call on problem p alone (decode_plan with its N)
hipError_t launch_decode_group(const GroupTable &tab, bool bf16, int M, int K, int group, int fmt,
                               const DecodePlan *plans, void *workspace, hipStream_t stream);
// Workspace of that grouped launch: every problem's row-block counters, then
// the partials of the problems that split (0 when none does).
size_t decode_group_workspace_bytes(const DecodePlan *plans, int count, int64_t M, const int *N);
// workspace: prefill_workspace_bytes(plan) bytes (the stream-K partials and
// flags), may be NULL when that is 0
hipError_t launch_gemm(const void *x, bool bf16, const void *qweight, const void *scales,
                       const void *zeros, void *y, int M, int N, int K, int group, int fmt,
                       const GemmPlan &plan, void *workspace, hipStream_t stream);
hipError_t launch_prefill(const void *x, bool bf16, const void *qweight, const void *scales,
                          const void *zeros, void *y, int M, int N, int K, int group, int fmt,
                          const GemmPlan &plan, void *workspace, hipStream_t stream);
int prefill_tile(int64_t M, int64_t N);

// The kernels of one format, each compiled in a translation unit of its own.
#define W4A16_LINEAR_PARAMS const void *x, bool bf16, const void *qweight, const void *scales, const void *zeros, \
                            void *y, int M, int N, int K, int group
template <int FMT>
hipError_t launch_decode_fmt(W4A16_LINEAR_PARAMS, const float *act_mul, const DecodePlan &plan, void *workspace,
                             hipStream_t stream);
template <int FMT>
hipError_t launch_decode_group_fmt(const GroupTable &tab, bool bf16, int M, int K, int group, const DecodePlan *plans,
                                   void *workspace, hipStream_t stream);
template <int FMT> hipError_t launch_skinny_fmt(W4A16_LINEAR_PARAMS, const GemmPlan &plan, hipStream_t stream);
template <int FMT>
hipError_t launch_prefill_fmt(W4A16_LINEAR_PARAMS, const GemmPlan &plan, void *workspace, hipStream_t stream);
template <int FMT>
hipError_t launch_skinny_group_fmt(const GroupTable &tab, bool bf16, int M, int K, int group, const GemmPlan &plan,
                                   hipStream_t stream);
#define W4A16_EXTERN_FMT(F)                                                                              \
    extern template hipError_t launch_decode_fmt<F>(W4A16_LINEAR_PARAMS, const float *, const DecodePlan &, \
                                                    void *, hipStream_t);                                 \
    extern template hipError_t launch_decode_group_fmt<F>(const GroupTable &, bool, int, int, int,        \
                                                          const DecodePlan *, void *, hipStream_t);       \
    extern template hipError_t launch_skinny_fmt<F>(W4A16_LINEAR_PARAMS, const GemmPlan &, hipStream_t); \
    extern template hipError_t launch_prefill_fmt<F>(W4A16_LINEAR_PARAMS, const GemmPlan &, void *, hipStream_t); \
    extern template hipError_t launch_skinny_group_fmt<F>(const GroupTable &, bool, int, int, int,        \
                                                          const GemmPlan &, hipStream_t);
W4A16_EXTERN_FMT(kAsym4)
W4A16_EXTERN_FMT(kSym4)
W4A16_EXTERN_FMT(kSym8)
W4A16_EXTERN_FMT(kKq4)
#undef W4A16_EXTERN_FMT

__device__ inline uint16_t f32_to_f16_bits(float v) {
    _Float16 h = (_Float16)v;
    return __builtin_bit_cast(uint16_t, h);
}
__device__ inline uint16_t f32_to_bf16_bits(float v) {
    __bf16 h = (__bf16)v;
    return __builtin_bit_cast(uint16_t, h);
}

}  // namespace w4a16
