// Matrix-core GEMM of the W4A16 linear layer for larger batches and prefill
// (M above the small-batch kernels' range): y[m][n] = sum_k x[m][k] * w_hat[n][k].
//
// At prefill the same packed weights serve many tokens, so the layer turns
// compute bound and the dequantisation sits on the critical path of a dense
// matrix product ("Weight-Only Quantisation", the FAQ answers on batch size
// and on where the time goes; "Weight-Only Quantization Explained", the
// section on where the method stops paying). Each workgroup therefore
// rebuilds its weight tile once, in LDS, as 16-bit values w_hat = s*(q - z)
// (one rounding from the exact product), and feeds the matrix cores from
// there ("Weight-Only Quantisation": the low-bit weights are turned back into
// 16-bit values right before the multiply).
//
// Tiling (gfx950, wave64): a workgroup computes a BM x BN tile of y with
// WM x WN waves (4, or 8 for the 256 x 256 tile: two per SIMD), each owning a
// (BM/WM) x (BN/WN) sub-tile as 32x32 blocks of
// v_mfma_f32_32x32x16 accumulators (fp32). K advances in steps of 64 through
// two LDS buffers: while the waves multiply out of one buffer they write the
// next step's activations and dequantised weights into the other, and the
// global loads for the step after that are already in flight. Both LDS tiles
// are [row][64 k] 16-bit with the eight 16-byte units of a row XOR-swizzled
// (swz below), so the MFMA operand reads (32 rows, same k) and the tile writes
// are free of bank conflicts. The packed weights arrive one 128-weight
// column at a time (16-byte records, one KiB per 16 rows) and serve two steps.
// Weight formats (FMT) differ only in the dequantisation into LDS: a fixed
// zero (symmetric 4-bit), c - 128 rebuilt from two code planes (8-bit), or
// S q - M per 32-weight sub-block from the super-block record (K-quant), each
// formed in fp32 and rounded once to 16 bit.
#pragma once

#include <stdlib.h>

#include "decode_common.hpp"

namespace w4a16 {
namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f16_t __attribute__((ext_vector_type(16)));

constexpr int kStepK = 64;                    // k per LDS step
struct Plain { static constexpr bool value = false; };
struct Masked { static constexpr bool value = true; };
constexpr Plain kPlain{};
constexpr Masked kMasked{};
// the weight column to prefetch: any column, or one known to hold all four chunks
struct AnyColumn { static constexpr bool value = false; };
struct FullColumn { static constexpr bool value = true; };
constexpr AnyColumn kAnyColumn{};
constexpr FullColumn kFullColumn{};
constexpr int kUnits = kStepK / 8;            // 16-byte units per tile row

template <bool BF>
__device__ inline f16_t mfma32x32x16(const uint4 &a, const uint4 &b, f16_t c) {
    if constexpr (BF)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(b8_t, a), __builtin_bit_cast(b8_t, b),
                                                        c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8_t, a), __builtin_bit_cast(h8_t, b),
                                                       c, 0, 0, 0);
}

// Unit u of tile row `row` sits at position u ^ f(row), f(row) = (row % 8) ^
// ((row / 8) % 2). Any 8 consecutive rows get 8 different positions, and so
// do the 8 even (or odd) rows of any aligned 16: 16-byte accesses of 8 or 16
// lanes at a time that walk down the rows hit all banks once whether the LDS
// serves 128 or 256 bytes per cycle.
__device__ inline int swz(int row, int unit) { return row * kUnits + (unit ^ (row & 7) ^ ((row >> 3) & 1)); }

// One dword of codes (k = 0..7 of a slice, even k in the low half-word) ->
// eight 16-bit values (bf16, or fp16) s*(q - z) in k order. The magic-number unpack gives the
// exact fp16 values 1024 + q (low nibble of a byte) and 1024 + 16 q (high
// nibble); one fma with an fp16 operand (v_fma_mix_f32) then forms
// s*(1024+q) - s*(1024+z) = s*(q - z), or (s/16)*(1024+16q) - s*(64+z), where
// every product and both constants are exact in fp32 (at most 22 significant
// bits), so the fma returns s*(q - z) exactly (15 significant bits at most) and
// the conversion to bf16 (or fp16: v_cvt_pk_f16_f32) is its one rounding, to
// nearest even. For fp16 this is the value an fp16 multiply of the exact
// (q - z) by s gives (one rounding of the same exact product); going through
// fp32 keeps fewer packed intermediates live than the fp16 route.
struct DequantConsts {
    float s, c_lo, s16, c_hi;   // s, -s*(1024+z), s/16, -s*(64+z)
};
__device__ inline DequantConsts dequant_consts(float s, uint32_t z) {
    return DequantConsts{s, -s * (float)(1024u + z), s * 0.0625f, -s * (float)(64u + z)};
}
template <bool BF>
__device__ inline uint4 dequant_16(uint32_t d, const DequantConsts &c, const UnpackConsts &uc) {
    const uint32_t d8 = d >> 8;
    const half2_t h0 = __builtin_bit_cast(half2_t, and_or(d, uc.lo_mask, uc.f16_magic));    // k0, k1
    const half2_t h1 = __builtin_bit_cast(half2_t, and_or(d, uc.hi_mask, uc.f16_magic));    // k2, k3 (x16)
    const half2_t h2 = __builtin_bit_cast(half2_t, and_or(d8, uc.lo_mask, uc.f16_magic));   // k4, k5
    const half2_t h3 = __builtin_bit_cast(half2_t, and_or(d8, uc.hi_mask, uc.f16_magic));   // k6, k7 (x16)
    auto lo = [&](_Float16 h) { return fmaf(c.s, (float)h, c.c_lo); };
    auto hi = [&](_Float16 h) { return fmaf(c.s16, (float)h, c.c_hi); };
    auto pk = [](float a, float b) {
        if constexpr (BF)
            return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{a, b}, bf162_t));
        else
            return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{a, b}, half2_t));
    };
    return make_uint4(pk(lo(h0.x), lo(h0.y)), pk(hi(h1.x), hi(h1.y)), pk(lo(h2.x), lo(h2.y)),
                      pk(hi(h3.x), hi(h3.y)));
}

// 8-bit codes (two planes, dwords d and dh of the same k-slice): the exact
// fp16 integers c - 128, then s*(c - 128) in fp32 (at most 19 significant
// bits: exact) and its one rounding to bf16.
__device__ inline uint4 dequant_bf16_s8(uint32_t d, uint32_t dh, float s, const UnpackConsts &uc) {
    uint32_t t[4];
    unpack_f16_s8(d, dh, uc, t);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const half2_t h = __builtin_bit_cast(half2_t, t[i]);
        o[i] = __builtin_bit_cast(uint32_t,
                                  __builtin_convertvector(float2_t{s * (float)h.x, s * (float)h.y}, bf162_t));
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// kq4 sub-block (scale S, minimum M): the exact codes q as fp16 pairs, then
// w_hat = S q - M by one fp32 fma (rounded once) and one rounding to 16 bit.
template <bool BF>
__device__ inline uint4 dequant_kq(uint32_t d, const KqParams &P, const UnpackConsts &uc) {
    uint32_t t[4];
    unpack_f16(d, 0u, uc, t);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const half2_t h = __builtin_bit_cast(half2_t, t[i]);
        const float2_t v = {fmaf(P.S, (float)h.x, -P.M), fmaf(P.S, (float)h.y, -P.M)};
        if constexpr (BF)
            o[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf162_t));
        else
            o[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, half2_t));
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// Same for fp16: exact (code - z) pairs, then one fp16 multiply by s.
template <int FMT>
__device__ inline uint4 dequant_f16(uint32_t d, uint32_t dh, uint32_t z, _Float16 sh, const UnpackConsts &uc) {
    uint32_t t[4];
    unpack_f16_fmt<FMT>(d, dh, z, uc, t);
    const half2_t s2 = {sh, sh};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, t[i]) * s2);
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// SK: compiled with the stream-K segments; without (every workgroup one whole
// tile) the segment loop and hand-over code vanish, so the whole-tile
// launches keep the registers of a plain tiled kernel.
template <int BM, int BN, int WM, int WN, int GROUP, bool BF, int FMT, bool SK>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(WM * WN / 4, WM * WN / 4))) void prefill_kernel(
    const uint16_t *__restrict__ x, const uint4 *__restrict__ qw, const uint4 *__restrict__ qw_hi,
    const uint16_t *__restrict__ scales, const uint32_t *__restrict__ zeros, uint16_t *__restrict__ y, int M,
    int N, int K, int m_tiles, int n_tiles, int mshift, int dp_tiles, int sk_wgs, int raster, int splits,
    int split_cols, float4 *__restrict__ partials,
    unsigned long long *__restrict__ flags, unsigned long long token, unsigned long long wait_token,
    unsigned int *__restrict__ err) {
    using FT = FormatTraits<FMT>;
    constexpr int NT = 64 * WM * WN;                 // threads
    constexpr int TM = BM / WM / 32, TN = BN / WN / 32;   // 32x32 blocks per wave
    constexpr int RB = BN / kRowBlock;               // row blocks per tile
    constexpr int WREC = RB * 64 / NT;               // packed records per thread per column
    constexpr int XREC = BM * kUnits / NT;           // activation units per thread per step
    constexpr int CPG = GROUP / kChunk;
    constexpr int GPC = kColumn / GROUP;
    static_assert(RB * 64 % NT == 0 && BM * kUnits % NT == 0, "tile / thread mismatch");

    extern __shared__ __align__(16) unsigned char smem[];

    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;

    const int C = K / kChunk;
    const int T = (C + kColChunks - 1) / kColChunks;
    const int steps = (C + 1) / 2;                   // 64-k steps (the last may hold one chunk)
    const int nblocks = (N + kRowBlock - 1) / kRowBlock;
    const int t_full = C / kColChunks;               // columns with all four chunks

    // ---- schedule. Tile ids walk M first, so the M tiles that share a
    // weight tile run side by side. Workgroups are dealt to the eight XCDs
    // round-robin: ids are remapped so each XCD gets a contiguous range (and
    // keeps the shared weight tiles in its own L2).
    // Workgroups below dp_tiles compute one whole tile each. The other sk_wgs
    // workgroups (stream-K) split the remaining tiles' columns evenly: workgroup
    // s takes units [s U / sk_wgs, (s+1) U / sk_wgs) of the U = tiles x T
    // (tile, column) units, at least T of them, so it touches at most three
    // tiles and a tile is shared by at most two workgroups. It runs its whole
    // tiles first, then the head (first columns) of its last tile, whose fp32
    // partial it leaves in `partials` slot s and announces with flags[s] =
    // token, and last the tail of its first tile, which it finishes with the
    // partial of workgroup s - 1. A workgroup waits only after producing, and
    // only for a lower s (dispatched earlier except across an XCD's range
    // boundary, where the producer never waits before producing), so every
    // wait ends. The partial is added after the workgroup's own columns, always
    // in this order, so results do not depend on timing.
    const int tiles = m_tiles * n_tiles;
    int ft, lt, fb, le, s_sk = -1;   // first / last tile, first column of the first, end column of the last
    // K split (4-wave tiles, plan.splits > 1): workgroup id takes columns
    // [j c, min((j + 1) c, T)) of tile id / S, j = id % S, c = split_cols
    constexpr bool kCanSplit = SK && WM * WN == 4 && BM <= 128;
    int piece = -1;
    if (kCanSplit && splits > 1) {
        piece = (int)blockIdx.x % splits;
        ft = lt = (int)blockIdx.x / splits;
        fb = piece * split_cols;
        le = min(fb + split_cols, T);
    } else if ((int)blockIdx.x < dp_tiles) {
        int id = blockIdx.x;
        if (raster) {
            // M bands: XCD j takes the band of m_tiles / 8 M tiles j * band ..
            // and every N tile, band first, so its activation rows (one band:
            // 2.6 MB at BM = 256, K = 5120) stay in its L2 and each weight
            // tile is read once per XCD (raster set only when m_tiles % 8 == 0
            // and dp_tiles is a multiple of m_tiles)
            const int band = m_tiles >> 3, xcd = id & 7, l = id >> 3;
            id = (l / band) * m_tiles + xcd * band + l % band;
        } else if (dp_tiles % 8 == 0) {
            id = (id % 8) * (dp_tiles / 8) + id / 8;
        }
        ft = lt = id;
        fb = 0;
        le = T;
    } else {
        const int b = blockIdx.x - dp_tiles;
        s_sk = (sk_wgs % 8 == 0) ? (b % 8) * (sk_wgs / 8) + b / 8 : b;
        const int64_t U = (int64_t)(tiles - dp_tiles) * T;
        const int64_t lo = (int64_t)s_sk * U / sk_wgs, hi = (int64_t)(s_sk + 1) * U / sk_wgs;
        ft = (int)(lo / T);
        lt = (int)((hi - 1) / T);
        fb = (int)(lo - (int64_t)ft * T);
        le = (int)(hi - (int64_t)lt * T);
        ft += dp_tiles;
        lt += dp_tiles;
    }
    // (uniform: keep the schedule in scalar registers)
    ft = __builtin_amdgcn_readfirstlane(ft);
    lt = __builtin_amdgcn_readfirstlane(lt);
    fb = __builtin_amdgcn_readfirstlane(fb);
    le = __builtin_amdgcn_readfirstlane(le);
    s_sk = __builtin_amdgcn_readfirstlane(s_sk);
    piece = __builtin_amdgcn_readfirstlane(piece);
    const bool split_piece = kCanSplit && piece >= 0;
    const int full_lo = fb == 0 ? ft : ft + 1;     // whole tiles full_lo..full_hi
    const int full_hi = le == T ? lt : lt - 1;
    const int n_full = split_piece ? 0 : max(0, full_hi - full_lo + 1);
    const bool has_head = !split_piece && le < T, has_tail = !split_piece && fb > 0;
    const int n_seg = split_piece ? 1 : n_full + (has_head ? 1 : 0) + (has_tail ? 1 : 0);

    const int G8 = meta_slots(K, GROUP << mshift);   // metadata slots per row (group 256: mshift = 1)
    const ColScales<GPC> *scol = reinterpret_cast<const ColScales<GPC> *>(scales);
    const uint4 *kqrec = reinterpret_cast<const uint4 *>(scales);
    const UnpackConsts uc = unpack_consts();
    const uint4 *xg = reinterpret_cast<const uint4 *>(x);
    const int k8_total = K / 8;
    // LDS: activations [2][BM][8] then weights [2][BN][8] (16-byte units, two buffers)
    uint4 *xs0 = reinterpret_cast<uint4 *>(smem), *xs1 = xs0 + BM * kUnits;
    uint4 *ws0 = xs0 + 2 * BM * kUnits, *ws1 = ws0 + BN * kUnits;

    for (int seg = 0; seg < (SK ? n_seg : 1); ++seg) {
        // segment seg: a whole tile, the head [0, le) of tile lt, or the tail
        // [fb, T) of tile ft
        // (kind 3: a piece [fb, le) of tile ft of the K split)
        const int kind = __builtin_amdgcn_readfirstlane(
            split_piece ? 3 : (seg < n_full ? 0 : ((seg == n_full && has_head) ? 1 : 2)));
        const int id = __builtin_amdgcn_readfirstlane(kind == 0 ? full_lo + seg : (kind == 1 ? lt : ft));
        const int tb = (kind == 2 || kind == 3) ? fb : 0, te = (kind == 1 || kind == 3) ? le : T;
        const int mt = __builtin_amdgcn_readfirstlane(id % m_tiles), nt = __builtin_amdgcn_readfirstlane(id / m_tiles);
        const int m0 = mt * BM, n0 = nt * BN;
        if (seg > 0) __syncthreads();   // the previous segment's last reads of both LDS buffers are done
        // The thread's per-segment values (offsets, LDS addresses) derive from a
        // copy of its index that the compiler cannot see through, so they are
        // computed per segment instead of being hoisted out of the segment loop
        // and kept live (spilled) through the hand-over code.
        int tid_v = (int)threadIdx.x;
        asm volatile("" : "+v"(tid_v));
        const int tid = tid_v;
        const int lane = tid & 63;
        const int d = lane >> 4, r = lane & 15;
        const int xu = tid % kUnits;

        // ---- weight records of this thread: row block i * waves + wave of the
        // tile, record = lane (d = lane / 16, r = lane % 16: dword d of the
        // column's four chunks of row r). Offsets are 32-bit element indices.
        uint32_t woff[WREC], wstep[WREC], soff[WREC], zoff[WREC];
        int wrow[WREC], wrows[WREC];
#pragma unroll
        for (int i = 0; i < WREC; ++i) {
            const int rb = i * (NT / 64) + wave;
            const int b = min(n0 / kRowBlock + rb, nblocks - 1);   // past the last block: repeat it (not stored)
            const int rows = min(kRowBlock, N - b * kRowBlock);
            const int rl = r < rows ? r : r - rows;                 // lanes past a short block re-read a valid row
            const int n = b * kRowBlock + rl;
            wrows[i] = rows;
            woff[i] = (uint32_t)b * (uint32_t)(K / 2) + (uint32_t)(d * rows + rl);    // uint4 index, column 0 (a block is K/2 uint4)
            wstep[i] = (uint32_t)(kColChunks * rows);                                 // uint4 per column
            // the row's metadata: ColScales index of its first column (kq4: its
            // first super-block record) and its first zero-point word
            soff[i] = FT::kquant ? (uint32_t)n * (uint32_t)(K / 256) : (uint32_t)n * (uint32_t)(G8 / GPC);
            zoff[i] = (uint32_t)n * (uint32_t)(G8 / 8);
            wrow[i] = rb * kRowBlock + r;                                             // LDS row
        }
        struct WCol {
            uint4 rec[WREC], rec_hi[WREC];   // rec_hi: high-nibble plane of 8-bit codes
            uint4 kq[WREC];                  // kq4: the super-block record of the column's row
            ColScales<GPC> sc[WREC];
            uint32_t zw[WREC];               // zero-point words as loaded
            int zsh;                         // bit offset of the column's first zero-point in zw
            int par;                         // kq4: column parity (half of the super-block)
        };
        // (with `full` known true the column's loads have no branch: whole-tile
        // launches keep them in the loop body's one basic block, as 16-byte loads)
        auto load_wcol = [&](int t, WCol &u, auto full) __attribute__((always_inline)) {
            u.par = t & 1;
#pragma unroll
            for (int i = 0; i < WREC; ++i) {
                if (decltype(full)::value || t < t_full) {
                    u.rec[i] = qw[woff[i] + (uint32_t)t * wstep[i]];
                    if constexpr (FT::two_planes) u.rec_hi[i] = qw_hi[woff[i] + (uint32_t)t * wstep[i]];
                } else {   // partial last column: nc dwords per (d, row), missing chunks are zero codes
                    const int nc = C - t * kColChunks;
                    const int rl = r < wrows[i] ? r : r - wrows[i];
                    const uint32_t blk = woff[i] - (uint32_t)(d * wrows[i] + rl);   // row block base, uint4
                    const size_t off = (size_t)t * wrows[i] * 16 + (size_t)(d * wrows[i] + rl) * nc;
                    const uint32_t *col = reinterpret_cast<const uint32_t *>(qw + blk) + off;
                    uint32_t v[4];
#pragma unroll
                    for (int j = 0; j < kColChunks; ++j) v[j] = j < nc ? col[j] : 0u;
                    u.rec[i] = make_uint4(v[0], v[1], v[2], v[3]);
                    if constexpr (FT::two_planes) {
                        const uint32_t *colh = reinterpret_cast<const uint32_t *>(qw_hi + blk) + off;
#pragma unroll
                        for (int j = 0; j < kColChunks; ++j) v[j] = j < nc ? colh[j] : 0u;
                        u.rec_hi[i] = make_uint4(v[0], v[1], v[2], v[3]);
                    }
                }
                // metadata slot of column t: t >> mshift (group 256: one slot per
                // two columns); the zero-point word is shifted where it is used
                // (a shift here would wait for the load at once, and for every
                // load issued before it)
                const uint32_t tm = (uint32_t)(t >> mshift);
                u.zsh = (int)(4 * ((tm * GPC) & 7));
                if constexpr (FT::kquant) {
                    u.kq[i] = kqrec[soff[i] + (uint32_t)(t >> 1)];
                } else {
                    u.sc[i] = scol[soff[i] + tm];
                    if constexpr (FT::has_zeros)
                        u.zw[i] = zeros[zoff[i] + ((tm * GPC) >> 3)];
                    else
                        u.zw[i] = 0;
                }
            }
        };
        // dequantise half h (chunks 2h, 2h+1) of weight record i into LDS;
        // chunks past K (partial last column) have zero codes and zero scale
        auto store_w_rec = [&](const WCol &u, int i, int h, uint4 *wbuf) __attribute__((always_inline)) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const uint32_t dw = h ? (jj ? u.rec[i].w : u.rec[i].z) : (jj ? u.rec[i].y : u.rec[i].x);
                const uint32_t dh = h ? (jj ? u.rec_hi[i].w : u.rec_hi[i].z) : (jj ? u.rec_hi[i].y : u.rec_hi[i].x);
                const int e = (2 * h + jj) / CPG;
                uint32_t z = FT::fixed_zero;
                if constexpr (FT::has_zeros) z = (u.zw[i] >> (u.zsh + 4 * e)) & 0xFu;
                uint4 v;
                if constexpr (FT::kquant) {
                    v = dequant_kq<BF>(dw, kq_sub(kq_half(u.kq[i], u.par != 0), 2 * h + jj), uc);
                    wbuf[swz(wrow[i], 4 * jj + d)] = v;
                    continue;
                }
                const float s = u.sc[i].get(e);
                if constexpr (BF && FT::two_planes)
                    v = dequant_bf16_s8(dw, dh, s, uc);
                else if constexpr (!FT::two_planes && (BF || GROUP >= 128))
                    // (fp16 through fp32 too at group 128 (and 256), where it is
                    // faster: M = 2048, N = 13824, K = 5120: 282 against 298 us,
                    // M = 512: 98 against 106 us; at groups 32 and 64 the packed
                    // fp16 route, with fewer per-group constants, is faster:
                    // 282 against 292 us, 92 against 97 us)
                    v = dequant_16<BF>(dw, dequant_consts(s, z), uc);
                else
                    v = dequant_f16<FMT>(dw, dh, z, (_Float16)s, uc);
                wbuf[swz(wrow[i], 4 * jj + d)] = v;
            }
        };

        // ---- activation units of this thread: tile row (i * NT + tid) / 8, unit
        // tid % 8 of the step; units past K read as zero
        uint32_t xoff[XREC];
#pragma unroll
        for (int i = 0; i < XREC; ++i) {
            const int row = (i * NT + tid) / kUnits;
            xoff[i] = (uint32_t)min(m0 + row, M - 1) * (uint32_t)(K / 8) + (uint32_t)xu;   // rows past M repeat the last
        }
        // Steps that may reach past K (the partial last column) zero those units:
        // the address is clamped into the row and the value masked, so the load
        // stays unconditional (no branch splits the interleaved step).
        auto load_x_unit = [&](int i, int step_idx, auto masked) __attribute__((always_inline)) {
            if constexpr (!decltype(masked)::value) return xg[xoff[i] + (uint32_t)(step_idx * kUnits)];
            const int k8 = step_idx * kUnits + xu;
            uint4 v = xg[xoff[i] + (uint32_t)(min(k8, k8_total - 1) - xu)];
            const uint32_t keep = 0u - (uint32_t)(k8 < k8_total);
            v.x &= keep;
            v.y &= keep;
            v.z &= keep;
            v.w &= keep;
            return v;
        };
        uint4 xv[XREC];

        f16_t acc[TM][TN];
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int b = 0; b < TN; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

        // One 64-k step out of LDS (4 sub-steps of 16 k), with the operands of
        // the next step written into the other buffer in between: sub-step kk
        // also dequantises weight record kk (both of its chunks of half h) and
        // moves every fourth activation unit from registers to LDS, reloading the
        // register with the unit of the step after (x_next). Fragment reads run
        // one sub-step ahead of the MFMAs that use them.
        auto step = [&](const uint4 *xb, const uint4 *wb, const WCol &u, int h, uint4 *wdst, uint4 *xdst,
                        int x_next, auto masked) __attribute__((always_inline)) {
            const int rsel = lane & 31, khalf = lane >> 5;
            if constexpr (!SK) {
                // whole tiles: each sub-step's activation load is issued ahead
                // of its eight MFMAs, where the scheduler would otherwise sink
                // all four to the end of the step and leave the next step's
                // first LDS write waiting on them (measured 2-4 % faster:
                // M = 2048, N = 13824, K = 5120 286 -> 279.5 us, M = 1024
                // 145.6 -> 141.8 us; the stream-K segments keep the
                // scheduler's own order, measured faster for them)
#pragma unroll
                for (int g = 0; g < kStepK / 16; ++g) {
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one vector-memory read
                    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);   // eight MFMAs
                }
            }
            uint4 af[2][TM], bfr[2][TN];
            auto read = [&](int kk, uint4 (&a_)[TM], uint4 (&b_)[TN]) __attribute__((always_inline)) {
#pragma unroll
                for (int a = 0; a < TM; ++a) a_[a] = xb[swz(wm * (BM / WM) + 32 * a + rsel, 2 * kk + khalf)];
#pragma unroll
                for (int b = 0; b < TN; ++b) b_[b] = wb[swz(wn * (BN / WN) + 32 * b + rsel, 2 * kk + khalf)];
            };
            // one wave per SIMD: fragment reads run one sub-step ahead; two waves
            // per SIMD: read just before use (the other wave covers the latency,
            // and the registers are needed for its accumulators)
            constexpr bool kAhead = WM * WN == 4;
            read(0, af[0], bfr[0]);
#pragma unroll
            for (int kk = 0; kk < kStepK / 16; ++kk) {
                if constexpr (kAhead) {
                    if (kk + 1 < kStepK / 16) read(kk + 1, af[(kk + 1) & 1], bfr[(kk + 1) & 1]);
                } else if (kk > 0) {
                    read(kk, af[kk & 1], bfr[kk & 1]);
                }
                if (kk < WREC) store_w_rec(u, kk, h, wdst);
#pragma unroll
                for (int i = kk; i < XREC; i += kStepK / 16) {
                    xdst[swz((i * NT + tid) / kUnits, xu)] = xv[i];
                    xv[i] = load_x_unit(i, x_next, masked);
                }
#pragma unroll
                for (int a = 0; a < TM; ++a)
#pragma unroll
                    for (int b = 0; b < TN; ++b)
                        acc[a][b] = mfma32x32x16<BF>(af[kk & 1][a], bfr[kk & 1][b], acc[a][b]);
            }
        };

        // ---- main loop over the segment's full columns [tb, te): iteration t
        // multiplies steps 2t (buffer 0) and 2t+1 (buffer 1) and writes steps
        // 2t+1 and 2t+2. Loads past the end of the segment or of K are clamped to
        // valid addresses; what they bring is written into a buffer that is never
        // multiplied.
        WCol wcur, wnext;
        load_wcol(tb, wcur, kAnyColumn);
#pragma unroll
        for (int i = 0; i < XREC; ++i) xv[i] = load_x_unit(i, 2 * tb, kMasked);
        load_wcol(min(tb + 1, T - 1), wnext, kAnyColumn);
#pragma unroll
        for (int i = 0; i < WREC; ++i) store_w_rec(wcur, i, 0, ws0);
#pragma unroll
        for (int i = 0; i < XREC; ++i) {
            xs0[swz((i * NT + tid) / kUnits, xu)] = xv[i];
            xv[i] = load_x_unit(i, min(2 * tb + 1, steps - 1), kMasked);
        }
        __syncthreads();
        // (the activation loads of the last full column reach the steps after it:
        // those are the masked ones)
        auto column = [&](int t, auto masked, auto next_full) __attribute__((always_inline)) {
            step(xs0, ws0, wcur, 1, ws1, xs1, min(2 * t + 2, steps - 1), masked);
            __syncthreads();
            wcur = wnext;
            load_wcol(min(t + 2, T - 1), wnext, next_full);
            step(xs1, ws1, wcur, 0, ws0, xs0, min(2 * t + 3, steps - 1), masked);
            __syncthreads();
        };
        const int te_full = min(te, t_full);
        int t = tb;
        // whole tiles: the steady state, where the column two ahead is a full one
        if constexpr (!SK)
            for (; t + 1 < te_full && t + 2 < t_full; ++t) column(t, kPlain, kFullColumn);
        for (; t + 1 < te_full; ++t) column(t, kPlain, kAnyColumn);
        if (te_full > tb) column(te_full - 1, kMasked, kAnyColumn);
        // the partial last column (K % 128 != 0; only a segment that ends the
        // tile's K has it): one or two more steps; its missing chunks have zero
        // codes and zero activations
        if (te == T && t_full < T) {
            const int s0 = 2 * t_full;
            const bool two = s0 + 1 < steps;
            step(xs0, ws0, wcur, 1, ws1, xs1, min(s0 + 2, steps - 1), kMasked);
            __syncthreads();
            if (two) step(xs1, ws1, wcur, 0, ws0, xs0, min(s0 + 2, steps - 1), kMasked);
        }

        // ---- K split: this piece's fp32 partial into slot (tile, piece), then
        // the arrival on the tile's counter; the last arrival adds the S
        // partials in split order (so the result does not depend on which one
        // is last) and stores the tile. Partials are written and read with
        // device-scope atomic accesses (coherent across the XCDs' L2 caches
        // without a fence); every wave waits for its stores to complete before
        // the barrier, the arrival is counted after it, and the last arrival
        // reads the partials only after its count returned. The counter holds
        // the launch's token in bits 8..63, so it needs no initialisation, and
        // the last arrival clears it, so a replayed graph counts from zero.
        if constexpr (kCanSplit) {
            if (kind == 3) {
                constexpr int kSlot = TM * TN * 16 * NT;   // floats of one partial tile
                float *pt = reinterpret_cast<float *>(partials) + (size_t)ft * splits * kSlot;
                float *mine = pt + (size_t)piece * kSlot;
#pragma unroll
                for (int a = 0; a < TM; ++a)
#pragma unroll
                    for (int b = 0; b < TN; ++b)
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            __hip_atomic_store(mine + ((a * TN + b) * 16 + v) * NT + tid, acc[a][b][v],
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __shared__ int split_last;
                __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
                __syncthreads();
                if (tid == 0) {
                    unsigned long long *c = flags + ft;
                    unsigned long long old = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    unsigned long long nv;
                    do {
                        nv = (old & ~0xFFull) == token ? old + 1 : (token | 1ull);
                    } while (!__hip_atomic_compare_exchange_strong(c, &old, nv, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                                   __HIP_MEMORY_SCOPE_AGENT));
                    split_last = (int)(nv & 0xFFull) == splits;
                    if (split_last) __hip_atomic_store(c, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                __syncthreads();
                if (!split_last) continue;
                // slot by slot, every load of a slot issued before its adds (one
                // memory round trip per slot); the sum runs in split order
                auto load_slot = [&](int j, f16_t (&dst)[TM][TN]) __attribute__((always_inline)) {
                    const float *src = pt + (size_t)j * kSlot + tid;
#pragma unroll
                    for (int a = 0; a < TM; ++a)
#pragma unroll
                        for (int b = 0; b < TN; ++b)
#pragma unroll
                            for (int v = 0; v < 16; ++v)
                                dst[a][b][v] = __hip_atomic_load(src + ((a * TN + b) * 16 + v) * NT, __ATOMIC_RELAXED,
                                                                 __HIP_MEMORY_SCOPE_AGENT);
                };
                load_slot(0, acc);
                for (int j = 1; j < splits; ++j) {
                    f16_t part[TM][TN];
                    load_slot(j, part);
#pragma unroll
                    for (int a = 0; a < TM; ++a)
#pragma unroll
                        for (int b = 0; b < TN; ++b) acc[a][b] += part[a][b];
                }
            }
        }

        // ---- stream-K hand-over. Partial slots hold each thread's accumulators
        // as float4 [TM][TN][4][NT] (coalesced; producer and consumer run the same
        // tile shape, so thread tid reads back exactly what thread tid wrote).
        constexpr int kPart = TM * TN * 4;   // float4 per thread
        if (SK && kind == 1) {
            float4 *slot = partials + (size_t)s_sk * kPart * NT;
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int b = 0; b < TN; ++b)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        slot[((a * TN + b) * 4 + q) * NT + tid] =
                            make_float4(acc[a][b][4 * q], acc[a][b][4 * q + 1], acc[a][b][4 * q + 2], acc[a][b][4 * q + 3]);
            // every wave waits until its stores have reached the L2 (vmcnt(0));
            // after the barrier one write-back of the L2 (the agent-scope release
            // of thread 0) makes the whole partial visible to the other XCDs
            // before the flag, itself a device-coherent store
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();
            if (tid == 0) {
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                __hip_atomic_store(&flags[s_sk], token, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            continue;
        }
        if (SK && kind == 2) {
            __shared__ float sk_poison;
            if (tid == 0) {
                // bounded wait (about a second): the producer never waits before
                // producing, so this ends; the bound only keeps a broken launch
                // from holding the device. Relaxed polls (device-coherent loads);
                // the acquire below then orders the partial's loads after them.
                // (a launch testing the expiry waits for another token, briefly)
                const int spin_limit = wait_token == token ? (1 << 21) : 64;
                int ready = 0;
                for (int spin = 0; spin < spin_limit; ++spin) {
                    if (__hip_atomic_load(&flags[s_sk - 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == wait_token) {
                        ready = 1;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
                // the wait ran out: the tile is written as NaN (the partial gets a
                // NaN term) and the process's error word (host memory) is set, so
                // the failure shows both in the output and in the status of the
                // next call
                if (!ready && err != nullptr) {
                    __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");
                }
                sk_poison = ready ? 0.0f : __builtin_nanf("");
                // invalidates this CU's L1 and this XCD's L2, which all waves of
                // the workgroup read through: no stale line of the partial is left
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            }
            __syncthreads();
            const float poison = sk_poison;
            const float4 *slot = partials + (size_t)(s_sk - 1) * kPart * NT;
            // all 32 loads of the thread's part issue back to back (one round
            // trip). The fix-up costs more than that: every workgroup reaches it
            // at about the same time, so the 256 KB partials of all of them are
            // read together (64 MB on 256 CUs, ~16 us); see the plan's threshold
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int b = 0; b < TN; ++b)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float4 p = slot[((a * TN + b) * 4 + q) * NT + tid];
                        acc[a][b][4 * q] += p.x + poison;
                        acc[a][b][4 * q + 1] += p.y + poison;
                        acc[a][b][4 * q + 2] += p.z + poison;
                        acc[a][b][4 * q + 3] += p.w + poison;
                    }
            // the flag of this launch is consumed: clear it, so a replay of the
            // same launch (same token, e.g. from a graph) waits again
            if (tid == 0) __hip_atomic_store(&flags[s_sk - 1], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }

        // ---- epilogue: lane holds rows (v/4)*8 + (lane/32)*4 + v%4 of column
        // lane%32 of each 32x32 block (a store instruction covers two 64-byte
        // runs of two rows; measured faster than the transposed layout's 8-byte
        // stores over 32 rows). Tiles inside the matrix store without per-element
        // checks (a branch per element splits the accumulators' live ranges and
        // spills them).
        const bool inside = m0 + BM <= M && n0 + BN <= N;
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int b = 0; b < TN; ++b) {
                const int n = n0 + wn * (BN / WN) + 32 * b + (lane & 31);
                const int mb = m0 + wm * (BM / WM) + 32 * a + (lane >> 5) * 4;
                uint16_t *yb = y + (int64_t)mb * N + n;
                if (inside) {
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        yb[(int64_t)((v / 4) * 8 + (v % 4)) * N] =
                            BF ? f32_to_bf16_bits(acc[a][b][v]) : f32_to_f16_bits(acc[a][b][v]);
                } else if (n < N) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int m = mb + (v / 4) * 8 + (v % 4);
                        if (m < M)
                            yb[(int64_t)((v / 4) * 8 + (v % 4)) * N] =
                                BF ? f32_to_bf16_bits(acc[a][b][v]) : f32_to_f16_bits(acc[a][b][v]);
                    }
                }
            }
    }   // segments
}

// One tiled launch: dp_tiles whole tiles, then sk_wgs stream-K workgroups
// (0: every tile whole) with their partials and flags in `ws`.
struct SkArgs {
    int dp_tiles, sk_wgs;
    int splits, split_cols;   // K split (splits > 1; exclusive with stream-K)
    void *ws;
    bool expire_test;   // consumers wait for a token no producer writes (tests the expiry path)
};

template <int BM, int BN, int WM, int WN, int GROUP, bool BF, int FMT>
hipError_t launch_tile(const void *x, const void *qw, const void *qh, const void *sc, const void *zp, void *y, int M,
                       int N, int K, int ms, const SkArgs &sk, hipStream_t stream) {
    static_assert(BN == kTileCols, "tile columns");
    const bool ksplit = WM * WN == 4 && BM <= 128 && sk.splits > 1;
    const bool split = sk.sk_wgs > 0 || ksplit;
    auto kern = split ? prefill_kernel<BM, BN, WM, WN, GROUP, BF, FMT, true>
                      : prefill_kernel<BM, BN, WM, WN, GROUP, BF, FMT, false>;
    const size_t lds = (size_t)2 * (BM + BN) * kUnits * 16;
    static DynLdsAttr attr[2];
    hipError_t e = raise_dyn_lds(reinterpret_cast<const void *>(kern), lds, attr[split ? 1 : 0]);
    if (e != hipSuccess) return e;
    const int m_tiles = (int)ceil_div(M, BM), n_tiles = (int)ceil_div(N, BN);
    const int tiles = m_tiles * n_tiles;
    int dp = tiles, skw = 0, splits = 1, grid = tiles;
    float4 *part = nullptr;
    unsigned long long *flags = nullptr;
    unsigned long long token = 0ull;
    if (ksplit) {   // partials [tiles][splits][BM x BN] fp32, then a counter per tile
        if (sk.ws == nullptr || sk.split_cols < 1 || (int64_t)(sk.splits - 1) * sk.split_cols >= ceil_div(K / kChunk, kColChunks))
            return hipErrorInvalidValue;
        splits = sk.splits;
        dp = 0;
        grid = tiles * splits;
        part = reinterpret_cast<float4 *>(sk.ws);
        flags = reinterpret_cast<unsigned long long *>(static_cast<char *>(sk.ws) +
                                                       (size_t)tiles * splits * BM * BN * 4);
        token = next_sk_token() & ~0xFFull;   // the counters keep the arrivals in bits 0..7
        if (token == 0) token = 0x100ull;
    } else if (sk.sk_wgs > 0) {   // the plan guarantees dp_tiles + sk_wgs <= tiles (each share >= one tile)
        if (sk.ws == nullptr || sk.dp_tiles + sk.sk_wgs > tiles) return hipErrorInvalidValue;
        dp = sk.dp_tiles;
        skw = sk.sk_wgs;
        grid = dp + skw;
        part = reinterpret_cast<float4 *>(sk.ws);
        flags = reinterpret_cast<unsigned long long *>(static_cast<char *>(sk.ws) + (size_t)skw * BM * BN * 4);
        token = next_sk_token();
    }
    // stream-K consumers wait for the token their producer writes; a launch
    // that tests the expiry of the wait gives them one no producer writes and
    // a short bound
    const unsigned long long wait_token = sk.expire_test ? token ^ 0xA5A5A5A5A5A5A5A5ull : token;
    const int raster = (!ksplit && m_tiles % 8 == 0 && dp % m_tiles == 0 &&
                        tuning_knob("W4A16_PREFILL_RASTER", 1) == 1) ? 1 : 0;
    unsigned int *err = skw > 0 ? kernel_error_word() : nullptr;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * WM * WN), lds, stream,
                       reinterpret_cast<const uint16_t *>(x), reinterpret_cast<const uint4 *>(qw),
                       reinterpret_cast<const uint4 *>(qh), reinterpret_cast<const uint16_t *>(sc),
                       reinterpret_cast<const uint32_t *>(zp), reinterpret_cast<uint16_t *>(y), M, N, K, m_tiles,
                       n_tiles, ms, dp, skw, raster, splits, sk.split_cols, part, flags, token, wait_token, err);
    return hipGetLastError();
}

template <int GROUP, bool BF, int FMT>
hipError_t launch_group(int tile, const void *x, const void *qw, const void *qh, const void *sc, const void *zp,
                        void *y, int M, int N, int K, int ms, const SkArgs &sk, hipStream_t stream) {
    switch (tile) {
        case kTile64x256: return launch_tile<64, 256, 1, 4, GROUP, BF, FMT>(x, qw, qh, sc, zp, y, M, N, K, ms, sk, stream);
        case kTile128x256: return launch_tile<128, 256, 2, 2, GROUP, BF, FMT>(x, qw, qh, sc, zp, y, M, N, K, ms, sk, stream);
        case kTile256x256w8: return launch_tile<256, 256, 2, 4, GROUP, BF, FMT>(x, qw, qh, sc, zp, y, M, N, K, ms, sk, stream);
        default: return launch_tile<256, 256, 2, 2, GROUP, BF, FMT>(x, qw, qh, sc, zp, y, M, N, K, ms, sk, stream);
    }
}

}  // namespace

// The tiled launches of one weight format. Group 256 runs the group-128
// kernels with one metadata slot per two columns (mshift = 1).
template <int FMT>
hipError_t launch_prefill_fmt(const void *x, bool bf16, const void *qweight, const void *scales, const void *zeros,
                              void *y, int M, int N, int K, int group, const GemmPlan &plan, void *workspace,
                              hipStream_t stream) {
    const SkArgs sk{plan.dp_tiles, plan.sk_wgs, plan.splits, plan.split_cols, workspace, plan.sk_expire_test != 0};
    const int ms = group == 256 ? 1 : 0;
    const void *qh = FormatTraits<FMT>::two_planes
                         ? static_cast<const void *>(static_cast<const char *>(qweight) + (size_t)N * K / 2)
                         : qweight;
    const int t = plan.tile;
    if constexpr (FormatTraits<FMT>::kquant) {   // one 32-weight sub-block per chunk
        return bf16 ? launch_group<32, true, FMT>(t, x, qweight, qh, scales, zeros, y, M, N, K, 0, sk, stream)
                    : launch_group<32, false, FMT>(t, x, qweight, qh, scales, zeros, y, M, N, K, 0, sk, stream);
    } else {
    if (bf16) {
        switch (group) {
            case 32: return launch_group<32, true, FMT>(t, x, qweight, qh, scales, zeros, y, M, N, K, ms, sk, stream);
            case 64: return launch_group<64, true, FMT>(t, x, qweight, qh, scales, zeros, y, M, N, K, ms, sk, stream);
            default: return launch_group<128, true, FMT>(t, x, qweight, qh, scales, zeros, y, M, N, K, ms, sk, stream);
        }
    }
    switch (group) {
        case 32: return launch_group<32, false, FMT>(t, x, qweight, qh, scales, zeros, y, M, N, K, ms, sk, stream);
        case 64: return launch_group<64, false, FMT>(t, x, qweight, qh, scales, zeros, y, M, N, K, ms, sk, stream);
        default: return launch_group<128, false, FMT>(t, x, qweight, qh, scales, zeros, y, M, N, K, ms, sk, stream);
    }    }
}

}  // namespace w4a16
