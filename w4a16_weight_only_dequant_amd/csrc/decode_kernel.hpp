// Decode kernel of the W4A16 linear layer for the smallest batches (M <= 8):
// y[m][n] = sum_k x[m][k] * w_hat[n][k], with 16-bit dot products and fp32
// accumulation.
//
// At decode every weight is read once per token and used for M multiply-adds,
// so the weight stream from HBM sets the time ("Weight-Only Quantisation",
// first two FAQ answers; "Weight-Only Quantization Explained", "Where it stops
// being the right answer"). The weights stay packed until they reach
// registers ("Quantization Is Not a Zip File", section 8) and are rebuilt as
// 16-bit values right before the multiply ("Weight-Only Quantisation",
// definition).
//
// What a launch costs on gfx950: a cold launch that reads B bytes takes about
// 1.45 us + B / 7 TB/s when every wave has issued all of its loads before it
// waits for any; every instruction a wave executes before its last load is
// issued, or after its data arrives, adds to that. The kernel is shaped by it:
//
// * Issue order. A wave loads, in this order and before any wait: its slice
//   of the activations (registers), its rows' scales and zero-points for the
//   slice (a few wide loads: the metadata of one row is contiguous along K),
//   and the codes of all NCOL columns of its slice (one 16-byte load per lane
//   and column). Vector-memory loads retire in issue order, so one wait
//   covers the activations and metadata while the weight loads stay in
//   flight, and each column is computed as soon as its own load is in. NCOL
//   is a compile-time constant so that every wait counts exactly the loads
//   issued after the one it waits for (a loop or a conditional load would
//   make the compiler wait for all of them).
// * Arithmetic per weight. fp16 activations, 4-bit codes: one shift and four
//   v_and_or per dword of codes give the exact magic operands 1024 + q (k0,k1
//   and k4,k5) and 1024 + 16 q (k2,k3 and k6,k7); four v_dot2_f32_f16
//   accumulate them against the activations into two fp32 sums. The magic
//   offsets are taken off once per group with the sums of the group's
//   activations (formed once per wave while the weights are in flight), the
//   16x sum is scaled by 1/16 (exact), and the group scale multiplies the
//   result. bf16 activations (a bf16 exponent has no room for the 16x
//   operand) and 8-bit codes use 128 + q / 1024 + q at every position (three
//   shifts, four v_and_or). The matrix cores are not used at M <= 8: on this
//   layer one v_mfma_f32_16x16x32 per dword of codes measured about twice the
//   time of the dot products.
//
// Mapping: a workgroup owns one block of 16 output rows and all of K; its
// waves take consecutive slices of NCOL 128-weight columns. Lane l = 16 s + r
// loads, per column, dword s of the column's four chunks of row r (one
// contiguous KiB per wave) and accumulates row r over the k-slices 8s..8s+7
// of the column's chunks; the four lanes of a row meet by cross-lane moves at
// the end, the waves through LDS, always in the same order, so results are
// deterministic and no partial sum leaves the workgroup.
//
// Weight formats (FMT) change the operands and the per-group terms: a fixed
// zero (symmetric 4-bit), a second code plane (8-bit codes, operands
// 16 (magic + hi)), or the per-chunk scale S and minimum M of a K-quant
// super-block: S * sum x q - M * sum x.
#pragma once

#include "decode_common.hpp"

namespace w4a16 {
namespace {

constexpr int kDecMaxWaves = 16;

template <bool BF>
__device__ inline float dec_dot2(uint32_t w, uint32_t x, float acc) {
    if constexpr (BF)
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, w), __builtin_bit_cast(bf162_t, x), acc,
                                               false);
    else
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w), __builtin_bit_cast(half2_t, x), acc, false);
}

// v + (v of the lane N below in the same row of 16 lanes; 0 past the row's
// start): one VALU op with a DPP row shift
template <int N>
__device__ inline float dpp_add_shr(float v) {
    const int o = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x110 + N, 0xF, 0xF, true);
    return v + __builtin_bit_cast(float, o);
}

// Bytes of one row's metadata in a slice of ncol columns: fp16 scales (one
// per group), or 16-byte super-block records; and of its zero-point words.
__host__ __device__ constexpr int dec_meta_row_bytes(int ncol, int group, int fmt) {
    return fmt == kKq4 ? ncol / 2 * 16 : (group >= 256 ? ncol : ncol * (128 / group) * 2);
}
__host__ __device__ constexpr int dec_zero_words(int ncol, int group, int fmt) {
    return fmt != kAsym4 ? 0 : (group >= 256 ? (ncol / 2 + 7) / 8 : (ncol * (128 / group) + 7) / 8);
}
// Per-wave LDS (bytes) for MT activation rows and ncol columns: activations
// [MT][ncol * 256], activation sums [MT][units][4 slices][2] floats, the 16
// rows' scales (or records) [16][meta_row_bytes] and zero-points [16][words],
// and 16 spare bytes.
struct DecLds {
    int x, sums, meta, zeros, spare, total;
};
__host__ __device__ constexpr DecLds dec_lds(int mt, int ncol, int group, int fmt) {
    const int upc = fmt == kKq4 ? 4 : (group >= 128 ? 1 : 128 / group);   // closing units per column
    const int x = mt * ncol * 256;
    const int sums = mt * ncol * upc * 4 * 2 * 4;
    const int meta = 16 * dec_meta_row_bytes(ncol, group, fmt);
    const int zeros = 16 * dec_zero_words(ncol, group, fmt) * 4;
    return DecLds{0, x, x + sums, x + sums + meta, x + sums + meta + zeros, x + sums + meta + zeros + 16};
}

// GROUP: 32, 64, 128 or 256 (K-quant super-blocks: 256, closed per 32-weight
// chunk). MT: activation rows held (1, 2, 4 or 8; rows m >= M repeat row
// M - 1 and are never stored). NCOL: columns per wave (8 or 16; 16 for group
// 256). AWQ: act_mul holds fp32 multipliers [K] applied to the activations as
// they are loaded (AWQ's run-time scaling: x' = rne16(x * m)).
// Metadata (layout 3): scales [N][G8] fp16 and zero-points [N][G8 / 8] words
// of eight 4-bit values (group g in bits 4 (g % 8)), G8 = K / group rounded up
// to a multiple of 8; super-block records [N][K / 256] of 16 bytes.
template <int GROUP, int MT, bool BF, int FMT, int NCOL, bool AWQ>
__global__ __launch_bounds__(64 * kDecMaxWaves) void decode_kernel(
    const uint16_t *__restrict__ x, const uint4 *__restrict__ qw, const uint4 *__restrict__ qw_hi,
    const uint16_t *__restrict__ scales, const uint32_t *__restrict__ zeros, uint16_t *__restrict__ y, int M,
    int N, int K, const float *__restrict__ act_mul) {
    using FT = FormatTraits<FMT>;
    constexpr int GC = GROUP > kColumn ? kColumn : GROUP;   // closing granularity along K (<= a column)
    constexpr int CPG = GC / kChunk;                       // chunks per group (1, 2, 4)
    constexpr int GPC = kColumn / GC;                      // groups per column (4, 2, 1)
    constexpr int UPC = FT::kquant ? kColChunks : GPC;     // closing units per column
    constexpr int CPU = FT::kquant ? 1 : CPG;              // chunks per closing unit
    constexpr bool HI = !BF && !FT::two_planes;            // fp16 4-bit codes: 16x operands at k2,k3,k6,k7
    constexpr DecLds L = dec_lds(MT, NCOL, GROUP, FMT);
    constexpr int MRB = dec_meta_row_bytes(NCOL, GROUP, FMT);
    constexpr int MPARTS = (MRB + 15) / 16;                // 16-byte parts of one row's metadata
    constexpr int MJ = (MPARTS + 3) / 4;                   // metadata loads per lane (LDS path)
    constexpr int ZW = dec_zero_words(NCOL, GROUP, FMT);   // zero-point words of one row
    constexpr int ZJ = (ZW + 3) / 4;                       // zero-point loads per lane (LDS path)
    constexpr int XQ = NCOL / 4;                           // 16-byte activation loads per lane and row
    // small metadata runs (groups 128 and 256) stay in each lane's registers
    constexpr bool MREG = !FT::kquant && MRB <= 32 && ZW <= 2;
    static_assert(NCOL % 4 == 0 && (MRB % 16 == 0 || (MREG && MRB == 8)),
                  "a slice covers whole 16-byte metadata parts (or one 8-byte run kept in registers)");
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ float red[kDecMaxWaves][MT][kRowBlock];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15;
    const int s = lane >> 4;
    const int b = blockIdx.x;
    const int rows_b = min(kRowBlock, N - b * kRowBlock);
    const int rl = r < rows_b ? r : r - rows_b;   // lanes past a short last block re-read a valid row
    const int C = K >> 5;                          // chunks along K
    const int T = (C + 3) >> 2;                    // columns (the last may be partial)
    const int t0 = wave * NCOL;                    // this wave's columns [t0, t0 + NCOL)
    const int nfull = min(max((C >> 2) - t0, 0), NCOL);
    const int c_lo = t0 * kColChunks;
    const int nchunks = max(min((t0 + NCOL) * kColChunks, C) - c_lo, 0);
    const int G8 = ((K / GROUP) + 7) & ~7;         // metadata slots per row (scales)
    const int gs0 = (int)((int64_t)t0 * kColumn / GROUP);   // first group of the slice (K-quant: record)

    unsigned char *wl = smem + wave * L.total;
    unsigned char *xl = wl + L.x;                          // [MT][NCOL * 256]
    float *xs = reinterpret_cast<float *>(wl + L.sums);   // [MT][NCOL * UPC][4] of (B, S)
    unsigned char *ml = wl + L.meta;                       // [16][MRB]      (LDS path)
    uint32_t *zl = reinterpret_cast<uint32_t *>(wl + L.zeros);   // [16][ZW] (LDS path)

    // 1. activations of the slice, 16 bytes per lane and load (positions past
    // the slice re-read its last unit and are never used)
    const int xlast = max(nchunks * 4 - 1, 0);
    uint4 xr[MT][XQ];
    float4 amr[AWQ ? XQ : 1][2];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const uint4 *src = reinterpret_cast<const uint4 *>(x + (size_t)min(m, M - 1) * K) + (size_t)c_lo * 4;
#pragma unroll
        for (int i = 0; i < XQ; ++i) xr[m][i] = src[min(i * 64 + lane, xlast)];
    }
    if constexpr (AWQ) {
        const float4 *src = reinterpret_cast<const float4 *>(act_mul) + (size_t)c_lo * 8;
#pragma unroll
        for (int i = 0; i < XQ; ++i) {
            const int q = min(i * 64 + lane, xlast);
            amr[i][0] = src[2 * q];
            amr[i][1] = src[2 * q + 1];
        }
    }

    // 2. metadata of the slice. Small runs: every lane loads its own row's run
    // into registers. Larger ones: lane l loads 16-byte parts l / 16 + 4 j of
    // row l % 16's run (and zero-point words the same way), for LDS. Parts
    // past the end of a row re-read its last one (never used).
    const int mp = lane >> 4;
    uint4 mreg[MREG ? MPARTS : MJ];
    uint32_t zreg[MREG ? (ZW > 0 ? ZW : 1) : (ZJ > 0 ? ZJ : 1)];
    {
        const int mrow = b * kRowBlock + rl;
        const unsigned char *base;
        int last_part;
        if constexpr (FT::kquant) {
            base = reinterpret_cast<const unsigned char *>(scales) + (size_t)mrow * (K / 256) * 16;
            last_part = K / 256 - 1;
        } else {
            base = reinterpret_cast<const unsigned char *>(scales) + (size_t)mrow * G8 * 2;
            last_part = G8 / 8 - 1;
        }
        const int part0 = FT::kquant ? gs0 : gs0 / 8;   // the slice's first part in the row
        const uint32_t *zb = zeros + (size_t)mrow * (G8 / 8);
        if constexpr (MREG) {
            if constexpr (MRB == 8) {   // an 8-byte run (8-byte aligned)
                const uint2 v = *reinterpret_cast<const uint2 *>(base + (size_t)min(gs0, G8 - 4) * 2);
                mreg[0] = make_uint4(v.x, v.y, 0u, 0u);
            } else {
#pragma unroll
                for (int j = 0; j < MPARTS; ++j)
                    mreg[j] = *reinterpret_cast<const uint4 *>(base + (size_t)min(part0 + j, last_part) * 16);
            }
#pragma unroll
            for (int j = 0; j < ZW; ++j) zreg[j] = zb[min(gs0 / 8 + j, G8 / 8 - 1)];
        } else {
#pragma unroll
            for (int j = 0; j < MJ; ++j)
                mreg[j] = *reinterpret_cast<const uint4 *>(base + (size_t)min(part0 + mp + 4 * j, last_part) * 16);
            if constexpr (ZJ > 0) {
#pragma unroll
                for (int j = 0; j < ZJ; ++j) zreg[j] = zb[min(gs0 / 8 + mp + 4 * j, G8 / 8 - 1)];
            }
        }
    }

    // 3. the codes of every column of the slice, all in flight at once (a
    // position past the slice re-reads its last full column: never used)
    const unsigned char *qb = reinterpret_cast<const unsigned char *>(qw) + (size_t)b * 8 * K;
    const unsigned char *qhb = reinterpret_cast<const unsigned char *>(qw_hi) + (size_t)b * 8 * K;
    const uint32_t col_bytes = (uint32_t)rows_b * 64;
    const uint32_t lane_off = nfull > 0 ? (uint32_t)(s * rows_b + rl) * 16u : 0u;
    const int tlast = min(t0 + max(nfull - 1, 0), T - 1);
    uint4 rec[NCOL], rech[NCOL];
#pragma unroll
    for (int p = 0; p < NCOL; ++p) {
        const uint32_t cb = (uint32_t)min(t0 + p, tlast) * col_bytes;
        rec[p] = nt_load(reinterpret_cast<const uint4 *>((qb + cb) + lane_off));
        if constexpr (FT::two_planes) rech[p] = nt_load(reinterpret_cast<const uint4 *>((qhb + cb) + lane_off));
        // keep each load where it is: sinking it towards its use would
        // serialise the stream
        __builtin_amdgcn_sched_barrier(0);
    }

    // 4. wait for the activations and metadata only (the codes issued after
    // them stay in flight) and store them in LDS, the activations scaled
    // (AWQ); stores are unconditional (lanes without a part write a spare
    // slot), so no load is moved into a branch behind the code loads
    {
        constexpr int V = NCOL * (FT::two_planes ? 2 : 1);
        __builtin_amdgcn_s_waitcnt((V & 15) | (7 << 4) | (15 << 8) | ((V >> 4) << 14));
    }
    if constexpr (!MREG) {
#pragma unroll
        for (int j = 0; j < MJ; ++j) {
            const int part = mp + 4 * j;
            *reinterpret_cast<uint4 *>(part < MPARTS ? ml + r * MRB + part * 16 : wl + L.spare) = mreg[j];
        }
        if constexpr (ZJ > 0) {
#pragma unroll
            for (int j = 0; j < ZJ; ++j) {
                const int w = mp + 4 * j;
                *(w < ZW ? zl + r * ZW + w : reinterpret_cast<uint32_t *>(wl + L.spare)) = zreg[j];
            }
        }
    }
    // per closing unit and slice s: S = the sum of its activations and B the
    // magic-offset term (a fixed zero-point folded in), so that the unit's
    // sum of x * (code - zero) over slice s is lo + f hi - B - z S. A lane
    // per 16-byte unit (chunk c, slice s); DPP row shifts add the chunks of a
    // unit (a row of 16 lanes is 4 chunks x 4 slices) in a fixed order.
    constexpr uint32_t one2 = BF ? 0x3F803F80u : 0x3C003C00u;   // (1, 1)
    constexpr float kMagic = BF ? 128.0f : 1024.0f;
    constexpr float kFixedZ = FT::has_zeros ? 0.0f : (float)FT::fixed_zero;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int i = 0; i < XQ; ++i) {
            uint4 v = xr[m][i];
            if constexpr (AWQ) v = scale8<BF>(v, amr[i][0], amr[i][1]);
            const int q = i * 64 + lane;
            *reinterpret_cast<uint4 *>(xl + m * (NCOL * 256) + q * 16) = v;
            float lo = dec_dot2<BF>(v.z, one2, dec_dot2<BF>(v.x, one2, 0.0f));   // k0,k1,k4,k5
            float hi = dec_dot2<BF>(v.w, one2, dec_dot2<BF>(v.y, one2, 0.0f));   // k2,k3,k6,k7
            if constexpr (CPU >= 2) {
                lo = dpp_add_shr<4>(lo);
                hi = dpp_add_shr<4>(hi);
            }
            if constexpr (CPU >= 4) {
                lo = dpp_add_shr<8>(lo);
                hi = dpp_add_shr<8>(hi);
            }
            const int c = q >> 2;
            const float S = lo + hi;
            float B;
            if constexpr (FT::two_planes)
                B = (BF ? 2304.0f : 17536.0f) * S;   // (magic + 16 magic) + 128
            else if constexpr (HI)
                B = fmaf(kMagic, lo, fmaf(64.0f, hi, kFixedZ * S));
            else
                B = (kMagic + kFixedZ) * S;
            float *o = c % CPU == CPU - 1 ? xs + (((m * NCOL * UPC) + c / CPU) * 4 + (q & 3)) * 2
                                          : reinterpret_cast<float *>(wl + L.spare);
            *reinterpret_cast<float2 *>(o) = make_float2(B, S);
        }
    }
    // every LDS store above precedes every LDS read below (same wave, in order)
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

    // 5. the columns in order, straight-line: a column past the slice is
    // computed from copies and not added (a select, not a branch, so the
    // compiler may read the next column's operands early)
    const UnpackConsts uc = unpack_consts();
    const unsigned char *xa = xl + s * 16;
    const unsigned char *mrow_l = ml + r * MRB;
    const uint32_t *zrow_l = zl + r * (ZW > 0 ? ZW : 1);
    float acc[MT], lo[MT], hi[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = lo[m] = hi[m] = 0.0f;
    // the four operand pairs of a dword, in dot-sum order (lo: k0,k1 and k4,k5;
    // hi: k2,k3 and k6,k7)
    auto unpack = [&](uint32_t d, uint32_t (&w)[4]) {
        if constexpr (HI) {
            const uint32_t d8 = d >> 8;
            w[0] = and_or(d, uc.lo_mask, uc.f16_magic);
            w[1] = and_or(d, uc.hi_mask, uc.f16_magic);
            w[2] = and_or(d8, uc.lo_mask, uc.f16_magic);
            w[3] = and_or(d8, uc.hi_mask, uc.f16_magic);
        } else {
            const uint32_t magic = BF ? uc.bf16_magic : uc.f16_magic;
            w[0] = and_or(d, uc.lo_mask, magic);
            w[1] = and_or(d >> 4, uc.lo_mask, magic);
            w[2] = and_or(d >> 8, uc.lo_mask, magic);
            w[3] = and_or(d >> 12, uc.lo_mask, magic);
        }
    };
    auto unpack16 = [&](uint32_t d, uint32_t (&w)[4]) {   // the high-nibble plane of 8-bit codes
        const uint32_t magic = BF ? uc.bf16_magic16 : uc.f16_magic16;
        w[0] = and_or(d, uc.lo_mask, magic);
        w[1] = and_or(d >> 4, uc.lo_mask, magic);
        w[2] = and_or(d >> 8, uc.lo_mask, magic);
        w[3] = and_or(d >> 12, uc.lo_mask, magic);
    };
    const int zoff = gs0 & 7;   // the slice's first zero-point nibble in its first word
    auto zero_of = [&](int g) -> uint32_t {   // g: group within the slice
        if constexpr (!FT::has_zeros) return 0u;
        else if constexpr (MREG) return (zreg[(g + zoff) >> 3] >> (4 * ((g + zoff) & 7))) & 0xFu;
        else return (zrow_l[g >> 3] >> (4 * (g & 7))) & 0xFu;
    };
    auto scale_of = [&](int g) -> float {     // g: group within the slice
        if constexpr (MREG) {
            const uint4 v = mreg[g >> 3];
            const uint32_t w = (g & 7) < 2 ? v.x : ((g & 7) < 4 ? v.y : ((g & 7) < 6 ? v.z : v.w));
            return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> (16 * (g & 1))));
        } else {
            return (float)*reinterpret_cast<const _Float16 *>(mrow_l + g * 2);
        }
    };
    // closing unit u of the slice with scale sc, zero-point z; K-quant: S and
    // the minimum mn; `on`: the column is part of the slice
    constexpr float kF = HI ? 0.0625f : 1.0f;
    auto close = [&](int u, float sc, float mn, uint32_t z, bool on) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const float2 bs = *reinterpret_cast<const float2 *>(xs + (((m * NCOL * UPC) + u) * 4 + s) * 2);
            float part = fmaf(kF, hi[m], lo[m]) - bs.x;
            if constexpr (FT::has_zeros) part = fmaf(-(float)z, bs.y, part);
            float na = fmaf(sc, part, acc[m]);
            if constexpr (FT::kquant) na = fmaf(-mn, bs.y, na);
            acc[m] = on ? na : acc[m];
            lo[m] = 0.0f;
            hi[m] = 0.0f;
        }
    };
    auto load_x = [&](int c, uint4 (&xv)[MT]) {   // c: chunk within the slice
#pragma unroll
        for (int m = 0; m < MT; ++m) xv[m] = *reinterpret_cast<const uint4 *>(xa + m * (NCOL * 256) + c * 64);
    };
    auto chunk = [&](const uint4 (&xv)[MT], uint32_t d, uint32_t dh) {
        uint32_t w[4], wh[4];
        unpack(d, w);
        if constexpr (FT::two_planes) unpack16(dh, wh);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            lo[m] = dec_dot2<BF>(w[0], xv[m].x, lo[m]);
            hi[m] = dec_dot2<BF>(w[1], xv[m].y, hi[m]);
            lo[m] = dec_dot2<BF>(w[2], xv[m].z, lo[m]);
            hi[m] = dec_dot2<BF>(w[3], xv[m].w, hi[m]);
            if constexpr (FT::two_planes) {
                lo[m] = dec_dot2<BF>(wh[0], xv[m].x, lo[m]);
                hi[m] = dec_dot2<BF>(wh[1], xv[m].y, hi[m]);
                lo[m] = dec_dot2<BF>(wh[2], xv[m].z, lo[m]);
                hi[m] = dec_dot2<BF>(wh[3], xv[m].w, hi[m]);
            }
        }
    };
#pragma unroll
    for (int p = 0; p < NCOL; ++p) {
        const bool on = p < nfull;
        const uint32_t dws[4] = {rec[p].x, rec[p].y, rec[p].z, rec[p].w};
        const uint32_t dwh[4] = {rech[p].x, rech[p].y, rech[p].z, rech[p].w};
#pragma unroll
        for (int j = 0; j < kColChunks; ++j) {
            uint4 xv[MT];
            load_x(p * kColChunks + j, xv);
            chunk(xv, dws[j], dwh[j]);
            if ((j + 1) % CPU == 0) {
                const int u = (p * kColChunks + j) / CPU;   // closing unit within the slice
                if constexpr (FT::kquant) {
                    const KqHalf hf = kq_half(*reinterpret_cast<const uint4 *>(mrow_l + (p >> 1) * 16), (p & 1) != 0);
                    const KqParams P = kq_sub(hf, j);
                    close(u, P.S, P.M, 0u, on);
                } else {
                    const int g = GROUP > kColumn ? (p >> 1) : u;   // group within the slice
                    close(u, scale_of(g), 0.0f, zero_of(g), on);
                }
            }
        }
    }

    // 6. the partial last column of K (K % 128 != 0, groups 32 and 64): nc < 4
    // chunks, whose nc dwords of a lane are consecutive; its groups are whole
    if constexpr (!FT::kquant && GROUP < kColumn) {
        if (nfull < NCOL && t0 + nfull == T - 1 && T > (C >> 2)) {
            const int tl = T - 1;
            const int nc = C - tl * kColChunks;
            const size_t off = (size_t)tl * rows_b * 16 + (size_t)s * rows_b * nc + (size_t)rl * nc;
            const uint32_t *col = reinterpret_cast<const uint32_t *>(qb) + off;
            const uint32_t *colh = reinterpret_cast<const uint32_t *>(qhb) + off;
            for (int j = 0; j < nc; ++j) {
                const int c = nfull * kColChunks + j;   // chunk within the slice
                uint4 xv[MT];
                load_x(c, xv);
                chunk(xv, col[j], FT::two_planes ? colh[j] : 0u);
                if ((j + 1) % CPG == 0 || j == nc - 1) close(c / CPG, scale_of(c / CPG), 0.0f, zero_of(c / CPG), true);
            }
        }
    }

    // 7. reduce: the four lanes of a row (its k-slices), then the waves, in a
    // fixed order
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        float v = acc[m];
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        acc[m] = v;
    }
    if (s == 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m) red[wave][m][r] = acc[m];
    }
    __syncthreads();
    const int waves = blockDim.x >> 6;
    for (int i = threadIdx.x; i < M * kRowBlock; i += blockDim.x) {
        const int m = i >> 4, rr = i & 15;
        if (rr < rows_b) {
            float v = red[0][m][rr];
            for (int w = 1; w < waves; ++w) v += red[w][m][rr];
            y[(int64_t)m * N + b * kRowBlock + rr] = BF ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
        }
    }
}

template <int GROUP, int MT, bool BF, int FMT, int NC, bool AWQ>
hipError_t launch_dec_one(const void *x, const void *qw, const void *qh, const void *sc, const void *zp, void *y,
                          int M, int N, int K, const float *am, const DecodePlan &p, hipStream_t stream) {
    auto kern = decode_kernel<GROUP, MT, BF, FMT, NC, AWQ>;
    static DynLdsAttr attr;
    hipError_t e = raise_dyn_lds(reinterpret_cast<const void *>(kern), p.lds, attr);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)ceil_div(N, kRowBlock)), dim3(64 * p.waves), p.lds, stream,
                       reinterpret_cast<const uint16_t *>(x), reinterpret_cast<const uint4 *>(qw),
                       reinterpret_cast<const uint4 *>(qh), reinterpret_cast<const uint16_t *>(sc),
                       reinterpret_cast<const uint32_t *>(zp), reinterpret_cast<uint16_t *>(y), M, N, K, am);
    return hipGetLastError();
}

// the instantiated (rows, columns per wave, AWQ) combinations: the ones
// decode_plan chooses
template <int GROUP, bool BF, int FMT>
hipError_t launch_dec_group(const void *x, const void *qw, const void *qh, const void *sc, const void *zp, void *y,
                            int M, int N, int K, const float *am, const DecodePlan &p, hipStream_t stream) {
#define W4A16_DEC(MT_, NC_, AWQ_) \
    launch_dec_one<GROUP, MT_, BF, FMT, NC_, AWQ_>(x, qw, qh, sc, zp, y, M, N, K, am, p, stream)
    const bool awq = am != nullptr;
    switch (p.mt * 100 + p.ncol * 2 + (awq ? 1 : 0)) {
        case 116: return W4A16_DEC(1, 8, false);
        case 132: return W4A16_DEC(1, 16, false);
        case 117: return W4A16_DEC(1, 8, true);
        case 216: return W4A16_DEC(2, 8, false);
        case 232: return W4A16_DEC(2, 16, false);
        case 217: return W4A16_DEC(2, 8, true);
        case 416: return W4A16_DEC(4, 8, false);
        case 417: return W4A16_DEC(4, 8, true);
        case 816: return W4A16_DEC(8, 8, false);
        case 817: return W4A16_DEC(8, 8, true);
        default: return hipErrorInvalidValue;
    }
#undef W4A16_DEC
}

}  // namespace

// The launches of one weight format. K-quant super-blocks: group 256.
template <int FMT>
hipError_t launch_decode_fmt(const void *x, bool bf16, const void *qweight, const void *scales, const void *zeros,
                             void *y, int M, int N, int K, int group, const float *am, const DecodePlan &plan,
                             hipStream_t stream) {
    if (!plan.ok) return hipErrorInvalidValue;
    const void *qh = FormatTraits<FMT>::two_planes
                         ? static_cast<const void *>(static_cast<const char *>(qweight) + (size_t)N * K / 2)
                         : qweight;
#define W4A16_DEC_G(G_, BF_) launch_dec_group<G_, BF_, FMT>(x, qweight, qh, scales, zeros, y, M, N, K, am, plan, stream)
    if constexpr (FormatTraits<FMT>::kquant) {
        return bf16 ? W4A16_DEC_G(256, true) : W4A16_DEC_G(256, false);
    } else {
        switch (group) {
            case 32: return bf16 ? W4A16_DEC_G(32, true) : W4A16_DEC_G(32, false);
            case 64: return bf16 ? W4A16_DEC_G(64, true) : W4A16_DEC_G(64, false);
            case 128: return bf16 ? W4A16_DEC_G(128, true) : W4A16_DEC_G(128, false);
            default: return bf16 ? W4A16_DEC_G(256, true) : W4A16_DEC_G(256, false);
        }
    }
#undef W4A16_DEC_G
}

}  // namespace w4a16
