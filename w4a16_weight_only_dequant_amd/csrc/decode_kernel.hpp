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
// Mapping: a workgroup owns one block of 16 output rows and one of S equal
// ranges of K's columns (S = 1: all of K); its waves take consecutive slices
// of NCOL 128-weight columns. Lane l = 16 s + r loads, per column, dword s of
// the column's four chunks of row r (one contiguous KiB per wave) and
// accumulates row r over the k-slices 8s..8s+7 of the column's chunks; the
// four lanes of a row meet by cross-lane moves at the end, the waves through
// LDS, always in the same order.
// * Split K. A launch needs several workgroups per compute unit to keep the
//   weight stream going (a row block is 16 rows, so N = 5120 gives only 320
//   of them for 256 compute units). With S > 1 the S workgroups of a row
//   block each leave an fp32 partial [M][16] in the workspace and count their
//   arrival on the block's counter; the last to arrive adds the S partials in
//   split order (the result does not depend on which one is last) and writes
//   y. The counter holds the launch's token in its upper 56 bits, so it needs
//   no initialisation, and the last arrival clears it, so a replayed graph
//   (same token) counts again from zero.
//
// Weight formats (FMT) change the operands and the per-group terms: a fixed
// zero (symmetric 4-bit), a second code plane (8-bit codes, operands
// 16 (magic + hi)), or the per-chunk scale S and minimum M of a K-quant
// super-block: S * sum x q - M * sum x.
#pragma once

#include <algorithm>

#include "decode_common.hpp"

namespace w4a16 {
namespace {

constexpr int kDecMaxWaves = 16;

// Split of K over the workgroups of a row block (see the mapping above).
struct DecSplit {
    int splits;                  // workgroups per row block
    int cols;                    // columns of K per workgroup (the last range may be shorter)
    float *part;                 // [blocks][splits][M][16] fp32 partials (splits > 1)
    unsigned long long *cnt;     // [blocks] arrival counters (splits > 1)
    unsigned long long token;    // this launch's token in bits 8..63, bits 0..7 zero
};

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
// LDS row strides of the 16 rows' metadata: one row's run plus 16 bytes (scales,
// records) and plus one word (zero-points), so that the 16 lanes reading the
// same group of their 16 rows hit 16 different banks (an unpadded run of 64 or
// 128 bytes would put them on 4 or 2 banks)
__host__ __device__ constexpr int dec_meta_stride(int ncol, int group, int fmt) {
    return dec_meta_row_bytes(ncol, group, fmt) + 16;
}
__host__ __device__ constexpr int dec_zero_stride(int ncol, int group, int fmt) {
    return dec_zero_words(ncol, group, fmt) + 1;
}
// Per-wave LDS (bytes) for MT activation rows and ncol columns: activations
// [MT][ncol * 256], activation sums [MT][units][4 slices][2] floats, the 16
// rows' scales (or records) and zero-points at the strides above, and 16 spare
// bytes.
struct DecLds {
    int x, sums, meta, zeros, spare, total;
};
// Static LDS of a workgroup: the waves' reduction buffer red[kDecMaxWaves][MT][16]
// floats and the split's arrival flag (rounded up)
__host__ __device__ constexpr int dec_static_lds(int mt) { return kDecMaxWaves * mt * 16 * 4 + 64; }
__host__ __device__ constexpr DecLds dec_lds(int mt, int ncol, int group, int fmt) {
    const int upc = fmt == kKq4 ? 4 : (group >= 128 ? 1 : 128 / group);   // closing units per column
    const int x = mt * ncol * 256;
    const int sums = mt * ncol * upc * 4 * 2 * 4;
    const int meta = 16 * dec_meta_stride(ncol, group, fmt);
    const int zeros = dec_zero_words(ncol, group, fmt) > 0 ? 16 * dec_zero_stride(ncol, group, fmt) * 4 : 0;
    return DecLds{0, x, x + sums, x + sums + meta, x + sums + meta + zeros, x + sums + meta + zeros + 16};
}

// GROUP: 32, 64, 128 or 256 (K-quant super-blocks: 256, closed per 32-weight
// chunk). MT: activation rows held (1, 2, 4 or 8; rows m >= M repeat row
// M - 1 and are never stored). NCOL: columns per wave (4, 8 or 16); a
// workgroup's range of columns (sp.cols) is a multiple of NCOL, so every slice
// starts at a multiple of NCOL columns and its metadata run at a whole
// 16-byte part (or, runs of 4 or 8 bytes, at their own alignment). AWQ: act_mul holds fp32 multipliers [K] applied to the activations as
// they are loaded (AWQ's run-time scaling: x' = rne16(x * m)).
// Metadata (layout 3): scales [N][G8] fp16 and zero-points [N][G8 / 8] words
// of eight 4-bit values (group g in bits 4 (g % 8)), G8 = K / group rounded up
// to a multiple of 8; super-block records [N][K / 256] of 16 bytes.
// b: the row block, h: the range of K (split), blk: the block's index in the
// launch's partials and counters.
template <int GROUP, int MT, bool BF, int FMT, int NCOL, bool AWQ>
__device__ __forceinline__ void decode_body(
    const uint16_t *__restrict__ x, const uint4 *__restrict__ qw, const uint4 *__restrict__ qw_hi,
    const uint16_t *__restrict__ scales, const uint32_t *__restrict__ zeros, uint16_t *__restrict__ y, int M,
    int N, int K, const float *__restrict__ act_mul, int b, int h, int blk, const DecSplit &sp) {
    using FT = FormatTraits<FMT>;
    constexpr int GC = GROUP > kColumn ? kColumn : GROUP;   // closing granularity along K (<= a column)
    constexpr int CPG = GC / kChunk;                       // chunks per group (1, 2, 4)
    constexpr int GPC = kColumn / GC;                      // groups per column (4, 2, 1)
    constexpr int UPC = FT::kquant ? kColChunks : GPC;     // closing units per column
    constexpr int CPU = FT::kquant ? 1 : CPG;              // chunks per closing unit
    constexpr bool HI = !BF && !FT::two_planes;            // fp16 4-bit codes: 16x operands at k2,k3,k6,k7
    constexpr DecLds L = dec_lds(MT, NCOL, GROUP, FMT);
    constexpr int MRB = dec_meta_row_bytes(NCOL, GROUP, FMT);
    constexpr int MRS = dec_meta_stride(NCOL, GROUP, FMT);  // LDS row stride of the metadata (bytes)
    constexpr int ZRS = dec_zero_stride(NCOL, GROUP, FMT);  // LDS row stride of the zero-points (words)
    constexpr int MPARTS = (MRB + 15) / 16;                // 16-byte parts of one row's metadata
    constexpr int MJ = (MPARTS + 3) / 4;                   // metadata loads per lane (LDS path)
    constexpr int ZW = dec_zero_words(NCOL, GROUP, FMT);   // zero-point words of one row
    constexpr int ZJ = (ZW + 3) / 4;                       // zero-point loads per lane (LDS path)
    constexpr int XQ = NCOL / 4;                           // 16-byte activation loads per lane and row
    // small metadata runs (groups 128 and 256) stay in each lane's registers
    constexpr bool MREG = !FT::kquant && MRB <= 32 && ZW <= 2;
    static_assert(NCOL % 4 == 0 && (MRB % 16 == 0 || (MREG && MRB <= 8)),
                  "a slice covers whole 16-byte metadata parts (or a run of at most 8 bytes kept in registers)");
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ float red[kDecMaxWaves][MT][kRowBlock];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15;
    const int s = lane >> 4;
    const int rows_b = min(kRowBlock, N - b * kRowBlock);
    const int rl = r < rows_b ? r : r - rows_b;   // lanes past a short last block re-read a valid row
    const int C = K >> 5;                          // chunks along K
    const int T = (C + 3) >> 2;                    // columns (the last may be partial)
    const int t0 = h * sp.cols + wave * NCOL;      // this wave's columns [t0, min(t0 + NCOL, tend))
    const int tend = min(h * sp.cols + sp.cols, T);
    // a wave past its range's end (the last range may be shorter) reads valid
    // memory at the last slice start before T (a multiple of NCOL, as every
    // slice start is, so its metadata reads stay aligned) and adds nothing
    const int tb = min(t0, ((T - 1) / NCOL) * NCOL);
    const int nfull = min(max(min(C >> 2, tend) - t0, 0), NCOL);
    const int c_lo = tb * kColChunks;
    const int nchunks = max(min(min(t0 + NCOL, tend) * kColChunks, C) - t0 * kColChunks, 0);
    const int G8 = ((K / GROUP) + 7) & ~7;         // metadata slots per row (scales)
    const int gs0 = (int)((int64_t)tb * kColumn / GROUP);   // first group of the slice (K-quant: record)

    unsigned char *wl = smem + wave * L.total;
    unsigned char *xl = wl + L.x;                          // [MT][NCOL * 256]
    float *xs = reinterpret_cast<float *>(wl + L.sums);   // [MT][NCOL * UPC][4] of (B, S)
    unsigned char *ml = wl + L.meta;                       // [16][MRS bytes] (LDS path)
    uint32_t *zl = reinterpret_cast<uint32_t *>(wl + L.zeros);   // [16][ZRS words] (LDS path)

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
    constexpr int NMR = MREG ? MPARTS : MJ;
    constexpr int NZR = MREG ? (ZW > 0 ? ZW : 1) : (ZJ > 0 ? ZJ : 1);
    // (held in one value returned by the loading code: as separate arrays
    // the compiler kept about 14 more registers live in the large-K kernels)
    struct MetaRegs {
        uint4 m[NMR];
        uint32_t z[NZR];
    };
    const MetaRegs meta = [&] {
        MetaRegs mr;
        uint4 *mreg = mr.m;
        uint32_t *zreg = mr.z;
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
            if constexpr (MRB == 8) {   // an 8-byte run (gs0 is a multiple of 4: aligned)
                const uint2 v = *reinterpret_cast<const uint2 *>(base + (size_t)gs0 * 2);
                mreg[0] = make_uint4(v.x, v.y, 0u, 0u);
            } else if constexpr (MRB == 4) {   // a 4-byte run (gs0 even)
                mreg[0] = make_uint4(*reinterpret_cast<const uint32_t *>(base + (size_t)gs0 * 2), 0u, 0u, 0u);
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
        return mr;
    }();
    const uint4 (&mreg)[NMR] = meta.m;
    const uint32_t (&zreg)[NZR] = meta.z;

    // 3. the codes of every column of the slice, all in flight at once (a
    // position past the slice re-reads its last full column: never used)
    const unsigned char *qb = reinterpret_cast<const unsigned char *>(qw) + (size_t)b * 8 * K;
    const unsigned char *qhb = reinterpret_cast<const unsigned char *>(qw_hi) + (size_t)b * 8 * K;
    const uint32_t col_bytes = (uint32_t)rows_b * 64;
    const uint32_t lane_off = nfull > 0 ? (uint32_t)(s * rows_b + rl) * 16u : 0u;
    const int tlast = min(tb + max(nfull - 1, 0), T - 1);
    uint4 rec[NCOL], rech[NCOL];
#pragma unroll
    for (int p = 0; p < NCOL; ++p) {
        const uint32_t cb = (uint32_t)min(tb + p, tlast) * col_bytes;
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
            *reinterpret_cast<uint4 *>(part < MPARTS ? ml + r * MRS + part * 16 : wl + L.spare) = mreg[j];
        }
        if constexpr (ZJ > 0) {
#pragma unroll
            for (int j = 0; j < ZJ; ++j) {
                const int w = mp + 4 * j;
                *(w < ZW ? zl + r * ZRS + w : reinterpret_cast<uint32_t *>(wl + L.spare)) = zreg[j];
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
    const unsigned char *mrow_l = ml + r * MRS;
    const uint32_t *zrow_l = zl + r * ZRS;
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
        if constexpr (!FT::has_zeros) {
            return 0u;
        } else if constexpr (MREG) {
            // one word: the slice's groups sit at nibbles zoff.. of it; two:
            // the slice starts a word (zoff = 0), so the index is static
            if constexpr (ZW <= 1) return (zreg[0] >> (4 * ((g + zoff) & 7))) & 0xFu;
            else return (zreg[g >> 3] >> (4 * (g & 7))) & 0xFu;
        } else {
            return (zrow_l[g >> 3] >> (4 * (g & 7))) & 0xFu;
        }
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
    // the same for a group known only at run time (the partial last column):
    // the register runs are read through selects, not a dynamic index (which
    // would put them in scratch memory)
    auto scale_dyn = [&](int g) -> float {
        if constexpr (MREG) {
            uint32_t w = 0;
#pragma unroll
            for (int q = 0; q < MPARTS; ++q) {
                w = (g >> 3) == q && (g & 7) < 2 ? mreg[q].x : w;
                w = (g >> 3) == q && ((g & 7) >> 1) == 1 ? mreg[q].y : w;
                w = (g >> 3) == q && ((g & 7) >> 1) == 2 ? mreg[q].z : w;
                w = (g >> 3) == q && ((g & 7) >> 1) == 3 ? mreg[q].w : w;
            }
            return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> (16 * (g & 1))));
        } else {
            return scale_of(g);
        }
    };
    auto zero_dyn = [&](int g) -> uint32_t {
        if constexpr (FT::has_zeros && MREG && ZW > 1) {
            const uint32_t w = (g >> 3) == 0 ? zreg[0] : zreg[1];
            return (w >> (4 * (g & 7))) & 0xFu;
        } else {
            return zero_of(g);
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
        if (nfull < NCOL && t0 + nfull == T - 1 && T > (C >> 2) && tend == T) {
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
                if ((j + 1) % CPG == 0 || j == nc - 1) close(c / CPG, scale_dyn(c / CPG), 0.0f, zero_dyn(c / CPG), true);
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
    if (sp.splits == 1) {
        for (int i = threadIdx.x; i < M * kRowBlock; i += blockDim.x) {
            const int m = i >> 4, rr = i & 15;
            if (rr < rows_b) {
                float v = red[0][m][rr];
                for (int w = 1; w < waves; ++w) v += red[w][m][rr];
                y[(int64_t)m * N + b * kRowBlock + rr] = BF ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
            }
        }
        return;
    }
    // split K: this range's partial, then the arrival; the last arrival adds
    // the S partials in split order and writes y. The partials are written
    // and read with device-scope atomic accesses (coherent across the XCDs'
    // L2 caches, which an agent-scope fence would otherwise write back and
    // invalidate whole, thousands of times per launch): every wave waits for
    // its stores to complete (vmcnt(0)) before the barrier, the arrival is
    // counted after it, and the last arrival reads the partials only after its
    // count returned.
    const int MR = M * kRowBlock;
    float *pb = sp.part + (size_t)blk * sp.splits * MR;
    for (int i = threadIdx.x; i < MR; i += blockDim.x) {
        const int m = i >> 4, rr = i & 15;
        float v = red[0][m][rr];
        for (int w = 1; w < waves; ++w) v += red[w][m][rr];
        __hip_atomic_store(pb + (size_t)h * MR + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __shared__ int last;
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long *c = sp.cnt + blk;
        unsigned long long old = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        unsigned long long nv;
        do {
            nv = (old & ~0xFFull) == sp.token ? old + 1 : (sp.token | 1ull);
        } while (!__hip_atomic_compare_exchange_strong(c, &old, nv, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT));
        last = (int)(nv & 0xFFull) == sp.splits;
        // the block is complete: clear its counter (a replay with this token
        // counts from zero again)
        if (last) __hip_atomic_store(c, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last) return;
    for (int i = threadIdx.x; i < MR; i += blockDim.x) {
        const int m = i >> 4, rr = i & 15;
        if (rr < rows_b) {
            float v = __hip_atomic_load(pb + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int j = 1; j < sp.splits; ++j)
                v += __hip_atomic_load(pb + (size_t)j * MR + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            y[(int64_t)m * N + b * kRowBlock + rr] = BF ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
        }
    }
}

// One activation row, no split, K a whole number of 128-weight columns, 4-bit
// codes: the same sums as decode_body in the same order (so the same bits),
// with less held per wave, so that two workgroups of up to 16 waves fit on a
// compute unit at once instead of one:
// * activations stay in registers: lane (s, r) holds slice s of chunks
//   16 q + r of its wave's slice (q = 0 .. NCOL / 4 - 1), and each chunk's
//   slice reaches the 16 lanes of row s by a DPP row broadcast (row_newbcast)
//   from the lane that holds it, instead of being staged through LDS;
// * the per-group activation sums (the magic-offset and zero-point terms) are
//   formed in those lanes, combined over a group's lanes by DPP row shifts in
//   the order decode_body uses, and reach the group's close as the DPP
//   source operand of the subtraction and the fused multiply-add that use
//   them (no broadcast instruction of their own);
// * the codes stream through a ring of D columns per wave: after column p is
//   used, column p + D is loaded into its registers.
// LDS holds only the 16 rows' metadata of each wave's slice (groups 32 and
// 64) and the waves' reduction buffer.
__host__ __device__ constexpr bool dec_bcast_meta_lds(int ncol, int group, int fmt) {
    return dec_meta_row_bytes(ncol, group, fmt) > 32 || dec_zero_words(ncol, group, fmt) > 2;
}
__host__ __device__ constexpr int dec_bcast_lds(int ncol, int group, int fmt) {
    return (dec_bcast_meta_lds(ncol, group, fmt)
                ? 16 * dec_meta_stride(ncol, group, fmt) +
                      (dec_zero_words(ncol, group, fmt) > 0 ? 16 * dec_zero_stride(ncol, group, fmt) * 4 : 0)
                : 0) + 16;
}

// the value of lane j of each row of 16 lanes, in every lane of that row
template <int J>
__device__ inline uint32_t row_bcast(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x150 + J, 0xF, 0xF, false);
}
// The same broadcast as the DPP source operand of the instruction that uses
// it (gfx950 VOP2 forms), so it costs no instruction of its own. Each starts
// with wait states (a VALU write of a register right before a DPP read of it
// needs them, and the compiler does not look inside these), and each is
// volatile: the compiler takes a plain asm statement for a function of its
// own lane's inputs and may move it into code that runs with some lanes
// inactive, where a DPP read returns stale values.
// v - b_J
template <int J>
__device__ inline float sub_rowbcast(float v, float b) {
    asm volatile("s_nop 4\n\tv_subrev_f32_dpp %0, %1, %0 row_newbcast:%2 row_mask:0xf bank_mask:0xf" : "+v"(v) : "v"(b), "n"(J));
    return v;
}
// v + s_J * (-z), one rounding (fma)
template <int J>
__device__ inline float fma_negz_rowbcast(float v, float s, float z) {
    asm volatile("s_nop 4\n\tv_fmac_f32_dpp %0, %1, -%2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
        : "+v"(v) : "v"(s), "v"(z), "n"(J));
    return v;
}

template <int GROUP, bool BF, int FMT, int NCOL, int D>
__global__ __launch_bounds__(64 * kDecMaxWaves) void decode_bcast_kernel(
    const uint16_t *__restrict__ x, const uint4 *__restrict__ qw, const uint16_t *__restrict__ scales,
    const uint32_t *__restrict__ zeros, uint16_t *__restrict__ y, int N, int K) {
    using FT = FormatTraits<FMT>;
    static_assert(!FT::two_planes && !FT::kquant, "4-bit codes with a scale (and zero-point) per group");
    static_assert(NCOL % 4 == 0 && D >= 1 && D <= NCOL, "ring of D columns within a slice of NCOL");
    constexpr int GC = GROUP > kColumn ? kColumn : GROUP;
    constexpr int CPG = GC / kChunk;
    constexpr bool HI = !BF;
    constexpr int MRB = dec_meta_row_bytes(NCOL, GROUP, FMT);
    constexpr int MRS = dec_meta_stride(NCOL, GROUP, FMT);
    constexpr int ZRS = dec_zero_stride(NCOL, GROUP, FMT);
    constexpr int MPARTS = (MRB + 15) / 16;
    constexpr int MJ = (MPARTS + 3) / 4;
    constexpr int ZW = dec_zero_words(NCOL, GROUP, FMT);
    constexpr int ZJ = (ZW + 3) / 4;
    constexpr int XQ = NCOL / 4;                 // activation registers (16 chunks each) per lane
    constexpr bool MREG = !dec_bcast_meta_lds(NCOL, GROUP, FMT);
    constexpr int LDS = dec_bcast_lds(NCOL, GROUP, FMT);
    static_assert(MRB % 16 == 0 || (MREG && MRB <= 8), "whole 16-byte metadata parts");
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ float red[kDecMaxWaves][kRowBlock];

    const int b = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15;
    const int s = lane >> 4;
    const int rows_b = min(kRowBlock, N - b * kRowBlock);
    const int rl = r < rows_b ? r : r - rows_b;
    const int T = K >> 7;                          // columns (K % 128 == 0)
    const int t0 = wave * NCOL;
    const int tb = min(t0, ((T - 1) / NCOL) * NCOL);
    const int nfull = min(max(T - t0, 0), NCOL);
    const int nchunks = nfull * kColChunks;
    const int G8 = ((K / GROUP) + 7) & ~7;
    const int gs0 = (int)((int64_t)tb * kColumn / GROUP);

    unsigned char *wl = smem + wave * LDS;
    unsigned char *ml = wl;                                          // [16][MRS bytes] (LDS path)
    uint32_t *zl = reinterpret_cast<uint32_t *>(wl + 16 * MRS);     // [16][ZRS words] (LDS path)
    unsigned char *spare = wl + LDS - 16;

    // 1. activations: lane (s, r) loads slice s of chunks 16 q + r of the
    // slice (chunks past the slice re-read its first one; never used)
    const uint4 *xsrc = reinterpret_cast<const uint4 *>(x) + (size_t)tb * kColChunks * 4;
    uint4 xq[XQ];
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
        const int cc = 16 * q + r;
        xq[q] = xsrc[(cc < nchunks ? cc : 0) * 4 + s];
    }

    // 2. metadata of the slice (as decode_body: registers for short runs, else LDS rows)
    const int mp = lane >> 4;
    constexpr int NMR = MREG ? MPARTS : MJ;
    constexpr int NZR = MREG ? (ZW > 0 ? ZW : 1) : (ZJ > 0 ? ZJ : 1);
    struct MetaRegs {
        uint4 m[NMR];
        uint32_t z[NZR];
    };
    const MetaRegs meta = [&] {
        MetaRegs mr;
        uint4 *mreg = mr.m;
        uint32_t *zreg = mr.z;
        const int mrow = b * kRowBlock + rl;
        const unsigned char *base = reinterpret_cast<const unsigned char *>(scales) + (size_t)mrow * G8 * 2;
        const int last_part = G8 / 8 - 1;
        const int part0 = gs0 / 8;
        const uint32_t *zb = zeros + (size_t)mrow * (G8 / 8);
        if constexpr (MREG) {
            if constexpr (MRB == 8) {
                const uint2 v = *reinterpret_cast<const uint2 *>(base + (size_t)gs0 * 2);
                mreg[0] = make_uint4(v.x, v.y, 0u, 0u);
            } else if constexpr (MRB == 4) {
                mreg[0] = make_uint4(*reinterpret_cast<const uint32_t *>(base + (size_t)gs0 * 2), 0u, 0u, 0u);
            } else {
#pragma unroll
                for (int j = 0; j < MPARTS; ++j)
                    mreg[j] = *reinterpret_cast<const uint4 *>(base + (size_t)min(part0 + j, last_part) * 16);
            }
            if constexpr (FT::has_zeros) {
#pragma unroll
                for (int j = 0; j < ZW; ++j) zreg[j] = zb[min(gs0 / 8 + j, G8 / 8 - 1)];
            }
        } else {
#pragma unroll
            for (int j = 0; j < MJ; ++j)
                mreg[j] = *reinterpret_cast<const uint4 *>(base + (size_t)min(part0 + mp + 4 * j, last_part) * 16);
            if constexpr (ZJ > 0) {
#pragma unroll
                for (int j = 0; j < ZJ; ++j) zreg[j] = zb[min(gs0 / 8 + mp + 4 * j, G8 / 8 - 1)];
            }
        }
        return mr;
    }();
    const uint4 (&mreg)[NMR] = meta.m;
    const uint32_t (&zreg)[NZR] = meta.z;

    // 3. the first D columns of codes
    const unsigned char *qb = reinterpret_cast<const unsigned char *>(qw) + (size_t)b * 8 * K;
    const uint32_t col_bytes = (uint32_t)rows_b * 64;
    const uint32_t lane_off = nfull > 0 ? (uint32_t)(s * rows_b + rl) * 16u : 0u;
    const int tlast = min(tb + max(nfull - 1, 0), T - 1);
    uint4 rec[D];
    auto load_col = [&](int p) -> uint4 {
        const uint32_t cb = (uint32_t)min(tb + p, tlast) * col_bytes;
        return nt_load(reinterpret_cast<const uint4 *>((qb + cb) + lane_off));
    };
#pragma unroll
    for (int p = 0; p < D; ++p) {
        rec[p] = load_col(p);
        __builtin_amdgcn_sched_barrier(0);
    }

    // 4. metadata to LDS; the activation sums per closing unit and slice:
    // lane (s, r) forms them for chunk 16 q + r, the lanes of a unit are
    // added by row shifts (the unit's sum lands in its last lane)
    __builtin_amdgcn_s_waitcnt((D & 15) | (7 << 4) | (15 << 8) | ((D >> 4) << 14));
    if constexpr (!MREG) {
#pragma unroll
        for (int j = 0; j < MJ; ++j) {
            const int part = mp + 4 * j;
            *reinterpret_cast<uint4 *>(part < MPARTS ? ml + r * MRS + part * 16 : spare) = mreg[j];
        }
        if constexpr (ZJ > 0) {
#pragma unroll
            for (int j = 0; j < ZJ; ++j) {
                const int w = mp + 4 * j;
                *(w < ZW ? zl + r * ZRS + w : reinterpret_cast<uint32_t *>(spare)) = zreg[j];
            }
        }
    }
    constexpr uint32_t one2 = BF ? 0x3F803F80u : 0x3C003C00u;
    constexpr float kMagic = BF ? 128.0f : 1024.0f;
    constexpr float kFixedZ = FT::has_zeros ? 0.0f : (float)FT::fixed_zero;
    float Bq[XQ], Sq[XQ];
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
        const uint4 v = xq[q];
        float lo = dec_dot2<BF>(v.z, one2, dec_dot2<BF>(v.x, one2, 0.0f));
        float hi = dec_dot2<BF>(v.w, one2, dec_dot2<BF>(v.y, one2, 0.0f));
        if constexpr (CPG >= 2) {
            lo = dpp_add_shr<1>(lo);
            hi = dpp_add_shr<1>(hi);
        }
        if constexpr (CPG >= 4) {
            lo = dpp_add_shr<2>(lo);
            hi = dpp_add_shr<2>(hi);
        }
        const float S = lo + hi;
        Sq[q] = S;
        if constexpr (HI)
            Bq[q] = fmaf(kMagic, lo, fmaf(64.0f, hi, kFixedZ * S));
        else
            Bq[q] = (kMagic + kFixedZ) * S;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

    // 5. the columns in order (a column past the slice is computed from copies
    // and not added)
    const UnpackConsts uc = unpack_consts();
    const unsigned char *mrow_l = ml + r * MRS;
    const uint32_t *zrow_l = zl + r * ZRS;
    float acc = 0.0f, lo = 0.0f, hi = 0.0f;
    const int zoff = gs0 & 7;
    auto zero_of = [&](int g) -> uint32_t {
        if constexpr (!FT::has_zeros) {
            return 0u;
        } else if constexpr (MREG) {
            if constexpr (ZW <= 1) return (zreg[0] >> (4 * ((g + zoff) & 7))) & 0xFu;
            else return (zreg[g >> 3] >> (4 * (g & 7))) & 0xFu;
        } else {
            return (zrow_l[g >> 3] >> (4 * (g & 7))) & 0xFu;
        }
    };
    auto scale_of = [&](int g) -> float {
        if constexpr (MREG) {
            const uint4 v = mreg[g >> 3];
            const uint32_t w = (g & 7) < 2 ? v.x : ((g & 7) < 4 ? v.y : ((g & 7) < 6 ? v.z : v.w));
            return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> (16 * (g & 1))));
        } else {
            return (float)*reinterpret_cast<const _Float16 *>(mrow_l + g * 2);
        }
    };
    constexpr float kF = HI ? 0.0625f : 1.0f;
#pragma unroll
    for (int p = 0; p < NCOL; ++p) {
        const bool on = p < nfull;
        const uint4 cur = rec[p % D];
        const uint32_t dws[4] = {cur.x, cur.y, cur.z, cur.w};
#pragma unroll
        for (int j = 0; j < kColChunks; ++j) {
            const int cc = p * kColChunks + j;   // chunk within the slice (compile-time)
            const uint4 xs_q = xq[cc >> 4];
            uint32_t w[4];
            const uint32_t d = dws[j];
            if constexpr (HI) {
                const uint32_t d8 = d >> 8;
                w[0] = and_or(d, uc.lo_mask, uc.f16_magic);
                w[1] = and_or(d, uc.hi_mask, uc.f16_magic);
                w[2] = and_or(d8, uc.lo_mask, uc.f16_magic);
                w[3] = and_or(d8, uc.hi_mask, uc.f16_magic);
            } else {
                const uint32_t magic = uc.bf16_magic;
                w[0] = and_or(d, uc.lo_mask, magic);
                w[1] = and_or(d >> 4, uc.lo_mask, magic);
                w[2] = and_or(d >> 8, uc.lo_mask, magic);
                w[3] = and_or(d >> 12, uc.lo_mask, magic);
            }
            // slice s of chunk cc is held by lane cc % 16 of row s
            switch (cc & 15) {
#define W4A16_BC(J) case J: \
                lo = dec_dot2<BF>(w[0], row_bcast<J>(xs_q.x), lo); hi = dec_dot2<BF>(w[1], row_bcast<J>(xs_q.y), hi); \
                lo = dec_dot2<BF>(w[2], row_bcast<J>(xs_q.z), lo); hi = dec_dot2<BF>(w[3], row_bcast<J>(xs_q.w), hi); \
                break;
                W4A16_BC(0) W4A16_BC(1) W4A16_BC(2) W4A16_BC(3) W4A16_BC(4) W4A16_BC(5) W4A16_BC(6) W4A16_BC(7)
                W4A16_BC(8) W4A16_BC(9) W4A16_BC(10) W4A16_BC(11) W4A16_BC(12) W4A16_BC(13) W4A16_BC(14)
                W4A16_BC(15)
#undef W4A16_BC
            }
            if ((j + 1) % CPG == 0) {
                const int u = cc / CPG;                  // closing unit within the slice
                const int cl = u * CPG + CPG - 1;       // its last chunk: the lane holding its sums
                const int g = GROUP > kColumn ? (p >> 1) : u;
                float part = fmaf(kF, hi, lo);
                const float zf = (float)zero_of(g);
                switch (cl & 15) {
#define W4A16_BS(J) case J: \
                    part = sub_rowbcast<J>(part, Bq[cl >> 4]); \
                    if constexpr (FT::has_zeros) part = fma_negz_rowbcast<J>(part, Sq[cl >> 4], zf); \
                    break;
                    W4A16_BS(0) W4A16_BS(1) W4A16_BS(2) W4A16_BS(3) W4A16_BS(4) W4A16_BS(5) W4A16_BS(6)
                    W4A16_BS(7) W4A16_BS(8) W4A16_BS(9) W4A16_BS(10) W4A16_BS(11) W4A16_BS(12) W4A16_BS(13)
                    W4A16_BS(14) W4A16_BS(15)
#undef W4A16_BS
                }
                (void)zf;
                const float na = fmaf(scale_of(g), part, acc);
                acc = on ? na : acc;
                lo = 0.0f;
                hi = 0.0f;
            }
        }
        if (p + D < NCOL) {
            __builtin_amdgcn_sched_barrier(0);
            rec[p % D] = load_col(p + D);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // 6. reduce: the four lanes of a row, then the waves, in a fixed order
    acc += __shfl_xor(acc, 16, 64);
    acc += __shfl_xor(acc, 32, 64);
    if (s == 0) red[wave][r] = acc;
    __syncthreads();
    const int waves = blockDim.x >> 6;
    if (threadIdx.x < kRowBlock && (int)threadIdx.x < rows_b) {
        const int rr = threadIdx.x;
        float v = red[0][rr];
        for (int w2 = 1; w2 < waves; ++w2) v += red[w2][rr];
        y[b * kRowBlock + rr] = BF ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
    }
}

template <int GROUP, int MT, bool BF, int FMT, int NCOL, bool AWQ>
__global__ __launch_bounds__(64 * kDecMaxWaves) void decode_kernel(
    const uint16_t *__restrict__ x, const uint4 *__restrict__ qw, const uint4 *__restrict__ qw_hi,
    const uint16_t *__restrict__ scales, const uint32_t *__restrict__ zeros, uint16_t *__restrict__ y, int M,
    int N, int K, const float *__restrict__ act_mul, DecSplit sp) {
    const int id = blockIdx.x;
    const int b = id / sp.splits, h = id - b * sp.splits;
    decode_body<GROUP, MT, BF, FMT, NCOL, AWQ>(x, qw, qw_hi, scales, zeros, y, M, N, K, act_mul, b, h, b, sp);
}

// Several independent problems (same M, K, group, format and type) in one
// launch: workgroups [first[p], first[p+1]) belong to problem p, which keeps
// the split of a call on it alone (splits[p] workgroups of cols[p] columns
// per row block: the same partial sums, so the same bits); its counters and
// partials start at blk0[p] and part0[p] of the launch's.
struct DecGroupTable {
    const void *x[kMaxGroup];
    const void *qweight[kMaxGroup];
    const void *scales[kMaxGroup];
    const void *zeros[kMaxGroup];
    void *y[kMaxGroup];
    int N[kMaxGroup];
    int splits[kMaxGroup];
    int cols[kMaxGroup];
    int first[kMaxGroup + 1];
    int blk0[kMaxGroup];
    int64_t part0[kMaxGroup];
    int count;
};

template <int GROUP, int MT, bool BF, int FMT, int NCOL, bool AWQ>
__global__ __launch_bounds__(64 * kDecMaxWaves) void decode_group_kernel(DecGroupTable tab, int M, int K,
                                                                         DecSplit sp) {
    int p = 0;
    while (p + 1 < tab.count && (int)blockIdx.x >= tab.first[p + 1]) ++p;   // uniform
    const int id = (int)blockIdx.x - tab.first[p];
    const DecSplit spp{tab.splits[p], tab.cols[p], sp.part ? sp.part + tab.part0[p] : nullptr,
                       sp.cnt ? sp.cnt + tab.blk0[p] : nullptr, sp.token};
    const int b = id / spp.splits, h = id - b * spp.splits;
    const uint4 *qw = reinterpret_cast<const uint4 *>(tab.qweight[p]);
    decode_body<GROUP, MT, BF, FMT, NCOL, AWQ>(
        reinterpret_cast<const uint16_t *>(tab.x[p]), qw,
        FormatTraits<FMT>::two_planes ? qw + (size_t)tab.N[p] * (K / 32) : qw,   // second plane (8-bit codes)
        reinterpret_cast<const uint16_t *>(tab.scales[p]), reinterpret_cast<const uint32_t *>(tab.zeros[p]),
        reinterpret_cast<uint16_t *>(tab.y[p]), M, tab.N[p], K, nullptr, b, h, b, spp);
}

// The split's view of the workspace: counters [blocks] (8 bytes each, the
// array padded to 256 bytes), then partials [blocks][splits][M][16] fp32.
inline DecSplit dec_split(const DecodePlan &p, void *ws, int blocks) {
    DecSplit sp{p.splits, p.cols, nullptr, nullptr, 0ull};
    if (ws != nullptr) {
        sp.cnt = static_cast<unsigned long long *>(ws);
        sp.part = reinterpret_cast<float *>(static_cast<char *>(ws) + align_up((size_t)blocks * 8, 256));
        unsigned long long t = next_sk_token() & ~0xFFull;
        sp.token = t != 0 ? t : 0x9E3779B97F4A7C00ull;
    }
    return sp;
}

// One launch of the kernel instantiated for (MT, NCOL, AWQ); `grouped` picks
// the several-problem kernel (its table in `tab`).
template <int GROUP, int MT, bool BF, int FMT, int NC, bool AWQ>
hipError_t launch_dec_one(const void *x, const void *qw, const void *qh, const void *sc, const void *zp, void *y,
                          int M, int N, int K, const float *am, const DecodePlan &p, const DecGroupTable *tab,
                          void *ws, hipStream_t stream) {
    auto kern = decode_kernel<GROUP, MT, BF, FMT, NC, AWQ>;
    static DynLdsAttr attr[2];
    if (tab) {   // (the grouped kernel has no activation multipliers)
        if constexpr (AWQ) {
            return hipErrorInvalidValue;
        } else {
            auto gkern = decode_group_kernel<GROUP, MT, BF, FMT, NC, false>;
            hipError_t e = raise_dyn_lds(reinterpret_cast<const void *>(gkern), p.lds, attr[1]);
            if (e != hipSuccess) return e;
            const int blocks = tab->blk0[tab->count - 1] + (int)ceil_div(tab->N[tab->count - 1], kRowBlock);
            hipLaunchKernelGGL(gkern, dim3((unsigned)tab->first[tab->count]), dim3(64 * p.waves), p.lds, stream,
                               *tab, M, K, dec_split(p, ws, blocks));   // (per-problem splits in the table)
        }
    } else {
        hipError_t e = raise_dyn_lds(reinterpret_cast<const void *>(kern), p.lds, attr[0]);
        if (e != hipSuccess) return e;
        const int blocks = (int)ceil_div(N, kRowBlock);
        hipLaunchKernelGGL(kern, dim3((unsigned)(blocks * p.splits)), dim3(64 * p.waves), p.lds, stream,
                           reinterpret_cast<const uint16_t *>(x), reinterpret_cast<const uint4 *>(qw),
                           reinterpret_cast<const uint4 *>(qh), reinterpret_cast<const uint16_t *>(sc),
                           reinterpret_cast<const uint32_t *>(zp), reinterpret_cast<uint16_t *>(y), M, N, K, am,
                           dec_split(p, ws, blocks));
    }
    return hipGetLastError();
}

// A launch of decode_bcast_kernel (plan.bcast: sixteen columns per wave): one
// workgroup per row block, four columns of codes in flight per wave (measured
// on K = 28672, group 32: 29.6 us, against 32.1 / 32.6 us with six / eight,
// and 30.8-31.1 us for decode_kernel on the same device).
template <int GROUP, bool BF, int FMT>
hipError_t launch_dec_bcast(const void *x, const void *qw, const void *sc, const void *zp, void *y, int N, int K,
                            const DecodePlan &p, hipStream_t stream) {
    constexpr int NC = 16, kD = 4;
    auto kern = decode_bcast_kernel<GROUP, BF, FMT, NC, kD>;
    const size_t lds = (size_t)p.waves * dec_bcast_lds(NC, GROUP, FMT);
    static DynLdsAttr attr;
    hipError_t e = raise_dyn_lds(reinterpret_cast<const void *>(kern), lds, attr);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)ceil_div(N, kRowBlock)), dim3(64 * p.waves), lds, stream,
                       reinterpret_cast<const uint16_t *>(x), reinterpret_cast<const uint4 *>(qw),
                       reinterpret_cast<const uint16_t *>(sc), reinterpret_cast<const uint32_t *>(zp),
                       reinterpret_cast<uint16_t *>(y), N, K);
    return hipGetLastError();
}

// the instantiated (rows, columns per wave, AWQ) combinations: the ones
// decode_plan chooses
template <int GROUP, bool BF, int FMT>
hipError_t launch_dec_group(const void *x, const void *qw, const void *qh, const void *sc, const void *zp, void *y,
                            int M, int N, int K, const float *am, const DecodePlan &p, const DecGroupTable *tab,
                            void *ws, hipStream_t stream) {
#define W4A16_DEC(MT_, NC_, AWQ_) \
    launch_dec_one<GROUP, MT_, BF, FMT, NC_, AWQ_>(x, qw, qh, sc, zp, y, M, N, K, am, p, tab, ws, stream)
    const bool awq = am != nullptr;
    if constexpr (FMT == kAsym4 || FMT == kSym4) {
        if (p.bcast && tab == nullptr) {   // one activation row, no split, no multipliers, K % 128 == 0
            if (awq || p.mt != 1 || p.splits != 1 || p.ncol != 16 || K % kColumn != 0) return hipErrorInvalidValue;
            return launch_dec_bcast<GROUP, BF, FMT>(x, qw, sc, zp, y, N, K, p, stream);
        }
    }
    switch (p.mt * 100 + p.ncol * 2 + (awq ? 1 : 0)) {
        case 108: return W4A16_DEC(1, 4, false);
        case 109: return W4A16_DEC(1, 4, true);
        case 116: return W4A16_DEC(1, 8, false);
        case 117: return W4A16_DEC(1, 8, true);
        case 132: return W4A16_DEC(1, 16, false);
        case 133: return W4A16_DEC(1, 16, true);
        case 208: return W4A16_DEC(2, 4, false);
        case 209: return W4A16_DEC(2, 4, true);
        case 216: return W4A16_DEC(2, 8, false);
        case 217: return W4A16_DEC(2, 8, true);
        case 232: return W4A16_DEC(2, 16, false);
        case 233: return W4A16_DEC(2, 16, true);
        case 408: return W4A16_DEC(4, 4, false);
        case 409: return W4A16_DEC(4, 4, true);
        case 416: return W4A16_DEC(4, 8, false);
        case 417: return W4A16_DEC(4, 8, true);
        case 808: return W4A16_DEC(8, 4, false);
        case 809: return W4A16_DEC(8, 4, true);
        case 816: return W4A16_DEC(8, 8, false);
        case 817: return W4A16_DEC(8, 8, true);
        default: return hipErrorInvalidValue;
    }
#undef W4A16_DEC
}

template <bool BF, int FMT>
hipError_t launch_dec_groups(const void *x, const void *qw, const void *qh, const void *sc, const void *zp, void *y,
                             int M, int N, int K, int group, const float *am, const DecodePlan &p,
                             const DecGroupTable *tab, void *ws, hipStream_t stream) {
#define W4A16_DEC_G(G_) launch_dec_group<G_, BF, FMT>(x, qw, qh, sc, zp, y, M, N, K, am, p, tab, ws, stream)
    if constexpr (FormatTraits<FMT>::kquant) {
        return W4A16_DEC_G(256);
    } else {
        switch (group) {
            case 32: return W4A16_DEC_G(32);
            case 64: return W4A16_DEC_G(64);
            case 128: return W4A16_DEC_G(128);
            default: return W4A16_DEC_G(256);
        }
    }
#undef W4A16_DEC_G
}

}  // namespace

// The launches of one weight format. K-quant super-blocks: group 256.
template <int FMT>
hipError_t launch_decode_fmt(const void *x, bool bf16, const void *qweight, const void *scales, const void *zeros,
                             void *y, int M, int N, int K, int group, const float *am, const DecodePlan &plan,
                             void *workspace, hipStream_t stream) {
    if (!plan.ok || (plan.splits > 1 && workspace == nullptr)) return hipErrorInvalidValue;
    const void *qh = FormatTraits<FMT>::two_planes
                         ? static_cast<const void *>(static_cast<const char *>(qweight) + (size_t)N * K / 2)
                         : qweight;
    return bf16 ? launch_dec_groups<true, FMT>(x, qweight, qh, scales, zeros, y, M, N, K, group, am, plan, nullptr,
                                               workspace, stream)
                : launch_dec_groups<false, FMT>(x, qweight, qh, scales, zeros, y, M, N, K, group, am, plan, nullptr,
                                                workspace, stream);
}

// plans[p]: each problem's own plan (the same mt and ncol for all); the
// launch runs the most waves and LDS any of them needs. Workspace: counters
// for every problem's row blocks (padded to 256 bytes), then the partials of
// the problems that split, in order.
template <int FMT>
hipError_t launch_decode_group_fmt(const GroupTable &gt, bool bf16, int M, int K, int group, const DecodePlan *plans,
                                   void *workspace, hipStream_t stream) {
    if (gt.count < 1 || gt.count > kMaxGroup) return hipErrorInvalidValue;
    DecGroupTable tab{};
    tab.count = gt.count;
    DecodePlan plan = plans[0];
    bool split = false;
    int wgs = 0, blocks = 0;
    int64_t part = 0;
    for (int i = 0; i < gt.count; ++i) {
        const DecodePlan &q = plans[i];
        if (!q.ok || q.mt != plan.mt || q.ncol != plan.ncol) return hipErrorInvalidValue;
        plan.waves = std::max(plan.waves, q.waves);
        plan.lds = std::max(plan.lds, q.lds);
        tab.x[i] = gt.x[i];
        tab.qweight[i] = gt.qweight[i];
        tab.scales[i] = gt.scales[i];
        tab.zeros[i] = gt.zeros[i];
        tab.y[i] = gt.y[i];
        tab.N[i] = gt.N[i];
        tab.splits[i] = q.splits;
        tab.cols[i] = q.cols;
        tab.first[i] = wgs;
        tab.blk0[i] = blocks;
        tab.part0[i] = part;
        const int nb = (int)ceil_div(gt.N[i], kRowBlock);
        wgs += nb * q.splits;
        blocks += nb;
        if (q.splits > 1) {
            part += (int64_t)nb * q.splits * M * kRowBlock;
            split = true;
        }
    }
    if (split && workspace == nullptr) return hipErrorInvalidValue;
    if (!split) workspace = nullptr;
    tab.first[gt.count] = wgs;
    return bf16 ? launch_dec_groups<true, FMT>(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, M, 0, K, group,
                                               nullptr, plan, &tab, workspace, stream)
                : launch_dec_groups<false, FMT>(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, M, 0, K, group,
                                                nullptr, plan, &tab, workspace, stream);
}

}  // namespace w4a16
