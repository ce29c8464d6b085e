// Matrix-core (MFMA) path of the W4A16 linear layer for small and medium
// batches: y[m][n] = sum_k x[m][k] * w_hat[n][k], x taken 16 rows at a time.
//
// Up to a batch of a few dozen tokens the layer still reads every weight once
// per call and does little arithmetic per byte, so it stays bound by the
// weight stream ("Weight-Only Quantisation", the FAQ answer on when the
// method stops paying; "Weight-Only Quantization Explained", the section on
// where it stops being the right answer). What changes with M is the
// arithmetic per weight: the dot-product kernel spends M multiply-adds per
// weight in the vector ALUs, this kernel spends one matrix instruction per 32
// weights of a row for all M (padded to 16) at once.
//
// Mapping (gfx950, wave64). Same stream as the dot-product kernel: a
// workgroup owns R blocks of 16 output rows and all of K; its waves split K
// into slices of 128-weight columns; lane l = 16 s + r loads, per column and
// row block, dword s of the column's four chunks of row r, plus row r's scales
// and zero-points of the column. Each of those dwords is the B operand of one
// v_mfma_f32_16x16x32 (column n = r, k-slice [8s, 8s+8) of the chunk); the A
// operand is x[m][k-slice] for m = l % 16, loaded straight from memory (it is
// shared by every workgroup and lives in the caches), and reused by the R row
// blocks. The result lane l holds y[4 s + v][r] (v = 0..3).
//
// fp16 activations: the dword unpacks to the exact integers (q - z) in fp16;
// the group's MFMAs accumulate sum x*(q-z) in fp32 and the group scale
// multiplies that sum. bf16 activations: the dword unpacks to exact bf16
// (128 + q); a second MFMA against a B of ones gives sum x over the same k,
// and sum x*(128+q) - (128+z)*sum x = sum x*(q-z), all in fp32. Weight
// formats (FMT): symmetric codes use a fixed zero; 8-bit codes add a second
// MFMA per chunk on the high-nibble plane (2048 + 16 hi in bf16); K-quant
// super-blocks close every chunk with its own scale and minimum
// (S * sum x q - M * sum x, sum x from the MFMA against ones).
#pragma once

#include <stdlib.h>

#include "decode_common.hpp"

namespace w4a16 {
namespace {

constexpr int kSkinnyMaxWaves = 8;   // two waves per SIMD at most: up to 256 VGPRs each

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

template <bool BF>
__device__ inline f4_t mfma16x16x32(const uint4 &a, const uint4 &b, f4_t c) {
    if constexpr (BF)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8_t, a), __builtin_bit_cast(b8_t, b),
                                                        c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a), __builtin_bit_cast(h8_t, b),
                                                       c, 0, 0, 0);
}

// The body of one workgroup; `id` is its index within its problem.
template <int GROUP, int R, bool BF, int FMT>
__device__ __forceinline__ void skinny_body(const uint16_t *__restrict__ x, const uint4 *__restrict__ qw,
                                            const uint4 *__restrict__ qw_hi,
                                            const uint16_t *__restrict__ scales,
                                            const uint32_t *__restrict__ zeros, uint16_t *__restrict__ y,
                                            int M, int N, int K, int mtiles, int mshift, int id) {
    using FT = FormatTraits<FMT>;
    constexpr int CPG = GROUP / kChunk;    // chunks per group (1, 2, 4)
    constexpr int GPC = kColumn / GROUP;   // groups per column (4, 2, 1)
    constexpr int PF = R == 1 ? 4 : (R == 2 ? 3 : 2);   // columns in flight ahead of the one computing
    __shared__ f4_t red[4 * kSkinnyMaxWaves][64];   // [wave * R + i][lane]

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int waves = blockDim.x >> 6;
    const int r = lane & 15;
    const int s = lane >> 4;
    const int nblocks = (N + kRowBlock - 1) / kRowBlock;
    const Slice sl = wave_slice<GROUP>(K, wave, waves);
    // workgroup = (group of R row blocks, 16-row tile of x); the x tiles of one
    // weight group are neighbours in launch order, so they share its stream
    // through the caches
    const int mtile = id % mtiles;
    const int wg = id / mtiles;
    const int M_loc = min(16, M - 16 * mtile);
    x += (size_t)16 * mtile * K;
    y += (size_t)16 * mtile * N;

    // per row block i of this workgroup: packed base, lane record, metadata
    // row; a workgroup past the last block repeats the last one (not stored)
    const uint4 *qw_b[R], *qwh_b[R];
    uint32_t lane_rec[R], col_rec[R];
    const ColScales<GPC> *sc_row[R];   // the row's scales, in units of one column's GPC values
    const uint4 *kq_row[R];            // kq4: the row's super-block records
    const uint32_t *zp_row[R];         // the row's zero-point words
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int b = min(wg * R + i, nblocks - 1);
        const int rows = min(kRowBlock, N - b * kRowBlock);
        const int rl = r < rows ? r : r - rows;   // lanes past a short block re-read a valid row
        qw_b[i] = qw + (size_t)b * (K / 2);
        qwh_b[i] = qw_hi + (size_t)b * (K / 2);   // 8-bit codes: the high-nibble plane
        lane_rec[i] = (uint32_t)(s * rows + rl);
        col_rec[i] = (uint32_t)(kColChunks * rows);
        const int n = b * kRowBlock + rl;
        const int G8 = meta_slots(K, GROUP << mshift);   // (group 256 runs these kernels with mshift = 1)
        sc_row[i] = reinterpret_cast<const ColScales<GPC> *>(scales + (size_t)n * G8);
        kq_row[i] = reinterpret_cast<const uint4 *>(scales) + (size_t)n * (K / 256);
        zp_row[i] = zeros + (size_t)n * (G8 / 8);
    }
    // A operand rows: lane row r, clamped to the last real row of x (rows of
    // the 16-row tile past M produce outputs that are never stored)
    const uint4 *xrow = reinterpret_cast<const uint4 *>(x) + (size_t)min(r, M_loc - 1) * (K / 8) + s;
    const UnpackConsts uc = unpack_consts();
    constexpr uint32_t one2 = BF ? 0x3F803F80u : 0x3C003C00u;   // (1.0, 1.0) in the activation type
    const uint4 ones = make_uint4(one2, one2, one2, one2);

    struct Buf {
        uint4 xa[kColChunks];
        uint4 rec[R], rec_hi[R], kq[R];
        ColScales<GPC> sc[R];
        uint32_t zw[R];
        int zsh;   // bit offset of the column's first zero-point in zw
        int par;   // column parity: which half of the super-block (kq4)
    };
    // metadata slot of column t: t >> mshift (group 256: one slot per two
    // columns). The zero-point word is kept as loaded and shifted where it is
    // used: a shift here would make the wave wait for the load at once, and
    // (loads complete in order) for every prefetch issued before it.
    auto load_meta = [&](int t, Buf &u) {
        const int tm = t >> mshift;
        u.par = t & 1;
        u.zsh = 4 * ((tm * GPC) & 7);
#pragma unroll
        for (int i = 0; i < R; ++i) {
            if constexpr (FT::kquant) {
                u.kq[i] = kq_row[i][t >> 1];
            } else {
                u.sc[i] = sc_row[i][tm];
                if constexpr (FT::has_zeros) u.zw[i] = zp_row[i][(tm * GPC) >> 3];
                else u.zw[i] = 0;
            }
        }
    };
    auto load_col = [&](int t, Buf &u) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            u.rec[i] = nt_load(&qw_b[i][(uint32_t)t * col_rec[i] + lane_rec[i]]);
            if constexpr (FT::two_planes) u.rec_hi[i] = nt_load(&qwh_b[i][(uint32_t)t * col_rec[i] + lane_rec[i]]);
        }
#pragma unroll
        for (int j = 0; j < kColChunks; ++j) u.xa[j] = xrow[(size_t)(t * kColChunks + j) * 4];
        load_meta(t, u);
        __builtin_amdgcn_sched_barrier(0);
    };

    f4_t acc[R];
#pragma unroll
    for (int i = 0; i < R; ++i) acc[i] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // chunk j of a column: dword d of row block i, A fragment xa; group sums
    // in g (and, bf16, sum x in sx); at the group's end scale into acc
    // (dh: the same dword of the high-nibble plane of 8-bit codes)
    auto chunk = [&](const uint4 &xa, uint32_t d, uint32_t dh, uint32_t z, f4_t &g, f4_t &sx) {
        uint32_t w[4];
        if constexpr (BF) {
            unpack_bf16_magic(d, uc, w);
            g = mfma16x16x32<BF>(xa, make_uint4(w[0], w[1], w[2], w[3]), g);
            if constexpr (FT::two_planes) {
                unpack_bf16_magic16(dh, uc, w);
                g = mfma16x16x32<BF>(xa, make_uint4(w[0], w[1], w[2], w[3]), g);
            }
            sx = mfma16x16x32<BF>(xa, ones, sx);
        } else {
            unpack_f16_fmt<FMT>(d, dh, z, uc, w);
            g = mfma16x16x32<BF>(xa, make_uint4(w[0], w[1], w[2], w[3]), g);
            if constexpr (FT::kquant) sx = mfma16x16x32<BF>(xa, ones, sx);   // sum x for the minimum
        }
    };
    auto zero_of = [&](uint32_t zw, int zsh, int e) -> uint32_t {
        if constexpr (FT::has_zeros) return (zw >> (zsh + 4 * e)) & 0xFu;
        else return FT::fixed_zero;
    };
    auto close_group = [&](int i, float sc, uint32_t z, f4_t &g, f4_t &sx) {
        if constexpr (BF) {
            const float zb = -bf16_magic_bias<FMT>(z);
#pragma unroll
            for (int v = 0; v < 4; ++v) g[v] = fmaf(zb, sx[v], g[v]);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][v] = fmaf(sc, g[v], acc[i][v]);
        g = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
        sx = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
    };
    // kq4: chunk j is a 32-weight sub-block: acc += S * sum x q - M * sum x
    auto close_kq = [&](int i, const KqParams &P, f4_t &g, f4_t &sx) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float gq = BF ? fmaf(-128.0f, sx[v], g[v]) : g[v];   // bf16 operands carry 128 + q
            acc[i][v] = fmaf(P.S, gq, fmaf(-P.M, sx[v], acc[i][v]));
        }
        g = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
        sx = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
    };
    auto compute_col = [&](const Buf &u) {
        if constexpr (FT::kquant) {
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const uint32_t dk[4] = {u.rec[i].x, u.rec[i].y, u.rec[i].z, u.rec[i].w};
                f4_t g = {0.0f, 0.0f, 0.0f, 0.0f}, sx = {0.0f, 0.0f, 0.0f, 0.0f};
                const KqHalf hf = kq_half(u.kq[i], u.par != 0);
#pragma unroll
                for (int j = 0; j < kColChunks; ++j) {
                    chunk(u.xa[j], dk[j], 0u, 0u, g, sx);
                    close_kq(i, kq_sub(hf, j), g, sx);
                }
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const uint32_t dws[4] = {u.rec[i].x, u.rec[i].y, u.rec[i].z, u.rec[i].w};
            const uint32_t dwh[4] = {u.rec_hi[i].x, u.rec_hi[i].y, u.rec_hi[i].z, u.rec_hi[i].w};
            f4_t g = {0.0f, 0.0f, 0.0f, 0.0f}, sx = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int j = 0; j < kColChunks; ++j) {
                const int e = j / CPG;
                const uint32_t z = zero_of(u.zw[i], u.zsh, e);
                chunk(u.xa[j], dws[j], dwh[j], z, g, sx);
                if ((j + 1) % CPG == 0) close_group(i, u.sc[i].get(e), z, g, sx);
            }
        }
    };

    // stream the full columns: column t computes while t+1..t+PF are in
    // flight; the ring is indexed by compile-time positions
    Buf ring[PF + 1];
#pragma unroll
    for (int i = 0; i < PF; ++i)
        if (sl.t_begin + i < sl.t_full) load_col(sl.t_begin + i, ring[i]);
    int t = sl.t_begin;
    for (; t + PF + 1 <= sl.t_full; t += PF + 1) {
#pragma unroll
        for (int i = 0; i <= PF; ++i) {
            load_col(min(t + i + PF, sl.t_full - 1), ring[(i + PF) % (PF + 1)]);
            compute_col(ring[i]);
        }
    }
#pragma unroll
    for (int i = 0; i <= PF; ++i)
        if (t + i < sl.t_full) compute_col(ring[i]);

    // the partial last column of K (K % 128 != 0): nc < 4 chunks, each lane's
    // nc dwords are consecutive
    if (!FT::kquant && sl.t_end > sl.t_full) {   // (kq4: K % 256 == 0, every column is full)
        const int tl = sl.t_end - 1;
        const int nc = sl.C - tl * kColChunks;
        Buf u;
        load_meta(tl, u);
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int rows = (int)(col_rec[i] / kColChunks);
            const size_t off = (size_t)tl * rows * 16 + (size_t)s * rows * nc + (size_t)(lane_rec[i] - s * rows) * nc;
            const uint32_t *col = reinterpret_cast<const uint32_t *>(qw_b[i]) + off;
            const uint32_t *colh = reinterpret_cast<const uint32_t *>(qwh_b[i]) + off;
            f4_t g = {0.0f, 0.0f, 0.0f, 0.0f}, sx = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int j = 0; j < nc; ++j) {
                const int e = j / CPG;
                const uint32_t z = zero_of(u.zw[i], u.zsh, e);
                chunk(xrow[(size_t)(tl * kColChunks + j) * 4], col[j], FT::two_planes ? colh[j] : 0u, z, g, sx);
                if ((j + 1) % CPG == 0 || j == nc - 1) close_group(i, u.sc[i].get(e), z, g, sx);
            }
        }
    }

    // reduce over the waves in a fixed order; lane l holds y[4 s + v][r]
#pragma unroll
    for (int i = 0; i < R; ++i) red[wave * R + i][lane] = acc[i];
    __syncthreads();
    for (int o = threadIdx.x; o < R * 256; o += blockDim.x) {
        const int i = o / 256, m = (o / 16) % 16, rr = o % 16;
        const int b = wg * R + i;
        if (b >= nblocks || m >= M_loc) continue;
        const int rows = min(kRowBlock, N - b * kRowBlock);
        if (rr >= rows) continue;
        const int src = 16 * (m / 4) + rr, v = m % 4;
        float acc_o = red[i][src][v];
        for (int w = 1; w < waves; ++w) acc_o += red[w * R + i][src][v];
        y[(int64_t)m * N + b * kRowBlock + rr] = BF ? f32_to_bf16_bits(acc_o) : f32_to_f16_bits(acc_o);
    }
}

template <int GROUP, int R, bool BF, int FMT>
__global__ __launch_bounds__(64 * kSkinnyMaxWaves) void skinny_kernel(
    const uint16_t *__restrict__ x, const uint4 *__restrict__ qw, const uint4 *__restrict__ qw_hi,
    const uint16_t *__restrict__ scales, const uint32_t *__restrict__ zeros, uint16_t *__restrict__ y, int M,
    int N, int K, int mtiles, int mshift) {
    skinny_body<GROUP, R, BF, FMT>(x, qw, qw_hi, scales, zeros, y, M, N, K, mtiles, mshift, blockIdx.x);
}

// Several independent problems (same M, K, group, format and type) in one
// launch: workgroups [first[p], first[p+1]) belong to problem p.
template <int GROUP, int R, bool BF, int FMT>
__global__ __launch_bounds__(64 * kSkinnyMaxWaves) void skinny_group_kernel(GroupTable tab, int M, int K,
                                                                            int mtiles, int mshift) {
    int p = 0;
    while (p + 1 < tab.count && (int)blockIdx.x >= tab.first[p + 1]) ++p;   // uniform
    const uint4 *qw = reinterpret_cast<const uint4 *>(tab.qweight[p]);
    skinny_body<GROUP, R, BF, FMT>(reinterpret_cast<const uint16_t *>(tab.x[p]), qw,
                                   qw + (size_t)tab.N[p] * (K / 32),   // second plane (8-bit codes)
                                   reinterpret_cast<const uint16_t *>(tab.scales[p]),
                                   reinterpret_cast<const uint32_t *>(tab.zeros[p]),
                                   reinterpret_cast<uint16_t *>(tab.y[p]), M, tab.N[p], K, mtiles, mshift,
                                   (int)blockIdx.x - tab.first[p]);
}

template <int GROUP, bool BF, int FMT>
hipError_t launch_skinny_group(GroupTable tab, int M, int K, int ms, const GemmPlan &plan, hipStream_t stream) {
    const int mtiles = (int)ceil_div(M, 16);
    const int R = plan.rows_per_wg;
    int total = 0;
    for (int p = 0; p < tab.count; ++p) {
        tab.first[p] = total;
        total += (int)ceil_div(ceil_div(tab.N[p], kRowBlock), R) * mtiles;
    }
    tab.first[tab.count] = total;
    const dim3 grid((unsigned)total), block(64 * plan.waves);
    switch (R) {
        case 1: hipLaunchKernelGGL((skinny_group_kernel<GROUP, 1, BF, FMT>), grid, block, 0, stream, tab, M, K, mtiles, ms); break;
        case 2: hipLaunchKernelGGL((skinny_group_kernel<GROUP, 2, BF, FMT>), grid, block, 0, stream, tab, M, K, mtiles, ms); break;
        default: hipLaunchKernelGGL((skinny_group_kernel<GROUP, 4, BF, FMT>), grid, block, 0, stream, tab, M, K, mtiles, ms); break;
    }
    return hipGetLastError();
}

template <int GROUP, bool BF, int FMT>
hipError_t launch_skinny(const void *x, const void *qw, const void *qh, const void *sc, const void *zp, void *y,
                         int M, int N, int K, int ms, const GemmPlan &plan, hipStream_t stream) {
    const int nblocks = (int)ceil_div(N, kRowBlock);
    const dim3 block(64 * plan.waves);
    auto args = [&](auto kern, int R) {
        const int mtiles = (int)ceil_div(M, 16);
        hipLaunchKernelGGL(kern, dim3((unsigned)(ceil_div(nblocks, R) * mtiles)), block, 0, stream,
                           reinterpret_cast<const uint16_t *>(x), reinterpret_cast<const uint4 *>(qw),
                           reinterpret_cast<const uint4 *>(qh), reinterpret_cast<const uint16_t *>(sc),
                           reinterpret_cast<const uint32_t *>(zp), reinterpret_cast<uint16_t *>(y), M, N, K,
                           mtiles, ms);
    };
    switch (plan.rows_per_wg) {
        case 1: args(skinny_kernel<GROUP, 1, BF, FMT>, 1); break;
        case 2: args(skinny_kernel<GROUP, 2, BF, FMT>, 2); break;
        default: args(skinny_kernel<GROUP, 4, BF, FMT>, 4); break;
    }
    return hipGetLastError();
}

}  // namespace

// The small-batch launches of one weight format. Group 256 runs the
// group-128 kernels with one metadata slot per two columns (mshift = 1).
template <int FMT>
hipError_t launch_skinny_fmt(const void *x, bool bf16, const void *qweight, const void *scales, const void *zeros,
                             void *y, int M, int N, int K, int group, const GemmPlan &plan, hipStream_t stream) {
    const int ms = group == 256 ? 1 : 0;
    const void *qh = FormatTraits<FMT>::two_planes
                         ? static_cast<const void *>(static_cast<const char *>(qweight) + (size_t)N * K / 2)
                         : qweight;
    if constexpr (FormatTraits<FMT>::kquant) {   // one 32-weight sub-block per chunk
        return bf16 ? launch_skinny<32, true, FMT>(x, qweight, qh, scales, zeros, y, M, N, K, 0, plan, stream)
                    : launch_skinny<32, false, FMT>(x, qweight, qh, scales, zeros, y, M, N, K, 0, plan, stream);
    } else {
    if (bf16) {
        switch (group) {
            case 32: return launch_skinny<32, true, FMT>(x, qweight, qh, scales, zeros, y, M, N, K, ms, plan, stream);
            case 64: return launch_skinny<64, true, FMT>(x, qweight, qh, scales, zeros, y, M, N, K, ms, plan, stream);
            default: return launch_skinny<128, true, FMT>(x, qweight, qh, scales, zeros, y, M, N, K, ms, plan, stream);
        }
    }
    switch (group) {
        case 32: return launch_skinny<32, false, FMT>(x, qweight, qh, scales, zeros, y, M, N, K, ms, plan, stream);
        case 64: return launch_skinny<64, false, FMT>(x, qweight, qh, scales, zeros, y, M, N, K, ms, plan, stream);
        default: return launch_skinny<128, false, FMT>(x, qweight, qh, scales, zeros, y, M, N, K, ms, plan, stream);
    }    }
}

template <int FMT>
hipError_t launch_skinny_group_fmt(const GroupTable &tab, bool bf16, int M, int K, int group, const GemmPlan &plan,
                                   hipStream_t stream) {
    const int ms = group == 256 ? 1 : 0;
    if constexpr (FormatTraits<FMT>::kquant) {
        return bf16 ? launch_skinny_group<32, true, FMT>(tab, M, K, 0, plan, stream)
                    : launch_skinny_group<32, false, FMT>(tab, M, K, 0, plan, stream);
    } else {
    if (bf16) {
        switch (group) {
            case 32: return launch_skinny_group<32, true, FMT>(tab, M, K, ms, plan, stream);
            case 64: return launch_skinny_group<64, true, FMT>(tab, M, K, ms, plan, stream);
            default: return launch_skinny_group<128, true, FMT>(tab, M, K, ms, plan, stream);
        }
    }
    switch (group) {
        case 32: return launch_skinny_group<32, false, FMT>(tab, M, K, ms, plan, stream);
        case 64: return launch_skinny_group<64, false, FMT>(tab, M, K, ms, plan, stream);
        default: return launch_skinny_group<128, false, FMT>(tab, M, K, ms, plan, stream);
    }    }
}

}  // namespace w4a16
