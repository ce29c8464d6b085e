// Decode GEMV for the W4A16 linear layer, y[m][n] = sum_k x[m][k] * w_hat[n][k],
// for small M (1..8), with fp16/bf16 dot products and fp32 accumulation.
//
// At small batch each weight is read once per token and used for only M
// multiply-adds, so the weight stream from HBM is the bottleneck
// ("Weight-Only Quantisation", first two FAQ answers; "Weight-Only
// Quantization Explained", "Where it stops being the right answer"). The
// weights stay packed until they reach registers ("Quantization Is Not a Zip
// File", section 8) and are rebuilt as 16-bit values just before the multiply
// ("Weight-Only Quantisation", definition).
//
// Mapping (gfx950, wave64). A workgroup owns one block of 16 output rows and
// all of K; its waves split K into slices of 128-weight columns. Lane
// l = 16 s + r holds, for every column, dword s of the column's four chunks of
// row r (one non-temporal 16-byte load per lane; one contiguous KiB per wave),
// together with row r's scales and zero-points of that column (one small load
// each, from the per-column metadata layout), prefetched several columns ahead
// in a register ring. The activations of the slice are staged in the wave's
// own LDS region (multiplied there by AWQ's per-channel factors when given).
// The four lanes of a row meet through cross-lane shuffles at the end, the
// waves through LDS, always in the same order, so results are deterministic
// and no partial sum leaves the workgroup.
//
// fp16 activations: each dword unpacks to four exact (q - z) fp16 pairs and
// v_dot2_f32_f16 multiplies them with the activation pairs, accumulating in
// fp32; the group scale multiplies the fp32 group sum. bf16 activations: the
// dword unpacks to bf16 pairs (128 + q); the sum of x*(128+q) over the
// dword's 8 weights minus (128 + z) times the sum of those 8 activations is
// the sum of x*(q - z), both in fp32. The other weight formats (FMT) change
// only the unpack and the per-group terms: a fixed zero (symmetric), a second
// code plane (8-bit), or a per-chunk scale and minimum (K-quant super-blocks).
#pragma once

#include <stdlib.h>

#include "decode_common.hpp"

namespace w4a16 {
namespace {

constexpr int kMaxWaves = kGemvMaxWaves;
// Rows of one workgroup: 16 (a block of the layout; a wave load is one column
// of it) or 8 (half a block; a wave load covers two columns of those rows).
// Eight-row workgroups double the workgroup count, which a plain streaming
// read rewards (35 MB: 12.9 us with 320 workgroups, 7.7 us with 640), but
// here they split every 256-byte segment of a column between two workgroups
// and measured 3% faster at 5120 x 5120 and 4-25% slower on the other decode
// shapes, so 16 is the default.
constexpr int kRowsPerWg = kGemvRowsPerWg;
#ifndef W4A16_GEMV_PREFETCH
#define W4A16_GEMV_PREFETCH 6
#endif
constexpr int kPrefetch = W4A16_GEMV_PREFETCH;   // columns in flight ahead of the one computing

template <bool BF>
__device__ inline float dot_pair(uint32_t w, uint32_t x, float acc) {
    if constexpr (BF)
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, w),
                                               __builtin_bit_cast(bf162_t, x), acc, false);
    else
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w),
                                      __builtin_bit_cast(half2_t, x), acc, false);
}

// Eight 16-bit activations times eight fp32 multipliers, each product rounded
// once to the activation type (round to nearest even).
template <bool BF>
__device__ inline uint4 scale8(const uint4 &v, const float4 &a, const float4 &b) {
    const float m[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    const uint32_t in[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float lo, hi;
        if constexpr (BF) {
            lo = __builtin_bit_cast(float, in[i] << 16);
            hi = __builtin_bit_cast(float, in[i] & 0xFFFF0000u);
        } else {
            const half2_t h = __builtin_bit_cast(half2_t, in[i]);
            lo = (float)h.x;
            hi = (float)h.y;
        }
        const float2_t p = {lo * m[2 * i], hi * m[2 * i + 1]};
        if constexpr (BF)
            out[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf162_t));
        else
            out[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, half2_t));
    }
    return make_uint4(out[0], out[1], out[2], out[3]);
}

// LDS bytes of one wave: activations [MT][xcols*128] (16-bit) and, when
// `sums` (bf16 activations, or super-block minima), their sums over every 8
// consecutive k ([MT][xcols*16] fp32).
__host__ __device__ inline size_t wave_lds_bytes(int MT, int xcols, bool sums) {
    return (size_t)MT * xcols * 256 + (sums ? (size_t)MT * xcols * 64 : 0);
}

// act_mul: NULL, or fp32 multipliers [K] applied to the activations as they
// are staged (AWQ's run-time scaling: x' = rne16(x * m)).
template <int GROUP, int MT, bool BF, int FMT>
__global__ __launch_bounds__(64 * kMaxWaves) __attribute__((amdgpu_waves_per_eu(1, 4))) void gemv_kernel(
    const uint16_t *__restrict__ x, const uint4 *__restrict__ qw, const uint4 *__restrict__ qw_hi,
    const uint16_t *__restrict__ scales, const uint32_t *__restrict__ zeros, uint16_t *__restrict__ y, int N,
    int K, int xcols, int mshift, const float *__restrict__ act_mul) {
    using FT = FormatTraits<FMT>;
    constexpr int CPG = GROUP / kChunk;   // chunks per group (1, 2, 4)
    constexpr int PF0 = MT == 1 ? kPrefetch : (MT == 2 ? 4 : (MT <= 4 ? 3 : 2));
    // 8-bit: the same bytes in flight; kq4: room for the super-block record
    constexpr int PF = FormatTraits<FMT>::two_planes ? (PF0 + 1) / 2 : (FormatTraits<FMT>::kquant ? PF0 - 1 : PF0);
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int RW = kRowsPerWg;          // rows of this workgroup
    constexpr int CPW = kRowBlock / RW;     // columns covered by one wave load (1 or 2)
    __shared__ float red[kMaxWaves][MT][RW];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int waves = blockDim.x >> 6;
    const int r = lane % RW;               // row within the workgroup's rows
    const int s = (lane / RW) & 3;         // dword position: k-slice [8s, 8s+8) of each chunk
    const int cw = lane / (4 * RW);        // which column of the wave load (0 when CPW = 1)
    const int n0 = blockIdx.x * RW;        // first row of the workgroup
    const int b = n0 / kRowBlock;          // its 16-row block of the layout
    const int rows_b = min(kRowBlock, N - b * kRowBlock);
    const int rows = min(RW, N - n0);
    const int rl = r < rows ? r : r - rows;   // lanes past a short last block re-read a valid row
    const int rib = n0 % kRowBlock + rl;       // row within the 16-row block

    constexpr int GPC = kColumn / GROUP;   // groups per column (4, 2, 1)
    const Slice sl = wave_slice<GROUP>(K, wave, waves);
    const int nchunks = sl.c_hi - sl.c_lo;

    // this wave's LDS region
    constexpr bool kSums = BF || FT::kquant;   // sums of every 8 activations are staged
    unsigned char *wbase = smem + (size_t)wave * wave_lds_bytes(MT, xcols, kSums);
    uint4 *xw = reinterpret_cast<uint4 *>(wbase);                                        // [MT][xcols*16]
    float *xsw = reinterpret_cast<float *>(wbase + (size_t)MT * xcols * 256);           // [MT][xcols*16]

    // weights: block base, full column t at t*4*rows_b uint4, lane at s*rows_b + rib
    const uint4 *qw_b = qw + (size_t)b * (K / 2);
    const uint4 *qwh_b = qw_hi + (size_t)b * (K / 2);   // 8-bit codes: the high-nibble plane
    const uint32_t lane_rec = (uint32_t)(s * rows_b + rib);
    const uint32_t col_rec = (uint32_t)(kColChunks * rows_b);
    const UnpackConsts uc = unpack_consts();
    // per-column metadata of row n: GPC scales at (t*N + n)*GPC, GPC zero
    // nibbles starting at nibble (t*N + n)*GPC of the zero words, where t is
    // the column >> mshift (group 256: one metadata slot serves two columns)
    const int n = n0 + rl;
    const ColScales<GPC> *sc_row = reinterpret_cast<const ColScales<GPC> *>(scales) + n;
    const uint32_t *zp_row = zeros + (n * GPC) / 8;
    const int zshift = 4 * ((n * GPC) % 8);

    // super-block records (kq4): one per 256 weights of row n, [K/256][N]
    const uint4 *kq_row = reinterpret_cast<const uint4 *>(scales) + n;
    struct Buf {
        uint4 rec, rec_hi, kq;
        ColScales<GPC> sc;
        uint32_t zw;
        int t;       // the lane's column
        float on;    // 1, or 0 for a lane past the slice's last full column (CPW = 2)
    };
    auto load_meta = [&](int t, Buf &u) {
        if constexpr (FT::kquant) {
            u.kq = kq_row[(size_t)(t >> 1) * N];
        } else {
            const int tm = t >> mshift;
            u.sc = sc_row[(size_t)tm * N];
            if constexpr (FT::has_zeros) u.zw = zp_row[(size_t)tm * (N * GPC / 8)];
            else u.zw = 0;
        }
    };
    // iteration p of the wave covers columns t_begin + CPW p + cw of its slice
    const int iters = (sl.t_full - sl.t_begin + CPW - 1) / CPW;
    auto load_col = [&](int p, Buf &u) {
        const int tc = sl.t_begin + CPW * p + cw;
        const bool in = CPW == 1 || tc < sl.t_full;
        const int t = in ? tc : sl.t_full - 1;   // a lane past the last full column re-reads one (weight 0)
        u.t = t;
        u.on = in ? 1.0f : 0.0f;
        u.rec = nt_load(&qw_b[(uint32_t)t * col_rec + lane_rec]);
        if constexpr (FT::two_planes) u.rec_hi = nt_load(&qwh_b[(uint32_t)t * col_rec + lane_rec]);
        load_meta(t, u);
        // keep the prefetch where it is: the scheduler may not sink these
        // loads towards their use (which would serialise the stream)
        __builtin_amdgcn_sched_barrier(0);
    };

    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
    Buf ring[PF + 1];

    // 1. stage: activation loads first, weight prefetch right behind them,
    // then the LDS stores (vector-memory counters retire in
    // order, so the stores wait for the stage loads only)
    {
        const uint4 *xg = reinterpret_cast<const uint4 *>(x);
        const int per_m = nchunks * 4;                 // uint4 of one activation row in the slice
        const int xtotal = MT * per_m;
        auto xsrc = [&](int i) {
            i = max(min(i, xtotal - 1), 0);
            const int m = i / per_m;
            return xg[(size_t)m * (K / 8) + sl.c_lo * 4 + (i - m * per_m)];
        };
        auto xdst = [&](int i, const uint4 &v) {
            if (i < xtotal) {
                const int m = i / per_m;
                xw[(size_t)m * xcols * 16 + (i - m * per_m)] = v;
            }
        };
        for (int base = 0; base < xtotal; base += 8 * 64) {
            const uint4 v0 = xsrc(base + 0 * 64 + lane), v1 = xsrc(base + 1 * 64 + lane);
            const uint4 v2 = xsrc(base + 2 * 64 + lane), v3 = xsrc(base + 3 * 64 + lane);
            const uint4 v4 = xsrc(base + 4 * 64 + lane), v5 = xsrc(base + 5 * 64 + lane);
            const uint4 v6 = xsrc(base + 6 * 64 + lane), v7 = xsrc(base + 7 * 64 + lane);
            if (base == 0) {
#pragma unroll
                for (int i = 0; i < PF; ++i)
                    if (i < iters) load_col(i, ring[i]);
            }
            xdst(base + 0 * 64 + lane, v0); xdst(base + 1 * 64 + lane, v1);
            xdst(base + 2 * 64 + lane, v2); xdst(base + 3 * 64 + lane, v3);
            xdst(base + 4 * 64 + lane, v4); xdst(base + 5 * 64 + lane, v5);
            xdst(base + 6 * 64 + lane, v6); xdst(base + 7 * 64 + lane, v7);
        }
        if (act_mul != nullptr) {
            // AWQ: scale the staged activations in place (each lane rewrites
            // the entries it stored; the multiplier loads retire after the
            // weight prefetch, which the first column waits for anyway)
            const float4 *mv = reinterpret_cast<const float4 *>(act_mul);
            for (int i = lane; i < xtotal; i += 64) {
                const int m = i / per_m, q = i - m * per_m;
                const int k8 = sl.c_lo * 4 + q;   // 8-activation unit along K
                uint4 &slot = xw[(size_t)m * xcols * 16 + q];
                slot = scale8<BF>(slot, mv[2 * k8], mv[2 * k8 + 1]);
            }
        }
        if constexpr (kSums) {
            // sum of every 8 activations (one k-slice of one chunk)
            constexpr uint32_t one2 = BF ? 0x3F803F80u : 0x3C003C00u;   // (1.0, 1.0)
            for (int i = lane; i < MT * nchunks * 4; i += 64) {
                const int m = i / (nchunks * 4), q = i - m * (nchunks * 4);
                const uint4 v = xw[(size_t)m * xcols * 16 + q];
                float sum = 0.0f;
                sum = dot_pair<BF>(v.x, one2, sum);
                sum = dot_pair<BF>(v.y, one2, sum);
                sum = dot_pair<BF>(v.z, one2, sum);
                sum = dot_pair<BF>(v.w, one2, sum);
                xsw[(size_t)m * xcols * 16 + q] = sum;
            }
        }
        // every LDS store above precedes every LDS read below (same wave, in order)
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }

    // one dword of chunk c (this lane's k-slice; dh: the same dword of the
    // high-nibble plane of 8-bit codes), group e of the column: adds its dot
    // product to p
    auto dword_dot = [&](int c, uint32_t d, uint32_t dh, uint32_t z, float (&p)[MT]) {
        uint32_t w[4], wh[4];
        if constexpr (BF) {
            unpack_bf16_magic(d, uc, w);
            if constexpr (FT::two_planes) unpack_bf16_magic16(dh, uc, wh);
        } else {
            unpack_f16_fmt<FMT>(d, dh, z, uc, w);
        }
        const int q = (c - sl.c_lo) * 4 + s;   // uint4 index of this k-slice in the wave's x
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint4 xv = xw[(size_t)m * xcols * 16 + q];
            float t = dot_pair<BF>(w[0], xv.x, 0.0f);
            t = dot_pair<BF>(w[1], xv.y, t);
            t = dot_pair<BF>(w[2], xv.z, t);
            t = dot_pair<BF>(w[3], xv.w, t);
            if constexpr (BF && FT::two_planes) {
                t = dot_pair<BF>(wh[0], xv.x, t);
                t = dot_pair<BF>(wh[1], xv.y, t);
                t = dot_pair<BF>(wh[2], xv.z, t);
                t = dot_pair<BF>(wh[3], xv.w, t);
            }
            if constexpr (BF) t = fmaf(-bf16_magic_bias<FMT>(z), xsw[(size_t)m * xcols * 16 + q], t);
            p[m] += t;
        }
    };
    auto zero_of = [&](uint32_t zw, int e) -> uint32_t {
        if constexpr (FT::has_zeros) return (zw >> (zshift + 4 * e)) & 0xFu;
        else return FT::fixed_zero;
    };
    auto close_group = [&](float sc, float (&p)[MT]) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            acc[m] = fmaf(sc, p[m], acc[m]);
            p[m] = 0.0f;
        }
    };
    // kq4: chunk c is one 32-weight sub-block with its own scale S and
    // minimum M; its contribution is S * sum x q - M * sum x, added to acc
    // (both types take the magic operands 128 + q / 1024 + q and remove the
    // offset with the chunk's activation sum, which the minimum needs anyway)
    auto dword_kq = [&](int c, uint32_t d, const KqParams &P) {
        uint32_t w[4];
        if constexpr (BF)
            unpack_bf16_magic(d, uc, w);
        else
            unpack_f16_magic(d, uc, w);
        const int q = (c - sl.c_lo) * 4 + s;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint4 xv = xw[(size_t)m * xcols * 16 + q];
            const float xs = xsw[(size_t)m * xcols * 16 + q];
            float t = dot_pair<BF>(w[0], xv.x, 0.0f);
            t = dot_pair<BF>(w[1], xv.y, t);
            t = dot_pair<BF>(w[2], xv.z, t);
            t = dot_pair<BF>(w[3], xv.w, t);
            t = fmaf(BF ? -128.0f : -1024.0f, xs, t);   // the magic operands carry 128 + q / 1024 + q
            acc[m] = fmaf(P.S, t, fmaf(-P.M, xs, acc[m]));
        }
    };
    auto compute_col = [&](const Buf &u) {
        const int t = u.t;
        if constexpr (FT::kquant) {
            const uint32_t dk[4] = {u.rec.x, u.rec.y, u.rec.z, u.rec.w};
            const KqHalf hf = kq_half(u.kq, (t & 1) != 0);
#pragma unroll
            for (int j = 0; j < kColChunks; ++j) {
                KqParams P = kq_sub(hf, j);
                if constexpr (CPW > 1) {   // (one column per wave load: every lane is on)
                    P.S *= u.on;
                    P.M *= u.on;
                }
                dword_kq(t * kColChunks + j, dk[j], P);
            }
            return;
        }
        const uint32_t dws[4] = {u.rec.x, u.rec.y, u.rec.z, u.rec.w};
        const uint32_t dwh[4] = {u.rec_hi.x, u.rec_hi.y, u.rec_hi.z, u.rec_hi.w};
        float p[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) p[m] = 0.0f;
#pragma unroll
        for (int j = 0; j < kColChunks; ++j) {
            const int e = j / CPG;
            const uint32_t z = zero_of(u.zw, e);
            dword_dot(t * kColChunks + j, dws[j], dwh[j], z, p);
            if ((j + 1) % CPG == 0) close_group(u.sc.get(e) * u.on, p);
        }
    };

    // 2. stream the full columns: column t computes while t+1..t+PF are in
    // flight. The ring is indexed by compile-time positions (the loop is
    // unrolled by the ring size), so no register with a load in flight is
    // ever copied, and the loop body has no lane-dependent branch.
    int it = 0;
    for (; it + PF + 1 <= iters; it += PF + 1) {
#pragma unroll
        for (int i = 0; i <= PF; ++i) {
            load_col(min(it + i + PF, iters - 1), ring[(i + PF) % (PF + 1)]);
            compute_col(ring[i]);
        }
    }
#pragma unroll
    for (int i = 0; i <= PF; ++i)
        if (it + i < iters) compute_col(ring[i]);

    // 3. the partial last column of K (K % 128 != 0): nc < 4 chunks, each
    // lane's nc dwords are consecutive; its metadata has the usual layout
    if (!FT::kquant && sl.t_end > sl.t_full && cw == 0) {   // (kq4: K % 256 == 0, every column is full)
        const int tl = sl.t_end - 1;
        const int nc = sl.C - tl * kColChunks;
        const size_t off = (size_t)tl * rows_b * 16 + (size_t)s * rows_b * nc + (size_t)rib * nc;
        const uint32_t *col = reinterpret_cast<const uint32_t *>(qw_b) + off;
        const uint32_t *colh = reinterpret_cast<const uint32_t *>(qwh_b) + off;
        Buf u;
        load_meta(tl, u);
        float p[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) p[m] = 0.0f;
        for (int j = 0; j < nc; ++j) {
            const int e = j / CPG;
            const uint32_t z = zero_of(u.zw, e);
            dword_dot(tl * kColChunks + j, col[j], FT::two_planes ? colh[j] : 0u, z, p);
            if ((j + 1) % CPG == 0 || j == nc - 1) close_group(u.sc.get(e), p);
        }
    }

    // 4. reduce: the lanes of a row (its four k-slices and, when CPW = 2, its
    // two columns), then the waves (fixed order)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        float v = acc[m];
#pragma unroll
        for (int off = RW; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
        acc[m] = v;
    }
    if (lane < RW) {
#pragma unroll
        for (int m = 0; m < MT; ++m) red[wave][m][r] = acc[m];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < MT * RW; i += blockDim.x) {
        const int m = i / RW;
        const int rr = i % RW;
        if (rr < rows) {
            float v = red[0][m][rr];
            for (int w = 1; w < waves; ++w) v += red[w][m][rr];
            y[(int64_t)m * N + n0 + rr] = BF ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
        }
    }
}

template <int GROUP, bool BF, int MT, int FMT>
hipError_t launch_one(const void *x, const void *qw, const void *qw_hi, const void *sc, const void *zp, void *y,
                      int N, int K, int mshift, const float *am, const GemvPlan &plan, hipStream_t stream) {
    const int xcols = gemv_xcols(K, plan.waves);
    const size_t lds = wave_lds_bytes(MT, xcols, BF || FormatTraits<FMT>::kquant) * plan.waves;
    auto kern = gemv_kernel<GROUP, MT, BF, FMT>;
    static DynLdsAttr attr;
    hipError_t e = raise_dyn_lds(reinterpret_cast<const void *>(kern), lds, attr);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(plan.row_blocks), dim3(64 * plan.waves), lds, stream,
                       reinterpret_cast<const uint16_t *>(x), reinterpret_cast<const uint4 *>(qw),
                       reinterpret_cast<const uint4 *>(qw_hi), reinterpret_cast<const uint16_t *>(sc),
                       reinterpret_cast<const uint32_t *>(zp), reinterpret_cast<uint16_t *>(y), N, K, xcols,
                       mshift, am);
    return hipGetLastError();
}

template <int GROUP, bool BF, int FMT>
hipError_t launch_m(int M, const void *x, const void *qw, const void *qh, const void *sc, const void *zp, void *y,
                    int N, int K, int ms, const float *am, const GemvPlan &plan, hipStream_t stream) {
    switch (M) {
        case 1: return launch_one<GROUP, BF, 1, FMT>(x, qw, qh, sc, zp, y, N, K, ms, am, plan, stream);
        case 2: return launch_one<GROUP, BF, 2, FMT>(x, qw, qh, sc, zp, y, N, K, ms, am, plan, stream);
        case 3: return launch_one<GROUP, BF, 3, FMT>(x, qw, qh, sc, zp, y, N, K, ms, am, plan, stream);
        case 4: return launch_one<GROUP, BF, 4, FMT>(x, qw, qh, sc, zp, y, N, K, ms, am, plan, stream);
        case 5: return launch_one<GROUP, BF, 5, FMT>(x, qw, qh, sc, zp, y, N, K, ms, am, plan, stream);
        case 6: return launch_one<GROUP, BF, 6, FMT>(x, qw, qh, sc, zp, y, N, K, ms, am, plan, stream);
        case 7: return launch_one<GROUP, BF, 7, FMT>(x, qw, qh, sc, zp, y, N, K, ms, am, plan, stream);
        default: return launch_one<GROUP, BF, 8, FMT>(x, qw, qh, sc, zp, y, N, K, ms, am, plan, stream);
    }
}

}  // namespace

// The launches of one weight format. Group 256 runs the group-128 kernels
// with one metadata slot per two columns (mshift = 1).
template <int FMT>
hipError_t launch_gemv_fmt(const void *x, bool bf16, const void *qweight, const void *scales, const void *zeros,
                           void *y, int M, int N, int K, int group, const float *am, const GemvPlan &plan,
                           hipStream_t stream) {
    const int ms = group == 256 ? 1 : 0;
    const void *qh = FormatTraits<FMT>::two_planes
                         ? static_cast<const void *>(static_cast<const char *>(qweight) + (size_t)N * K / 2)
                         : qweight;
    if constexpr (FormatTraits<FMT>::kquant) {   // one 32-weight sub-block per chunk
        return bf16 ? launch_m<32, true, FMT>(M, x, qweight, qh, scales, zeros, y, N, K, 0, am, plan, stream)
                    : launch_m<32, false, FMT>(M, x, qweight, qh, scales, zeros, y, N, K, 0, am, plan, stream);
    } else {
    if (bf16) {
        switch (group) {
            case 32: return launch_m<32, true, FMT>(M, x, qweight, qh, scales, zeros, y, N, K, ms, am, plan, stream);
            case 64: return launch_m<64, true, FMT>(M, x, qweight, qh, scales, zeros, y, N, K, ms, am, plan, stream);
            default: return launch_m<128, true, FMT>(M, x, qweight, qh, scales, zeros, y, N, K, ms, am, plan, stream);
        }
    }
    switch (group) {
        case 32: return launch_m<32, false, FMT>(M, x, qweight, qh, scales, zeros, y, N, K, ms, am, plan, stream);
        case 64: return launch_m<64, false, FMT>(M, x, qweight, qh, scales, zeros, y, N, K, ms, am, plan, stream);
        default: return launch_m<128, false, FMT>(M, x, qweight, qh, scales, zeros, y, N, K, ms, am, plan, stream);
    }    }
}

}  // namespace w4a16
