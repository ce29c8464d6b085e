// Decode GEMV for the W4A16 linear layer, y[m][n] = sum_k x[m][k] * w_hat[n][k],
// for small M (1..8).
//
// At small batch each weight is read once per token and used for only M
// multiply-adds, so the kernel is bound by the weight stream from HBM
// ("Weight-Only Quantisation", first two FAQ answers; "Weight-Only
// Quantization Explained", "Where it stops being the right answer"). The
// weights stay packed until they reach registers ("Quantization Is Not a Zip
// File", section 8) and are rebuilt as 16-bit values just before the multiply
// ("Weight-Only Quantisation", definition).
//
// Mapping (gfx950, wave64). A workgroup owns 16 output rows and all of K; its
// W waves split K into contiguous slices of 128-weight columns. Inside a wave,
// lane (r, s) = (lane / 4, lane % 4) handles row r and chunk s of every
// column, so one wave load is four 256-byte runs of 16-byte records (16 rows x
// 4 chunks). Because a workgroup covers all of K, no partial sum ever leaves
// the workgroup: the four chunk lanes of a row meet through DPP (quad
// shuffles), the waves through LDS, always in the same order, so results are
// deterministic and no cross-workgroup synchronisation (or L2 writeback) is
// needed. Narrow N still fills the chip because the waves per workgroup grow
// as N shrinks. The activations of the workgroup are staged once in LDS; for
// bf16 the stage also stores each 32-weight chunk's activation sum.
//
// Unpack, fp16 activations: for a dword d holding k0..k7 (even k in the low
// half-word), (d & 0x000F000F) | 0x64006400 is the fp16 pair (1024+q0, 1024+q1)
// and (d & 0x00F000F0) | 0x64006400 is (1024+16 q2, 1024+16 q3); subtracting
// (1024+z), or scaling by 1/16 and subtracting (64+z), gives q - z exactly,
// and v_dot2_f32_f16 multiplies by the fp16 activation pair with fp32
// accumulation. The group's scale multiplies the fp32 chunk sum.
// bf16 activations: ((d >> 4i) & 0x000F000F) | 0x43004300 is the bf16 pair
// (128+q, 128+q'); the chunk sum of x*(128+q) minus (128+z) times the chunk
// sum of x is the chunk sum of x*(q-z) (both sums in fp32).
#include <stdlib.h>

#include "w4a16_internal.hpp"

namespace w4a16 {
namespace {

constexpr int kRowsPerWave = 16;
constexpr int kChunkLanes = 4;
constexpr int kMaxWaves = 16;
#ifndef W4A16_GEMV_PREFETCH
#define W4A16_GEMV_PREFETCH 6
#endif
constexpr int kPrefetch = W4A16_GEMV_PREFETCH;   // columns in flight ahead of the one computing

// A 32-bit constant materialised in a VGPR. VOP3 instructions (v_and_or_b32)
// cannot take two literal operands on gfx9, so the masks and magic numbers of
// the unpack live in registers, which lets (d & mask) | magic issue as one
// v_and_or_b32 instead of a v_and + v_or pair.
__device__ inline uint32_t vconst(uint32_t c) {
    uint32_t r;
    asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
    return r;
}

struct UnpackConsts {
    uint32_t lo_mask, hi_mask, f16_magic, bf16_magic;
};

__device__ inline UnpackConsts unpack_consts() {
    return UnpackConsts{vconst(0x000F000Fu), vconst(0x00F000F0u), vconst(0x64006400u), vconst(0x43004300u)};
}

__device__ inline uint32_t and_or(uint32_t a, uint32_t mask, uint32_t bits) { return (a & mask) | bits; }

template <bool BF>
__device__ inline float dot_pair(uint32_t w, uint32_t x, float acc) {
    if constexpr (BF)
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, w),
                                               __builtin_bit_cast(bf162_t, x), acc, false);
    else
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w),
                                      __builtin_bit_cast(half2_t, x), acc, false);
}

// One record (32 weights of one row, one group) -> 16 activation-ready pairs.
// fp16: the pairs are q - z exactly. bf16: the pairs are 128 + q.
template <bool BF>
__device__ inline void unpack_record(const uint4 &rec, uint32_t z, const UnpackConsts &uc,
                                     uint32_t (&t)[16]) {
    const uint32_t dws[4] = {rec.x, rec.y, rec.z, rec.w};
    if constexpr (BF) {
        (void)z;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t d = dws[j];
            t[4 * j + 0] = and_or(d, uc.lo_mask, uc.bf16_magic);
            t[4 * j + 1] = and_or(d >> 4, uc.lo_mask, uc.bf16_magic);
            t[4 * j + 2] = and_or(d >> 8, uc.lo_mask, uc.bf16_magic);
            t[4 * j + 3] = and_or(d >> 12, uc.lo_mask, uc.bf16_magic);
        }
    } else {
        const half2_t a = __builtin_bit_cast(half2_t, (0xE400u | z) * 0x00010001u);          // -(1024+z)
        const half2_t b = __builtin_bit_cast(half2_t, (0xD400u + 16u * z) * 0x00010001u);    // -(64+z)
        const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t d = dws[j];
            const uint32_t d8 = d >> 8;
            half2_t h0 = __builtin_bit_cast(half2_t, and_or(d, uc.lo_mask, uc.f16_magic));
            half2_t h1 = __builtin_bit_cast(half2_t, and_or(d, uc.hi_mask, uc.f16_magic));
            half2_t h2 = __builtin_bit_cast(half2_t, and_or(d8, uc.lo_mask, uc.f16_magic));
            half2_t h3 = __builtin_bit_cast(half2_t, and_or(d8, uc.hi_mask, uc.f16_magic));
            t[4 * j + 0] = __builtin_bit_cast(uint32_t, h0 + a);
            t[4 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(h1, sixteenth, b));
            t[4 * j + 2] = __builtin_bit_cast(uint32_t, h2 + a);
            t[4 * j + 3] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(h3, sixteenth, b));
        }
    }
}

template <int GROUP, int MT, bool BF>
__global__ __launch_bounds__(1024) void gemv_kernel(const uint16_t *__restrict__ x,
                                                    const uint4 *__restrict__ qw,
                                                    const uint16_t *__restrict__ scales,
                                                    const uint32_t *__restrict__ zeros,
                                                    uint16_t *__restrict__ y, int N, int K) {
    // LDS image of the activations: x[m][k] as 16-bit values, then (bf16 only)
    // the fp32 sum of every 32-weight chunk of every row, [MT][K/32].
    extern __shared__ __align__(16) unsigned char smem[];
    uint4 *xs16 = reinterpret_cast<uint4 *>(smem);
    float *xsum = reinterpret_cast<float *>(smem + (size_t)MT * K * 2);
    __shared__ float red[kMaxWaves][MT][kRowsPerWave];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int waves = blockDim.x >> 6;
    const int r = lane >> 2;          // row within the workgroup's 16
    const int s = lane & 3;           // chunk within a 128-weight column
    const int n0 = blockIdx.x * kRowsPerWave;
    const int rows = min(kRowsPerWave, N - n0);
    const bool row_ok = r < rows;
    const int n = n0 + (row_ok ? r : 0);

    // this wave's slice of 128-weight columns
    const int C = K / kChunk;                 // chunks along K
    const int T = (C + kChunkLanes - 1) / kChunkLanes;
    const int t_begin = (int)(((int64_t)wave * T) / waves);
    const int t_end = (int)(((int64_t)(wave + 1) * T) / waves);

    // record (n, chunk c) sits at uint4 index rb*2K + c*rows_b + (n % 64)
    const int rb = n / kRowBlock;
    const int rows_b = min(kRowBlock, N - rb * kRowBlock);
    const uint4 *rec_base = qw + (int64_t)rb * 2 * K + (n % kRowBlock);
    const uint16_t *sc_base = scales + n;
    const uint32_t *zp_base = zeros + (n >> 3);
    const int zshift = 4 * (n & 7);
    const UnpackConsts uc = unpack_consts();

    struct Buf {
        uint4 rec;
        uint32_t sc, zw;
    };
    // This lane's chunk of column t, clamped into range: a clamped lane
    // re-reads a valid record and its result is dropped in compute_col.
    auto load_col = [&](int t, Buf &b) {
        const int c = min(t * kChunkLanes + s, C - 1);
        const uint32_t g = (uint32_t)(c * kChunk) / GROUP;
        b.rec = rec_base[(uint32_t)c * (uint32_t)rows_b];
        b.sc = sc_base[(size_t)g * (uint32_t)N];
        b.zw = zp_base[(size_t)g * (uint32_t)(N / 8)];
        // keep the prefetch where it is: the scheduler may not sink these
        // loads towards their use (which would serialise the stream)
        __builtin_amdgcn_sched_barrier(0);
    };

    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;

    auto compute_col = [&](int t, const Buf &b) {
        const int c = t * kChunkLanes + s;
        if (c < C) {
            const uint32_t z = (b.zw >> zshift) & 0xFu;
            uint32_t w[16];
            unpack_record<BF>(b.rec, z, uc, w);
            const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)b.sc);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const uint4 *xp = xs16 + ((size_t)m * K + (size_t)c * kChunk) / 8;
                float p = 0.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint4 xv = xp[j];
                    p = dot_pair<BF>(w[4 * j + 0], xv.x, p);
                    p = dot_pair<BF>(w[4 * j + 1], xv.y, p);
                    p = dot_pair<BF>(w[4 * j + 2], xv.z, p);
                    p = dot_pair<BF>(w[4 * j + 3], xv.w, p);
                }
                if constexpr (BF) p = fmaf(-(float)(128u + z), xsum[(size_t)m * C + c], p);
                acc[m] = fmaf(sc, p, acc[m]);
            }
        }
    };

    // 1. start the weight stream before anything else
    Buf ring[kPrefetch + 1];
#pragma unroll
    for (int i = 0; i < kPrefetch; ++i)
        if (t_begin + i < t_end) load_col(t_begin + i, ring[i]);

    // 2. stage the activations (and the bf16 chunk sums) in LDS
    {
        const int per_row = K / 8;                 // uint4 per activation row
        const uint4 *xg = reinterpret_cast<const uint4 *>(x);
        for (int i = threadIdx.x; i < MT * per_row; i += blockDim.x) xs16[i] = xg[i];
        if constexpr (BF) {
            __syncthreads();
            for (int i = threadIdx.x; i < MT * C; i += blockDim.x) {
                const uint4 *xp = xs16 + (size_t)i * 4;   // chunk i of the [MT][C] grid
                float sum = 0.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint4 v = xp[j];
                    sum = dot_pair<true>(v.x, 0x3F803F80u, sum);
                    sum = dot_pair<true>(v.y, 0x3F803F80u, sum);
                    sum = dot_pair<true>(v.z, 0x3F803F80u, sum);
                    sum = dot_pair<true>(v.w, 0x3F803F80u, sum);
                }
                xsum[i] = sum;
            }
        }
        __syncthreads();
    }

    // 3. stream: column t computes while t+1..t+kPrefetch are in flight. The
    // ring is indexed by compile-time positions (the loop is unrolled by the
    // ring size), so no register with a load in flight is ever copied.
    int t = t_begin;
    for (; t + kPrefetch + 1 <= t_end; t += kPrefetch + 1) {
#pragma unroll
        for (int i = 0; i <= kPrefetch; ++i) {
            const int tl = t + i + kPrefetch;
            if (tl < t_end) load_col(tl, ring[(i + kPrefetch) % (kPrefetch + 1)]);
            compute_col(t + i, ring[i]);
        }
    }
#pragma unroll
    for (int i = 0; i <= kPrefetch; ++i)
        if (t + i < t_end) compute_col(t + i, ring[i]);

    // 4. reduce: the four chunk lanes of a row (DPP quad shuffles), then the waves
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        float v = acc[m];
        v += __shfl_xor(v, 1, 64);
        v += __shfl_xor(v, 2, 64);
        acc[m] = v;
    }
    if (s == 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m) red[wave][m][r] = acc[m];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < MT * kRowsPerWave; i += blockDim.x) {
        const int m = i / kRowsPerWave;
        const int rr = i % kRowsPerWave;
        if (rr < rows) {
            float v = red[0][m][rr];
            for (int w = 1; w < waves; ++w) v += red[w][m][rr];
            y[(int64_t)m * N + n0 + rr] = BF ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
        }
    }
}

template <int GROUP, bool BF, int MT>
hipError_t launch_one(const void *x, const void *qw, const void *sc, const void *zp, void *y, int N,
                      int K, const GemvPlan &plan, hipStream_t stream) {
    const size_t lds = gemv_lds_bytes(MT, K, BF);
    auto kern = gemv_kernel<GROUP, MT, BF>;
    if (lds > 48 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(plan.row_blocks), dim3(64 * plan.waves), lds, stream,
                       reinterpret_cast<const uint16_t *>(x), reinterpret_cast<const uint4 *>(qw),
                       reinterpret_cast<const uint16_t *>(sc), reinterpret_cast<const uint32_t *>(zp),
                       reinterpret_cast<uint16_t *>(y), N, K);
    return hipGetLastError();
}

template <int GROUP, bool BF>
hipError_t launch_m(int M, const void *x, const void *qw, const void *sc, const void *zp, void *y, int N,
                    int K, const GemvPlan &plan, hipStream_t stream) {
    switch (M) {
        case 1: return launch_one<GROUP, BF, 1>(x, qw, sc, zp, y, N, K, plan, stream);
        case 2: return launch_one<GROUP, BF, 2>(x, qw, sc, zp, y, N, K, plan, stream);
        case 3: return launch_one<GROUP, BF, 3>(x, qw, sc, zp, y, N, K, plan, stream);
        case 4: return launch_one<GROUP, BF, 4>(x, qw, sc, zp, y, N, K, plan, stream);
        case 5: return launch_one<GROUP, BF, 5>(x, qw, sc, zp, y, N, K, plan, stream);
        case 6: return launch_one<GROUP, BF, 6>(x, qw, sc, zp, y, N, K, plan, stream);
        case 7: return launch_one<GROUP, BF, 7>(x, qw, sc, zp, y, N, K, plan, stream);
        default: return launch_one<GROUP, BF, 8>(x, qw, sc, zp, y, N, K, plan, stream);
    }
}

}  // namespace

size_t gemv_lds_bytes(int64_t M, int64_t K, bool bf16) {
    return (size_t)M * K * 2 + (bf16 ? (size_t)M * (K / kChunk) * 4 : 0);
}

GemvPlan gemv_plan(int64_t M, int64_t N, int64_t K, int32_t group) {
    (void)M;
    (void)group;
    static const int forced_waves = [] {
        const char *v = getenv("W4A16_GEMV_WAVES");
        return v ? atoi(v) : 0;
    }();
    GemvPlan p{};
    p.row_blocks = (int)ceil_div(N, kRowsPerWave);
    const int64_t columns = ceil_div(K / kChunk, kChunkLanes);
    // about 16 resident waves per CU over 256 CUs, at least 2 columns per wave
    int64_t w = ceil_div(4096, p.row_blocks);
    if (w > columns / 2) w = columns / 2;
    if (forced_waves > 0) w = forced_waves;
    if (w > kMaxWaves) w = kMaxWaves;
    if (w < 1) w = 1;
    p.waves = (int)w;
    return p;
}

hipError_t launch_gemv(const void *x, bool bf16, const void *qweight, const void *scales,
                       const void *zeros, void *y, int M, int N, int K, int group,
                       const GemvPlan &plan, hipStream_t stream) {
    if (bf16) {
        switch (group) {
            case 32: return launch_m<32, true>(M, x, qweight, scales, zeros, y, N, K, plan, stream);
            case 64: return launch_m<64, true>(M, x, qweight, scales, zeros, y, N, K, plan, stream);
            default: return launch_m<128, true>(M, x, qweight, scales, zeros, y, N, K, plan, stream);
        }
    }
    switch (group) {
        case 32: return launch_m<32, false>(M, x, qweight, scales, zeros, y, N, K, plan, stream);
        case 64: return launch_m<64, false>(M, x, qweight, scales, zeros, y, N, K, plan, stream);
        default: return launch_m<128, false>(M, x, qweight, scales, zeros, y, N, K, plan, stream);
    }
}

}  // namespace w4a16
