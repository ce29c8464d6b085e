// Device helpers shared by the small-M kernels (the dot-product GEMV and the
// matrix-core skinny GEMM): unpacking 4-bit codes and the per-wave K-slice.
//
// Both kernels give a workgroup one block of 16 output rows and all of K; its
// waves split K into contiguous slices of 128-weight columns. A wave stages
// the activations of its own slice in its own LDS region (no workgroup
// barrier: a wave reads only what it wrote), issuing those loads before its
// first weight loads.
#pragma once

#include "w4a16_internal.hpp"

namespace w4a16 {

constexpr int kColumn = kChunk * kColChunks;   // 128 weights of K per column

// A 16-byte load marked non-temporal: the packed weights of the small-M
// kernels are read once per call, so they need not displace the activations
// and metadata in the caches (measured 2-4% faster on the decode shapes).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ inline uint4 nt_load(const uint4 *p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

typedef float float2_t __attribute__((ext_vector_type(2)));

// A 32-bit constant materialised in a VGPR. VOP3 instructions (v_and_or_b32)
// cannot take two literal operands on gfx9, so the masks and magic numbers of
// the unpack live in registers, which lets (d & mask) | magic issue as one
// v_and_or_b32 instead of a v_and + v_or pair.
__device__ inline uint32_t vconst(uint32_t c) {
    uint32_t r;
    asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
    return r;
}

__device__ inline uint32_t and_or(uint32_t a, uint32_t mask, uint32_t bits) { return (a & mask) | bits; }

// f16_magic16 / bf16_magic16 are the same magic numbers times 16 (exponent
// + 4): (d & 0x000F000F) | magic16 is (16384 + 16 q) in fp16, (2048 + 16 q)
// in bf16, the high nibble of an 8-bit code already weighted by 16.
struct UnpackConsts {
    uint32_t lo_mask, hi_mask, f16_magic, bf16_magic, f16_magic16, bf16_magic16;
};

__device__ inline UnpackConsts unpack_consts() {
    return UnpackConsts{vconst(0x000F000Fu), vconst(0x00F000F0u), vconst(0x64006400u),
                        vconst(0x43004300u), vconst(0x74007400u), vconst(0x45004500u)};
}

// Weight formats (compile-time kernel parameter): kAsym4 reads a 4-bit
// zero-point per group, kSym4 and kSym8 have the fixed zero 8 / 128 and no
// zero-point loads; kSym8 codes are two 4-bit planes (low nibbles, then high
// nibbles), each in the packed layout of the 4-bit formats.
// kKq4 (K-quant-style super-blocks) has no zero-point either: the codes are
// used as they are (zero 0) and each 32-weight chunk takes its own scale S and
// minimum M from the super-block record (kq_params).
template <int FMT> struct FormatTraits {
    static constexpr bool has_zeros = FMT == kAsym4;
    static constexpr bool two_planes = FMT == kSym8;
    static constexpr bool kquant = FMT == kKq4;
    static constexpr uint32_t fixed_zero = FMT == kSym8 ? 128u : (FMT == kKq4 ? 0u : 8u);
};

// Sub-block jj (0..7) of a super-block record {d | dmin << 16, 48-bit field
// of eight 6-bit scales, 48-bit field of eight 6-bit minima}: S = d * sc_jj,
// M = dmin * mq_jj (fp32 products of an fp16 value and a 6-bit integer: exact).
struct KqParams {
    float S, M;
};
__device__ inline KqParams kq_params(const uint4 &rec, int jj) {
    const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)(rec.x & 0xFFFFu));
    const float dm = (float)__builtin_bit_cast(_Float16, (uint16_t)(rec.x >> 16));
    const uint64_t scf = (uint64_t)rec.y | ((uint64_t)(rec.z & 0xFFFFu) << 32);
    const uint64_t mqf = (uint64_t)(rec.z >> 16) | ((uint64_t)rec.w << 16);
    const uint32_t sc = (uint32_t)(scf >> (6 * jj)) & 63u;
    const uint32_t mq = (uint32_t)(mqf >> (6 * jj)) & 63u;
    return KqParams{d * (float)sc, dm * (float)mq};
}

// The same for the four sub-blocks of one half (upper: sub-blocks 4-7) of a
// record, for kernels that take all four at once (the decode GEMV): their
// fields sit in bits 0-23 of a 32-bit window of each 48-bit field (the upper
// half's window 24 bits up), so one funnel shift per field and one bit-field
// extract per sub-block replace the 64-bit shifts. (Kernels that take one
// sub-block at a time keep kq_params: there the two windows' selects cost
// registers.)
struct KqHalf {
    float d, dm;
    uint32_t scw, mqw;
};
__device__ inline KqHalf kq_half(const uint4 &rec, bool upper) {
    KqHalf h;
    h.d = (float)__builtin_bit_cast(_Float16, (uint16_t)(rec.x & 0xFFFFu));
    h.dm = (float)__builtin_bit_cast(_Float16, (uint16_t)(rec.x >> 16));
    // scale field: rec.y | rec.z[15:0] << 32; minimum field: rec.z[31:16] | rec.w << 16
    // (a funnel shift by 0 returns the low word: no select for the scales)
    h.scw = __builtin_amdgcn_alignbit(rec.z, rec.y, upper ? 24u : 0u);
    const uint32_t mlo = __builtin_amdgcn_alignbit(rec.w, rec.z, 16), mhi = rec.w >> 8;
    h.mqw = upper ? mhi : mlo;
    return h;
}
__device__ inline KqParams kq_sub(const KqHalf &h, int j) {
    const uint32_t sc = (h.scw >> (6 * j)) & 63u;
    const uint32_t mq = (h.mqw >> (6 * j)) & 63u;
    return KqParams{h.d * (float)sc, h.dm * (float)mq};
}

// One dword (8 codes of one k-slice, even k in the low half-word) -> four
// fp16 pairs (k0,k1) (k2,k3) (k4,k5) (k6,k7) holding q - z exactly.
// (d & 0x000F000F) | 0x64006400 is (1024+q0, 1024+q1); (d & 0x00F000F0) |
// 0x64006400 is (1024+16 q2, 1024+16 q3); subtracting (1024+z), or scaling by
// 1/16 and subtracting (64+z), leaves small integers, so every step is exact.
__device__ inline void unpack_f16(uint32_t d, uint32_t z, const UnpackConsts &uc, uint32_t (&t)[4]) {
    const half2_t a = __builtin_bit_cast(half2_t, (0xE400u | z) * 0x00010001u);         // -(1024+z)
    const half2_t b = __builtin_bit_cast(half2_t, (0xD400u + 16u * z) * 0x00010001u);   // -(64+z)
    const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const uint32_t d8 = d >> 8;
    const half2_t h0 = __builtin_bit_cast(half2_t, and_or(d, uc.lo_mask, uc.f16_magic));
    const half2_t h1 = __builtin_bit_cast(half2_t, and_or(d, uc.hi_mask, uc.f16_magic));
    const half2_t h2 = __builtin_bit_cast(half2_t, and_or(d8, uc.lo_mask, uc.f16_magic));
    const half2_t h3 = __builtin_bit_cast(half2_t, and_or(d8, uc.hi_mask, uc.f16_magic));
    t[0] = __builtin_bit_cast(uint32_t, h0 + a);
    t[1] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(h1, sixteenth, b));
    t[2] = __builtin_bit_cast(uint32_t, h2 + a);
    t[3] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(h3, sixteenth, b));
}

// Two dwords of the two planes of 8-bit codes c = lo + 16 hi (the same
// k-slice) -> four fp16 pairs holding c - 128 exactly. Pairs (k0,k1): from
// 1024 + lo and 16384 + 16 hi, (16384 + 16 hi - 17536) + (1024 + lo); pairs
// (k2,k3): from 1024 + 16 lo and 16384 + 256 hi, both scaled by 1/16 in two
// fmas. Every intermediate is an integer below 2048 in magnitude, so exact.
__device__ inline void unpack_f16_s8(uint32_t dl, uint32_t dh, const UnpackConsts &uc, uint32_t (&t)[4]) {
    const half2_t c0 = {(_Float16)-17536.0f, (_Float16)-17536.0f};
    const half2_t c1 = {(_Float16)-1216.0f, (_Float16)-1216.0f};
    const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const uint32_t dl8 = dl >> 8, dh8 = dh >> 8;
    auto even = [&](uint32_t a, uint32_t b) {
        const half2_t l = __builtin_bit_cast(half2_t, and_or(a, uc.lo_mask, uc.f16_magic));
        const half2_t h = __builtin_bit_cast(half2_t, and_or(b, uc.lo_mask, uc.f16_magic16));
        return __builtin_bit_cast(uint32_t, (h + c0) + l);
    };
    auto odd = [&](uint32_t a, uint32_t b) {
        const half2_t l = __builtin_bit_cast(half2_t, and_or(a, uc.hi_mask, uc.f16_magic));
        const half2_t h = __builtin_bit_cast(half2_t, and_or(b, uc.hi_mask, uc.f16_magic16));
        return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(
                                                l, sixteenth, __builtin_elementwise_fma(h, sixteenth, c1)));
    };
    t[0] = even(dl, dh);
    t[1] = odd(dl, dh);
    t[2] = even(dl8, dh8);
    t[3] = odd(dl8, dh8);
}

// One dword -> four fp16 pairs holding 1024 + q (exact), in the pair order of
// unpack_f16: (k0,k1) (k2,k3) (k4,k5) (k6,k7); three shifts and four and_or.
__device__ inline void unpack_f16_magic(uint32_t d, const UnpackConsts &uc, uint32_t (&t)[4]) {
    t[0] = and_or(d, uc.lo_mask, uc.f16_magic);
    t[1] = and_or(d >> 4, uc.lo_mask, uc.f16_magic);
    t[2] = and_or(d >> 8, uc.lo_mask, uc.f16_magic);
    t[3] = and_or(d >> 12, uc.lo_mask, uc.f16_magic);
}

// The fp16 operands of one k-slice of a format: exact (code - zero) pairs.
template <int FMT>
__device__ inline void unpack_f16_fmt(uint32_t d, uint32_t dh, uint32_t z, const UnpackConsts &uc,
                                      uint32_t (&t)[4]) {
    if constexpr (FormatTraits<FMT>::two_planes)
        unpack_f16_s8(d, dh, uc, t);
    else
        unpack_f16(d, z, uc, t);
}

// One dword -> four bf16 pairs holding 128 + q (exact: 7 mantissa bits).
__device__ inline void unpack_bf16_magic(uint32_t d, const UnpackConsts &uc, uint32_t (&t)[4]) {
    t[0] = and_or(d, uc.lo_mask, uc.bf16_magic);
    t[1] = and_or(d >> 4, uc.lo_mask, uc.bf16_magic);
    t[2] = and_or(d >> 8, uc.lo_mask, uc.bf16_magic);
    t[3] = and_or(d >> 12, uc.lo_mask, uc.bf16_magic);
}

// The high-nibble plane of 8-bit codes -> four bf16 pairs holding
// 16 (128 + hi) = 2048 + 16 hi (exact: 16 times an 8-bit integer).
__device__ inline void unpack_bf16_magic16(uint32_t d, const UnpackConsts &uc, uint32_t (&t)[4]) {
    t[0] = and_or(d, uc.lo_mask, uc.bf16_magic16);
    t[1] = and_or(d >> 4, uc.lo_mask, uc.bf16_magic16);
    t[2] = and_or(d >> 8, uc.lo_mask, uc.bf16_magic16);
    t[3] = and_or(d >> 12, uc.lo_mask, uc.bf16_magic16);
}

// Offset that the bf16 magic operands of a format add per activation: a dot
// product of x with them equals sum x (code - z) + bias(z) * sum x, where
// bias = 128 + z for 4-bit codes and 128 + 16 * 128 + 128 = 2304 for 8-bit ones.
template <int FMT>
__device__ inline float bf16_magic_bias(uint32_t z) {
    if constexpr (FormatTraits<FMT>::two_planes)
        return 2304.0f;
    else
        return (float)(128u + z);
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

// The K-slice of one wave, in columns [t_begin, t_end); t_full ends the run of
// full (4-chunk) columns; the last column of K may be partial.
struct Slice {
    int C;          // chunks along K
    int T;          // columns along K
    int t_begin, t_end, t_full;
    int c_lo, c_hi;   // chunk range of the slice
    int g_lo, g_hi;   // group range of the slice
};

template <int GROUP>
__device__ inline Slice wave_slice(int K, int wave, int waves) {
    Slice sl;
    sl.C = K / kChunk;
    sl.T = (sl.C + kColChunks - 1) / kColChunks;
    sl.t_begin = (int)(((int64_t)wave * sl.T) / waves);
    sl.t_end = (int)(((int64_t)(wave + 1) * sl.T) / waves);
    sl.t_full = min(sl.t_end, sl.C / kColChunks);
    sl.c_lo = sl.t_begin * kColChunks;
    sl.c_hi = min(sl.t_end * kColChunks, sl.C);
    sl.g_lo = sl.c_lo * kChunk / GROUP;
    sl.g_hi = (sl.c_hi * kChunk + GROUP - 1) / GROUP;
    return sl;
}

// The scales of one row in one column (GPC fp16 values) as raw bits.
template <int GPC> struct ColScales;
template <> struct ColScales<1> { uint16_t v; __device__ float get(int) const { return (float)__builtin_bit_cast(_Float16, v); } };
template <> struct ColScales<2> { uint32_t v; __device__ float get(int e) const { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> (16 * e))); } };
template <> struct ColScales<4> { uint2 v; __device__ float get(int e) const { const uint32_t h = e < 2 ? v.x : v.y; return (float)__builtin_bit_cast(_Float16, (uint16_t)(h >> (16 * (e & 1)))); } };

}  // namespace w4a16
