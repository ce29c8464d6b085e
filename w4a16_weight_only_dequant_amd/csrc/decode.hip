// Decode kernel, host side: launch plan and the dispatch over the weight
// formats. The kernel is in decode_kernel.hpp; each weight format is compiled
// in its own translation unit (this one: the 4-bit zero-point format;
// decode_sym4.hip, decode_sym8.hip, decode_kq4.hip).
#include "decode_kernel.hpp"

namespace w4a16 {

namespace {
constexpr int kDecLdsLimit = 160 * 1024;   // gfx950: LDS of one workgroup
constexpr int kDecMaxSplits = 32;
}  // namespace

// The split: one workgroup per row block (S = 1) while its LDS fits, else S
// doubled until it does. (Splitting K only to give the compute units more
// workgroups measured slower on every decode shape here: the device-scope
// hand-over at the end adds microseconds to each workgroup, as much as the
// better balance gains.) Columns per wave: four for eight activation rows
// (their registers), and when the row blocks fill the compute units once but
// not twice (more waves per block then shorten the blocks that share a
// compute unit: N = 5120 on 256 compute units, 5.8 against 6.2 us); sixteen
// for one or two activation rows when eight would need more than sixteen
// waves; eight otherwise. Columns per workgroup: ceil(T / S) rounded up to
// whole waves (S recomputed so that no range is empty). The plan does not
// depend on `awq`: with activation multipliers the kernel sums in the same
// order, so its result is the plain launch's on the pre-scaled activations.
DecodePlan decode_plan(int64_t M, int64_t N, int64_t K, int32_t group, int fmt, bool awq) {
    DecodePlan p{};
    p.ok = false;
    if (M < 1 || M > kDecodeMaxM || K <= 0 || N <= 0 || K > 65536) return p;
    const int64_t T = ceil_div(K / kChunk, kColChunks);   // 128-weight columns of K
    const int64_t nb = ceil_div(N, kRowBlock);
    const int mt = M <= 1 ? 1 : (M <= 2 ? 2 : (M <= 4 ? 4 : 8));
    const int g = fmt == kKq4 ? 256 : group;
    int cus = device_cu_count();
    if (cus <= 0) cus = 256;
    int S = tuning_knob("W4A16_DEC_SPLIT", 0);
    const int forced_ncol = tuning_knob("W4A16_DEC_NCOL", 0);
    if (S <= 0) S = 1;
    for (;; S *= 2) {
        if (S > kDecMaxSplits) return p;
        const int64_t want = ceil_div(T, S);
        int ncol = 8;
        if (forced_ncol == 4 || forced_ncol == 8 || forced_ncol == 16) ncol = forced_ncol;
        else if (mt == 8 || (nb > cus && nb < 2 * cus)) ncol = 4;
        if (ceil_div(want, ncol) > kDecMaxWaves) ncol = (mt <= 2 && ceil_div(want, 8) > kDecMaxWaves) ? 16 : 8;
        if (ncol == 16 && mt > 2) ncol = 8;
        // a range is a whole number of slices (the kernel's metadata reads
        // rely on slices starting at multiples of ncol columns)
        const int64_t cols = ceil_div(want, ncol) * ncol;
        const int s_eff = (int)ceil_div(T, cols);
        const int64_t waves = cols / ncol;
        const size_t lds = (size_t)waves * (size_t)dec_lds(mt, ncol, g, fmt).total;
        // (the limit holds the dynamic LDS and the kernel's static buffers)
        if (waves > kDecMaxWaves || lds + (size_t)dec_static_lds(mt) > (size_t)kDecLdsLimit) {
            if (want <= 4) return p;
            continue;
        }
        p.mt = mt;
        p.ncol = ncol;
        p.waves = (int)waves;
        p.splits = s_eff;
        p.cols = (int)cols;
        p.lds = lds;
        // one activation row, 4-bit codes with a scale per group, whole
        // 128-weight columns, sixteen columns per wave (K > 16384): the
        // variant that keeps the activations in registers, two workgroups per
        // compute unit (same sums, same order, so the same bits). It is
        // slower at eight or four columns per wave (K = 5120 and 13824:
        // 5.7-13.1 against 5.1-10.9 us), where the broadcasts add to the
        // shorter slices' work.
        p.bcast = mt == 1 && ncol == 16 && s_eff == 1 && !awq && (fmt == kAsym4 || fmt == kSym4) &&
                  K % kColumn == 0 && tuning_knob("W4A16_DEC_BCAST", 1) == 1;
        p.ok = true;
        return p;
    }
}

size_t decode_static_lds(const DecodePlan &plan) { return (size_t)dec_static_lds(plan.mt); }

size_t decode_workspace_bytes(const DecodePlan &plan, int64_t M, int64_t N) {
    if (!plan.ok || plan.splits <= 1) return 0;
    const int64_t nb = ceil_div(N, kRowBlock);
    return align_up((size_t)nb * 8, 256) + (size_t)nb * plan.splits * M * kRowBlock * sizeof(float);
}

hipError_t launch_decode(const void *x, bool bf16, const void *qweight, const void *scales, const void *zeros,
                         void *y, int M, int N, int K, int group, int fmt, const float *act_mul,
                         const DecodePlan &plan, void *workspace, hipStream_t stream) {
    switch (fmt) {
        case kSym4: return launch_decode_fmt<kSym4>(x, bf16, qweight, scales, zeros, y, M, N, K, group, act_mul, plan, workspace, stream);
        case kSym8: return launch_decode_fmt<kSym8>(x, bf16, qweight, scales, zeros, y, M, N, K, group, act_mul, plan, workspace, stream);
        case kKq4: return launch_decode_fmt<kKq4>(x, bf16, qweight, scales, zeros, y, M, N, K, group, act_mul, plan, workspace, stream);
        default: return launch_decode_fmt<kAsym4>(x, bf16, qweight, scales, zeros, y, M, N, K, group, act_mul, plan, workspace, stream);
    }
}

size_t decode_group_workspace_bytes(const DecodePlan *plans, int count, int64_t M, const int *N) {
    int64_t blocks = 0, part = 0;
    for (int i = 0; i < count; ++i) {
        const int64_t nb = ceil_div(N[i], kRowBlock);
        blocks += nb;
        if (plans[i].ok && plans[i].splits > 1) part += nb * plans[i].splits * M * kRowBlock;
    }
    return part > 0 ? align_up((size_t)blocks * 8, 256) + (size_t)part * sizeof(float) : 0;
}

hipError_t launch_decode_group(const GroupTable &tab, bool bf16, int M, int K, int group, int fmt,
                               const DecodePlan *plans, void *workspace, hipStream_t stream) {
    switch (fmt) {
        case kSym4: return launch_decode_group_fmt<kSym4>(tab, bf16, M, K, group, plans, workspace, stream);
        case kSym8: return launch_decode_group_fmt<kSym8>(tab, bf16, M, K, group, plans, workspace, stream);
        case kKq4: return launch_decode_group_fmt<kKq4>(tab, bf16, M, K, group, plans, workspace, stream);
        default: return launch_decode_group_fmt<kAsym4>(tab, bf16, M, K, group, plans, workspace, stream);
    }
}

template hipError_t launch_decode_fmt<kAsym4>(const void *, bool, const void *, const void *, const void *, void *,
                                              int, int, int, int, const float *, const DecodePlan &, void *,
                                              hipStream_t);
template hipError_t launch_decode_group_fmt<kAsym4>(const GroupTable &, bool, int, int, int, const DecodePlan *,
                                                    void *, hipStream_t);

}  // namespace w4a16
