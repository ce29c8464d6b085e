// C ABI of the gfx950 W4A16 library: argument checks, workspace sizing,
// device check and dispatch on M. Declarations and contracts: include/w4a16.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/w4a16.h"
#include "w4a16_internal.hpp"

using namespace w4a16;

namespace {

constexpr int kMaxDevices = 64;
// 0 = not queried yet, 1 = gfx950, 2 = other device
std::atomic<int> g_device_kind[kMaxDevices];

// Largest M routed to the decode kernel by w4a16_linear (the decode kernel
// itself accepts M <= 8): measured faster than the matrix-core kernel up to
// M = 2 (N = 15360, K = 5120: 11.4 against 14.2 us), slower from M = 4.
int gemv_max_m() { return 2; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool shape_ok(int64_t N, int64_t K, int32_t group) {
    if (group != 32 && group != 64 && group != 128 && group != 256) return false;
    if (N < 8 || N % 8 != 0) return false;
    if (K < group || K % group != 0) return false;
    // 32-bit index limits of the kernels
    if (N > (1LL << 30) || K > (1LL << 30) || (N / 8) * K > (1LL << 31)) return false;
    return true;
}

bool fmt_ok(int32_t fmt) {
    return fmt == W4A16_FMT_ASYM4 || fmt == W4A16_FMT_SYM4 || fmt == W4A16_FMT_SYM8 || fmt == W4A16_FMT_KQ4;
}
// K-quant super-blocks are 256 weights: that format takes group 256 only
bool fmt_group_ok(int32_t fmt, int32_t group) { return fmt_ok(fmt) && (fmt != W4A16_FMT_KQ4 || group == 256); }

// Byte sizes of the packed buffers: codes (one 4-bit plane, two for 8-bit
// codes), then scales and zero-points row-major, each row's groups padded to
// a multiple of 8 (G8 slots); K-quant: one 16-byte record per (row,
// super-block). The symmetric formats store no zero-points.
void meta_bytes(int64_t N, int64_t K, int32_t group, int32_t fmt, size_t *q, size_t *sb, size_t *zb) {
    if (fmt == W4A16_FMT_KQ4) {   // one 16-byte record per (row, super-block)
        *q = (size_t)(N * K / 2);
        *sb = (size_t)(16 * (K / 256) * N);
        *zb = 0;
        return;
    }
    const int64_t G8 = (K / group + 7) / 8 * 8;
    *q = (size_t)(N * K / 2) * (fmt == W4A16_FMT_SYM8 ? 2 : 1);
    *sb = (size_t)(2 * G8 * N);
    *zb = fmt == W4A16_FMT_ASYM4 ? (size_t)(G8 * N / 2) : 0;
}

struct Range {
    uintptr_t lo, hi;
};
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }
Range range_of(const void *p, size_t bytes) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + bytes};
}

// Process-wide kernel error word: pinned host memory, mapped into every
// device's address space and coherent (kernels write it with system-scope
// stores, the host reads it without a copy). Allocated once by the first
// w4a16_init; g_err_dev holds its address on each initialised device.
std::mutex g_init_mu;
unsigned int *g_err_host = nullptr;
std::atomic<unsigned int *> g_err_dev[kMaxDevices];
std::atomic<int> g_ready[kMaxDevices];   // 1 once w4a16_init succeeded on the device

// Scratch of w4a16_linear_noalloc: the stream-K partial tiles and flags of the
// tiled GEMM, which need at most (256 x 256 x 4 + 8) bytes per compute unit,
// 64 MiB + 2 KiB on 256 compute units. Each device holds its own copy for the
// life of the process. The name is a host-side stand-in: host code uses only
// the device address that w4a16_init stores in g_scratch.
constexpr size_t kScratchBytes = W4A16_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::atomic<void *> g_scratch[kMaxDevices];

w4a16_status init_device(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return W4A16_ERR_INVALID_ARG;
    if (g_ready[dev].load(std::memory_order_acquire)) return W4A16_OK;
    std::lock_guard<std::mutex> lock(g_init_mu);
    if (g_ready[dev].load(std::memory_order_acquire)) return W4A16_OK;
    if (g_err_host == nullptr) {
        void *p = nullptr;
        if (hipHostMalloc(&p, 256, hipHostMallocMapped | hipHostMallocPortable | hipHostMallocCoherent) != hipSuccess)
            return W4A16_ERR_HIP;
        std::memset(p, 0, 256);
        g_err_host = static_cast<unsigned int *>(p);
    }
    void *d = nullptr;
    if (hipHostGetDevicePointer(&d, g_err_host, 0) != hipSuccess) return W4A16_ERR_HIP;
    g_err_dev[dev].store(static_cast<unsigned int *>(d), std::memory_order_release);
    void *sp = nullptr;
    if (hipGetSymbolAddress(&sp, HIP_SYMBOL(scratch)) != hipSuccess || sp == nullptr) return W4A16_ERR_HIP;
    g_scratch[dev].store(sp, std::memory_order_release);
    g_ready[dev].store(1, std::memory_order_release);
    return W4A16_OK;
}

// A kernel error recorded since the last call (a stream-K wait that ran out):
// taken once, reported as W4A16_ERR_HIP by the call that finds it.
bool take_kernel_error() {
    unsigned int *p = g_err_host;
    return p != nullptr && __atomic_exchange_n(p, 0u, __ATOMIC_SEQ_CST) != 0u;
}

// The device check of every compute call: a gfx950, set up (w4a16_init on
// first use), and no kernel error pending.
w4a16_status check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return W4A16_ERR_HIP;
    w4a16_status st = w4a16_device_supported(dev);
    if (st != W4A16_OK) return st;
    st = init_device(dev);
    if (st != W4A16_OK) return st;
    return take_kernel_error() ? W4A16_ERR_HIP : W4A16_OK;
}

// Argument checks shared by gemv / gemm / linear. The symmetric formats do
// not read `zeros` (it may be NULL). An empty batch (M = 0) checks the shape,
// type and format arguments only: no pointer is read, and the callers return
// before anything is enqueued.
w4a16_status check_linear(const void *x, int32_t dtype, const void *qweight, const void *scales,
                          const void *zeros, void *y, int64_t M, int64_t N, int64_t K, int32_t group,
                          int32_t fmt, void *workspace, size_t workspace_bytes, size_t need) {
    if (!fmt_group_ok(fmt, group)) return W4A16_ERR_INVALID_ARG;
    if (dtype != W4A16_F16 && dtype != W4A16_BF16) return W4A16_ERR_INVALID_ARG;
    if (M < 0 || M > (1LL << 24) || !shape_ok(N, K, group)) return W4A16_ERR_INVALID_ARG;
    if (M == 0) return W4A16_OK;
    const bool zp = fmt == W4A16_FMT_ASYM4;
    if (!x || !qweight || !scales || (zp && !zeros) || !y) return W4A16_ERR_INVALID_ARG;
    if (M * K >= (1LL << 34)) return W4A16_ERR_INVALID_ARG;   // 32-bit activation indices (in 16-byte units)
    if (!aligned16(x) || !aligned16(qweight) || !aligned16(scales) || (zp && !aligned16(zeros)) ||
        !aligned16(y))
        return W4A16_ERR_INVALID_ARG;
    size_t qb, sb, zb;
    meta_bytes(N, K, group, fmt, &qb, &sb, &zb);
    const Range ry = range_of(y, (size_t)(M * N * 2));
    if (overlap(ry, range_of(x, (size_t)(M * K * 2))) || overlap(ry, range_of(qweight, qb)) ||
        overlap(ry, range_of(scales, sb)) || overlap(ry, range_of(zeros, zb)))
        return W4A16_ERR_INVALID_ARG;
    if (need > 0) {   // the kernels write the workspace: it may overlap nothing else
        if (!workspace || workspace_bytes < need) return W4A16_ERR_WORKSPACE;
        if (!aligned16(workspace)) return W4A16_ERR_INVALID_ARG;
        const Range rw = range_of(workspace, need);
        if (overlap(ry, rw) || overlap(rw, range_of(x, (size_t)(M * K * 2))) || overlap(rw, range_of(qweight, qb)) ||
            overlap(rw, range_of(scales, sb)) || overlap(rw, range_of(zeros, zb)))
            return W4A16_ERR_INVALID_ARG;
    }
    return W4A16_OK;
}

std::mutex g_attr_mutex;
std::atomic<int> g_cus[kMaxDevices];
}  // namespace

int w4a16::tuning_knob(const char *name, int fallback) {
#ifdef W4A16_TUNING_KNOBS
    const char *v = std::getenv(name);
    if (!v || !*v) return fallback;
    char *end = nullptr;
    const long r = std::strtol(v, &end, 10);
    return (end && *end == 0) ? (int)r : fallback;
#else
    (void)name;
    return fallback;
#endif
}

int w4a16::device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int v = g_cus[dev].load(std::memory_order_acquire);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return 0;
        g_cus[dev].store(v, std::memory_order_release);
    }
    return v;
}

hipError_t w4a16::raise_dyn_lds(const void *kern, size_t bytes, DynLdsAttr &attr) {
    if (bytes <= 48 * 1024) return hipSuccess;   // within the default limit
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kAttrDevices)
        return hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (attr.set[dev].load(std::memory_order_acquire) >= (int)bytes) return hipSuccess;
    std::lock_guard<std::mutex> lock(g_attr_mutex);
    if (attr.set[dev].load(std::memory_order_relaxed) >= (int)bytes) return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) attr.set[dev].store((int)bytes, std::memory_order_release);
    return e;
}

namespace {
// Largest LDS allocation of one workgroup on the current device (cached per device).
std::atomic<int> g_max_lds[kMaxDevices];
size_t max_lds_per_block() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 64 * 1024;
    int v = g_max_lds[dev].load(std::memory_order_acquire);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0)
            v = 64 * 1024;
        g_max_lds[dev].store(v, std::memory_order_release);
    }
    return (size_t)v;
}

// The decode kernel takes M <= 8 and K <= 65536 (its plan splits K until a
// workgroup's LDS fits).
bool decode_fits(int64_t M, int64_t N, int64_t K, int32_t group, int32_t fmt, bool awq) {
    if (M < 1 || M > kDecodeMaxM) return false;
    const DecodePlan p = decode_plan(M, N, K, group, fmt, awq);
    return p.ok && p.lds + decode_static_lds(p) <= max_lds_per_block();
}

// Workspace of a decode launch over N rows (the split's counters and
// partials; 0 without a split or outside the kernel's range).
size_t decode_need(int64_t M, int64_t N, int64_t K, int32_t group, int32_t fmt, bool awq) {
    if (M < 1 || M > kDecodeMaxM) return 0;
    const DecodePlan p = decode_plan(M, N, K, group, fmt, awq);
    return p.ok ? decode_workspace_bytes(p, M, N) : 0;
}
// A grouped decode launch: every problem keeps its own plan (0 when a plan
// does not fit).
size_t group_decode_need(int count, int64_t M, const int64_t *N, int64_t K, int32_t group, int32_t fmt) {
    DecodePlan plans[kMaxGroup];
    int n[kMaxGroup];
    for (int p = 0; p < count; ++p) {
        plans[p] = decode_plan(M, N[p], K, group, fmt, false);
        n[p] = (int)N[p];
    }
    return decode_group_workspace_bytes(plans, count, M, n);
}
// The same for any weight format (w4a16_workspace_bytes takes none).
size_t decode_need_any(int64_t M, int64_t N, int64_t K, int32_t group) {
    size_t need = 0;
    for (int32_t fmt : {W4A16_FMT_ASYM4, W4A16_FMT_SYM4, W4A16_FMT_SYM8, W4A16_FMT_KQ4})
        if (fmt_group_ok(fmt, group)) need = std::max(need, decode_need(M, N, K, group, fmt, false));
    return need;
}

// w4a16_linear's choice: the decode kernel at M <= gemv_max_m(), the
// matrix-core kernels otherwise.
bool prefer_gemv(int64_t M, int64_t N, int64_t K, int32_t group, int32_t dtype, int32_t fmt) {
    return M >= 1 && M <= gemv_max_m() && shape_ok(N, K, group) && (dtype == W4A16_F16 || dtype == W4A16_BF16) &&
           decode_fits(M, N, K, group, fmt, false);
}

// Workspace of a matrix-core call: the stream-K partials and flags of the
// tiled kernel when its plan splits tiles (0 otherwise).
size_t gemm_need(int64_t M, int64_t N, int64_t K, int32_t group) {
    return prefill_workspace_bytes(gemm_plan(M, N, K, group));
}

}  // namespace

extern "C" {

const char *w4a16_status_string(int status) {
    switch (status) {
        case W4A16_OK: return "ok";
        case W4A16_ERR_INVALID_ARG: return "invalid argument";
        case W4A16_ERR_UNSUPPORTED: return "device is not a gfx950";
        case W4A16_ERR_HIP: return "HIP runtime error";
        case W4A16_ERR_WORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

int w4a16_layout_version(void) { return W4A16_LAYOUT_VERSION; }

w4a16_status w4a16_init(int device) {
    w4a16_status st = w4a16_device_supported(device);
    if (st != W4A16_OK) return st;
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return W4A16_ERR_HIP;
    if (cur != device && hipSetDevice(device) != hipSuccess) return W4A16_ERR_HIP;
    st = init_device(device);
    if (cur != device && hipSetDevice(cur) != hipSuccess) return W4A16_ERR_HIP;
    return st;
}

int32_t w4a16_gemv_max_m(void) { return gemv_max_m(); }

int32_t w4a16_linear_kernel(int64_t M, int64_t N, int64_t K, int32_t group, int32_t dtype) {
    // the same choice for every weight format
    if (M < 1 || M > (1LL << 24) || !shape_ok(N, K, group) || (dtype != W4A16_F16 && dtype != W4A16_BF16))
        return -1;
    if (prefer_gemv(M, N, K, group, dtype, W4A16_FMT_ASYM4)) return 0;
    return gemm_plan(M, N, K, group).kind == 0 ? 1 : 2;
}

int32_t w4a16_linear_launch_shape(int64_t M, int64_t N, int64_t K, int32_t group, int32_t dtype, int32_t fmt,
                                  int64_t *workgroups, int32_t *threads) {
    if (M < 1 || M > (1LL << 24) || !shape_ok(N, K, group) || !fmt_group_ok(fmt, group) ||
        (dtype != W4A16_F16 && dtype != W4A16_BF16))
        return -1;
    int64_t wg = 0;
    int32_t th = 0;
    int32_t kind;
    if (prefer_gemv(M, N, K, group, dtype, fmt)) {
        const DecodePlan p = decode_plan(M, N, K, group, fmt, false);
        kind = 0;
        wg = ceil_div(N, kRowBlock) * p.splits;
        th = 64 * p.waves;
    } else {
        const GemmPlan p = gemm_plan(M, N, K, group);
        if (p.kind == 0) {
            kind = 1;
            wg = ceil_div(ceil_div(N, kRowBlock), p.rows_per_wg) * ceil_div(M, 16);
            th = 64 * p.waves;
        } else {
            kind = 2;
            const int64_t tiles = ceil_div(M, tile_rows(p.tile)) * ceil_div(N, kTileCols);
            wg = p.sk_wgs > 0 ? (int64_t)p.dp_tiles + p.sk_wgs : (p.splits > 1 ? tiles * p.splits : tiles);
            th = p.tile == kTile256x256w8 ? 512 : 256;
        }
    }
    if (workgroups) *workgroups = wg;
    if (threads) *threads = th;
    return kind;
}

w4a16_status w4a16_device_supported(int device) {
    if (device < 0) return W4A16_ERR_INVALID_ARG;
    if (device < kMaxDevices) {
        int k = g_device_kind[device].load(std::memory_order_acquire);
        if (k == 1) return W4A16_OK;
        if (k == 2) return W4A16_ERR_UNSUPPORTED;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return W4A16_ERR_HIP;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (device < kMaxDevices) g_device_kind[device].store(ok ? 1 : 2, std::memory_order_release);
    return ok ? W4A16_OK : W4A16_ERR_UNSUPPORTED;
}

w4a16_status w4a16_packed_bytes(int64_t N, int64_t K, int32_t group, size_t *qweight_bytes,
                                size_t *scales_bytes, size_t *zeros_bytes) {
    return w4a16_packed_bytes_fmt(N, K, group, W4A16_FMT_ASYM4, qweight_bytes, scales_bytes, zeros_bytes);
}

w4a16_status w4a16_packed_bytes_fmt(int64_t N, int64_t K, int32_t group, int32_t fmt, size_t *qweight_bytes,
                                    size_t *scales_bytes, size_t *zeros_bytes) {
    if (!shape_ok(N, K, group) || !fmt_group_ok(fmt, group)) return W4A16_ERR_INVALID_ARG;
    size_t q, sb, zb;
    meta_bytes(N, K, group, fmt, &q, &sb, &zb);
    if (qweight_bytes) *qweight_bytes = q;
    if (scales_bytes) *scales_bytes = sb;
    if (zeros_bytes) *zeros_bytes = zb;
    return W4A16_OK;
}

w4a16_status w4a16_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group, size_t *bytes) {
    if (!bytes || M < 0 || M > (1LL << 24) || !shape_ok(N, K, group)) return W4A16_ERR_INVALID_ARG;
    *bytes = M == 0 ? 0 : std::max(gemm_need(M, N, K, group), decode_need_any(M, N, K, group));
    return W4A16_OK;
}

w4a16_status w4a16_group_workspace_bytes(int32_t count, int64_t M, const int64_t *N, int64_t K, int32_t group,
                                         int32_t fmt, size_t *bytes) {
    if (!bytes || !N || count < 1 || count > kMaxGroup || M < 0 || M > (1LL << 24) || !fmt_group_ok(fmt, group))
        return W4A16_ERR_INVALID_ARG;
    size_t need = 0;
    for (int p = 0; p < count; ++p) {
        if (!shape_ok(N[p], K, group)) return W4A16_ERR_INVALID_ARG;
        if (M > 0) need = std::max(need, std::max(gemm_need(M, N[p], K, group), decode_need(M, N[p], K, group, fmt, false)));
    }
    if (M > 0 && M <= kDecodeMaxM) need = std::max(need, group_decode_need(count, M, N, K, group, fmt));
    *bytes = need;
    return W4A16_OK;
}

w4a16_status w4a16_pack(const float *w, int64_t N, int64_t K, int32_t group, void *qweight,
                        void *scales, void *zeros, void *stream) {
    return w4a16_pack_fmt(w, N, K, group, W4A16_FMT_ASYM4, qweight, scales, zeros, stream);
}

w4a16_status w4a16_pack_fmt(const float *w, int64_t N, int64_t K, int32_t group, int32_t fmt, void *qweight,
                            void *scales, void *zeros, void *stream) {
    if (!fmt_group_ok(fmt, group)) return W4A16_ERR_INVALID_ARG;
    const bool zp = fmt == W4A16_FMT_ASYM4;
    if (!w || !qweight || !scales || (zp && !zeros) || !shape_ok(N, K, group)) return W4A16_ERR_INVALID_ARG;
    if (!aligned16(w) || !aligned16(qweight) || !aligned16(scales) || (zp && !aligned16(zeros)))
        return W4A16_ERR_INVALID_ARG;
    if (((K / 32 + 3) / 4) * N > (1LL << 31)) return W4A16_ERR_INVALID_ARG;
    w4a16_status st = check_device();
    if (st != W4A16_OK) return st;
    hipError_t e = launch_pack(w, (int)N, (int)K, group, fmt, qweight, scales, zeros,
                               reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

w4a16_status w4a16_unpack(const void *qweight, const void *scales, const void *zeros, int64_t N,
                          int64_t K, int32_t group, uint8_t *codes, uint16_t *scales_out,
                          uint8_t *zeros_out, void *stream) {
    return w4a16_unpack_fmt(qweight, scales, zeros, N, K, group, W4A16_FMT_ASYM4, codes, scales_out, zeros_out,
                            stream);
}

w4a16_status w4a16_unpack_fmt(const void *qweight, const void *scales, const void *zeros, int64_t N,
                              int64_t K, int32_t group, int32_t fmt, uint8_t *codes, uint16_t *scales_out,
                              uint8_t *zeros_out, void *stream) {
    if (!fmt_group_ok(fmt, group)) return W4A16_ERR_INVALID_ARG;
    const bool zp = fmt == W4A16_FMT_ASYM4;
    const bool meta = fmt != W4A16_FMT_KQ4;   // kq4: codes only (its records are already canonical)
    if (!qweight || (meta && !scales) || (zp && !zeros) || !codes || (meta && (!scales_out || !zeros_out)) ||
        !shape_ok(N, K, group))
        return W4A16_ERR_INVALID_ARG;
    if (!aligned16(qweight) || !aligned16(codes)) return W4A16_ERR_INVALID_ARG;
    w4a16_status st = check_device();
    if (st != W4A16_OK) return st;
    hipError_t e = launch_unpack(qweight, scales, zeros, (int)N, (int)K, group, fmt, codes, scales_out,
                                 zeros_out, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

w4a16_status w4a16_gemv_fmt(const void *x, int32_t dtype, const void *qweight, const void *scales,
                            const void *zeros, void *y, int64_t M, int64_t N, int64_t K, int32_t group, int32_t fmt,
                            void *workspace, size_t workspace_bytes, void *stream) {
    if (M > kDecodeMaxM) return W4A16_ERR_INVALID_ARG;
    const size_t need = (M >= 1 && shape_ok(N, K, group) && fmt_group_ok(fmt, group))
                            ? decode_need(M, N, K, group, fmt, false) : 0;
    w4a16_status st = check_linear(x, dtype, qweight, scales, zeros, y, M, N, K, group, fmt, workspace,
                                   workspace_bytes, need);
    if (st != W4A16_OK || M == 0) return st;
    st = check_device();
    if (st != W4A16_OK) return st;
    if (!decode_fits(M, N, K, group, fmt, false)) return W4A16_ERR_INVALID_ARG;
    const DecodePlan plan = decode_plan(M, N, K, group, fmt, false);
    hipError_t e = launch_decode(x, dtype == W4A16_BF16, qweight, scales, zeros, y, (int)M, (int)N, (int)K, group,
                                 fmt, nullptr, plan, workspace, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

w4a16_status w4a16_gemv(const void *x, int32_t dtype, const void *qweight, const void *scales,
                        const void *zeros, void *y, int64_t M, int64_t N, int64_t K, int32_t group,
                        void *workspace, size_t workspace_bytes, void *stream) {
    return w4a16_gemv_fmt(x, dtype, qweight, scales, zeros, y, M, N, K, group, W4A16_FMT_ASYM4, workspace,
                          workspace_bytes, stream);
}

// The matrix-core kernels with a plan of kind `kind` (-1: the dispatch's).
static w4a16_status run_gemm(int kind, const void *x, int32_t dtype, const void *qweight, const void *scales,
                      const void *zeros, void *y, int64_t M, int64_t N, int64_t K, int32_t group, int32_t fmt,
                      void *workspace, size_t workspace_bytes, void *stream) {
    const size_t need = (M >= 1 && M <= (1LL << 24) && shape_ok(N, K, group))
                            ? prefill_workspace_bytes(gemm_plan(M, N, K, group, kind)) : 0;
    w4a16_status st = check_linear(x, dtype, qweight, scales, zeros, y, M, N, K, group, fmt, workspace,
                                   workspace_bytes, need);
    if (st != W4A16_OK || M == 0) return st;
    st = check_device();
    if (st != W4A16_OK) return st;
    GemmPlan plan = gemm_plan(M, N, K, group, kind);
    if (prefill_workspace_bytes(plan) > need) return W4A16_ERR_WORKSPACE;   // (the same plan: never)
    hipError_t e = launch_gemm(x, dtype == W4A16_BF16, qweight, scales, zeros, y, (int)M, (int)N,
                               (int)K, group, fmt, plan, workspace, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

w4a16_status w4a16_gemm_fmt(const void *x, int32_t dtype, const void *qweight, const void *scales,
                            const void *zeros, void *y, int64_t M, int64_t N, int64_t K, int32_t group, int32_t fmt,
                            void *workspace, size_t workspace_bytes, void *stream) {
    return run_gemm(-1, x, dtype, qweight, scales, zeros, y, M, N, K, group, fmt, workspace, workspace_bytes, stream);
}

w4a16_status w4a16_kernel_workspace_bytes(int32_t kernel, int64_t M, int64_t N, int64_t K, int32_t group,
                                          int32_t fmt, size_t *bytes) {
    if (!bytes || M < 0 || M > (1LL << 24) || !shape_ok(N, K, group) || !fmt_group_ok(fmt, group))
        return W4A16_ERR_INVALID_ARG;
    switch (kernel) {
        case 0:
            if (M > kDecodeMaxM) return W4A16_ERR_INVALID_ARG;
            *bytes = M == 0 ? 0 : decode_need(M, N, K, group, fmt, false);
            return W4A16_OK;
        case 1:
        case 2:
            *bytes = M == 0 ? 0 : prefill_workspace_bytes(gemm_plan(M, N, K, group, kernel - 1));
            return W4A16_OK;
        default: return W4A16_ERR_INVALID_ARG;
    }
}

w4a16_status w4a16_linear_run_fmt(int32_t kernel, const void *x, int32_t dtype, const void *qweight,
                                  const void *scales, const void *zeros, void *y, int64_t M, int64_t N, int64_t K,
                                  int32_t group, int32_t fmt, void *workspace, size_t workspace_bytes,
                                  void *stream) {
    switch (kernel) {
        case 0:
            return w4a16_gemv_fmt(x, dtype, qweight, scales, zeros, y, M, N, K, group, fmt, workspace,
                                  workspace_bytes, stream);
        case 1:
        case 2:
            return run_gemm(kernel - 1, x, dtype, qweight, scales, zeros, y, M, N, K, group, fmt, workspace,
                            workspace_bytes, stream);
        default: return W4A16_ERR_INVALID_ARG;
    }
}

w4a16_status w4a16_testing_gemm_expire(const void *x, int32_t dtype, const void *qweight, const void *scales,
                                       const void *zeros, void *y, int64_t M, int64_t N, int64_t K, int32_t group,
                                       int32_t fmt, void *workspace, size_t workspace_bytes, void *stream) {
    const bool shape = M >= 1 && M <= (1LL << 24) && shape_ok(N, K, group);
    const size_t need = shape ? gemm_need(M, N, K, group) : 0;
    // (only a stream-K plan has waits to expire; a K split does not wait)
    if (need == 0 || gemm_plan(M, N, K, group).sk_wgs == 0) return W4A16_ERR_INVALID_ARG;
    w4a16_status st = check_linear(x, dtype, qweight, scales, zeros, y, M, N, K, group, fmt, workspace,
                                   workspace_bytes, need);
    if (st != W4A16_OK) return st;
    st = check_device();
    if (st != W4A16_OK) return st;
    GemmPlan plan = gemm_plan(M, N, K, group);
    plan.sk_expire_test = 1;
    hipError_t e = launch_gemm(x, dtype == W4A16_BF16, qweight, scales, zeros, y, (int)M, (int)N, (int)K, group,
                               fmt, plan, workspace, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

w4a16_status w4a16_gemm(const void *x, int32_t dtype, const void *qweight, const void *scales,
                        const void *zeros, void *y, int64_t M, int64_t N, int64_t K, int32_t group,
                        void *workspace, size_t workspace_bytes, void *stream) {
    return w4a16_gemm_fmt(x, dtype, qweight, scales, zeros, y, M, N, K, group, W4A16_FMT_ASYM4, workspace,
                          workspace_bytes, stream);
}

w4a16_status w4a16_linear_group_fmt(int32_t count, const void *const *x, int32_t dtype,
                                    const void *const *qweight, const void *const *scales,
                                    const void *const *zeros, void *const *y, int64_t M, const int64_t *N,
                                    int64_t K, int32_t group, int32_t fmt, void *workspace, size_t workspace_bytes,
                                    void *stream) {
    const bool zp = fmt == W4A16_FMT_ASYM4;
    if (count < 1 || count > kMaxGroup || !N) return W4A16_ERR_INVALID_ARG;
    if (M == 0) {   // empty batch: shapes only
        for (int p = 0; p < count; ++p) {
            const w4a16_status st = check_linear(nullptr, dtype, nullptr, nullptr, nullptr, nullptr, 0, N[p], K,
                                                 group, fmt, nullptr, 0, 0);
            if (st != W4A16_OK) return st;
        }
        return W4A16_OK;
    }
    if (!x || !qweight || !scales || (zp && !zeros) || !y) return W4A16_ERR_INVALID_ARG;
    auto zero_ptr = [&](int p) -> const void * { return zp ? zeros[p] : nullptr; };
    int64_t n_total = 0;
    for (int p = 0; p < count; ++p) {
        if (!shape_ok(N[p], K, group)) return W4A16_ERR_INVALID_ARG;
        n_total += N[p];
    }
    // small batches: one decode launch over every problem's row blocks, each
    // problem with the plan of a call on it alone (the same bits)
    bool decode = true;
    for (int p = 0; p < count; ++p) decode = decode && prefer_gemv(M, N[p], K, group, dtype, fmt);
    const size_t dec_need = decode ? group_decode_need(count, M, N, K, group, fmt) : 0;
    for (int p = 0; p < count; ++p) {
        const w4a16_status st = check_linear(x[p], dtype, qweight[p], scales[p], zero_ptr(p), y[p], M, N[p], K,
                                             group, fmt, workspace, workspace_bytes, dec_need);
        if (st != W4A16_OK) return st;
    }
    // no output may overlap any other problem's buffers either
    for (int p = 0; p < count; ++p) {
        const Range ry = range_of(y[p], (size_t)(M * N[p] * 2));
        for (int q = 0; q < count; ++q) {
            if (q == p) continue;
            size_t qb, sb, zb;
            meta_bytes(N[q], K, group, fmt, &qb, &sb, &zb);
            if (overlap(ry, range_of(x[q], (size_t)(M * K * 2))) || overlap(ry, range_of(qweight[q], qb)) ||
                overlap(ry, range_of(scales[q], sb)) || (zp && overlap(ry, range_of(zeros[q], zb))) ||
                overlap(ry, range_of(y[q], (size_t)(M * N[q] * 2))))
                return W4A16_ERR_INVALID_ARG;
        }
    }
    w4a16_status st = check_device();
    if (st != W4A16_OK) return st;
    GroupTable tab{};
    tab.count = count;
    for (int p = 0; p < count; ++p) {
        tab.x[p] = x[p];
        tab.qweight[p] = qweight[p];
        tab.scales[p] = scales[p];
        tab.zeros[p] = zero_ptr(p);
        tab.y[p] = y[p];
        tab.N[p] = (int)N[p];
    }
    if (decode) {
        DecodePlan plans[kMaxGroup];
        bool same = true;
        for (int p = 0; p < count; ++p) {
            plans[p] = decode_plan(M, N[p], K, group, fmt, false);
            same = same && plans[p].mt == plans[0].mt && plans[p].ncol == plans[0].ncol;
        }
        size_t lds = 0;
        for (int p = 0; p < count; ++p) lds = std::max(lds, plans[p].lds + decode_static_lds(plans[p]));
        if (same && lds <= max_lds_per_block()) {
            hipError_t e = launch_decode_group(tab, dtype == W4A16_BF16, (int)M, (int)K, group, fmt, plans,
                                               workspace, reinterpret_cast<hipStream_t>(stream));
            return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
        }
        for (int p = 0; p < count; ++p) {   // plans of different shapes: one launch each
            st = w4a16_gemv_fmt(x[p], dtype, qweight[p], scales[p], zero_ptr(p), y[p], M, N[p], K, group, fmt,
                                workspace, workspace_bytes, stream);
            if (st != W4A16_OK) return st;
        }
        return W4A16_OK;
    }
    const GemmPlan plan = gemm_plan(M, n_total, K, group);
    if (plan.kind != 0) {   // large M: one tiled launch per problem
        for (int p = 0; p < count; ++p) {
            st = w4a16_gemm_fmt(x[p], dtype, qweight[p], scales[p], zero_ptr(p), y[p], M, N[p], K, group, fmt,
                                workspace, workspace_bytes, stream);
            if (st != W4A16_OK) return st;
        }
        return W4A16_OK;
    }
    hipError_t e = launch_gemm_group(tab, dtype == W4A16_BF16, (int)M, (int)K, group, fmt, plan,
                                     reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

w4a16_status w4a16_linear_noalloc(const void *x, int32_t dtype, const void *qweight, const void *scales,
                                  const void *zeros, void *y, int64_t M, int64_t N, int64_t K, int32_t group,
                                  int32_t fmt, void *stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return W4A16_ERR_HIP;
    // the set-up (and its one allocation) must have run on this device
    if (dev < 0 || dev >= kMaxDevices || !g_ready[dev].load(std::memory_order_acquire))
        return W4A16_ERR_INVALID_ARG;
    size_t need = 0;
    if (M >= 1 && M <= (1LL << 24) && shape_ok(N, K, group) && fmt_group_ok(fmt, group))
        need = prefer_gemv(M, N, K, group, dtype, fmt) ? decode_need(M, N, K, group, fmt, false)
                                                       : gemm_need(M, N, K, group);
    if (need > kScratchBytes) return W4A16_ERR_WORKSPACE;
    void *ws = need > 0 ? g_scratch[dev].load(std::memory_order_acquire) : nullptr;
    return w4a16_linear_fmt(x, dtype, qweight, scales, zeros, y, M, N, K, group, fmt, ws,
                            need > 0 ? kScratchBytes : 0, stream);
}

w4a16_status w4a16_linear_group(int32_t count, const void *const *x, int32_t dtype, const void *const *qweight,
                                const void *const *scales, const void *const *zeros, void *const *y, int64_t M,
                                const int64_t *N, int64_t K, int32_t group, void *workspace,
                                size_t workspace_bytes, void *stream) {
    return w4a16_linear_group_fmt(count, x, dtype, qweight, scales, zeros, y, M, N, K, group, W4A16_FMT_ASYM4,
                                  workspace, workspace_bytes, stream);
}

w4a16_status w4a16_linear_fmt(const void *x, int32_t dtype, const void *qweight, const void *scales,
                              const void *zeros, void *y, int64_t M, int64_t N, int64_t K, int32_t group,
                              int32_t fmt, void *workspace, size_t workspace_bytes, void *stream) {
    if (prefer_gemv(M, N, K, group, dtype, fmt))
        return w4a16_gemv_fmt(x, dtype, qweight, scales, zeros, y, M, N, K, group, fmt, workspace,
                              workspace_bytes, stream);
    return w4a16_gemm_fmt(x, dtype, qweight, scales, zeros, y, M, N, K, group, fmt, workspace,
                          workspace_bytes, stream);
}

w4a16_status w4a16_linear(const void *x, int32_t dtype, const void *qweight, const void *scales,
                          const void *zeros, void *y, int64_t M, int64_t N, int64_t K, int32_t group,
                          void *workspace, size_t workspace_bytes, void *stream) {
    return w4a16_linear_fmt(x, dtype, qweight, scales, zeros, y, M, N, K, group, W4A16_FMT_ASYM4, workspace,
                            workspace_bytes, stream);
}

w4a16_status w4a16_quant_error_workspace_bytes(int64_t N, int64_t K, int32_t group, size_t *bytes) {
    if (!bytes || !shape_ok(N, K, group)) return W4A16_ERR_INVALID_ARG;
    *bytes = quant_error_partial_bytes((int)N, (int)K);
    return W4A16_OK;
}

w4a16_status w4a16_quant_error(const float *w, const void *qweight, const void *scales, const void *zeros,
                               int64_t N, int64_t K, int32_t group, int32_t fmt, double *out, void *workspace,
                               size_t workspace_bytes, void *stream) {
    if (!fmt_group_ok(fmt, group) || !shape_ok(N, K, group)) return W4A16_ERR_INVALID_ARG;
    const bool zp = fmt == W4A16_FMT_ASYM4;
    if (!w || !qweight || !scales || (zp && !zeros) || !out) return W4A16_ERR_INVALID_ARG;
    if (!aligned16(w) || !aligned16(qweight) || !aligned16(out)) return W4A16_ERR_INVALID_ARG;
    const size_t need = quant_error_partial_bytes((int)N, (int)K);
    if (!workspace || workspace_bytes < need) return W4A16_ERR_WORKSPACE;
    if (!aligned16(workspace)) return W4A16_ERR_INVALID_ARG;
    size_t qb, sb, zb;
    meta_bytes(N, K, group, fmt, &qb, &sb, &zb);
    const Range ro = range_of(out, 8 * sizeof(double)), rw = range_of(workspace, need);
    const Range ins[4] = {range_of(w, (size_t)(N * K * 4)), range_of(qweight, qb), range_of(scales, sb),
                          range_of(zeros, zb)};
    for (const Range &r : ins)
        if (overlap(ro, r) || overlap(rw, r)) return W4A16_ERR_INVALID_ARG;
    if (overlap(ro, rw)) return W4A16_ERR_INVALID_ARG;
    w4a16_status st = check_device();
    if (st != W4A16_OK) return st;
    hipError_t e = launch_quant_error(w, qweight, scales, zeros, (int)N, (int)K, group, fmt, out,
                                      reinterpret_cast<double *>(workspace), reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

w4a16_status w4a16_scale_activations(const void *x, int32_t dtype, const float *act_mul, void *x_out, int64_t M,
                                     int64_t K, void *stream) {
    if (M < 0 || M > (1LL << 24) || K < 8 || K % 8 != 0 || K > (1LL << 30)) return W4A16_ERR_INVALID_ARG;
    if (dtype != W4A16_F16 && dtype != W4A16_BF16) return W4A16_ERR_INVALID_ARG;
    if (M == 0) return W4A16_OK;
    if (!x || !act_mul || !x_out) return W4A16_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(act_mul) || !aligned16(x_out)) return W4A16_ERR_INVALID_ARG;
    const Range ro = range_of(x_out, (size_t)(M * K * 2));
    if (overlap(ro, range_of(act_mul, (size_t)K * 4))) return W4A16_ERR_INVALID_ARG;
    if (x != x_out && overlap(ro, range_of(x, (size_t)(M * K * 2)))) return W4A16_ERR_INVALID_ARG;
    w4a16_status st = check_device();
    if (st != W4A16_OK) return st;
    hipError_t e = launch_scale_activations(x, dtype == W4A16_BF16, act_mul, x_out, M, (int)K,
                                            reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

w4a16_status w4a16_awq_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group, int32_t fmt, int32_t dtype,
                                       size_t *bytes) {
    if (!bytes || M < 0 || M > (1LL << 24) || !shape_ok(N, K, group) || !fmt_group_ok(fmt, group) ||
        (dtype != W4A16_F16 && dtype != W4A16_BF16))
        return W4A16_ERR_INVALID_ARG;
    (void)dtype;
    *bytes = M == 0 ? 0
             : decode_fits(M, N, K, group, fmt, true) ? decode_need(M, N, K, group, fmt, true)
                                                      : align_up((size_t)(M * K * 2), 256) + gemm_need(M, N, K, group);
    return W4A16_OK;
}

w4a16_status w4a16_linear_awq(const void *x, int32_t dtype, const float *act_mul, const void *qweight,
                              const void *scales, const void *zeros, void *y, int64_t M, int64_t N, int64_t K,
                              int32_t group, int32_t fmt, void *workspace, size_t workspace_bytes, void *stream) {
    w4a16_status st = check_linear(x, dtype, qweight, scales, zeros, y, M, N, K, group, fmt, nullptr, 0, 0);
    if (st != W4A16_OK || M == 0) return st;
    if (!act_mul || !aligned16(act_mul)) return W4A16_ERR_INVALID_ARG;
    if (overlap(range_of(y, (size_t)(M * N * 2)), range_of(act_mul, (size_t)K * 4))) return W4A16_ERR_INVALID_ARG;
    const bool fused = decode_fits(M, N, K, group, fmt, true);
    // not fused: the scaled activations, then the product's own workspace
    const size_t xbytes = align_up((size_t)(M * K * 2), 256);
    const size_t need = fused ? decode_need(M, N, K, group, fmt, true) : xbytes + gemm_need(M, N, K, group);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return W4A16_ERR_WORKSPACE;
        if (!aligned16(workspace)) return W4A16_ERR_INVALID_ARG;
        const Range rw = range_of(workspace, need);
        size_t qb, sb, zb;
        meta_bytes(N, K, group, fmt, &qb, &sb, &zb);
        if (overlap(rw, range_of(y, (size_t)(M * N * 2))) || overlap(rw, range_of(x, (size_t)(M * K * 2))) ||
            overlap(rw, range_of(act_mul, (size_t)K * 4)) || overlap(rw, range_of(qweight, qb)) ||
            overlap(rw, range_of(scales, sb)) || overlap(rw, range_of(zeros, zb)))
            return W4A16_ERR_INVALID_ARG;
    }
    st = check_device();
    if (st != W4A16_OK) return st;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (fused) {   // one launch: the decode kernel scales the activations as it loads them
        const DecodePlan plan = decode_plan(M, N, K, group, fmt, true);
        hipError_t e = launch_decode(x, dtype == W4A16_BF16, qweight, scales, zeros, y, (int)M, (int)N, (int)K,
                                     group, fmt, act_mul, plan, workspace, s);
        return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
    }
    hipError_t e = launch_scale_activations(x, dtype == W4A16_BF16, act_mul, workspace, M, (int)K, s);
    if (e != hipSuccess) return W4A16_ERR_HIP;
    return w4a16_gemm_fmt(workspace, dtype, qweight, scales, zeros, y, M, N, K, group, fmt,
                          static_cast<char *>(workspace) + xbytes, workspace_bytes - xbytes, stream);
}

}  // extern "C"

unsigned int *w4a16::kernel_error_word() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    return g_err_dev[dev].load(std::memory_order_acquire);
}
