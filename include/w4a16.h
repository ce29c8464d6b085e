/*
 * w4a16.h - C ABI of the MI355X (gfx950) W4A16 weight-only linear layer.
 *
 * The operation. Weights are stored as 4-bit integer codes with one fp16 scale
 * and one 4-bit zero-point per group of 32, 64, 128 or 256 consecutive input
 * channels; the kernels unpack and rescale the codes just before the multiply,
 * while the activations stay 16-bit and the accumulation is fp32
 * ("Weight-Only Quantisation", klaylearn glossary, definition; "Weight-Only
 * Quantization Explained", multigrid.ai, "What W4A16 actually names").
 *
 *   quantise (per output column n, group g of k):
 *     lo = min(0, min w), hi = max(0, max w)           fp32
 *     s  = fp16_rne((hi - lo) / 15), 0 -> 2^-24         (the stored scale)
 *     z  = clamp(rint(-lo / s), 0, 15)
 *     q  = clamp(rint(w / s) + z, 0, 15)                rint: ties to even
 *   dequantise:   w_hat[n][k] = s[g][n] * (q[n][k] - z[g][n])
 *   product:      y[m][n] = sum_k x[m][k] * w_hat[n][k]
 *
 * Two symmetric formats share the kernels (w4a16_format): codes without a
 * stored zero-point, 4-bit (SYM4) or 8-bit (SYM8, weight-only INT8: W8A16),
 *     s = fp16_rne(max|w| / qmax), 0 -> 2^-24         qmax = 7 or 127
 *     q = clamp(rint(w / s), -qmax-1, qmax) + qmax + 1   (stored code, unsigned)
 *     w_hat = s * (q - (qmax + 1))
 * (the symmetric INT8 scheme of the instagit comparison page, "INT8:
 * Symmetric Integer Quantization", applied per group as the "Classic blocks"
 * row of the GGUF table in "Quantization Is Not a Zip File" does; INT4 or
 * INT8 weights under 16-bit activations: "Weight-Only Quantisation",
 * definition). Group 256 is the super-block size of that table's K-quant row.
 *
 * KQ4, K-quant-style super-blocks ("sub-block scales/minima inside
 * 256-weight super-blocks", the K-quant row of that table), group = 256:
 *   per 32-weight sub-block j:  lo, hi as above, s_j = (hi - lo)/15, mn_j = 0 - lo
 *   per super-block:  d = fp16_rne(max_j s_j / 63), dmin = fp16_rne(max_j mn_j / 63)
 *                     (0 -> 2^-24)
 *   sc_j = clamp(rint(s_j/d), 0, 63), mq_j = clamp(rint(mn_j/dmin), 0, 63)
 *   S_j = d*sc_j, M_j = dmin*mq_j, q = clamp(rint((w + M_j)/S_j), 0, 15) (0 if S_j = 0)
 *   w_hat = S_j * q - M_j
 *
 * Rounding to the nearest grid point of w / scale follows "Quantization Is Not
 * a Zip File" (zhuai.tech), section 3; the per-group scale ("block locality")
 * is in the same section; the (q - zero) * scale reconstruction is the
 * zero-point example of the instagit comparison page ("Practical Code
 * Examples"). The quantiser runs once, offline; the packed data then stays
 * packed until the kernel consumes it ("Quantization Is Not a Zip File",
 * section 8).
 *
 * Layout (all little-endian, contiguous). C = K/32 chunks of 32 weights along
 * K, grouped into T = ceil(C/4) columns of 128 weights (the last column holds
 * nc = C - 4(T-1) chunks when K % 128 != 0). Rows come in blocks of 16 (the
 * last block holds rows_b = N - 16b when N % 16 == 8).
 *   w        fp32 [N][K]            input of w4a16_pack (PyTorch Linear order)
 *   qweight  N*K/2 bytes            block b occupies bytes [8Kb, 8K(b+1));
 *            inside it, column t starts at byte 64*rows_b*t. Dword d (0..3) of
 *            chunk c = 4t + j of row r = n%16 sits at byte
 *              8Kb + 64*rows_b*t + 4*(d*rows_b*nc + r*nc + j)
 *            (nc = 4 for a full column). It holds k = 32c + 8d + i (i = 0..7)
 *            in nibble i/2 + 4*(i%2): even k in the low half-word, odd k in
 *            the high half-word. A full column of a full block is one
 *            contiguous KiB in which the 16 bytes at 256d + 16r are dword d of
 *            the column's four chunks of row r.
 *   scales   fp16 [N][G8]           row n's group scales in k order, G = K/group
 *                                   and G8 = G rounded up to a multiple of 8
 *                                   (slots g >= G hold 0): one row's scales
 *                                   along K are contiguous
 *   zeros    uint32 [N][G8/8]       4-bit zero-points: group g of row n is
 *                                   bits 4*(g%8) .. 4*(g%8)+3 of word n*G8/8 + g/8
 *                                   (slots g >= G hold 0)
 *            With G % 8 == 0 the sizes are the canonical 2*G*N and G*N/2 bytes.
 *   SYM4     qweight as above (codes q + 8), scales as above, no zeros.
 *   SYM8     qweight N*K bytes: two 4-bit planes in the layout above, the low
 *            nibbles of every code in bytes [0, N*K/2), the high nibbles in
 *            [N*K/2, N*K); scales as above, no zeros.
 *   KQ4      qweight as above; `scales` holds one 16-byte record per
 *            (row n, super-block u) in [N][K/256] order: four little-endian
 *            words {d | dmin << 16, sc bits 0-31, sc bits 32-47 | mq bits 0-15
 *            << 16, mq bits 16-47}, sc and mq being 48-bit fields of eight
 *            6-bit values (sub-block j at bits 6j..6j+5); no zeros. K % 256 == 0.
 *   x        fp16 or bf16 [M][K], row-major
 *   y        same type as x, [M][N], row-major; fp32 accumulation, rounded
 *            once to the output type (round to nearest even)
 *
 * Ownership: the caller owns every buffer; no call allocates or frees device
 * memory. Every pointer passed to a compute call is a device pointer. Calls
 * enqueue work on `stream` (a hipStream_t; NULL = the null stream) and return
 * without synchronising; faults inside a kernel surface at the caller's next
 * synchronisation.
 *
 * Errors: every function returns a w4a16_status. Argument checks happen
 * before anything is enqueued, and a failed check leaves every buffer
 * untouched. W4A16_ERR_HIP reports a HIP runtime error (launch failure or a
 * device query that failed) or a kernel error of an earlier call (see
 * w4a16_init).
 *
 * Preconditions shared by the compute calls:
 *   0 <= M <= 2^24, M*K < 2^34, N >= 8, N % 8 == 0, group in {32, 64, 128, 256},
 *   K >= group, K % group == 0; pointers non-NULL and 16-byte aligned (zeros
 *   is not read, and may be NULL, for the symmetric formats); y does not
 *   overlap any input; the current device is a gfx950 (w4a16_device_supported).
 *   Weights given to w4a16_pack are finite with |w| < 2^18.
 *
 * Empty batch: with M = 0 the products (gemv, gemm, linear, linear_group,
 * linear_awq) and w4a16_scale_activations check the shape, type and format
 * arguments only, read no pointer (all may be NULL), enqueue nothing and
 * return W4A16_OK; the workspace queries return 0 bytes.
 *
 * Every call without a format argument works on W4A16_FMT_ASYM4; its `_fmt`
 * twin takes the format as the argument after `group` and is otherwise the
 * same call.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_LAYOUT_VERSION 3

typedef enum {
    W4A16_OK = 0,
    W4A16_ERR_INVALID_ARG = 1,   /* a precondition above does not hold */
    W4A16_ERR_UNSUPPORTED = 2,   /* the device is not a gfx950 */
    W4A16_ERR_HIP = 3,           /* HIP runtime error */
    W4A16_ERR_WORKSPACE = 4      /* workspace missing or smaller than required */
} w4a16_status;

typedef enum {
    W4A16_F16 = 0,
    W4A16_BF16 = 1
} w4a16_dtype;

typedef enum {
    W4A16_FMT_ASYM4 = 0,   /* 4-bit codes, fp16 scale and 4-bit zero-point per group */
    W4A16_FMT_SYM4 = 1,    /* 4-bit codes q + 8, fp16 scale per group, no zero-points */
    W4A16_FMT_SYM8 = 2,    /* 8-bit codes q + 128 (two 4-bit planes), fp16 scale per group: W8A16 */
    W4A16_FMT_KQ4 = 3      /* 4-bit codes in 256-weight super-blocks of eight 32-weight sub-blocks with
                              6-bit scales and minima (K-quant style, 4.5 bits/weight); group 256 */
} w4a16_format;

/* Human-readable name of a status code (static string, never NULL). */
const char *w4a16_status_string(int status);

/* Layout version of the packed format this library reads and writes. */
int w4a16_layout_version(void);

/* One-time set-up of `device` (a gfx950) for this library, safe to call again
 * and from several threads: the device check, the device address of the
 * library's static scratch array (w4a16_linear_noalloc) and, once per
 * process, a 256-byte block of pinned host memory mapped into every device
 * (the kernel error word below). Every compute call runs it on its device on
 * first use; call it at start-up to keep that allocation out of later calls.
 * Kernel errors: when the bounded wait of a stream-K hand-over (see
 * w4a16_workspace_bytes) runs out, which a correct launch never lets happen,
 * the waiting workgroup writes its whole output tile as NaN and sets the
 * process's error word; the next compute call (any entry point, any device)
 * clears it and returns W4A16_ERR_HIP before enqueuing anything.
 * W4A16_ERR_UNSUPPORTED for a device other than a gfx950, W4A16_ERR_HIP when
 * a runtime call fails. */
w4a16_status w4a16_init(int device);

/* W4A16_OK when `device` is a gfx950 (the only target of these kernels),
 * W4A16_ERR_UNSUPPORTED for any other device, W4A16_ERR_HIP if the query fails.
 * The four "support" states of "Quantization Is Not a Zip File" (section 8)
 * map to: format parsable (always), CPU reference (the separate test oracle),
 * device packed kernel (this call), default path (w4a16_linear). */
w4a16_status w4a16_device_supported(int device);

/* Byte sizes of the packed buffers for an N x K weight matrix: qweight
 * N*K/2, scales 2*G8*N, zeros G8*N/2 (G8 = K/group rounded up to a multiple
 * of 8). With (K/group) % 8 == 0 these are 2*G*N and G*N/2: 4 + 20/group
 * bits per weight, the 4.156 bits/weight at group 128 of "Weight-Only
 * Quantization Explained", "The memory arithmetic". Host-only; any
 * out-pointer may be NULL. */
w4a16_status w4a16_packed_bytes(int64_t N, int64_t K, int32_t group,
                                size_t *qweight_bytes, size_t *scales_bytes,
                                size_t *zeros_bytes);
/* Per format: qweight N*K/2 bytes (N*K for SYM8), scales as above (KQ4:
 * 16*(K/256)*N bytes of records), zeros 0 bytes for every format but ASYM4.
 * SYM4 stores 4 + 16/group bits per weight, SYM8 8 + 16/group, KQ4 4.5. KQ4
 * with a group other than 256 is W4A16_ERR_INVALID_ARG. */
w4a16_status w4a16_packed_bytes_fmt(int64_t N, int64_t K, int32_t group, int32_t fmt,
                                    size_t *qweight_bytes, size_t *scales_bytes,
                                    size_t *zeros_bytes);

/* Workspace bytes a w4a16_gemv / w4a16_gemm / w4a16_linear call of this shape
 * needs on the current device, in any weight format. Host-only (queries the
 * device's compute-unit count once). The decode kernel (M <= 8) needs some
 * when it splits K: an 8-byte counter per 16-row block (padded to 256 bytes)
 * and M x 16 fp32 partials per row block and split. The tiled GEMM (M > 32) needs
 * some when its last round of 256 x 256 (or 128 / 64-row) output tiles would
 * be at most half full on the device's compute units: it then splits the
 * last two rounds' tiles by K over one workgroup per compute unit
 * (stream-K), and a tile's two workgroups hand an fp32 partial tile and an
 * 8-byte flag over through the workspace: BM x 256 x 4 + 8 bytes per compute
 * unit (about 64 MiB on 256 compute units). It also needs some when its tiles
 * fill at most half of the compute units (mid-size batches): each tile's K
 * is then split over S workgroups (S up to 16), which leave fp32 partial
 * tiles, the last to arrive adding them in split order: tiles x S x
 * BM x 256 x 4 bytes plus an 8-byte counter per tile (padded to 256 bytes),
 * under 64 MiB. With 0 bytes the compute calls accept a NULL workspace.
 * The workspace is device memory owned by the caller, 16-byte aligned, and
 * must not overlap any argument of the call. Its contents need no
 * initialisation (each launch marks its hand-overs with a 64-bit token mixed
 * from a random per-process seed, which earlier contents match only by a
 * 2^-64 chance) and are meaningless after the call; calls that run at the
 * same time (other streams) must not share one. */
w4a16_status w4a16_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group,
                                   size_t *bytes);
/* Workspace bytes of a w4a16_linear_group_fmt call (count problems of N[p]
 * rows each, N a host array): the largest single-call need of any problem,
 * or, when the call runs one decode launch, the counters of every problem's
 * row blocks and the partials of those that split. Host-only. */
w4a16_status w4a16_group_workspace_bytes(int32_t count, int64_t M, const int64_t *N, int64_t K,
                                         int32_t group, int32_t fmt, size_t *bytes);

/* Quantise and pack: w fp32 [N][K] -> qweight, scales, zeros (layout above).
 * Bit-exact with the quantiser defined above (IEEE fp32, no reciprocal). */
w4a16_status w4a16_pack(const float *w, int64_t N, int64_t K, int32_t group,
                        void *qweight, void *scales, void *zeros, void *stream);
/* Same in any format: the symmetric quantiser above for SYM4 / SYM8 (zeros
 * not written, may be NULL). */
w4a16_status w4a16_pack_fmt(const float *w, int64_t N, int64_t K, int32_t group, int32_t fmt,
                            void *qweight, void *scales, void *zeros, void *stream);

/* Inverse view of the packed data in canonical form, for tests and tools:
 * codes uint8 [N][K], scales fp16 bits [G][N], zeros uint8 [G][N]. */
w4a16_status w4a16_unpack(const void *qweight, const void *scales, const void *zeros,
                          int64_t N, int64_t K, int32_t group,
                          uint8_t *codes, uint16_t *scales_out, uint8_t *zeros_out,
                          void *stream);
/* Same in any format: codes are the stored unsigned codes (0..255 for SYM8);
 * zeros_out receives the fixed zero (8 or 128) of a symmetric format. KQ4:
 * codes only (its records are already in canonical order; scales_out and
 * zeros_out are not written and may be NULL). */
w4a16_status w4a16_unpack_fmt(const void *qweight, const void *scales, const void *zeros,
                              int64_t N, int64_t K, int32_t group, int32_t fmt,
                              uint8_t *codes, uint16_t *scales_out, uint8_t *zeros_out,
                              void *stream);

/* Decode GEMV: y [M][N] = x [M][K] . w_hat^T for small M (M <= 8).
 * One pass over the packed weights: a workgroup per 16-row block and range of
 * K's 128-weight columns (up to 16 waves of four, eight or sixteen columns),
 * 128-bit loads, in-register unpack, packed fp16 / bf16 dot products with
 * fp32 accumulation, the group scale and zero-point applied once per group;
 * the waves meet in LDS in a fixed order. At M = 1 with K > 16384 (4-bit
 * codes, K a multiple of 128) the activations stay in registers and are
 * broadcast across lanes, with the same sums in the same order (the same
 * bits). Split K: only where a workgroup's LDS cannot hold its slice (long K
 * at the larger M and the smaller groups), S workgroups share a row block's K
 * and leave fp32 partials in the workspace (w4a16_workspace_bytes); the last
 * of them adds the S partials in a fixed order, so results are deterministic
 * and independent of timing. Range:
 * M <= 8 and K <= 65536; W4A16_ERR_INVALID_ARG outside it (w4a16_gemm and
 * w4a16_linear have no such limit), W4A16_ERR_WORKSPACE when the workspace is
 * smaller than w4a16_workspace_bytes. */
w4a16_status w4a16_gemv(const void *x, int32_t dtype, const void *qweight,
                        const void *scales, const void *zeros, void *y,
                        int64_t M, int64_t N, int64_t K, int32_t group,
                        void *workspace, size_t workspace_bytes, void *stream);
w4a16_status w4a16_gemv_fmt(const void *x, int32_t dtype, const void *qweight,
                            const void *scales, const void *zeros, void *y,
                            int64_t M, int64_t N, int64_t K, int32_t group, int32_t fmt,
                            void *workspace, size_t workspace_bytes, void *stream);

/* Matrix-core GEMM for any M (M*K < 2^34); the workspace is sized by
 * w4a16_workspace_bytes (W4A16_ERR_WORKSPACE when it is smaller). M <= 32: the packed weights
 * stream through registers as in the GEMV, and each unpacked dword feeds one
 * 16x16x32 MFMA per 16-row tile of x (exact integers q - z, group scale on the
 * fp32 sums; one workgroup per tile and group of row blocks). Larger M:
 * weight tiles are dequantised once per workgroup into LDS as 16-bit
 * s*(q - z) (one rounding) and fed to 32x32x16 MFMAs with fp32 accumulation
 * ("Weight-Only Quantisation", the FAQ answers on batch size: at prefill the
 * layer is compute bound and the dequantisation is on the critical path). */
w4a16_status w4a16_gemm(const void *x, int32_t dtype, const void *qweight,
                        const void *scales, const void *zeros, void *y,
                        int64_t M, int64_t N, int64_t K, int32_t group,
                        void *workspace, size_t workspace_bytes, void *stream);
w4a16_status w4a16_gemm_fmt(const void *x, int32_t dtype, const void *qweight,
                            const void *scales, const void *zeros, void *y,
                            int64_t M, int64_t N, int64_t K, int32_t group, int32_t fmt,
                            void *workspace, size_t workspace_bytes, void *stream);

/* Default path: dispatches on M between w4a16_gemv (small-batch decode, where
 * the weight stream is the bottleneck) and w4a16_gemm (larger batches and
 * prefill, where the multiply becomes the bottleneck; "Weight-Only
 * Quantization Explained", "Where it stops being the right answer"). */
w4a16_status w4a16_linear(const void *x, int32_t dtype, const void *qweight,
                          const void *scales, const void *zeros, void *y,
                          int64_t M, int64_t N, int64_t K, int32_t group,
                          void *workspace, size_t workspace_bytes, void *stream);
w4a16_status w4a16_linear_fmt(const void *x, int32_t dtype, const void *qweight,
                              const void *scales, const void *zeros, void *y,
                              int64_t M, int64_t N, int64_t K, int32_t group, int32_t fmt,
                              void *workspace, size_t workspace_bytes, void *stream);

/* Several independent linear layers of the same M, K, group and activation
 * type in one launch: y[p] = x[p] . w_hat[p]^T for p < count (1..8), problem p
 * with N[p] output rows. The arrays x, qweight, scales, zeros, y and N are
 * host arrays of `count` entries (device pointers / sizes); x[p] may be the
 * same pointer for several p (q/k/v or gate/up of one token batch). Every
 * problem must pass w4a16_linear's checks, and no y[p] may overlap any buffer
 * of any problem. The workspace is sized by w4a16_group_workspace_bytes. At
 * M <= w4a16_gemv_max_m all problems run in one launch of the decode kernel,
 * each with the split a call on it alone would use; for M up to 128 in one
 * launch of the small-batch matrix-core kernel; either pays the fixed cost of
 * a launch (the ramp-up and drain that dominate small decode layers) once.
 * For larger M it enqueues one tiled GEMM per problem, one after the other,
 * each using the workspace. Results are bit-identical to w4a16_linear on each
 * problem. This fuses the launches, not the math: the
 * pages' dual-output decode variant ("Quantization Is Not a Zip File", section
 * 2, paired gate/up projections) is the special case of two problems sharing x. */
w4a16_status w4a16_linear_group(int32_t count, const void *const *x, int32_t dtype,
                                const void *const *qweight, const void *const *scales,
                                const void *const *zeros, void *const *y, int64_t M,
                                const int64_t *N, int64_t K, int32_t group,
                                void *workspace, size_t workspace_bytes, void *stream);
/* Same, every problem in format `fmt` (zeros may be NULL for the symmetric formats). */
w4a16_status w4a16_linear_group_fmt(int32_t count, const void *const *x, int32_t dtype,
                                    const void *const *qweight, const void *const *scales,
                                    const void *const *zeros, void *const *y, int64_t M,
                                    const int64_t *N, int64_t K, int32_t group, int32_t fmt,
                                    void *workspace, size_t workspace_bytes, void *stream);

/* A kernel run by choice instead of w4a16_linear's dispatch: kernel 0 = the
 * decode kernel (w4a16_gemv's range), 1 = the small-batch matrix-core kernel,
 * 2 = the tiled matrix-core GEMM (with its stream-K split where its plan has
 * one), each at any M it takes; W4A16_ERR_INVALID_ARG for another kernel
 * number or a shape the kernel does not take. For measuring the dispatch's
 * crossovers and for callers that pin a kernel. Every other argument and the
 * results are those of w4a16_linear_fmt (kernel 1 and 2 at M <= 32 and
 * above give w4a16_gemm_fmt's bits where w4a16_gemm_fmt runs that kernel).
 * Workspace: w4a16_kernel_workspace_bytes (host-only). */
w4a16_status w4a16_kernel_workspace_bytes(int32_t kernel, int64_t M, int64_t N, int64_t K,
                                          int32_t group, int32_t fmt, size_t *bytes);
w4a16_status w4a16_linear_run_fmt(int32_t kernel, const void *x, int32_t dtype,
                                  const void *qweight, const void *scales, const void *zeros,
                                  void *y, int64_t M, int64_t N, int64_t K, int32_t group,
                                  int32_t fmt, void *workspace, size_t workspace_bytes,
                                  void *stream);

/* Largest M that w4a16_linear may send to the GEMV kernel. */
int32_t w4a16_gemv_max_m(void);

/* The kernel w4a16_linear picks for this shape on the current device:
 * 0 = decode GEMV, 1 = small-batch matrix-core kernel (M <= 32),
 * 2 = tiled matrix-core GEMM; -1 for M = 0 (no kernel runs) and for
 * arguments w4a16_linear would reject.
 * Host-only (queries the device's LDS size once). */
int32_t w4a16_linear_kernel(int64_t M, int64_t N, int64_t K, int32_t group, int32_t dtype);
/* The same choice for a weight format, with the launch geometry of that
 * kernel: *workgroups workgroups of *threads threads (either pointer may be
 * NULL). For profiles and benchmarks: a kernel trace's rows of one shape are
 * told apart by kernel, grid and workgroup size. Returns the kernel code as
 * w4a16_linear_kernel, -1 for arguments w4a16_linear_fmt rejects. Host-only
 * (queries the device's LDS size and compute units once). */
int32_t w4a16_linear_launch_shape(int64_t M, int64_t N, int64_t K, int32_t group, int32_t dtype,
                                  int32_t fmt, int64_t *workgroups, int32_t *threads);

/* ---- Quality report ----------------------------------------------------
 * How far the packed weights are from the fp32 weights they were made from:
 * out[8] (device, fp64) = {MSE, SNR in dB, cosine similarity, max |w - w_hat|,
 * sum (w - w_hat)^2, sum w^2, sum w_hat^2, sum w*w_hat} over all N*K weights,
 * w_hat rebuilt from the packed data as the kernels rebuild it. The four
 * figures are those of the error-analysis routine of the instagit comparison
 * page ("Implementation Architecture"): MSE = sum d^2 / (N K), SNR =
 * 10 log10(sum w^2 / sum d^2) (+inf when d = 0), cosine = sum w w_hat /
 * sqrt(sum w^2 sum w_hat^2) (1 when both are zero). w is the fp32 [N][K]
 * matrix given to the pack call; workspace (device, caller-owned) holds
 * per-workgroup partial sums, w4a16_quant_error_workspace_bytes of them; the
 * partials are folded in a fixed order, so the result is deterministic. */
w4a16_status w4a16_quant_error_workspace_bytes(int64_t N, int64_t K, int32_t group, size_t *bytes);
w4a16_status w4a16_quant_error(const float *w, const void *qweight, const void *scales,
                               const void *zeros, int64_t N, int64_t K, int32_t group, int32_t fmt,
                               double *out, void *workspace, size_t workspace_bytes, void *stream);

/* ---- AWQ run-time scaling ---------------------------------------------
 * AWQ scales salient input channels of the weights up before quantisation and
 * the activations down to compensate (instagit comparison page, "AWQ:
 * Activation-Aware Weight Quantization"); choosing the factors needs
 * calibration data and is not done here. The caller quantises
 * w'[n][k] = w[n][k] * a_k with any pack call and passes act_mul[k] = 1 / a_k
 * (fp32, device, 16-byte aligned, [K]).
 *
 * w4a16_scale_activations: x_out[m][k] = x[m][k] * act_mul[k], the fp32
 * product rounded once (to nearest even) to x's type. x_out may be x itself.
 *
 * w4a16_linear_awq: y = x_out . w_hat'^T. When the GEMV takes the shape
 * (M <= 8, K within its range above and K <= 16384) the scaling is folded into the
 * GEMV's activation staging: one launch, no workspace. Otherwise it runs
 * w4a16_scale_activations into the workspace (w4a16_awq_workspace_bytes:
 * M*K*2 rounded up to 256, then w4a16_workspace_bytes for the product)
 * followed by w4a16_gemm. Either way the result is
 * the one the same kernel gives for the pre-scaled activations. */
w4a16_status w4a16_scale_activations(const void *x, int32_t dtype, const float *act_mul, void *x_out,
                                     int64_t M, int64_t K, void *stream);
w4a16_status w4a16_awq_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group, int32_t fmt,
                                       int32_t dtype, size_t *bytes);
w4a16_status w4a16_linear_awq(const void *x, int32_t dtype, const float *act_mul, const void *qweight,
                              const void *scales, const void *zeros, void *y, int64_t M, int64_t N,
                              int64_t K, int32_t group, int32_t fmt, void *workspace,
                              size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid it): w4a16_linear_fmt
 * with no workspace argument. The tiled GEMM's stream-K partials and flags
 * (and the decode kernel's partials and counters where its plan splits K) go
 * to a static device array of W4A16_NOALLOC_SCRATCH_BYTES that each device
 * holds for the life of the process; the call makes no allocation of any
 * kind. It needs w4a16_init to have run on the current device
 * (W4A16_ERR_INVALID_ARG otherwise), and returns W4A16_ERR_WORKSPACE, with
 * nothing enqueued, for a shape whose plan needs more scratch than that
 * (none on a device of at most 256 compute units). All calls on one device
 * share the array, so calls that overlap in time on one device (other
 * streams, other threads) race and must not be made; consecutive calls are
 * safe (the array needs no clearing: its stale flags never match a later
 * launch's token). Everything else is as w4a16_linear_fmt. */
#define W4A16_NOALLOC_SCRATCH_BYTES ((size_t)(64u << 20) + (4u << 10))
w4a16_status w4a16_linear_noalloc(const void *x, int32_t dtype, const void *qweight,
                                  const void *scales, const void *zeros, void *y, int64_t M,
                                  int64_t N, int64_t K, int32_t group, int32_t fmt, void *stream);

/* Measurement helpers of the benchmark, not on the product path.
 * w4a16_measure_stream_read: reads `bytes` (a multiple of 16) at `src` with
 * 16-byte loads, workgroups of 256 threads each reading one contiguous share
 * with four loads per thread in flight: `workgroups` equal shares, or (0) as
 * many workgroups as 16 KiB shares; the achievable HBM read rate, a ceiling
 * reported beside the kernels. `sink` is one device word that is written only
 * if the data's fold equals a fixed constant.
 * w4a16_measure_copy: dst = src, `bytes` (a multiple of 16, non-overlapping)
 * with 16-byte loads and stores: a kernel of known traffic (bytes read and
 * bytes written) that scales a profiler's HBM byte counters.
 * Both enqueue on `stream`; W4A16_ERR_INVALID_ARG on a bad size, pointer or
 * alignment. */
w4a16_status w4a16_measure_stream_read(const void *src, size_t bytes, uint32_t *sink,
                                       int32_t workgroups, void *stream);
w4a16_status w4a16_measure_copy(const void *src, void *dst, size_t bytes, void *stream);

/* Testing hook, for the tests of the kernel error path only: w4a16_gemm_fmt
 * on a shape whose plan splits tiles by stream-K (W4A16_ERR_INVALID_ARG
 * otherwise, nothing enqueued), except that the waiting workgroups wait for a
 * token no producer writes and give up after a few microseconds. Every
 * kernel ends normally; the split tiles of y are NaN, every other tile is what
 * w4a16_gemm_fmt writes, and the error word is set (see w4a16_init). */
w4a16_status w4a16_testing_gemm_expire(const void *x, int32_t dtype, const void *qweight,
                                       const void *scales, const void *zeros, void *y, int64_t M,
                                       int64_t N, int64_t K, int32_t group, int32_t fmt,
                                       void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
