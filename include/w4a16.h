/*
 * w4a16.h - C ABI of the MI355X (gfx950) W4A16 weight-only linear layer.
 *
 * The operation. Weights are stored as 4-bit integer codes with one fp16 scale
 * and one 4-bit zero-point per group of 32, 64 or 128 consecutive input
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
 * Rounding to the nearest grid point of w / scale follows "Quantization Is Not
 * a Zip File" (zhuai.tech), section 3; the per-group scale ("block locality")
 * is in the same section; the (q - zero) * scale reconstruction is the
 * zero-point example of the instagit comparison page ("Practical Code
 * Examples"). The quantiser runs once, offline; the packed data then stays
 * packed until the kernel consumes it ("Quantization Is Not a Zip File",
 * section 8).
 *
 * Layout (all little-endian, row-major, contiguous):
 *   w        fp32 [N][K]            input of w4a16_pack (PyTorch Linear order)
 *   qweight  N*K/2 bytes            rows in blocks of 64 (the last block holds
 *            rows_b = min(64, N - 64b) rows), K in chunks of 32: the 16-byte
 *            record of (row n, chunk c) starts at byte
 *              64*b*(K/2) + c*rows_b*16 + r*16,   b = n/64, r = n%64, c = k/32.
 *            Dword j = (k%32)/8 of a record holds k = 32c + 8j + i (i = 0..7)
 *            in nibble i/2 + 4*(i%2): even k in the low half-word, odd k in the
 *            high half-word.
 *   scales   fp16 [G][N]            G = K / group
 *   zeros    uint32 [G][N/8]        nibble n%8 of word n/8 holds z[g][n]
 *   x        fp16 or bf16 [M][K]
 *   y        same type as x, [M][N]; fp32 accumulation, rounded once (RNE)
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
 * device query that failed).
 *
 * Preconditions shared by the compute calls:
 *   M >= 1, N >= 8, N % 8 == 0, group in {32, 64, 128}, K >= group,
 *   K % group == 0; pointers non-NULL and 16-byte aligned; y does not overlap
 *   any input; the current device is a gfx950 (w4a16_device_supported).
 *   Weights given to w4a16_pack are finite with |w| < 2^18.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_LAYOUT_VERSION 1

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

/* Human-readable name of a status code (static string, never NULL). */
const char *w4a16_status_string(int status);

/* Layout version of the packed format this library reads and writes. */
int w4a16_layout_version(void);

/* W4A16_OK when `device` is a gfx950 (the only target of these kernels),
 * W4A16_ERR_UNSUPPORTED for any other device, W4A16_ERR_HIP if the query fails.
 * The four "support" states of "Quantization Is Not a Zip File" (section 8)
 * map to: format parsable (always), CPU reference (the separate test oracle),
 * device packed kernel (this call), default path (w4a16_linear). */
w4a16_status w4a16_device_supported(int device);

/* Byte sizes of the packed buffers for an N x K weight matrix:
 * qweight N*K/2, scales 2*G*N, zeros G*N/2 (4 + 20/group bits per weight, the
 * 4.156 bits/weight at group 128 of "Weight-Only Quantization Explained",
 * "The memory arithmetic"). Host-only; any out-pointer may be NULL. */
w4a16_status w4a16_packed_bytes(int64_t N, int64_t K, int32_t group,
                                size_t *qweight_bytes, size_t *scales_bytes,
                                size_t *zeros_bytes);

/* Workspace bytes a w4a16_gemv / w4a16_gemm / w4a16_linear call of this shape
 * needs (split-K partial sums and arrival counters). Host-only. The workspace
 * must be zero-filled once before its first use; every completed call leaves
 * its counters at zero again. One workspace serves one call at a time. */
w4a16_status w4a16_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group,
                                   size_t *bytes);

/* Quantise and pack: w fp32 [N][K] -> qweight, scales, zeros (layout above).
 * Bit-exact with the quantiser defined above (IEEE fp32, no reciprocal). */
w4a16_status w4a16_pack(const float *w, int64_t N, int64_t K, int32_t group,
                        void *qweight, void *scales, void *zeros, void *stream);

/* Inverse view of the packed data in canonical form, for tests and tools:
 * codes uint8 [N][K], scales fp16 bits [G][N], zeros uint8 [G][N]. */
w4a16_status w4a16_unpack(const void *qweight, const void *scales, const void *zeros,
                          int64_t N, int64_t K, int32_t group,
                          uint8_t *codes, uint16_t *scales_out, uint8_t *zeros_out,
                          void *stream);

/* Decode GEMV: y [M][N] = x [M][K] . w_hat^T for small M (1 <= M <= 8).
 * One pass over the packed weights: 128-bit loads, in-register unpack, fp16
 * or bf16 dot products with fp32 accumulation, per-group scale, split-K with a
 * deterministic in-kernel reduction. Returns W4A16_ERR_INVALID_ARG for M > 8. */
w4a16_status w4a16_gemv(const void *x, int32_t dtype, const void *qweight,
                        const void *scales, const void *zeros, void *y,
                        int64_t M, int64_t N, int64_t K, int32_t group,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Matrix-core GEMM for any M >= 1: packed weight tiles are dequantised in
 * registers/LDS to fp16/bf16 and fed to MFMA with fp32 accumulation. */
w4a16_status w4a16_gemm(const void *x, int32_t dtype, const void *qweight,
                        const void *scales, const void *zeros, void *y,
                        int64_t M, int64_t N, int64_t K, int32_t group,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Default path: dispatches on M between w4a16_gemv (small-batch decode, where
 * the weight stream is the bottleneck) and w4a16_gemm (larger batches and
 * prefill, where the multiply becomes the bottleneck; "Weight-Only
 * Quantization Explained", "Where it stops being the right answer"). */
w4a16_status w4a16_linear(const void *x, int32_t dtype, const void *qweight,
                          const void *scales, const void *zeros, void *y,
                          int64_t M, int64_t N, int64_t K, int32_t group,
                          void *workspace, size_t workspace_bytes, void *stream);

/* Largest M that w4a16_linear sends to the GEMV kernel. */
int32_t w4a16_gemv_max_m(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
