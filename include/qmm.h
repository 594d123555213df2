/*
 * qmm.h -- C ABI of libqmm: affine group-quantized small-M matmul for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is y[M,N] = x[M,K] . dequant(Wq[N,K])^T, the transposed
 * quantized matmul of a speculative-decoding verify step (M = 4..6 rows for
 * 3..5 draft tokens) and of batched decode (M up to 64):
 *   - "How the NAX Verify Kernel Path Improves Decode Performance in MTPLX",
 *     sections "Architectural Differences" (verify shapes M = 4-6) and
 *     "Implementation and Configuration" (operands x, w_q, scales, biases;
 *     y has shape (M, N));
 *   - MLX issue #4720 "[BUG] qmm_splitk is chosen over qmm_nax on M5 ...",
 *     "To Reproduce" (quantize(w, group_size, bits) -> (wq, scales, biases);
 *     quantized_matmul(x, wq, scales, biases, transpose=True, ...)).
 * Supported formats follow "What Are NAX Verify Kernels and When Is the
 * Turbo Profile Activated in MTPLX?", "Supported Data Formats and
 * Quantization Schemes": 4-, 6- or 8-bit affine codes, group sizes 32, 64,
 * 128, fp16 or bf16 activations.
 *
 * Data layout (all arrays dense, row-major, caller-owned device memory):
 *   w       [N, K]            dtype dt (weights before quantization)
 *   wq      [N, K*bits/32]    uint32; each row is a little-endian bitstream
 *                             with code k at bits [bits*k, bits*k+bits):
 *                             4-bit = 8 codes per word, low nibble first;
 *                             8-bit = 4 codes per word; 6-bit = 4 codes per
 *                             24 bits (16 codes per 3 words)
 *   scales  [N, K/gs]         dtype dt
 *   biases  [N, K/gs]         dtype dt
 *   x       [M, K]            dtype dt
 *   y       [M, N]            dtype dt
 * Dequantized weight: w_hat = s*q + b.  Accumulation is fp32; y is rounded
 * once to dt (nearest-even).
 *
 * Quantizer (no formula is printed on the pages; this is the min/max affine
 * reading): per group, lo = min, hi = max,
 *   s = fp32 (hi - lo) / (2^bits - 1), stored in dt rounded toward +inf;
 *   b = lo;  q = clamp(rint_half_even(fp32 (w - b) / s), 0, 2^bits - 1),
 *   and q = 0 when s == 0 (constant group).
 *
 * Conventions shared by every entry point:
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *     No entry point synchronizes, allocates memory or keeps a pointer
 *     after it returns; the caller keeps buffers alive until the stream has
 *     passed the call.  Entry points are thread-safe.
 *   - Arguments are validated before any HIP call.  Return values:
 *       QMM_OK               success (also for empty problems: M == 0 or
 *                            N == 0 launch nothing and may pass NULL)
 *       QMM_ERR_INVALID_ARG  negative size, or NULL pointer for a non-empty
 *                            array
 *       QMM_ERR_UNSUPPORTED  dt not fp16/bf16, bits not 4/6/8, group size
 *                            not 32/64/128, K < 64 or K % 64 != 0,
 *                            K % group_size != 0, M > 64, unknown kernel id
 *       QMM_ERR_MISALIGNED   an array base pointer not 16-byte aligned
 *       QMM_ERR_HIP          the launch failed (asynchronous faults surface
 *                            at the caller's next synchronization)
 *   - Inputs must be finite; inputs to the quantizer must have a finite
 *     fp32 group range.  Output arrays must not alias input arrays.
 */
#ifndef QMM_H
#define QMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum qmm_dtype { QMM_F16 = 0, QMM_BF16 = 1 };

enum qmm_status {
    QMM_OK = 0,
    QMM_ERR_INVALID_ARG = -1,
    QMM_ERR_UNSUPPORTED = -2,
    QMM_ERR_MISALIGNED = -3,
    QMM_ERR_HIP = -4
};

/* Kernel variants for qmm_small_m_forced / qmm_select_kernel. */
enum qmm_kernel {
    QMM_KERNEL_VALU = 0,      /* split-free, VALU dot products, cross-lane K reduction */
    QMM_KERNEL_MFMA_REG = 1,  /* split-free, MFMA with in-register weight fragments, M <= 16 */
    QMM_KERNEL_MFMA_PASS = 2, /* split-free, MFMA, K walked in passes of 16 k-blocks, any K, M <= 64 */
    QMM_KERNEL_MFMA_TILE16 = 3, /* split-free, MFMA, 16-column tiles, activations shared through LDS, M <= 64 */
    QMM_KERNEL_MFMA_TILE64 = 4, /* as TILE16 with 64-column tiles (wide N) */
    QMM_KERNEL_COUNT = 5
};

/*
 * Quantize W [N, K] (dtype dt) into wq / scales / biases with the rule
 * above.  Bit-exact: the same inputs always give the same words, scales
 * and biases.
 */
int qmm_quantize(int dt, int bits, int group_size, int64_t N, int64_t K,
                 const void* w, uint32_t* wq, void* scales, void* biases,
                 void* stream);

/*
 * Dequantize into w_out [N, K] (dtype dt): w_out = RNE_dt(fp32(s*q + b)).
 * s*q is exact in fp32, so this is one fp32 rounding then one rounding to
 * dt.  Bit-exact.
 */
int qmm_dequantize(int dt, int bits, int group_size, int64_t N, int64_t K,
                   const uint32_t* wq, const void* scales, const void* biases,
                   void* w_out, void* stream);

/*
 * y [M, N] = x [M, K] . dequant(wq, scales, biases)^T with fp32
 * accumulation and one rounding to dt.  1 <= M <= 64 (M == 0 is an empty
 * no-op).  The kernel variant is chosen by qmm_select_kernel.
 * Deterministic: identical inputs give bit-identical outputs.
 */
int qmm_small_m(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K,
                const void* x, const uint32_t* wq, const void* scales,
                const void* biases, void* y, void* stream);

/* As qmm_small_m with the variant forced (measurement and tests).
 * QMM_ERR_UNSUPPORTED if the variant cannot run this shape
 * (QMM_KERNEL_MFMA_REG needs M <= 16 and K <= 4096; the TILE variants need
 * K to be a multiple of 128 for 4-bit codes, of 64 for 6- and 8-bit). */
int qmm_small_m_forced(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K,
                       const void* x, const uint32_t* wq, const void* scales,
                       const void* biases, void* y, void* stream, int kernel_id);

/* The variant qmm_small_m runs for this problem (a qmm_kernel value), or a
 * negative status if the problem is not supported.  Pure host logic. */
int qmm_select_kernel(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K);

/* 1 if variant `kernel_id` can run this problem, 0 if it cannot, or a
 * negative status if the problem itself is invalid or unsupported.  Pure
 * host logic. */
int qmm_kernel_supported(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K, int kernel_id);

/* uint32 words per packed row: K*bits/32 (-1 for unsupported bits or a K
 * that does not fill whole words). */
int64_t qmm_packed_words(int bits, int64_t K);

/* Static description of a status code. */
const char* qmm_strerror(int status);

/* Static name of a kernel variant ("?" if unknown). */
const char* qmm_kernel_name(int kernel_id);

/*
 * Measurement helpers (not part of the matmul path).
 *
 * qmm_probe_stream_read: read `bytes` (a multiple of 16) from device memory
 * `src` with coalesced 16-byte nontemporal loads, `grid` workgroups of 256
 * threads (0 = 2048; never more than the data needs), and discard the data.
 * `sink` is caller-owned device memory of at least 256 uint32 that the
 * kernel may write (practically never does).  It is the streaming-read
 * ceiling a matmul streaming the same bytes can approach.
 *
 * qmm_probe_copy: copy `bytes` (a multiple of 16) from `src` to `dst`
 * (device memory, not overlapping).  It reads and writes exactly `bytes`
 * each, so hardware byte counters taken on it give their scale.
 *
 * Both: 16-byte aligned pointers (QMM_ERR_MISALIGNED otherwise), negative
 * sizes -> QMM_ERR_INVALID_ARG, other sizes -> QMM_ERR_UNSUPPORTED, 0 bytes
 * -> QMM_OK with nothing launched; asynchronous on `stream` like the rest.
 */
int qmm_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int grid, void* stream);
int qmm_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
