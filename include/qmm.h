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
 *     passed the call (scratch, where a variant needs it, is a
 *     caller-provided workspace).  Entry points are thread-safe.
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
    QMM_KERNEL_MFMA_REG = 1,  /* split-free, MFMA with in-register weight fragments (16-row blocks above 16 rows) */
    QMM_KERNEL_MFMA_PASS = 2, /* split-free, MFMA, K walked in passes of 16 k-blocks, any K, M <= 64 */
    QMM_KERNEL_MFMA_TILE16 = 3, /* split-free, MFMA, 16-column tiles, activations shared through LDS, M <= 64 */
    QMM_KERNEL_MFMA_TILE64 = 4, /* as TILE16 with 64-column tiles (wide N) */
    QMM_KERNEL_MFMA_DQLDS = 5,  /* split-free, MFMA, weights dequantized into LDS (64-column tiles, M <= 64,
                                   N a multiple of 64, K a multiple of 256) */
    QMM_KERNEL_COUNT = 6
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

/*
 * Batched form: `batch` independent products, each with its own weights,
 *   y[b] [M, N] = x[b] [M, K] . dequant(wq[b], scales[b], biases[b])^T,
 * over dense arrays x [batch, M, K], wq [batch, N, K*bits/32],
 * scales / biases [batch, N, K/gs], y [batch, M, N] (entry b at b times one
 * entry's size).  MLX issue #4720, "Describe the bug", confines its dispatch
 * story to transposed, non-batched calls; this is the batched case of the
 * same product.  The variant is the one qmm_small_m picks for (M, N, K);
 * the register-resident variant runs every entry in one launch (entries
 * share its resident workgroups), the others launch once per entry.  Each
 * entry's result is bit-identical to qmm_small_m on that entry.
 * batch < 0 -> QMM_ERR_INVALID_ARG; batch == 0 (or M == 0 or N == 0) ->
 * QMM_OK with nothing launched (NULL allowed); with batch > 1 every entry's
 * arrays must start 16-byte aligned (M*K*2, N*K*bits/8, N*(K/gs)*2 and
 * M*N*2 bytes multiples of 16), else QMM_ERR_MISALIGNED.  Otherwise as
 * qmm_small_m.
 */
int qmm_small_m_batched(int dt, int bits, int group_size, int64_t batch, int64_t M, int64_t N, int64_t K,
                        const void* x, const uint32_t* wq, const void* scales, const void* biases,
                        void* y, void* stream);

/*
 * Non-transposed weights: y [M, N] = x [M, K] . dequant(wq, scales, biases),
 * with W stored [K, N] and quantized along N -- the other orientation of the
 * call in MLX issue #4720, "Describe the bug" (transposed weights there):
 *   wq      [K, N*bits/32]  row k = the packed codes of W[k, :] (same
 *                           bitstream as a transposed row)
 *   scales  [K, N/gs]       one scale and bias per gs consecutive columns
 *   biases  [K, N/gs]
 * (what qmm_quantize produces from a [K, N] matrix).  fp32 accumulation and
 * one rounding to dt; deterministic.  N obeys the rules K obeys in
 * qmm_small_m (N >= 64, N % 64 == 0, N % gs == 0); K must be a positive
 * multiple of 32; 1 <= M <= 64 (M == 0: QMM_OK, nothing launched).
 * Otherwise as qmm_small_m.
 */
int qmm_small_m_nt(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K,
                   const void* x, const uint32_t* wq, const void* scales,
                   const void* biases, void* y, void* stream);

/*
 * Non-transposed weights with K split across workgroups: as qmm_small_m_nt,
 * with column-block workgroups each taking one slice of K and leaving fp32
 * partial outputs ([split][M][N]) in a caller-provided workspace; a second
 * kernel adds them in slice order and rounds once (deterministic).  4/8-bit
 * codes with N >= 4096: 256-column blocks on the fewest slices of whole
 * 16 KiB chunks dividing K that give 224..512 workgroups (at most 32 slices;
 * unsplit from 256 blocks); otherwise 128-column blocks on at most 16 slices
 * for about 256 workgroups.
 * Where the plan does not split (wide N, short K) the workspace may be NULL
 * and the call is exactly qmm_small_m_nt.
 * qmm_small_m_nt_workspace_bytes: bytes of workspace the call needs (0: no
 * split), or a negative status.  Pure host logic.
 * qmm_small_m_nt_ws: workspace is caller-owned device memory of
 * workspace_bytes >= that, 16-byte aligned, not aliasing the other arrays;
 * too small or NULL when needed -> QMM_ERR_INVALID_ARG, misaligned ->
 * QMM_ERR_MISALIGNED.  Two calls in flight need two workspaces.
 */
int64_t qmm_small_m_nt_workspace_bytes(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K);
int qmm_small_m_nt_ws(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K,
                      const void* x, const uint32_t* wq, const void* scales, const void* biases,
                      void* y, void* workspace, int64_t workspace_bytes, void* stream);

/* As qmm_small_m with the variant forced (measurement and tests): the
 * counterpart of timing qmm_nax forced against the stock dispatch in MLX
 * issue #4720, "Expected behavior".
 * QMM_ERR_UNSUPPORTED if the variant cannot run this shape
 * (QMM_KERNEL_MFMA_REG needs K <= 4096; for M = 17..64 it runs on 16-row
 * blocks and needs K to fill 16 wavefronts with whole k-blocks (above 1024
 * for 4-bit codes, above 512 for 6/8-bit) and N either to give more 4-bit
 * 16-column tiles than its row-block slots or at most one tile per resident
 * workgroup -- qmm_kernel_supported says which shapes; the TILE variants
 * need K to be a multiple of 128 for 4-bit codes, of 64 for 6- and 8-bit). */
int qmm_small_m_forced(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K,
                       const void* x, const uint32_t* wq, const void* scales,
                       const void* biases, void* y, void* stream, int kernel_id);

/*
 * K split across workgroups, for the shapes with few column tiles per CU
 * (the batched-decode down projection: N = 4096, K = 14336).  A split-free
 * kernel makes every CU read the whole activation matrix (M*K*2 bytes) for
 * its columns; with K split S ways a CU reads 1/S of it.  The partial
 * outputs (fp32, [S][M][N]) go to a caller-provided workspace and a second
 * kernel adds them in split order and rounds once, so results stay
 * deterministic.  This splits K the way MLX issue #4720 ("Describe the bug")
 * describes qmm_splitk; there it is the slow path on Apple parts, here it is
 * taken only where it measured faster.
 *
 * qmm_small_m_workspace_bytes: bytes qmm_small_m_ws needs for this problem
 * (0: it runs split-free, exactly as qmm_small_m), or a negative status.
 * Pure host logic.
 *
 * qmm_small_m_ws: as qmm_small_m, with `workspace` caller-owned device
 * memory of `workspace_bytes` >= qmm_small_m_workspace_bytes(...) bytes,
 * 16-byte aligned (may be NULL when that is 0).  The workspace is
 * overwritten by the call and must not alias x, wq, scales, biases or y;
 * two calls in flight at once need two workspaces.  Too small or NULL when
 * needed -> QMM_ERR_INVALID_ARG; misaligned -> QMM_ERR_MISALIGNED.  Nothing
 * is allocated.
 *
 * qmm_small_m_split_forced: the same with the variant and split forced
 * (measurement and tests).  split >= 1.  split > 1 with a TILE variant is
 * reduced to the largest count that gives every split part of K; with
 * QMM_KERNEL_MFMA_REG (4-bit; above 16 rows on 16-row blocks) K must be
 * exactly `split` slices of a depth that variant covers split-free
 * (K/split in {2048, 4096} with group sizes whose scale rows split evenly),
 * with more 16-column tiles than 256 / (split x row blocks), else
 * QMM_ERR_UNSUPPORTED -- that is how it runs K it cannot take whole.  The
 * workspace must hold that many [M][N] fp32 outputs.
 *
 * qmm_split_plan: the variant and split qmm_small_m_ws uses.  Pure host
 * logic.
 */
int64_t qmm_small_m_workspace_bytes(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K);
int qmm_small_m_ws(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K,
                   const void* x, const uint32_t* wq, const void* scales,
                   const void* biases, void* y, void* workspace, int64_t workspace_bytes, void* stream);
int qmm_small_m_split_forced(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K,
                             const void* x, const uint32_t* wq, const void* scales,
                             const void* biases, void* y, void* workspace, int64_t workspace_bytes,
                             void* stream, int kernel_id, int split);
int qmm_split_plan(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K,
                   int* kernel_id, int* split);

/*
 * For callers that cannot allocate device memory (code under HIP stream or
 * graph capture, serving loops and harnesses that forbid hipMalloc):
 * exactly qmm_small_m_ws -- the same plan, kernels and results -- with the
 * workspace in a library-owned static device array of
 * QMM_NOALLOC_SCRATCH_BYTES per GPU instead of a caller buffer.  Nothing is
 * allocated by the call (the array is part of the loaded library; each GPU
 * the library runs on holds its own copy until the process ends; its
 * address is looked up once per device, at the first call on it).
 *   - A problem whose planned workspace (qmm_small_m_workspace_bytes)
 *     exceeds QMM_NOALLOC_SCRATCH_BYTES -> QMM_ERR_UNSUPPORTED, checked
 *     before any HIP call; use qmm_small_m_ws with a caller buffer there.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's partial sums: calls that overlap on one GPU (two streams, two
 *     threads) race and must be ordered by the caller.  Sequential calls
 *     need no clearing (each split overwrites the partials it reads).
 * Otherwise as qmm_small_m.
 */
#define QMM_NOALLOC_SCRATCH_BYTES (8 * 1024 * 1024)
int qmm_small_m_noalloc(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K,
                        const void* x, const uint32_t* wq, const void* scales,
                        const void* biases, void* y, void* stream);

/* The variant qmm_small_m runs for this problem (a qmm_kernel value), or a
 * negative status if the problem is not supported.  Pure host logic.  The
 * selection is a table of measured crossovers over (dt, bits, group size, M,
 * N, K): MLX issue #4720 shows a dispatch keyed on M and N (its qmv cutoff
 * and split_k rule, "Describe the bug") misrouting shapes whose crossover
 * lies elsewhere ("Expected behavior": near M = 6-8 on 4096-class shapes). */
int qmm_select_kernel(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K);

/* 1 if variant `kernel_id` can run this problem, 0 if it cannot, or a
 * negative status if the problem itself is invalid or unsupported.  Pure
 * host logic. */
int qmm_kernel_supported(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K, int kernel_id);

/* uint32 words per packed row: K*bits/32 (-1 for unsupported bits or a K
 * that does not fill whole words). */
int64_t qmm_packed_words(int bits, int64_t K);

/* Hex digest (SHA-256, first 16 digits) of the source files this library
 * was built from, or "unknown" for a build that did not record it; callers
 * compare it with the sources they ship to detect a stale binary. */
const char* qmm_build_digest(void);

/* Static description of a status code. */
const char* qmm_strerror(int status);

/* Static name of a kernel variant ("?" if unknown). */
const char* qmm_kernel_name(int kernel_id);

/*
 * Measurement helpers (not part of the matmul path).
 *
 * qmm_probe_stream_read: read `bytes` (a multiple of 16) from device memory
 * `src` with coalesced 16-byte nontemporal loads and discard the data, in
 * one of two shapes: `shape` 0, a grid-stride loop over `grid` workgroups of
 * 256 threads (0 = 2048), four loads in flight per thread; `shape` 1, each
 * wavefront reading whole 8 KiB chunks (8 loads of 1 KiB in flight) in
 * `grid` workgroups of 1024 threads (0 = 512).  Never more workgroups than
 * the data needs; another shape -> QMM_ERR_INVALID_ARG.
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
int qmm_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int grid, int shape, void* stream);
int qmm_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);

/*
 * qmm_probe_small_m_loop: `passes` times over `count` weight sets, one
 * qmm_small_m call each (x, y and the formats shared), issued back to back
 * from this C loop on `stream`: the stream-launched rate of the matmul with
 * no interpreter between the calls.  `wq`, `scales`, `biases` are HOST
 * arrays of `count` device pointers (caller-owned, read during the call
 * only).  Stops at the first call that fails and returns its status;
 * count < 0, passes < 0 or a NULL pointer array -> QMM_ERR_INVALID_ARG;
 * count or passes 0 -> QMM_OK with nothing launched.
 */
int qmm_probe_small_m_loop(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K, const void* x,
                           const uint32_t* const* wq, const void* const* scales, const void* const* biases, void* y,
                           int count, int passes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
