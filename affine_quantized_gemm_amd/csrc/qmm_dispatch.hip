// Kernel selection for qmm_small_m.
#include "qmm.h"
#include "qmm_dispatch.hpp"

namespace qmm {

bool kernel_supports(int kid, int /*dt*/, int bits, int gs, int64_t M, int64_t N, int64_t K) {
    switch (kid) {
        case QMM_KERNEL_VALU: return M <= 64;
        case QMM_KERNEL_MFMA_REG: return mfma_reg_supports(bits, gs, M, N, K);
        case QMM_KERNEL_MFMA_PASS: return M <= 64;
        case QMM_KERNEL_MFMA_TILE16: return mfma_tile_supports(bits, M, K, TILE_CFG_16);
        case QMM_KERNEL_MFMA_TILE64: return mfma_tile_supports(bits, M, K, TILE_CFG_64);
        case QMM_KERNEL_MFMA_DQLDS: return mfma_dqlds_supports(bits, M, N, K);
        default: return false;
    }
}

// Crossovers measured on MI355X (graph-replayed calls over a weight stack
// larger than the Infinity Cache; affine_quantized_gemm_amd/sweep.py):
//   * M <= 16: the register-resident MFMA kernel wherever it can run
//     (K <= 4096): 5.0 us vs 7.4 us (pass) vs 14.2 us (VALU) at M = 6,
//     K = N = 4096, 4-bit; the pass kernel for longer K (18.4 us vs 25.2 us
//     for the 16-column tile kernel at M = 8 on the 4096 x 14336 down
//     projection);
//   * M 17..64, 4-bit, K <= 4096, more 16-column tiles than the row-block
//     grid's column slots: the register kernel on row blocks (one 16-row
//     block per workgroup layer, weights shared through the XCD's L2):
//     15.3 / 16.1 / 23.7 us vs 24.1 / 24.3 / 34.1 us (64-column tiles) at
//     M = 24 / 32 / 64 on the 14336 x 4096 gate/up projection, 9.5 / 11.3 /
//     11.9 us vs 12.9 (pass) / 16.0 / 20.6 (16-column tiles) at M = 24 / 36 /
//     64, K = N = 4096, 99 / 188 us vs 190 / 287 us on the LM head;
//   * M 17..64 where 16 rows take one tile per workgroup (N up to 4096 at
//     K <= 4096, any width): the register kernel on a grid of tiles x 16-row
//     blocks: 5.6 / 6.0 us vs 7.9 / 8.1 us (pass) at M = 24 / 64 on the
//     1024 x 4096 k/v projection; 8-bit K = N = 4096: 12.0 / 16.5 / 21.6 us
//     vs 17.3 / 19.9 / 27.9 us (16-column tiles) at M = 24 / 36 / 64, 6-bit
//     gs128 11.8 / 16.6 / 22.5 us vs 17.2 (pass) / 20.0 / 29.0 us;
//     Except 6/8-bit at group size 32 above 48 rows (N = 4096): there the
//     register kernel's 8 units per wavefront make the 16-column tile
//     kernel faster (22.8-23.8 us vs 24.3-25.6 us at M = 64, all four
//     formats; sweep.py --formats);
//   * otherwise (6/8-bit with more tiles than resident workgroups), M > 16,
//     wide N (>= 8192): for fp16 the weights dequantized into LDS (packed
//     fp16 dequantization, one pass per workgroup): 28.1-40.5 us vs
//     34.9-51.5 us for the 64-column tile kernel at M = 24 / 36 / 64 on
//     14336 x 4096, every fp16 6/8-bit format (sweep.py --formats); for bf16
//     (two matrix steps per weight, hi and lo) the 64-column tile kernel:
//     24.1 / 33.2 us vs 37.6 / 66.6 us (pass) at M = 24 / 64 on the
//     14336 x 4096 gate/up projection, 186 / 278 us vs 368 / 669 us on the
//     151936-column LM head;
//   * M > 32, N from 4096 (at least one 16-column tile per CU): the
//     16-column tile kernel: 46.0 / 64.7 us vs 56.1 / 65.5 us (pass) at
//     M = 36 / 64 on the down projection; with fewer tiles than CUs it idles
//     most of the chip (15.7 us vs 7.8 us for the pass kernel at M = 36,
//     N = 1024);
//   * everything else (M = 17..32 with N < 8192, or K the tile kernels do not
//     take): the pass kernel (37.3 us vs 47.7 us for the 16-column tiles at
//     M = 32 on the down projection);
//   * the VALU kernel is not selected (kept as an independent variant for
//     measurement and cross-checks).
// The pages' own dispatch is likewise a measured crossover in M per shape
// (MLX issue #4720: the dispatch rules under "Describe the bug", the
// crossover near M = 6-8 on Apple parts under "Expected behavior").
int select_kernel(int dt, int bits, int gs, int64_t M, int64_t N, int64_t K) {
    if (bits != 4 && gs == 32 && M > 48 && N >= 4096 && mfma_reg_single_tile_rows(bits, gs, M, N, K) &&
        kernel_supports(QMM_KERNEL_MFMA_TILE16, dt, bits, gs, M, N, K))
        return QMM_KERNEL_MFMA_TILE16;
    if (kernel_supports(QMM_KERNEL_MFMA_REG, dt, bits, gs, M, N, K)) return QMM_KERNEL_MFMA_REG;
    if (M <= 16) return QMM_KERNEL_MFMA_PASS;
    if (dt == QMM_F16 && bits != 4 && N >= 8192 && kernel_supports(QMM_KERNEL_MFMA_DQLDS, dt, bits, gs, M, N, K))
        return QMM_KERNEL_MFMA_DQLDS;
    if (kernel_supports(QMM_KERNEL_MFMA_TILE64, dt, bits, gs, M, N, K)) {
        if (N >= 8192) return QMM_KERNEL_MFMA_TILE64;
        if (M > 32 && N >= 4096) return QMM_KERNEL_MFMA_TILE16;
    }
    return QMM_KERNEL_MFMA_PASS;
}

// K split (workspace entry point).  Measured on MI355X (sweep.py --splits,
// graph-replayed): the 64-column tile kernel with K split 4 ways beats the
// other split-free variants from M = 24 when N gives 32..64 tiles of 64
// columns (down projection, 6/8-bit: it is the only split there); below
// that, with fewer than 32 such tiles (k/v, N = 1024: 14.5 vs 4.9 us at
// M = 8) or with 8 splits the partial-sum pass costs more than the
// activation bytes it saves.  So: split when N gives 32..64 tiles of 64
// columns and M >= 24, into min(4, 256 / tiles) parts.
//
// Where the register kernel runs split-free it is faster than any split
// (4-bit with K <= 4096; 6/8-bit K = N = 4096 at M = 24 / 36: 12.0 / 16.5 us
// vs 15.9 / 17.7 us split, 8-bit), except its single-tile row blocks above
// 48 rows (4 blocks, 4 workgroups per tile): there the split wins where it
// applies (6/8-bit K = N = 4096 at M = 64: 21.1 / 19.5 us vs 22.5 / 21.6 us;
// at M = 48 the row blocks still win, 17.2 vs 18.1 us at 8-bit).
//
// Before those: K the register kernel cannot take whole (the down
// projection, K = 14336): that kernel on K / S slices, the fewest that work
// (7 slices of 2048 at K = 14336), on 16-row blocks above 16 rows: 13.7 /
// 15.0 / 16.1 us vs 16.1 / 18.3 / 22.5 us for the split-free pass kernel at
// M = 1 / 8 / 16, and 21.0 / 20.4 / 26.3 / 31.7 us vs 27.0 / 27.0 / 32.3 /
// 36.6 us for the 64-column tile kernel split 4 ways at M = 24 / 32 / 48 /
// 64.
SplitPlan plan_split(int dt, int bits, int gs, int64_t M, int64_t N, int64_t K) {
    SplitPlan p{select_kernel(dt, bits, gs, M, N, K), 1};
    if (M < 1 || N < 1) return p;  // empty problem: nothing to split
    if (p.kernel == QMM_KERNEL_MFMA_REG && !(M > 48 && mfma_reg_single_tile_rows(bits, gs, M, N, K)))
        return p;  // faster than any split measured
    if (!mfma_reg_supports(bits, gs, 1, N, K))  // K deeper than the register kernel takes whole
        for (int s = 2; s <= 8; ++s)
            if (mfma_reg_split_supports(bits, gs, M, N, K, s)) return SplitPlan{QMM_KERNEL_MFMA_REG, s};
    if (!kernel_supports(QMM_KERNEL_MFMA_TILE64, dt, bits, gs, M, N, K)) return p;
    const int64_t ntiles = (N + 63) / 64;
    if (ntiles < 32 || ntiles > 64) return p;
    if (M < 24) return p;
    const int64_t want = 256 / ntiles < 4 ? 256 / ntiles : 4;
    const int split = tile_split(bits, K, TILE_CFG_64, static_cast<int>(want));
    if (split < 2) return p;
    return SplitPlan{QMM_KERNEL_MFMA_TILE64, split};
}

hipError_t launch_kernel(int kid, const MatmulArgs& a) {
    switch (kid) {
        case QMM_KERNEL_VALU: return launch_valu(a);
        case QMM_KERNEL_MFMA_REG: return launch_mfma_reg(a);
        case QMM_KERNEL_MFMA_PASS: return launch_mfma_pass(a);
        case QMM_KERNEL_MFMA_TILE16: return launch_mfma_tile(a, TILE_CFG_16);
        case QMM_KERNEL_MFMA_TILE64: return launch_mfma_tile(a, TILE_CFG_64);
        case QMM_KERNEL_MFMA_DQLDS: return launch_mfma_dqlds(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
