// Kernel selection for qmm_small_m.
#include "qmm.h"
#include "qmm_dispatch.hpp"

namespace qmm {

bool kernel_supports(int kid, int /*dt*/, int bits, int gs, int64_t M, int64_t /*N*/, int64_t K) {
    switch (kid) {
        case QMM_KERNEL_VALU: return M <= 64;
        case QMM_KERNEL_MFMA_REG: return mfma_reg_supports(bits, gs, M, K);
        case QMM_KERNEL_MFMA_PASS: return M <= 64;
        default: return false;
    }
}

// Crossovers measured on MI355X (graph-replayed calls over a weight stack
// larger than the Infinity Cache; affine_quantized_gemm_amd/sweep.py):
//   * the register-resident MFMA kernel is fastest wherever it can run
//     (M <= 16, K <= 4096): e.g. 5.0 us vs 7.3 us (pass kernel) vs 14.2 us
//     (VALU) at M = 6, K = N = 4096, 4-bit; 7.3 us vs 9.2 us (VALU) at M = 1,
//     8-bit;
//   * the pass kernel everywhere else: 15.3 us vs 18.9 us (VALU) at M = 1 on
//     the 14336-deep down projection, 84 us vs 294 us at M = 64;
//   * the VALU kernel is not selected (kept as an independent variant for
//     measurement and cross-checks).
// The pages' own dispatch is likewise a measured crossover in M per shape
// (MLX issue #4720, "Root cause"; crossover near M = 6-8 on Apple parts).
int select_kernel(int dt, int bits, int gs, int64_t M, int64_t N, int64_t K) {
    return kernel_supports(QMM_KERNEL_MFMA_REG, dt, bits, gs, M, N, K) ? QMM_KERNEL_MFMA_REG : QMM_KERNEL_MFMA_PASS;
}

hipError_t launch_kernel(int kid, const MatmulArgs& a) {
    switch (kid) {
        case QMM_KERNEL_VALU: return launch_valu(a);
        case QMM_KERNEL_MFMA_REG: return launch_mfma_reg(a);
        case QMM_KERNEL_MFMA_PASS: return launch_mfma_pass(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
