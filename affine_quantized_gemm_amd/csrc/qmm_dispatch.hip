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
//     (M <= 16, K <= 4096) -- e.g. 6.9 us vs 14.4 us (VALU) at M = 6, K = N =
//     4096, 4-bit -- except for 8-bit codes at M <= 2 on shapes up to
//     4096 x 4096, where the VALU kernel's single pass over the bytes wins
//     (9.2 us vs 9.9 us);
//   * elsewhere the pass kernel, except M <= 2 (VALU: 19.4 us vs 22.3 us on
//     the 14336-deep down projection);
//   * the VALU kernel loses everywhere from M = 3 up (M = 64, 4096 x 14336:
//     294 us vs 103 us).
// The pages' own dispatch is likewise a measured crossover in M per shape
// (MLX issue #4720, "Root cause"; crossover near M = 6-8 on Apple parts).
int select_kernel(int dt, int bits, int gs, int64_t M, int64_t N, int64_t K) {
    const bool reg_ok = kernel_supports(QMM_KERNEL_MFMA_REG, dt, bits, gs, M, N, K);
    if (M <= 2) {
        if (!reg_ok) return QMM_KERNEL_VALU;
        if (bits == 8 && N * K <= int64_t(4096) * 4096) return QMM_KERNEL_VALU;
    }
    return reg_ok ? QMM_KERNEL_MFMA_REG : QMM_KERNEL_MFMA_PASS;
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
