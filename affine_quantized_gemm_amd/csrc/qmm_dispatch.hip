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

int select_kernel(int dt, int bits, int gs, int64_t M, int64_t N, int64_t K) {
    if (kernel_supports(QMM_KERNEL_MFMA_REG, dt, bits, gs, M, N, K)) return QMM_KERNEL_MFMA_REG;
    return QMM_KERNEL_MFMA_PASS;
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
