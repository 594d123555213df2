// Kernel selection for qmm_small_m.
#include "qmm.h"
#include "qmm_dispatch.hpp"

namespace qmm {

bool kernel_supports(int kid, int /*dt*/, int /*bits*/, int /*gs*/, int64_t M, int64_t /*N*/, int64_t /*K*/) {
    switch (kid) {
        case QMM_KERNEL_VALU: return M <= 64;
        default: return false;
    }
}

int select_kernel(int /*dt*/, int /*bits*/, int /*gs*/, int64_t /*M*/, int64_t /*N*/, int64_t /*K*/) {
    return QMM_KERNEL_VALU;
}

hipError_t launch_kernel(int kid, const MatmulArgs& a) {
    switch (kid) {
        case QMM_KERNEL_VALU: return launch_valu(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
