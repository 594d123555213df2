// Register-kernel launcher for bf16 activations and 8-bit codes (all group sizes).
#include "qmm_mfma_reg.hpp"

namespace qmm {
QMM_REG_FMT_LAUNCHER(launch_mfma_reg_bf16_8, DT_BF16, 8)
}  // namespace qmm
