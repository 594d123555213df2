// Register-kernel launcher for fp16 activations and 8-bit codes (all group sizes).
#include "qmm_mfma_reg.hpp"

namespace qmm {
QMM_REG_FMT_LAUNCHER(launch_mfma_reg_f16_8, DT_F16, 8)
}  // namespace qmm
