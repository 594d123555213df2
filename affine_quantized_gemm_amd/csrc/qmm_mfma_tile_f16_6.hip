// Tile-kernel launcher for fp16 activations and 6-bit codes (all group sizes).
#include "qmm_mfma_tile.hpp"

namespace qmm {
QMM_TILE_FMT_LAUNCHER(launch_mfma_tile_f16_6, DT_F16, 6)
}  // namespace qmm
