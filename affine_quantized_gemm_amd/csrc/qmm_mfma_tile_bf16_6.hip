// Tile-kernel launcher for bf16 activations and 6-bit codes (all group sizes).
#include "qmm_mfma_tile.hpp"

namespace qmm {
QMM_TILE_FMT_LAUNCHER(launch_mfma_tile_bf16_6, DT_BF16, 6)
}  // namespace qmm
