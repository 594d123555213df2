// Tile-kernel launcher for bf16 activations and 8-bit codes (all group sizes).
#include "qmm_mfma_tile.hpp"

namespace qmm {
QMM_TILE_FMT_LAUNCHER(launch_mfma_tile_bf16_8, DT_BF16, 8)
}  // namespace qmm
