// Tile-kernel launcher for bf16 activations and 4-bit codes (all group sizes).
#include "qmm_mfma_tile.hpp"

namespace qmm {
QMM_TILE_FMT_LAUNCHER(launch_mfma_tile_bf16_4, DT_BF16, 4)
}  // namespace qmm
