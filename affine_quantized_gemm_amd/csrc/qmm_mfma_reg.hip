// Host side of the split-free register kernel (qmm_mfma_reg.hpp): which
// shapes it takes, and the launch dispatched over activation dtype and code
// width to the per-format translation units.
#include "qmm_mfma_reg.hpp"

namespace qmm {

bool mfma_reg_supports(int bits, int gs, int64_t M, int64_t N, int64_t K) {
    RegShape s;
    if (M > 16) return reg_rows_shape(bits, gs, M, N, K, s) || reg_rows1_shape(bits, gs, M, N, K, s);
    return pick_shape(bits, gs, K, s);
}

bool mfma_reg_single_tile_rows(int bits, int gs, int64_t M, int64_t N, int64_t K) {
    RegShape s;
    return reg_rows1_shape(bits, gs, M, N, K, s);
}

bool mfma_reg_split_supports(int bits, int gs, int64_t M, int64_t N, int64_t K, int split) {
    RegShape s;
    return reg_split_shape(bits, gs, M, N, K, split, s);
}

hipError_t launch_mfma_reg(const MatmulArgs& a) {
    switch (a.dt * 10 + a.bits) {
        case 4: return launch_mfma_reg_f16_4(a);
        case 6: return launch_mfma_reg_f16_6(a);
        case 8: return launch_mfma_reg_f16_8(a);
        case 14: return launch_mfma_reg_bf16_4(a);
        case 16: return launch_mfma_reg_bf16_6(a);
        case 18: return launch_mfma_reg_bf16_8(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
