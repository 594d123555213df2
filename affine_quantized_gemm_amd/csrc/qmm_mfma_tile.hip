// Host side of the shared-activation tile kernels (qmm_mfma_tile.hpp): which
// shapes they take, the split-count rule, the second kernel of every K split,
// and the launch dispatched to the per-format translation units.
#include "qmm_mfma_tile.hpp"

namespace qmm {

namespace {

// y = the split partial outputs added in split order (deterministic), then
// rounded once to dt.  part is [S][M*N] fp32.
template <int DT>
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float* __restrict__ part,
                                                              uint16_t* __restrict__ y, int S, int64_t mn) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= mn) return;
    float v = part[i];
    for (int s = 1; s < S; ++s) v += part[static_cast<int64_t>(s) * mn + i];
    y[i] = DtOps<DT>::rne(v);
}

}  // namespace

hipError_t launch_reduce_partials(int dt, const float* part, void* y, int split, int64_t mn, hipStream_t st) {
    if (mn <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((mn + 255) / 256));
    if (dt == 0)
        hipLaunchKernelGGL((reduce_partials_kernel<0>), grid, dim3(256), 0, st, part, static_cast<uint16_t*>(y), split, mn);
    else
        hipLaunchKernelGGL((reduce_partials_kernel<1>), grid, dim3(256), 0, st, part, static_cast<uint16_t*>(y), split, mn);
    return hipGetLastError();
}

int tile_split(int bits, int64_t K, int cfg, int split) {
    const int64_t kblk = bits == 4 ? 128 : 64;
    const int64_t kw = cfg == TILE_CFG_16 ? 4 : 2;  // k-blocks per pass (launch_tile_t)
    const int64_t P = (K / kblk + kw - 1) / kw;
    int64_t S = split < 1 ? 1 : split;
    if (S > P) S = P;
    const int64_t PP = (P + S - 1) / S;
    return static_cast<int>((P + PP - 1) / PP);
}

bool mfma_tile_supports(int bits, int64_t M, int64_t K, int /*cfg*/) {
    const int64_t kblk = bits == 4 ? 128 : 64;
    // (K <= 2^24 keeps every activation byte offset within 32 bits)
    return M >= 1 && M <= 16 * TILE_RBM && K % kblk == 0 && K <= (int64_t{1} << 24);
}

hipError_t launch_mfma_tile(const MatmulArgs& a, int cfg) {
    switch (a.dt * 10 + a.bits) {
        case 4: return launch_mfma_tile_f16_4(a, cfg);
        case 6: return launch_mfma_tile_f16_6(a, cfg);
        case 8: return launch_mfma_tile_f16_8(a, cfg);
        case 14: return launch_mfma_tile_bf16_4(a, cfg);
        case 16: return launch_mfma_tile_bf16_6(a, cfg);
        case 18: return launch_mfma_tile_bf16_8(a, cfg);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
