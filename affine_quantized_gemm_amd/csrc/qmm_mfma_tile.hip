// Host side of the shared-activation tile kernels (qmm_mfma_tile.hpp): which
// shapes they take, the split-count rule, the second kernel of every K split,
// and the launch dispatched to the per-format translation units.
#include "qmm_mfma_tile.hpp"

namespace qmm {

namespace {

// y = the split partial outputs added in split order (deterministic), then
// rounded once to dt.  part is [S][M*N] fp32.  A thread takes 4 consecutive
// outputs (16-byte loads) and keeps 16 slices' loads in flight before adding
// them in order: one slice at a time, each add waited for its load, made a
// 16-way split a chain of 16 round trips (8 in flight: two).  One wavefront
// per workgroup, so that a few thousand outputs still spread over many CUs.
template <int DT>
__global__ __launch_bounds__(64) void reduce_partials_kernel(const float* __restrict__ part,
                                                             uint16_t* __restrict__ y, int S, int64_t mn) {
    typedef float f4_t __attribute__((ext_vector_type(4)));
    const int64_t i = (static_cast<int64_t>(blockIdx.x) * 64 + threadIdx.x) * 4;
    if (i >= mn) return;
    if (i + 4 <= mn && mn % 4 == 0) {
        f4_t v = *reinterpret_cast<const f4_t*>(part + i);
        for (int s = 1; s < S; s += 16) {
            f4_t t[16];
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (s + j < S) t[j] = *reinterpret_cast<const f4_t*>(part + static_cast<int64_t>(s + j) * mn + i);
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (s + j < S) v += t[j];
        }
        uint32_t lo = DtOps<DT>::rne(v[0]) | (static_cast<uint32_t>(DtOps<DT>::rne(v[1])) << 16);
        uint32_t hi = DtOps<DT>::rne(v[2]) | (static_cast<uint32_t>(DtOps<DT>::rne(v[3])) << 16);
        *reinterpret_cast<uint2*>(y + i) = make_uint2(lo, hi);
        return;
    }
    for (int64_t e = i; e < i + 4 && e < mn; ++e) {
        float v = part[e];
        for (int s = 1; s < S; ++s) v += part[static_cast<int64_t>(s) * mn + e];
        y[e] = DtOps<DT>::rne(v);
    }
}

}  // namespace

hipError_t launch_reduce_partials(int dt, const float* part, void* y, int split, int64_t mn, hipStream_t st) {
    if (mn <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((mn + 255) / 256));  // 64 threads of 4 outputs
    if (dt == 0)
        hipLaunchKernelGGL((reduce_partials_kernel<0>), grid, dim3(64), 0, st, part, static_cast<uint16_t*>(y), split, mn);
    else
        hipLaunchKernelGGL((reduce_partials_kernel<1>), grid, dim3(64), 0, st, part, static_cast<uint16_t*>(y), split, mn);
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
