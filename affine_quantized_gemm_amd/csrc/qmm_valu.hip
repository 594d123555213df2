// Split-free small-M kernel on the vector ALUs.
//
// Structure taken from the verify-kernel design in "How the NAX Verify Kernel
// Path Improves Decode Performance in MTPLX" ("Architectural Differences" and
// "How the NAX Verify Kernel Path Eliminates Bottlenecks"): each wavefront
// exclusively owns a tile of BN = 4 output columns, walks the whole K
// dimension with its lanes strided over K, and reduces across its own lanes;
// there is no K split and no barrier.  On gfx950 the wavefront is 64 lanes
// and the final reduction is a butterfly over lane exchanges.
//
// Arithmetic is group-factored and exact up to fp32 rounding:
//   y[m,n] = sum_g ( s[n,g] * sum_{k in g} x[m,k] * q[n,k]  +  b[n,g] * sum_{k in g} x[m,k] )
// Each lane handles whole 32-code chunks (a chunk lies inside one group
// because group sizes are multiples of 32), so the scale/bias step is one
// fma per (row, column, chunk).
#include "qmm_device.hpp"
#include "qmm_internal.hpp"

namespace qmm {

namespace {

constexpr int kValuBN = 4;        // columns per wavefront
constexpr int kValuWaves = 4;     // wavefronts per workgroup

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// MB = rows per pass (accumulator block); passes cover all M rows.
template <int DT, int BITS, int GS, int MB>
__global__ __launch_bounds__(64 * kValuWaves) void valu_kernel(const uint16_t* __restrict__ x,
                                                               const uint32_t* __restrict__ wq,
                                                               const uint16_t* __restrict__ scales,
                                                               const uint16_t* __restrict__ biases,
                                                               uint16_t* __restrict__ y,
                                                               int M, int64_t N, int64_t K) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t n0 = (static_cast<int64_t>(blockIdx.x) * kValuWaves + wave) * kValuBN;
    if (n0 >= N) return;
    const int64_t chunks = K / 32;
    const int64_t row_words = K * BITS / 32;
    const int64_t G = K / GS;

    for (int m0 = 0; m0 < M; m0 += MB) {
        const int mrows = min(MB, M - m0);
        float acc[MB][kValuBN];
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int c = 0; c < kValuBN; ++c) acc[m][c] = 0.0f;

        for (int64_t ch = lane; ch < chunks; ch += 64) {
            // packed words, scale and bias of this chunk for each owned column
            uint32_t w[kValuBN][BITS];
            float s[kValuBN], b[kValuBN];
#pragma unroll
            for (int c = 0; c < kValuBN; ++c) {
                const int64_t n = min(n0 + c, N - 1);  // tail columns recompute the last one
                load_chunk_words<BITS>(wq + n * row_words + ch * BITS, w[c]);
                const int64_t gi = n * G + (ch * 32) / GS;
                s[c] = DtOps<DT>::to_f32(scales[gi]);
                b[c] = DtOps<DT>::to_f32(biases[gi]);
            }
            float p[MB][kValuBN];
            float xs[MB];
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                xs[m] = 0.0f;
#pragma unroll
                for (int c = 0; c < kValuBN; ++c) p[m][c] = 0.0f;
            }
#pragma unroll
            for (int sub = 0; sub < 4; ++sub) {  // 8 codes at a time
                float xv[MB][8];
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    uint4 u = make_uint4(0u, 0u, 0u, 0u);
                    if (m < mrows)
                        u = *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(m0 + m) * K + ch * 32 + sub * 8);
                    const uint32_t pr[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        xv[m][2 * j] = DtOps<DT>::to_f32(static_cast<uint16_t>(pr[j] & 0xFFFFu));
                        xv[m][2 * j + 1] = DtOps<DT>::to_f32(static_cast<uint16_t>(pr[j] >> 16));
                    }
#pragma unroll
                    for (int t = 0; t < 8; ++t) xs[m] += xv[m][t];
                }
#pragma unroll
                for (int c = 0; c < kValuBN; ++c) {
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const float q = static_cast<float>(chunk_code<BITS>(w[c], sub * 8 + t));
#pragma unroll
                        for (int m = 0; m < MB; ++m) p[m][c] = fmaf(xv[m][t], q, p[m][c]);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int c = 0; c < kValuBN; ++c) acc[m][c] = fmaf(s[c], p[m][c], fmaf(b[c], xs[m], acc[m][c]));
        }

#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int c = 0; c < kValuBN; ++c) acc[m][c] = wave_sum(acc[m][c]);

        if (lane == 0) {
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                if (m >= mrows) break;
#pragma unroll
                for (int c = 0; c < kValuBN; ++c)
                    if (n0 + c < N) y[static_cast<int64_t>(m0 + m) * N + n0 + c] = DtOps<DT>::rne(acc[m][c]);
            }
        }
    }
}

template <int DT, int BITS, int GS>
hipError_t launch_valu_t(const MatmulArgs& a) {
    const int64_t cols_per_block = kValuWaves * kValuBN;
    const int64_t grid = (a.N + cols_per_block - 1) / cols_per_block;
    const auto* x = static_cast<const uint16_t*>(a.x);
    const auto* s = static_cast<const uint16_t*>(a.scales);
    const auto* b = static_cast<const uint16_t*>(a.biases);
    auto* y = static_cast<uint16_t*>(a.y);
    const int M = static_cast<int>(a.M);
    if (M <= 2)
        hipLaunchKernelGGL((valu_kernel<DT, BITS, GS, 2>), dim3(grid), dim3(64 * kValuWaves), 0, a.stream, x, a.wq,
                           s, b, y, M, a.N, a.K);
    else if (M <= 4)
        hipLaunchKernelGGL((valu_kernel<DT, BITS, GS, 4>), dim3(grid), dim3(64 * kValuWaves), 0, a.stream, x, a.wq,
                           s, b, y, M, a.N, a.K);
    else if (M <= 6)
        hipLaunchKernelGGL((valu_kernel<DT, BITS, GS, 6>), dim3(grid), dim3(64 * kValuWaves), 0, a.stream, x, a.wq,
                           s, b, y, M, a.N, a.K);
    else
        hipLaunchKernelGGL((valu_kernel<DT, BITS, GS, 8>), dim3(grid), dim3(64 * kValuWaves), 0, a.stream, x, a.wq,
                           s, b, y, M, a.N, a.K);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_valu(const MatmulArgs& a) {
#define VCALL(D, B, G) launch_valu_t<D, B, G>(a)
    switch (a.dt * 100 + a.bits * 10 + a.gs / 32) {
        case 41: return VCALL(0, 4, 32);   case 42: return VCALL(0, 4, 64);   case 44: return VCALL(0, 4, 128);
        case 61: return VCALL(0, 6, 32);   case 62: return VCALL(0, 6, 64);   case 64: return VCALL(0, 6, 128);
        case 81: return VCALL(0, 8, 32);   case 82: return VCALL(0, 8, 64);   case 84: return VCALL(0, 8, 128);
        case 141: return VCALL(1, 4, 32);  case 142: return VCALL(1, 4, 64);  case 144: return VCALL(1, 4, 128);
        case 161: return VCALL(1, 6, 32);  case 162: return VCALL(1, 6, 64);  case 164: return VCALL(1, 6, 128);
        case 181: return VCALL(1, 8, 32);  case 182: return VCALL(1, 8, 64);  case 184: return VCALL(1, 8, 128);
        default: return hipErrorInvalidValue;
    }
#undef VCALL
}

}  // namespace qmm
