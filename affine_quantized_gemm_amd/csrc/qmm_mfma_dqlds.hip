// Split-free small-M kernel with the weights dequantized into LDS and fed to
// the matrix cores from there (M <= 64): the "dequantize to shared memory,
// then matrix-unit contraction" form of the M >= 16 path.
//
// Design source: MLX issue #4720 ("Describe the bug", "Expected behavior"):
// above a handful of rows the matrix-unit kernel (qmm_nax) is the path to
// beat, and a split-K dispatch of the same product halves its bandwidth.  On
// Apple GPUs that kernel stages dequantized weight tiles in threadgroup
// memory; this is that arrangement written for gfx950, kept beside the
// in-register forms (mfma_splitfree_pass / tile16 / tile64, which build
// the weight operand in registers) so that the two can be timed against
// each other on the same shapes.  It is a measured alternative, not a
// dispatch choice: the selection takes it nowhere (its sweep rows say why).
//
// Workgroup: 4 wavefronts own a tile of 64 output columns for every row of
// M (16-row blocks 0..RB-1) and walk K in chunks of KC values (256 at 4 bits,
// so that a column's chunk is one 128-byte line; 128 at 6 and 8 bits).  Per
// chunk:
//   * every thread dequantizes whole 32-code runs of one column (4 threads
//     per column, one or two runs each): w = s q + b in fp32, rounded once to
//     fp16 (error far inside the accepted bound), or for bf16 split into
//     hi = RNE(w) and lo = RNE(w - hi) (bf16's 8-bit significand would spend
//     most of the bound on one rounding), and writes them to the LDS tile
//     W[column][k];
//   * the activation rows of the chunk go to LDS beside it (rows past M stay
//     zero);
//   * after one barrier wavefront w reads the B operand of its 16 columns
//     (8 consecutive k of one column per lane: one 16-byte LDS read) and the
//     A operand of each row block (8 consecutive k of one row) in natural
//     order, and accumulates v_mfma_f32_16x16x32 steps in fp32 (two per step
//     for bf16: hi and lo).
// The next chunk's code words, scales, biases and activations are loaded into
// registers while the current chunk is computed (after the last chunk, the
// last one again: the same loads on every path).  Each weight is dequantized
// once per workgroup; the B operand crosses LDS once (its column owner reads
// it), the activations once per wavefront.
#include "qmm_device.hpp"
#include "qmm_internal.hpp"
#include "qmm_mfma_frag.hpp"

namespace qmm {

namespace {

using namespace mf;

constexpr int DQ_TN = 64;        // columns per workgroup
constexpr int DQ_THREADS = 256;  // 4 wavefronts, 16 columns each

template <int BITS>
struct DqFmt {
    static constexpr int KC = BITS == 4 ? 256 : 128;   // k values per chunk
    static constexpr int RUNS = KC / 32 / 4;            // 32-code runs per thread (4 threads per column)
    static constexpr int WS = KC + 8;                   // LDS row stride of W and x (16 bytes of padding)
};

template <int DT, int BITS, int RB>
__global__ __launch_bounds__(DQ_THREADS) void mfma_dqlds_kernel(const uint16_t* __restrict__ x,
                                                             const uint32_t* __restrict__ wq,
                                                             const uint16_t* __restrict__ scales,
                                                             const uint16_t* __restrict__ biases,
                                                             uint16_t* __restrict__ y, int M, int64_t N,
                                                             int64_t K, int gs) {
    using F = DqFmt<BITS>;
    constexpr int KC = F::KC, RUNS = F::RUNS, WS = F::WS;
    constexpr int NH = DT == DT_BF16 ? 2 : 1;          // bf16: hi and lo tiles
    constexpr int XP = (16 * RB * KC / 8 + DQ_THREADS - 1) / DQ_THREADS;  // 16-byte activation pieces per thread
    extern __shared__ __align__(16) uint16_t lds[];
    uint16_t* const w_lds = lds;                        // [NH][DQ_TN][WS]
    uint16_t* const x_lds = lds + NH * DQ_TN * WS;      // [16 RB][WS]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * DQ_TN;
    const int64_t G = K / gs;
    const int64_t row_words = K * BITS / 32;

    // activation rows M .. 16 RB - 1 stay zero
    for (int i = tid; i < (16 * RB - M) * WS; i += DQ_THREADS) x_lds[M * WS + i] = 0;

    // this thread's dequantization share: column c, runs r = q + 4 j
    const int c = tid >> 2, q = tid & 3;
    const uint32_t* const wrow = wq + (n0 + c) * row_words;

    typedef uint32_t v4u __attribute__((ext_vector_type(4)));  // (a native vector: stays in registers)
    struct Regs {
        uint32_t w[RUNS][BITS];
        uint16_t s[RUNS], b[RUNS];
        v4u xv[XP];
    };
    auto load = [&](int64_t k0, Regs& r) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < RUNS; ++j) {
            const int64_t kr = k0 + 32 * (q + 4 * j);      // first k of the run
            load_chunk_words<BITS>(wrow + kr * BITS / 32, r.w[j]);
            const int64_t gi = (n0 + c) * G + kr / gs;
            r.s[j] = scales[gi];
            r.b[j] = biases[gi];
        }
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            const int p = tid + DQ_THREADS * i;            // piece p: row p / (KC / 8), k 8 (p % (KC / 8))
            const int m = p / (KC / 8), kk = 8 * (p % (KC / 8));
            const int mm = m < M ? m : M - 1;              // (rows past M load a valid row, never staged)
            r.xv[i] = *reinterpret_cast<const v4u*>(x + static_cast<int64_t>(mm) * K + k0 + kk);
        }
    };
    auto stage = [&](const Regs& r) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < RUNS; ++j) {
            const float s = DtOps<DT>::to_f32(r.s[j]), b = DtOps<DT>::to_f32(r.b[j]);
            const int kl = 32 * (q + 4 * j);
#pragma unroll
            for (int e = 0; e < 32; e += 8) {
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float w0 = __fmaf_rn(s, static_cast<float>(chunk_code<BITS>(r.w[j], e + 2 * t)), b);
                    const float w1 = __fmaf_rn(s, static_cast<float>(chunk_code<BITS>(r.w[j], e + 2 * t + 1)), b);
                    const uint16_t h0 = DtOps<DT>::rne(w0), h1 = DtOps<DT>::rne(w1);
                    hi[t] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
                    if constexpr (NH == 2) {
                        const uint16_t l0 = DtOps<DT>::rne(w0 - DtOps<DT>::to_f32(h0));
                        const uint16_t l1 = DtOps<DT>::rne(w1 - DtOps<DT>::to_f32(h1));
                        lo[t] = static_cast<uint32_t>(l0) | (static_cast<uint32_t>(l1) << 16);
                    }
                }
                *reinterpret_cast<uint4*>(w_lds + c * WS + kl + e) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
                if constexpr (NH == 2)
                    *reinterpret_cast<uint4*>(w_lds + (DQ_TN + c) * WS + kl + e) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
            }
        }
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            const int p = tid + DQ_THREADS * i;
            const int m = p / (KC / 8), kk = 8 * (p % (KC / 8));
            if (m < M) *reinterpret_cast<v4u*>(x_lds + m * WS + kk) = r.xv[i];
        }
    };

    float4_t acc[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) acc[b] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int li = lane & 15, lq = lane >> 4;
    Regs regs;
    load(0, regs);
    for (int64_t k0 = 0; k0 < K; k0 += KC) {
        __syncthreads();  // the previous chunk's LDS reads are done
        stage(regs);
        __syncthreads();
        // the next chunk in flight during this chunk's steps (after the last
        // chunk the same loads again, never staged: registers loaded on one
        // path and not on another would be kept in scratch memory)
        load(k0 + KC < K ? k0 + KC : k0, regs);
#pragma unroll
        for (int st = 0; st < KC / 32; ++st) {
            const int kk = 32 * st + 8 * lq;
            Frag bh, bl;
            {
                const uint4 v = *reinterpret_cast<const uint4*>(w_lds + (16 * wave + li) * WS + kk);
                bh.v[0] = v.x; bh.v[1] = v.y; bh.v[2] = v.z; bh.v[3] = v.w;
            }
            if constexpr (NH == 2) {
                const uint4 v = *reinterpret_cast<const uint4*>(w_lds + (DQ_TN + 16 * wave + li) * WS + kk);
                bl.v[0] = v.x; bl.v[1] = v.y; bl.v[2] = v.z; bl.v[3] = v.w;
            }
#pragma unroll
            for (int b = 0; b < RB; ++b) {
                Frag a;
                const uint4 v = *reinterpret_cast<const uint4*>(x_lds + (16 * b + li) * WS + kk);
                a.v[0] = v.x; a.v[1] = v.y; a.v[2] = v.z; a.v[3] = v.w;
                acc[b] = mfma<DT>(a, bh, acc[b]);
                if constexpr (NH == 2) acc[b] = mfma<DT>(a, bl, acc[b]);
            }
        }
    }
    // D[4 lq + r][li] of row block b: output row 16 b + 4 lq + r, column
    // n0 + 16 wave + li
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 16 * b + 4 * lq + r;
            if (m < M) y[static_cast<int64_t>(m) * N + n0 + 16 * wave + li] = DtOps<DT>::rne(acc[b][r]);
        }
}

template <int DT, int BITS, int RB>
hipError_t launch_dqlds_t(const MatmulArgs& a) {
    using F = DqFmt<BITS>;
    constexpr int NH = DT == DT_BF16 ? 2 : 1;
    constexpr size_t lds = static_cast<size_t>(NH * DQ_TN + 16 * RB) * F::WS * sizeof(uint16_t);
    if (lds > 65536) {
        static std::atomic<uint64_t> raised{0};
        if (hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(&mfma_dqlds_kernel<DT, BITS, RB>), raised);
            e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((mfma_dqlds_kernel<DT, BITS, RB>), dim3(static_cast<unsigned>(a.N / DQ_TN)), dim3(DQ_THREADS),
                       lds, a.stream, static_cast<const uint16_t*>(a.x), a.wq,
                       static_cast<const uint16_t*>(a.scales), static_cast<const uint16_t*>(a.biases),
                       static_cast<uint16_t*>(a.y), static_cast<int>(a.M), a.N, a.K, a.gs);
    return hipGetLastError();
}

template <int DT, int BITS>
hipError_t launch_dqlds_b(const MatmulArgs& a) {
    switch ((a.M + 15) / 16) {
        case 1: return launch_dqlds_t<DT, BITS, 1>(a);
        case 2: return launch_dqlds_t<DT, BITS, 2>(a);
        case 3: return launch_dqlds_t<DT, BITS, 3>(a);
        case 4: return launch_dqlds_t<DT, BITS, 4>(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool mfma_dqlds_supports(int bits, int64_t M, int64_t N, int64_t K) {
    const int64_t kc = bits == 4 ? 256 : 128;
    // (K <= 2^24 keeps every activation and code offset well inside 32-bit
    // products of the index arithmetic)
    return M >= 1 && M <= 64 && N >= DQ_TN && N % DQ_TN == 0 && K >= kc && K % kc == 0 &&
           K <= (int64_t{1} << 24);
}

hipError_t launch_mfma_dqlds(const MatmulArgs& a) {
    if (!mfma_dqlds_supports(a.bits, a.M, a.N, a.K) || a.batch != 1) return hipErrorInvalidValue;
    switch (a.dt * 10 + a.bits) {
        case 4: return launch_dqlds_b<DT_F16, 4>(a);
        case 6: return launch_dqlds_b<DT_F16, 6>(a);
        case 8: return launch_dqlds_b<DT_F16, 8>(a);
        case 14: return launch_dqlds_b<DT_BF16, 4>(a);
        case 16: return launch_dqlds_b<DT_BF16, 6>(a);
        case 18: return launch_dqlds_b<DT_BF16, 8>(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
