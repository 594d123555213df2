// Split-free small-M kernel with the weights dequantized into LDS and fed to
// the matrix cores from there (M <= 64): the "dequantize to shared memory,
// then matrix-unit contraction" form of the M >= 16 path.
//
// Design source: MLX issue #4720 ("Describe the bug", "Expected behavior"):
// above a handful of rows the matrix-unit kernel (qmm_nax) is the path to
// beat, and a split-K dispatch of the same product halves its bandwidth.  On
// Apple GPUs that kernel stages dequantized weight tiles in threadgroup
// memory; this is that arrangement written for gfx950, beside the in-register
// forms (mfma_splitfree_reg / pass / tile16 / tile64, which build the weight
// operand in registers), and both are timed on every format.  The selection
// takes it for fp16 6/8-bit codes above 16 rows at wide N (8192 columns and
// more), where it beats the 64-column tile kernel by 5-23 %; elsewhere the
// in-register forms win (1.4x to 10x): the dequantized tile crosses LDS and
// each chunk waits on two barriers, and for bf16 every weight costs two
// matrix steps (hi and lo).
//
// Workgroup: 4 wavefronts own a tile of 64 output columns for every row of
// M (16-row blocks 0..RB-1) and walk K in chunks of 256 values (a column's
// chunk is one, one and a half or two 128-byte lines at 4, 6, 8 bits).  Per
// chunk:
//   * every thread dequantizes two 32-code runs of one column (4 threads per
//     column): for fp16, two codes at a time, as packed halves -- the codes
//     become exact fp16 values through the exponent pattern of 1024
//     (0x6400 | q, minus 1024), then one packed fused multiply-add gives
//     s q + b rounded once; for bf16, w = s q + b in fp32 split into
//     hi = RNE(w) and lo = RNE(w - hi) (bf16's 8-bit significand would spend
//     most of the accepted error on one rounding) -- and writes them to the
//     LDS tile W[column][k];
//   * the activation rows of the chunk go to LDS beside it (rows past M stay
//     zero);
//   * after one barrier wavefront w reads the B operand of its 16 columns
//     (8 consecutive k of one column per lane: one 16-byte LDS read) and the
//     A operand of each row block (8 consecutive k of one row) in natural
//     order, and accumulates v_mfma_f32_16x16x32 steps in fp32 (two per step
//     for bf16: hi and lo).
// Two chunks are in flight in registers (code words, scales, biases and
// activations) while one is computed; past the end of K the prefetch reads
// the last chunk again (the same loads on every path, never staged).  Each
// weight is dequantized once per workgroup; the B operand crosses LDS once
// (its column owner reads it), the activations once per wavefront.
#include "qmm_device.hpp"
#include "qmm_internal.hpp"
#include "qmm_mfma_frag.hpp"

namespace qmm {

namespace {

using namespace mf;

constexpr int DQ_TN = 64;        // columns per workgroup
constexpr int DQ_THREADS = 256;  // 4 wavefronts, 16 columns each

constexpr int DQ_KC = 256;        // k values per chunk
constexpr int DQ_WS = DQ_KC + 8;  // LDS row stride of W and x (16 bytes of padding)

template <int DT, int BITS, int RB>
__global__ __launch_bounds__(DQ_THREADS) void mfma_dqlds_kernel(const uint16_t* __restrict__ x,
                                                             const uint32_t* __restrict__ wq,
                                                             const uint16_t* __restrict__ scales,
                                                             const uint16_t* __restrict__ biases,
                                                             uint16_t* __restrict__ y, int M, int64_t N,
                                                             int64_t K, int gs) {
    constexpr int KC = DQ_KC, WS = DQ_WS;
    constexpr int RUNS = KC / 32 / 4;                  // 32-code runs per thread (4 threads per column)
    constexpr int NH = DT == DT_BF16 ? 2 : 1;          // bf16: hi and lo tiles
    constexpr int XP = 16 * RB * KC / 8 / DQ_THREADS;  // 16-byte activation pieces per thread
    extern __shared__ __align__(16) uint16_t lds[];
    uint16_t* const w_lds = lds;                        // [NH][DQ_TN][WS]
    uint16_t* const x_lds = lds + NH * DQ_TN * WS;      // [16 RB][WS]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * DQ_TN;
    const int64_t G = K / gs;
    const int64_t row_words = K * BITS / 32;

    // activation rows M .. 16 RB - 1 stay zero
    for (int i = tid; i < (16 * RB - M) * WS; i += DQ_THREADS) x_lds[M * WS + i] = 0;

    // this thread's dequantization share: column c, runs q and q + 4
    const int c = tid >> 2, q = tid & 3;
    const uint32_t* const wrow = wq + (n0 + c) * row_words;

    typedef uint32_t v4u __attribute__((ext_vector_type(4)));  // (a native vector: stays in registers)
    struct Regs {
        uint32_t w[RUNS][BITS];
        uint32_t sb[RUNS];  // scale | bias << 16
        v4u xv[XP];
    };
    // chunk k0 into r; past the end of K the last chunk again (never staged)
    auto load = [&](int64_t k0, Regs& r) __attribute__((always_inline)) {
        k0 = k0 < K ? k0 : K - KC;
#pragma unroll
        for (int j = 0; j < RUNS; ++j) {
            const int64_t kr = k0 + 32 * (q + 4 * j);      // first k of the run
            load_chunk_words<BITS>(wrow + kr * BITS / 32, r.w[j]);
            const int64_t gi = (n0 + c) * G + kr / gs;
            r.sb[j] = static_cast<uint32_t>(scales[gi]) | (static_cast<uint32_t>(biases[gi]) << 16);
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
            const int kl = 32 * (q + 4 * j);
#pragma unroll
            for (int e = 0; e < 32; e += 8) {
                uint32_t hi[4], lo[4];
                if constexpr (DT == DT_F16) {
                    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
                    const h2_t s2 = __builtin_bit_cast(h2_t, (r.sb[j] & 0xFFFFu) * 0x10001u);
                    const h2_t b2 = __builtin_bit_cast(h2_t, (r.sb[j] >> 16) * 0x10001u);
                    const h2_t k1024 = {static_cast<_Float16>(1024.0f), static_cast<_Float16>(1024.0f)};
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const uint32_t pr = chunk_code<BITS>(r.w[j], e + 2 * t) |
                                            (chunk_code<BITS>(r.w[j], e + 2 * t + 1) << 16);
                        const h2_t qv = __builtin_bit_cast(h2_t, pr | 0x64006400u) - k1024;  // exact codes
                        hi[t] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(qv, s2, b2));
                    }
                } else {
                    const float s = DtOps<DT>::to_f32(static_cast<uint16_t>(r.sb[j] & 0xFFFFu));
                    const float b = DtOps<DT>::to_f32(static_cast<uint16_t>(r.sb[j] >> 16));
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const float w0 = __fmaf_rn(s, static_cast<float>(chunk_code<BITS>(r.w[j], e + 2 * t)), b);
                        const float w1 = __fmaf_rn(s, static_cast<float>(chunk_code<BITS>(r.w[j], e + 2 * t + 1)), b);
                        const uint16_t h0 = DtOps<DT>::rne(w0), h1 = DtOps<DT>::rne(w1);
                        const uint16_t l0 = DtOps<DT>::rne(w0 - DtOps<DT>::to_f32(h0));
                        const uint16_t l1 = DtOps<DT>::rne(w1 - DtOps<DT>::to_f32(h1));
                        hi[t] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
                        lo[t] = static_cast<uint32_t>(l0) | (static_cast<uint32_t>(l1) << 16);
                    }
                }
                *reinterpret_cast<v4u*>(w_lds + c * WS + kl + e) = v4u{hi[0], hi[1], hi[2], hi[3]};
                if constexpr (NH == 2)
                    *reinterpret_cast<v4u*>(w_lds + (DQ_TN + c) * WS + kl + e) = v4u{lo[0], lo[1], lo[2], lo[3]};
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
    auto compute = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int st = 0; st < KC / 32; ++st) {
            const int kk = 32 * st + 8 * lq;
            Frag bh, bl;
            {
                const v4u v = *reinterpret_cast<const v4u*>(w_lds + (16 * wave + li) * WS + kk);
                bh.v[0] = v.x; bh.v[1] = v.y; bh.v[2] = v.z; bh.v[3] = v.w;
            }
            if constexpr (NH == 2) {
                const v4u v = *reinterpret_cast<const v4u*>(w_lds + (DQ_TN + 16 * wave + li) * WS + kk);
                bl.v[0] = v.x; bl.v[1] = v.y; bl.v[2] = v.z; bl.v[3] = v.w;
            }
#pragma unroll
            for (int b = 0; b < RB; ++b) {
                Frag a;
                const v4u v = *reinterpret_cast<const v4u*>(x_lds + (16 * b + li) * WS + kk);
                a.v[0] = v.x; a.v[1] = v.y; a.v[2] = v.z; a.v[3] = v.w;
                acc[b] = mfma<DT>(a, bh, acc[b]);
                if constexpr (NH == 2) acc[b] = mfma<DT>(a, bl, acc[b]);
            }
        }
    };
    // chunk i is staged from buffer i % 2, whose next load (chunk i + 2) is
    // then in flight during the compute of chunks i and i + 1
    auto step = [&](int64_t k0, Regs& r) __attribute__((always_inline)) {
        const bool in = k0 < K;
        if (in) stage(r);
        __syncthreads();
        load(k0 + 2 * KC, r);
        if (in) compute();
        __syncthreads();  // the chunk's LDS is overwritten next
    };
    Regs r0, r1;
    load(0, r0);
    load(KC, r1);
    for (int64_t k0 = 0; k0 < K; k0 += 2 * KC) {
        step(k0, r0);
        step(k0 + KC, r1);
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
    constexpr int NH = DT == DT_BF16 ? 2 : 1;
    constexpr size_t lds = static_cast<size_t>(NH * DQ_TN + 16 * RB) * DQ_WS * sizeof(uint16_t);
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
    (void)bits;
    // (K <= 2^24 keeps every activation and code offset well inside 32-bit
    // products of the index arithmetic)
    return M >= 1 && M <= 64 && N >= DQ_TN && N % DQ_TN == 0 && K >= DQ_KC && K % DQ_KC == 0 &&
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
