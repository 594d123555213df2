// Split-free small-M kernel with MFMA accumulation for any K and M <= 64:
// K is walked in passes.
//
// Design source: the verify kernels of "How the NAX Verify Kernel Path
// Improves Decode Performance in MTPLX" ("How the NAX Verify Kernel Path
// Eliminates Bottlenecks"): a column tile is owned by one workgroup, its
// weights are read once and K is never split across workgroups (the split-K
// dispatch that MLX issue #4720 measures as the slow path).  This variant
// covers the shapes the register-resident kernel cannot hold: long K (the
// 14336-wide down projection of the batched-decode workload) and M above 16
// (one 16-row block of M per blockIdx.y).
//
// A workgroup of 16 wavefronts owns a 16-column tile; in pass p wavefront w
// takes k-block p*16 + w, so a pass covers 16 k-blocks and the partial sums
// stay in registers across passes until the tile's last pass, when the
// wavefronts combine them once through LDS.  Each iteration (tile, pass)
// prefetches the next one's weight segment, scales, biases and activation
// block while it computes: the activation block (16 rows x one k-block) is
// read with coalesced 16-byte loads, staged through the wavefront's own LDS
// region and read back in fragment order.
//
// Arithmetic: codes become exact fp16/bf16 values q + off with one offset
// for every code, and per unit u (a run of K inside one group)
//   y += s_u * P_u + (b_u - off * s_u) * X_u,
// P_u = sum x * (q + off) and X_u = sum x on the matrix cores (the block
// changes every iteration, so the unit sums are recomputed each time and
// kept as cheap as possible: two per-lane FMAs per output and unit).
#include "qmm_device.hpp"
#include "qmm_internal.hpp"
#include "qmm_mfma_frag.hpp"

namespace qmm {

namespace {

using namespace mf;

constexpr int PW = 16;  // wavefronts per workgroup

template <int DT, int BITS, int GS>
struct PassFmt {
    using F = Fmt<DT, BITS, GS>;
    static constexpr int CPR = F::KBLK / 8;       // 16-byte activation chunks per row of a k-block
    static constexpr int XG = 16 * CPR / 64;      // chunks per lane for 16 rows
    static constexpr int XS_ROW = F::KBLK + 8;    // staged row stride in elements (16 bytes of padding)
    static constexpr int NU = F::PORTIONS;        // units per k-block
    static constexpr int RED_BYTES = 2 * PW * 4 * 64 * 4;
    static constexpr int LDS_BYTES = RED_BYTES + PW * 16 * XS_ROW * 2;
};

// Weight segment and per-unit scale and bias (raw 16-bit) of one iteration
// for one lane.
template <int DT, int BITS, int GS>
struct PassRegs {
    using F = Fmt<DT, BITS, GS>;
    uint32_t w[F::SEG_WORDS];
    uint32_t s[F::PORTIONS], b[F::PORTIONS];
};

// SV: K is a whole number of k-blocks and a row's group count is a multiple
// of the units per k-block, so a k-block's scales (and biases) are read with
// one aligned 4- or 8-byte load per lane instead of one per unit.
template <int DT, int BITS, int GS, bool SV>
__global__ __launch_bounds__(64 * PW, 4) void mfma_pass_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, uint16_t* __restrict__ y, int M, int64_t N, int64_t K) {
    using F = Fmt<DT, BITS, GS>;
    using PF = PassFmt<DT, BITS, GS>;
    using Regs = PassRegs<DT, BITS, GS>;
    // the code offset shared by every code (uniform unpack)
    constexpr float UOFF = F::off(0);
    extern __shared__ __align__(16) uint8_t lds[];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane & 15;
    const int jj = lane >> 4;
    float* red = reinterpret_cast<float*>(lds);
    uint16_t* xs = reinterpret_cast<uint16_t*>(lds + PF::RED_BYTES) + wave * 16 * PF::XS_ROW;

    // this workgroup's 16-row block of M
    const int row0 = static_cast<int>(blockIdx.y) * 16;
    const int Mloc = min(16, M - row0);
    x += static_cast<int64_t>(row0) * K;
    y += static_cast<int64_t>(row0) * N;

    const int64_t row_bytes = K * BITS / 8;
    const int64_t G = K / GS;
    const int64_t nkb = (K + F::KBLK - 1) / F::KBLK;
    const int P = static_cast<int>((nkb + PW - 1) / PW);
    const int64_t ntiles = (N + 15) / 16;
    const int64_t my_tiles = (ntiles - 1 - static_cast<int64_t>(blockIdx.x)) / gridDim.x + 1;
    const int64_t n_it = my_tiles * P;

    // As in the register-resident kernel: the last tile of a ragged N is
    // shifted back to end at column N (overlapping columns are recomputed
    // with identical values); for N < 16 the lanes clamp their row instead.
    const bool narrow = N < 16;
    const int64_t lane_row = narrow ? min(static_cast<int64_t>(c), N - 1) : c;
    auto tile_col0 = [&](int64_t tile) -> int64_t {
        const int64_t c0 = tile * 16;
        return (narrow || c0 + 16 <= N) ? c0 : N - 16;
    };

    // Loads of iteration (tile, pass): the activation
    // block first (into xg), then the weight segment, scales and biases.  A
    // wavefront whose k-block lies beyond K in the last pass reads valid
    // addresses and gets a zero activation block, so it adds exact zeros.
    uint4 xg[PF::XG];
    auto load_it = [&](int64_t tile, int pass, Regs& r) {
        const int64_t col0 = tile_col0(tile);
        const int64_t kb = static_cast<int64_t>(pass) * PW + wave;
        const bool kvalid = kb < nkb;
        const int64_t kbc = kvalid ? kb : nkb - 1;
#pragma unroll
        for (int j = 0; j < PF::XG; ++j) {
            const int t = lane + 64 * j;
            const int row = t / PF::CPR, piece = t % PF::CPR;
            const int64_t k = kb * F::KBLK + piece * 8;
            xg[j] = make_uint4(0u, 0u, 0u, 0u);
            if (kvalid && row < Mloc && k < K)
                xg[j] = *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(row) * K + k);
        }
        int64_t code0 = kbc * F::KBLK + jj * F::SEG;
        code0 = code0 < K ? code0 : K - F::SEG;
        const uint8_t* wrow = reinterpret_cast<const uint8_t*>(wq) + (col0 + lane_row) * row_bytes;
        load_segment<BITS, F::SEG_WORDS>(reinterpret_cast<const uint32_t*>(wrow + code0 * BITS / 8), r.w);
        if constexpr (SV && F::PORTIONS == 2) {
            const int64_t at = (col0 + lane_row) * G + kbc * 2;
            const uint32_t sw = *reinterpret_cast<const uint32_t*>(scales + at);
            const uint32_t bw = *reinterpret_cast<const uint32_t*>(biases + at);
            r.s[0] = sw; r.s[1] = sw >> 16;
            r.b[0] = bw; r.b[1] = bw >> 16;
        } else if constexpr (SV && F::PORTIONS == 4) {
            const int64_t at = (col0 + lane_row) * G + kbc * 4;
            const uint2 sw = *reinterpret_cast<const uint2*>(scales + at);
            const uint2 bw = *reinterpret_cast<const uint2*>(biases + at);
            r.s[0] = sw.x; r.s[1] = sw.x >> 16; r.s[2] = sw.y; r.s[3] = sw.y >> 16;
            r.b[0] = bw.x; r.b[1] = bw.x >> 16; r.b[2] = bw.y; r.b[3] = bw.y >> 16;
        } else {
#pragma unroll
            for (int p = 0; p < F::PORTIONS; ++p) {
                int64_t g = (kbc * F::KBLK + static_cast<int64_t>(p) * F::PC) / GS;
                g = g < G ? g : G - 1;
                r.s[p] = scales[(col0 + lane_row) * G + g];
                r.b[p] = biases[(col0 + lane_row) * G + g];
            }
        }
    };
    // the activation block of the loads just issued -> this wavefront's LDS
    // region (rows >= M are zero)
    auto stage_x = [&]() {
#pragma unroll
        for (int j = 0; j < PF::XG; ++j) {
            const int t = lane + 64 * j;
            const int row = t / PF::CPR, piece = t % PF::CPR;
            *reinterpret_cast<uint4*>(xs + row * PF::XS_ROW + piece * 8) = xg[j];
        }
    };

    const UnpackConsts uk = unpack_consts<DT>();


    float4_t yacc = {0.0f, 0.0f, 0.0f, 0.0f};
    int parity = 0;

    auto process = [&](int64_t tile, int pass, const Regs& r) {
        // this iteration's activation block, staged at the top of the
        // iteration, in fragment order
        Frag xa[F::STEPS];
#pragma unroll
        for (int s = 0; s < F::STEPS; ++s) {
            const int kk = F::src_lane(s, jj) * F::SEG + F::src_slot(s, jj) * 8;
            xa[s] = x_frag<BITS, DT>(*reinterpret_cast<const uint4*>(xs + c * PF::XS_ROW + kk));
        }
        // Every code carries the same offset UOFF here (fp16 4-bit codes
        // take their odd nibbles shifted down as well), so O_u = UOFF * X_u
        // and per unit u
        //   y += s_u * P_u + (b_u - UOFF * s_u) * X_u,
        // with P_u = sum x * (q + UOFF) and X_u = sum x both on the matrix
        // cores: X_u as the product with an all-ones B operand, which lands
        // in the accumulator layout directly (row sums repeated across the
        // columns), so both terms are per-lane FMAs.
        uint32_t wcopy[F::SEG_WORDS];
#pragma unroll
        for (int q = 0; q < F::SEG_WORDS; ++q) wcopy[q] = r.w[q];
        Frag bw[F::STEPS];
        segment_frags<DT, BITS, GS, F::SEG_WORDS, F::STEPS, true>(wcopy, bw, uk);
        Frag ones;
#pragma unroll
        for (int v = 0; v < 4; ++v) ones.v[v] = DtBits<DT>::one * 0x10001u;
#pragma unroll
        for (int p = 0; p < F::PORTIONS; ++p) {
            float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
            float4_t xs4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int st = 0; st < F::STEPS_PER_PORTION; ++st) {
                const int s = p * F::STEPS_PER_PORTION + st;
                acc = mfma<DT>(xa[s], bw[s], acc);
                xs4 = mfma<DT>(xa[s], ones, xs4);
            }
            const float sc = DtOps<DT>::to_f32(static_cast<uint16_t>(r.s[p]));
            const float bp = __fmaf_rn(-UOFF, sc, DtOps<DT>::to_f32(static_cast<uint16_t>(r.b[p])));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                yacc[q] = __fmaf_rn(sc, acc[q], yacc[q]);
                yacc[q] = __fmaf_rn(bp, xs4[q], yacc[q]);
            }
        }
        if (pass == P - 1) {
            // combine the wavefronts' partial tiles (parity double buffer,
            // one barrier per tile, as in the register-resident kernel)
            float* rb = red + parity * (PW * 4 * 64);
#pragma unroll
            for (int q = 0; q < 4; ++q) rb[(wave * 4 + q) * 64 + lane] = yacc[q];
            __syncthreads();
            if (wave < 4) {
                const int q = wave;
                float v = 0.0f;
#pragma unroll
                for (int w = 0; w < PW; ++w) v += rb[(w * 4 + q) * 64 + lane];
                const int64_t col = tile_col0(tile) + c;
                const int row = 4 * jj + q;
                if (col < N && row < Mloc) y[static_cast<int64_t>(row) * N + col] = DtOps<DT>::rne(v);
            }
            parity ^= 1;
            yacc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };

    // Iteration cur: its activation block (loaded one iteration earlier, and
    // issued before that iteration's weights, so waiting for it does not
    // wait for them) goes to LDS, replacing the previous block, whose
    // fragments this wavefront has already read (its LDS accesses execute in
    // order); then the next iteration's loads are issued, then cur computes.
    // (tile, pass) of the current and of the next iteration, advanced
    // without divisions; past the last iteration the prefetch re-reads the
    // last one
    Regs buf[2];
    const int64_t tstep = gridDim.x;
    int64_t tile = blockIdx.x;
    int pass = 0;
    int64_t ntile = tile;
    int npass = 0;
    auto advance = [&](int64_t& t, int& p) {
        if (++p == P) {
            p = 0;
            t += tstep;
        }
    };
    load_it(tile, 0, buf[0]);
    for (int64_t it = 0; it < n_it; it += 2) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (it + u >= n_it) break;
            stage_x();
            if (it + u + 1 < n_it) advance(ntile, npass);
            load_it(ntile, npass, buf[u ^ 1]);
            __builtin_amdgcn_sched_barrier(0);
            process(tile, pass, buf[u]);
            advance(tile, pass);
        }
    }
}

template <int DT, int BITS, int GS, bool SV>
hipError_t launch_pass_sv(const MatmulArgs& a) {
    using PF = PassFmt<DT, BITS, GS>;
    // For 2 or 4 row blocks, one resident workgroup per CU in all: the gy
    // 16-row blocks of a column slot run at the same time and walk the same
    // tiles, and (256 / gy being a multiple of 8, the XCD count) their linear
    // ids fall on the same XCD, so a tile's weights come from HBM once and
    // from that XCD's L2 for the other blocks.  For 3 blocks the slot counts
    // that keep that alignment split the tiles unevenly or idle a quarter of
    // the CUs (measured slower), so each row block walks the tiles on its own.
    const int64_t ntiles = (a.N + 15) / 16;
    const int gy = static_cast<int>((a.M + 15) / 16);
    const int64_t slots = (gy == 2 || gy == 4) ? 256 / gy : 256;
    const int64_t gx = ntiles < slots ? ntiles : slots;
    const size_t lds = static_cast<size_t>(PF::LDS_BYTES);
    if (lds > 65536) {
        static std::atomic<uint64_t> raised{0};
        if (hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(&mfma_pass_kernel<DT, BITS, GS, SV>), raised);
            e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((mfma_pass_kernel<DT, BITS, GS, SV>), dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy)),
                       dim3(64 * PW), lds, a.stream, static_cast<const uint16_t*>(a.x), a.wq,
                       static_cast<const uint16_t*>(a.scales), static_cast<const uint16_t*>(a.biases),
                       static_cast<uint16_t*>(a.y), static_cast<int>(a.M), a.N, a.K);
    return hipGetLastError();
}

template <int DT, int BITS, int GS>
hipError_t launch_pass_t(const MatmulArgs& a) {
    using F = Fmt<DT, BITS, GS>;
    const int64_t G = a.K / GS;
    const bool sv = F::PORTIONS > 1 && a.K % F::KBLK == 0 && G % F::PORTIONS == 0;
    return sv ? launch_pass_sv<DT, BITS, GS, true>(a) : launch_pass_sv<DT, BITS, GS, false>(a);
}

}  // namespace

hipError_t launch_mfma_pass(const MatmulArgs& a) {
#define PCALL(D, B, G) launch_pass_t<D, B, G>(a)
    switch (a.dt * 100 + a.bits * 10 + a.gs / 32) {
        case 41: return PCALL(0, 4, 32);   case 42: return PCALL(0, 4, 64);   case 44: return PCALL(0, 4, 128);
        case 61: return PCALL(0, 6, 32);   case 62: return PCALL(0, 6, 64);   case 64: return PCALL(0, 6, 128);
        case 81: return PCALL(0, 8, 32);   case 82: return PCALL(0, 8, 64);   case 84: return PCALL(0, 8, 128);
        case 141: return PCALL(1, 4, 32);  case 142: return PCALL(1, 4, 64);  case 144: return PCALL(1, 4, 128);
        case 161: return PCALL(1, 6, 32);  case 162: return PCALL(1, 6, 64);  case 164: return PCALL(1, 6, 128);
        case 181: return PCALL(1, 8, 32);  case 182: return PCALL(1, 8, 64);  case 184: return PCALL(1, 8, 128);
        default: return hipErrorInvalidValue;
    }
#undef PCALL
}

}  // namespace qmm
