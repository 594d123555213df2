// Split-free small-M kernel for the batched-decode shapes: M up to 64, any K
// that is a whole number of k-blocks, column tiles of 16 or 64 columns.
//
// Design source: the verify kernels of "How the NAX Verify Kernel Path
// Improves Decode Performance in MTPLX" ("How the NAX Verify Kernel Path
// Eliminates Bottlenecks": one workgroup owns a column tile, reads its
// weights once and never splits K across workgroups) and the batched-decode
// M sweep of MLX issue #4720 ("Expected behavior").  What changes with M: every
// column tile needs the whole activation matrix (M x K), which at M = 64 is
// several times the tile's own weight bytes, so here the activation block of
// a pass is brought into LDS once per workgroup and read there by every
// wavefront that needs it, and the weights stay the only thing a compute
// wavefront loads itself.
//
// Workgroup: CW x KW compute wavefronts and two loader wavefronts.
//   * Loader wavefronts copy the activation block of the next pass (all
//     rows, KW k-blocks) from global memory straight into LDS
//     (global_load_lds, 16 bytes per lane) while the compute wavefronts work
//     on the current one: two LDS buffers, one workgroup barrier per pass.
//   * Compute wavefront (cw, kw) owns NT 16-column tiles and every 16-row
//     block of M; in pass p it takes k-block p*KW + kw.  Its weight segments,
//     scales and biases are loaded D iterations ahead into a register ring.
//     Because a wavefront's loads retire in issue order, keeping the
//     activation traffic on other wavefronts is what lets that ring run deep:
//     a compute wavefront never waits on anything but its own weights.
//   * At a tile's last pass the KW partial tiles are added in a fixed order
//     (kw = 0, 1, ...) through LDS, so results are deterministic.
//
// Arithmetic as in the pass kernel: codes become exact values q + off with
// one offset for every code, and per unit u
//   y += s_u * P_u + (b_u - off * s_u) * X_u,
// P_u = sum x * (q + off) and X_u = sum x on the matrix cores (X_u with an
// all-ones operand; one X per row block and step serves all NT tiles).
//
// LDS activation layout: a pass block is [rows][RP pieces of 16 bytes]
// (RP = KW * KBLK / 8), row-major with no padding; piece q of row r is
// stored at slot q ^ (r & 15), so the 16 rows that one fragment read touches
// fall in 16 different bank groups.
#pragma once

#include "qmm_device.hpp"
#include "qmm_internal.hpp"
#include "qmm_mfma_frag.hpp"

namespace qmm {

namespace {

using namespace mf;

constexpr int TILE_LOADERS = 2; // activation-loading wavefronts per workgroup
constexpr int TILE_RBM = 4;     // 16-row blocks (M <= 64)

template <int DT, int BITS, int GS, int CW, int NT, int KW_>
struct TileFmt {
    using F = Fmt<DT, BITS, GS>;
    static constexpr int KW = KW_;
    static constexpr int CWAVES = CW * KW;
    static constexpr int WAVES = CWAVES + TILE_LOADERS;
    static constexpr int BN = 16 * NT * CW;       // columns per tile
    static constexpr int RP = KW * F::KBLK / 8;   // 16-byte pieces per activation row of a pass
    static constexpr int KPASS = KW * F::KBLK;    // codes per pass
    static_assert(RP % 16 == 0, "the slot swizzle needs 16 pieces per row");
    // LDS: NB activation buffers of 16*rb rows (three where they fit, else
    // two), then the partial-tile area of one k-group
    __host__ __device__ static constexpr int xbuf_bytes(int rb) { return 16 * rb * RP * 16; }
    __host__ __device__ static constexpr int red_bytes(int rb) { return CW * rb * NT * 1024; }
    __host__ __device__ static constexpr int nbuf(int rb) {
        return 3 * xbuf_bytes(rb) + red_bytes(rb) <= 160 * 1024 ? 3 : 2;
    }
    __host__ __device__ static constexpr int lds_bytes(int rb) { return nbuf(rb) * xbuf_bytes(rb) + red_bytes(rb); }
};

// One iteration's weight segments and raw scale/bias words for one lane.
template <int DT, int BITS, int GS, int NT>
struct TileSlot {
    using F = Fmt<DT, BITS, GS>;
    static constexpr int SW = F::PORTIONS == 4 ? 2 : 1;  // 32-bit words of unit scales
    uint32_t w[NT][F::SEG_WORDS];
    uint32_t s[NT][SW], b[NT][SW];
};

// 16-bit scale (or bias) of unit p from the words a TileSlot holds.
template <int PORTIONS, int SW>
__device__ __forceinline__ uint16_t unit_half(const uint32_t (&v)[SW], int p) {
    if constexpr (PORTIONS == 1) return static_cast<uint16_t>(v[0]);
    else return static_cast<uint16_t>(v[p >> 1] >> (16 * (p & 1)));
}

template <int DT, int BITS, int GS, int CW, int NT, int KW_, int D>
__global__ __launch_bounds__(64 * (CW * KW_ + TILE_LOADERS)) void mfma_tile_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, uint16_t* __restrict__ y, float* __restrict__ part, int M, int64_t N,
    int64_t K) {
    using F = Fmt<DT, BITS, GS>;
    using TF = TileFmt<DT, BITS, GS, CW, NT, KW_>;
    using Slot = TileSlot<DT, BITS, GS, NT>;
    constexpr int KW = TF::KW;
    constexpr int RP = TF::RP;
    constexpr float UOFF = F::off(0);
    extern __shared__ __align__(16) uint8_t lds[];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int RB = (M + 15) >> 4;
    const int xbuf = TF::xbuf_bytes(RB);
    const int nb = TF::nbuf(RB);

    const int64_t nkb = K / F::KBLK;
    const int P = static_cast<int>((nkb + KW - 1) / KW);
    // K split over gridDim.y workgroups: split s takes passes [pb, pe) of
    // every tile and leaves fp32 partial tiles in `part` ([split][M][N]);
    // the host makes every split non-empty.  Unsplit: pb = 0, pe = P.
    const int PP = (P + static_cast<int>(gridDim.y) - 1) / static_cast<int>(gridDim.y);
    const int pb = static_cast<int>(blockIdx.y) * PP;
    const int pe = min(P, pb + PP);
    const int64_t ntiles = (N + TF::BN - 1) / TF::BN;
    const int64_t my_tiles = (ntiles - 1 - static_cast<int64_t>(blockIdx.x)) / gridDim.x + 1;
    const int64_t n_it = my_tiles * (pe - pb);

    if (wave >= TF::CWAVES) {
        // ---- loader wavefronts: activation blocks -> LDS ----
        // Instruction i of a pass block fills slots 64i .. 64i+63: row
        // i*RPI + lane/RP, stored piece lane % RP, which holds activation
        // piece (lane % RP) ^ (row & 15).  Loader lw issues i = lw, lw+2, ...
        // Only the instructions that hold rows < M are issued: the rows of
        // the last 16-row block past M keep whatever the buffer held, and a
        // row of A only reaches the same row of the matrix products, whose
        // outputs are never stored.  (Within an instruction that does cover
        // row M - 1, the rows past it repeat row M - 1.)  A lane's source
        // offset within a pass does not depend on the pass, so it is computed
        // once; a last pass that runs past K takes the clamped path (pieces
        // past K read the row's first piece; their k-blocks are skipped by
        // the compute wavefronts).
        constexpr int RPI = 64 / RP;
        constexpr int MAXJ = TILE_RBM * RP / 4 / TILE_LOADERS;
        const int lw = wave - TF::CWAVES;
        const int n_ins = (M + RPI - 1) / RPI;  // instructions holding rows < M
        const int nj = (n_ins - lw + TILE_LOADERS - 1) / TILE_LOADERS;
        const int lrow = lane / RP;
        const int lpiece = lane % RP;
        uint32_t off[MAXJ];
#pragma unroll
        for (int j = 0; j < MAXJ; ++j) {
            const int row = (lw + TILE_LOADERS * j) * RPI + lrow;
            const int srow = row < M ? row : M - 1;
            const int piece = lpiece ^ (row & 15);
            off[j] = static_cast<uint32_t>((static_cast<int64_t>(srow) * K + piece * 8) * 2);
        }
        auto issue = [&](int pass, int b) {
            const int64_t k0 = static_cast<int64_t>(pass) * TF::KPASS;
            uint8_t* base = lds + b * xbuf;
            if (k0 + TF::KPASS <= K) {
                const uint8_t* src = reinterpret_cast<const uint8_t*>(x) + k0 * 2;
#pragma unroll
                for (int j = 0; j < MAXJ; ++j)
                    if (j < nj)
                        __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + off[j]), base + (lw + TILE_LOADERS * j) * 1024, 16, 0, 0);
            } else {
                for (int j = 0; j < nj; ++j) {
                    const int row = (lw + TILE_LOADERS * j) * RPI + lrow;
                    const int piece = lpiece ^ (row & 15);
                    int64_t k = k0 + piece * 8;
                    k = k < K ? k : 0;
                    const int srow = row < M ? row : M - 1;
                    __builtin_amdgcn_global_load_lds(static_cast<const void*>(x + static_cast<int64_t>(srow) * K + k),
                                                     base + (lw + TILE_LOADERS * j) * 1024, 16, 0, 0);
                }
            }
        };
        // Chunk = the block of one iteration.  Two buffers: iteration it
        // issues chunk it+1 and waits for it before the next barrier.  Three
        // buffers: iteration it waits for chunk it+1 (issued an iteration
        // earlier), then issues chunk it+2 into the buffer chunk it-1 used.
        int ipass = pb, ibuf = 0;
        int64_t iss = 0;
        auto issue_next = [&]() {
            if (iss < n_it) {
                issue(ipass, ibuf);
                ipass = ipass + 1 == pe ? pb : ipass + 1;
                ibuf = ibuf + 1 == nb ? 0 : ibuf + 1;
                ++iss;
            }
        };
        issue_next();
        if (nb == 3) issue_next();
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        int pass = pb;
        for (int64_t it = 0; it < n_it; ++it) {
            __syncthreads();  // chunk `it` is in LDS; chunk it-1's buffer is free
            if (nb == 2) {
                issue_next();
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            } else {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                issue_next();
            }
            if (pass == pe - 1) {
                // the compute wavefronts' ordered tile reduction
#pragma unroll
                for (int st = 0; st < KW - 1; ++st) __syncthreads();
            }
            pass = pass + 1 == pe ? pb : pass + 1;
        }
        return;
    }

    // ---- compute wavefronts ----
    const int c = lane & 15;
    const int jj = lane >> 4;
    const int cw = wave % CW;
    const int kw = wave / CW;
    const int64_t row_bytes = K * BITS / 8;
    const int64_t G = K / GS;
    const bool narrow = N < TF::BN;
    auto tile_col0 = [&](int64_t t) -> int64_t {
        if (narrow) return 0;
        const int64_t c0 = t * TF::BN;
        return c0 + TF::BN <= N ? c0 : N - TF::BN;
    };

    auto load_slot = [&](int64_t t, int pass, Slot& r) {
        const int64_t kb = static_cast<int64_t>(pass) * KW + kw;
        const int64_t kbc = kb < nkb ? kb : nkb - 1;
        const int64_t c0 = tile_col0(t);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            int64_t col = c0 + 16 * (cw * NT + nt) + c;
            col = col < N ? col : N - 1;
            const uint8_t* wrow = reinterpret_cast<const uint8_t*>(wq) + col * row_bytes;
            load_segment<BITS, F::SEG_WORDS>(
                reinterpret_cast<const uint32_t*>(wrow + (kbc * F::KBLK + jj * F::SEG) * BITS / 8), r.w[nt]);
            if constexpr (F::PORTIONS == 1) {
                const int64_t at = col * G + kbc * F::KBLK / GS;
                r.s[nt][0] = scales[at];
                r.b[nt][0] = biases[at];
            } else if constexpr (F::PORTIONS == 2) {
                const int64_t at = col * G + kbc * 2;
                r.s[nt][0] = *reinterpret_cast<const uint32_t*>(scales + at);
                r.b[nt][0] = *reinterpret_cast<const uint32_t*>(biases + at);
            } else {
                const int64_t at = col * G + kbc * 4;
                const uint2 sw = *reinterpret_cast<const uint2*>(scales + at);
                const uint2 bw = *reinterpret_cast<const uint2*>(biases + at);
                r.s[nt][0] = sw.x; r.s[nt][1] = sw.y;
                r.b[nt][0] = bw.x; r.b[nt][1] = bw.y;
            }
        }
    };

    const UnpackConsts uk = unpack_consts<DT>();
    Frag ones;
#pragma unroll
    for (int v = 0; v < 4; ++v) ones.v[v] = DtBits<DT>::one * 0x10001u;

    float4_t yacc[TILE_RBM][NT];
#pragma unroll
    for (int rb = 0; rb < TILE_RBM; ++rb)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) yacc[rb][nt] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // LDS byte offset of this lane's fragment piece for step s within a row
    // block (row c, the k-block of this k-group); row block rb adds
    // rb * 16 rows, a constant
    uint32_t xoff[F::STEPS];
#pragma unroll
    for (int s = 0; s < F::STEPS; ++s) {
        const int kk = F::src_lane(s, jj) * F::SEG + F::src_slot(s, jj) * 8;
        const int piece = (kw * F::KBLK + kk) >> 3;
        xoff[s] = static_cast<uint32_t>((c * RP + (piece ^ c)) << 4);
    }
    constexpr uint32_t RB_STRIDE = 16 * RP * 16;

    auto compute = [&](const Slot& r, int64_t kb, const uint8_t* xb) {
        if (kb >= nkb) return;  // past K in the last pass
        Frag bw[NT][F::STEPS];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            // The lane swaps rewrite their operands in place.  Copying the
            // ring words here, in a form the compiler keeps, ends the ring
            // registers' live range at this point; otherwise it may place
            // that copy at the loop latch, where it would wait for the
            // newest load of the ring.
            uint32_t wc[F::SEG_WORDS];
#pragma unroll
            for (int q = 0; q < F::SEG_WORDS; ++q) asm volatile("v_mov_b32 %0, %1" : "=v"(wc[q]) : "v"(r.w[nt][q]));
            segment_frags<DT, BITS, GS, F::SEG_WORDS, F::STEPS, true>(wc, bw[nt], uk);
        }
#pragma unroll
        for (int p = 0; p < F::PORTIONS; ++p) {
            float sc[NT], bp[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                sc[nt] = DtOps<DT>::to_f32(unit_half<F::PORTIONS, Slot::SW>(r.s[nt], p));
                bp[nt] = __fmaf_rn(-UOFF, sc[nt], DtOps<DT>::to_f32(unit_half<F::PORTIONS, Slot::SW>(r.b[nt], p)));
            }
#pragma unroll
            for (int rb = 0; rb < TILE_RBM; ++rb) {
                if (rb >= RB) break;
                float4_t acc[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) acc[nt] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
                float4_t xs4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int st = 0; st < F::STEPS_PER_PORTION; ++st) {
                    const int s = p * F::STEPS_PER_PORTION + st;
                    const uint4 u = *reinterpret_cast<const uint4*>(xb + xoff[s] + rb * RB_STRIDE);
                    const Frag a = x_frag<BITS, DT>(u);
                    xs4 = mfma<DT>(a, ones, xs4);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma<DT>(a, bw[nt][s], acc[nt]);
                }
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        yacc[rb][nt][q] = __fmaf_rn(sc[nt], acc[nt][q], yacc[rb][nt][q]);
                        yacc[rb][nt][q] = __fmaf_rn(bp[nt], xs4[q], yacc[rb][nt][q]);
                    }
            }
        }
    };

    // Ordered combination of the KW partial tiles: k-group 0 writes its
    // partial, each next k-group adds its own in turn, the last one rounds
    // and stores.  KW - 1 barriers, matched by the loader wavefronts.
    float* red = reinterpret_cast<float*>(lds + nb * xbuf);
    auto finish_tile = [&](int64_t t) {
        const int64_t c0 = tile_col0(t);
#pragma unroll
        for (int st = 0; st < KW; ++st) {
            if (kw == st) {
#pragma unroll
                for (int rb = 0; rb < TILE_RBM; ++rb) {
                    if (rb >= RB) break;
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int idx = (((cw * RB + rb) * NT + nt) * 4 + q) * 64 + lane;
                            float v = yacc[rb][nt][q];
                            if (st > 0) v = red[idx] + v;
                            if (st < KW - 1) {
                                red[idx] = v;
                            } else {
                                const int row = 16 * rb + 4 * jj + q;
                                const int64_t col = c0 + 16 * (cw * NT + nt) + c;
                                if (row < M && col < N) {
                                    if (part)
                                        part[(static_cast<int64_t>(blockIdx.y) * M + row) * N + col] = v;
                                    else
                                        y[static_cast<int64_t>(row) * N + col] = DtOps<DT>::rne(v);
                                }
                            }
                        }
                }
            }
            if (st < KW - 1) __syncthreads();
        }
#pragma unroll
        for (int rb = 0; rb < TILE_RBM; ++rb)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) yacc[rb][nt] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    };

    // Iteration `it` = (tile, pass).  The ring slot of iteration it was
    // loaded D iterations earlier; past the last iteration the prefetch
    // re-reads the last one.
    Slot ring[D];
    const int64_t tstep = gridDim.x;
    int64_t tile = blockIdx.x;
    int pass = pb;
    int64_t ptile = tile;
    int ppass = pb;
    int64_t pit = 0;
    auto advance = [&](int64_t& t, int& p) {
        if (++p == pe) {
            p = pb;
            t += tstep;
        }
    };
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load_slot(ptile, ppass, ring[d]);
        if (pit + 1 < n_it) {
            advance(ptile, ppass);
            ++pit;
        }
    }
    // Groups of D iterations.  An iteration past the end (last group) skips
    // its barrier and compute -- uniformly across the workgroup, as the
    // loaders skip theirs -- but still issues its ring load (a re-read of the
    // last iteration): every path through the group then issues the same
    // loads, so the waits the compiler places stay D iterations deep (a path
    // with fewer loads merged into the loop head would make them shallow).
    int xbi = 0;  // activation buffer of the current iteration
    for (int64_t it = 0; it < n_it; it += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            if (it + u < n_it) {
                __syncthreads();  // this pass's activation block is in LDS
                compute(ring[u], static_cast<int64_t>(pass) * KW + kw, lds + xbi * xbuf);
                xbi = xbi + 1 == nb ? 0 : xbi + 1;
            }
            load_slot(ptile, ppass, ring[u]);
            if (pit + 1 < n_it) {
                advance(ptile, ppass);
                ++pit;
            }
            if (it + u < n_it) {
                if (pass == pe - 1) finish_tile(tile);
                advance(tile, pass);
            }
        }
    }
}

template <int DT, int BITS, int GS, int CW, int NT, int KW, int D>
hipError_t launch_tile_cfg(const MatmulArgs& a) {
    using TF = TileFmt<DT, BITS, GS, CW, NT, KW>;
    const int rb = static_cast<int>((a.M + 15) / 16);
    const int64_t ntiles = (a.N + TF::BN - 1) / TF::BN;
    const int S = a.split > 1 ? a.split : 1;
    // about one workgroup per CU (its LDS use is most of a CU's), the K
    // splits of a column slot side by side in gridDim.y
    const int64_t slots = 256 / S > 1 ? 256 / S : 1;
    const int64_t gx = ntiles < slots ? ntiles : slots;
    const size_t lds = static_cast<size_t>(TF::lds_bytes(rb));
    static std::atomic<uint64_t> raised{0};
    if (hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(&mfma_tile_kernel<DT, BITS, GS, CW, NT, KW, D>),
                                       raised);
        e != hipSuccess)
        return e;
    hipLaunchKernelGGL((mfma_tile_kernel<DT, BITS, GS, CW, NT, KW, D>),
                       dim3(static_cast<unsigned>(gx), static_cast<unsigned>(S)), dim3(64 * TF::WAVES), lds,
                       a.stream, static_cast<const uint16_t*>(a.x), a.wq, static_cast<const uint16_t*>(a.scales),
                       static_cast<const uint16_t*>(a.biases), static_cast<uint16_t*>(a.y),
                       S > 1 ? a.part : nullptr, static_cast<int>(a.M), a.N, a.K);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || S == 1) return e;
    return launch_reduce_partials(DT, a.part, a.y, S, a.M * a.N, a.stream);
}

// Every shape runs 4 compute wavefronts and 2 loaders (6 wavefronts: at
// most 2 per SIMD, so 256 VGPRs each):
//   TILE16:  one 16-column tile per compute wavefront, 4 k-blocks per pass,
//            weights 8 iterations ahead;
//   TILE64:  two column groups of two tiles, 2 k-blocks per pass, 4 ahead.
// (KW per shape is also in tile_split.)
template <int DT, int BITS, int GS>
hipError_t launch_tile_t(const MatmulArgs& a, int cfg) {
    switch (cfg) {
        case TILE_CFG_16: return launch_tile_cfg<DT, BITS, GS, 1, 1, 4, 8>(a);
        case TILE_CFG_64: return launch_tile_cfg<DT, BITS, GS, 2, 2, 2, 4>(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Launch for one activation dtype and code width (every group size), each
// compiled in a translation unit of its own (qmm_mfma_tile_<dt>_<bits>.hip).
hipError_t launch_mfma_tile_f16_4(const MatmulArgs& a, int cfg);
hipError_t launch_mfma_tile_f16_6(const MatmulArgs& a, int cfg);
hipError_t launch_mfma_tile_f16_8(const MatmulArgs& a, int cfg);
hipError_t launch_mfma_tile_bf16_4(const MatmulArgs& a, int cfg);
hipError_t launch_mfma_tile_bf16_6(const MatmulArgs& a, int cfg);
hipError_t launch_mfma_tile_bf16_8(const MatmulArgs& a, int cfg);

#define QMM_TILE_FMT_LAUNCHER(NAME, DTV, BITSV)                       \
    hipError_t NAME(const MatmulArgs& a, int cfg) {                   \
        switch (a.gs) {                                               \
            case 32: return launch_tile_t<DTV, BITSV, 32>(a, cfg);    \
            case 64: return launch_tile_t<DTV, BITSV, 64>(a, cfg);    \
            case 128: return launch_tile_t<DTV, BITSV, 128>(a, cfg);  \
            default: return hipErrorInvalidValue;                     \
        }                                                             \
    }

}  // namespace qmm
