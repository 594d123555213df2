// Split-free small-M kernel with MFMA accumulation and in-register weight
// fragments (M <= 16).
//
// Design source: the verify kernels of "How the NAX Verify Kernel Path
// Improves Decode Performance in MTPLX" ("Architectural Differences",
// "How the NAX Verify Kernel Path Eliminates Bottlenecks"): each column tile
// is owned by one workgroup and its weights are read exactly once, there is
// no split of K across workgroups, and M is padded (there to 4 or 6, here to
// the 16 rows of the matrix-core tile).  What changes on gfx950:
//   * the multiply-accumulates run on the matrix cores
//     (v_mfma_f32_16x16x32_{f16,bf16}); at 4 bits the vector ALUs alone
//     cannot keep up with the HBM stream for M >= 6;
//   * the workgroup's wavefronts (up to 16) split K among themselves so that
//     each SIMD streams a distinct part of the tile, and their partial sums
//     are combined once per tile through LDS;
//   * each wavefront holds the activation fragments of its part of K in
//     registers for the whole kernel while the workgroup walks over column
//     tiles (persistent grid), so x is read once per workgroup, not once per
//     tile, and the inner loop touches no shared memory.
//
// Arithmetic (exact up to fp32 rounding).  Codes become fp16/bf16 values
// q + off with the "magic number" trick: off = 1024 (fp16; 64 for the odd
// codes of a 4-bit word, which are unpacked without a shift), 128 (bf16 at
// 4/6 bits) or 0 (8-bit bf16, converted exactly).  For column n, the sum
// splits into
//   y = sum_u s_u * P_u  +  sum_u b_u * X_u  -  sum_u s_u * O_u
// over "units" u (runs of K inside one quantization group), with
//   P_u = sum_{k in u} x_k * (q_k + off_k)   (matrix cores, per tile),
//   X_u = sum_{k in u} x_k,  O_u = sum_{k in u} x_k * off_k  (from x only).
// The first term is one fp32 FMA per output per unit; the other two are
// small products over units (X and O against the bias and scale vectors of
// the tile), done on the matrix cores with X and O split into a high and a
// low fp16/bf16 part so that they keep fp32-level accuracy.  The dequantized
// weight s*q + b is never rounded to the activation dtype.
//
// Operand layout of v_mfma_f32_16x16x32 (verified on the hardware): lane l
// supplies A[l%16][8*(l/16)+e] and B[8*(l/16)+e][l%16] for e = 0..7 and
// receives D[4*(l/16)+r][l%16], r = 0..3.  A lane thus serves row i = l%16 of
// x and column c = l%16 of the tile, in k-slot quarter jj = l/16.
#pragma once

#include <type_traits>

#include "qmm_device.hpp"
#include "qmm_internal.hpp"
#include "qmm_mfma_frag.hpp"

namespace qmm {

namespace {

using namespace mf;


// Scale/bias words of one tile for one lane.  Vector form (VEC): the
// wavefront's NG consecutive groups as NG/2 words (two 16-bit values per
// word) of scales and of biases.  Scalar form: one value per portion.
template <bool VEC, int NGW, int KPW, int NP>
struct ScaleRegs;
template <int NGW, int KPW, int NP>
struct ScaleRegs<true, NGW, KPW, NP> {
    uint32_t s[NGW], b[NGW];
    // from a cooperative block in LDS: scales at p, biases at p + bias_off
    __device__ __forceinline__ void from_lds(const uint8_t* p, int64_t bias_off) {
        load_words<NGW>(reinterpret_cast<const uint16_t*>(p), s);
        load_words<NGW>(reinterpret_cast<const uint16_t*>(p + bias_off), b);
    }
};
template <int NGW, int KPW, int NP>
struct ScaleRegs<false, NGW, KPW, NP> {
    uint32_t s[KPW][NP], b[KPW][NP];
    __device__ __forceinline__ void from_lds(const uint8_t*, int64_t) {}  // not used by the scalar form
};

// Weight words and raw scale/bias values of one tile for one lane.
template <bool VEC, int NGW, int KPW, int NW, int NP>
struct TileRegs {
    uint32_t w[KPW][NW];
    ScaleRegs<VEC, NGW, KPW, NP> sb;
    uint4 sch;  // cooperative form: this lane's chunk of the tile's scale/bias block
};

// LDS of one wavefront: its activation rows for its part of K (row stride
// padded by 16 bytes so that rows fall in different banks), staged once; the
// first 2 KB later hold its two partial-tile buffers (parities).
__host__ __device__ constexpr int xs_row_elems(int kpw, int kblk) { return kpw * kblk + 8; }
__host__ __device__ inline int wave_lds_bytes(int M, int kpw, int kblk) {
    const int x = M * xs_row_elems(kpw, kblk) * 2;
    return x > 2048 ? x : 2048;
}

// Whole-line weight loads (single-tile 4-bit vector form).  In the matrix-core
// layout a lane's 16 bytes of a k-block sit in the row of its tile column, so
// a wavefront's fragment loads touch 16 rows x 64 bytes -- half lines -- per
// instruction.  Here the wavefront loads its K range of the tile's 16 rows as
// whole 128-byte lines instead (consecutive lanes, consecutive 16-byte
// pieces of a row), writes them to its own LDS region (over its staged
// activations, which it has read back by then; rows padded by 16 bytes) and
// reads its fragments from there: no barrier, the region is the
// wavefront's own.  Measured against the fragment loads on one box (graph-
// replayed, alternated): verify 4096^2 at M = 1 / 4 / 6 / 8 4.78 / 4.85-4.91
// / 4.93 / 5.04 vs 5.06-5.10 / 5.12-5.14 / 5.14-5.16 / 5.20-5.23 us, but
// 12- and 16-row blocks 0.06-0.2 us slower (their activation staging keeps
// the LDS busy), so the host launches it for one block of at most 8 rows.
// (4- and 8-bit codes: a k-block is 64 bytes of a row, a lane's quarter 16.)
template <int BITS, bool MULTI, bool VEC>
__host__ __device__ constexpr bool reg_wl() {
    return !MULTI && VEC && (BITS == 4 || BITS == 8);
}
// bytes of one staged row: the wavefront's k-blocks, plus padding
__host__ __device__ constexpr int wl_row_bytes(int kpw, int kblk_bytes) { return kpw * kblk_bytes + 16; }
template <int BITS, bool MULTI, bool VEC>
__host__ __device__ inline int reg_wave_lds(int M, int kpw, int kblk) {
    const int x = wave_lds_bytes(M, kpw, kblk);
    const int w = reg_wl<BITS, MULTI, VEC>() ? 16 * wl_row_bytes(kpw, kblk * BITS / 8) : 0;
    return x > w ? x : w;
}

// Cooperative form of the scales and biases (multi-tile workgroups of the
// vector form): the 16 rows x G values of a tile are one contiguous block per
// array; the workgroup fetches it with one 16-byte chunk per lane (a few
// lines in all, instead of one line per row per wavefront) and keeps it in
// LDS: two tile parities x two arrays x 16 rows, row stride 2G + 16 bytes.
__host__ __device__ inline int64_t sb_row_bytes(int64_t G) { return 2 * G + 16; }

// Prefetch distance in tiles: two where the register budget allows.
template <int DT, int BITS, int GS, int KPW, bool VEC>
__host__ __device__ constexpr int reg_lead() {
    return (VEC && KPW * Fmt<DT, BITS, GS>::SEG_WORDS <= 8) ? 2 : 1;
}
// Cooperative scale/bias blocks (vector form) need a tile of lead: the chunk
// of tile t + step is staged to LDS at the end of tile t, so it is loaded an
// iteration earlier -- with that tile's weights at prefetch distance 2, in a
// ring of its own two tiles ahead at distance 1.
template <int DT, int BITS, int GS, int KPW, bool VEC>
__host__ __device__ constexpr bool reg_coop() {
    return VEC;
}
__host__ __device__ inline int64_t sb_lds_bytes(int64_t G) { return 4 * 16 * sb_row_bytes(G); }

// Weights through LDS (multi-tile 4-bit kernels).  Loaded straight into
// registers, a wavefront's slice of a tile arrives as 16 rows x 64 bytes per
// instruction -- the matrix-core layout puts the 16 tile columns on
// consecutive lanes -- and half-line requests cap a long stream near 5.7 TB/s
// on MI355X against 6.7-6.9 TB/s for whole 128-byte lines.  Here each
// wavefront brings its slice in with direct global-to-LDS loads whose
// consecutive lanes cover whole lines, into a ring of slots of its own, and
// reads its fragments from there; the prefetch ring then costs LDS instead
// of registers.  A tile's slot is read into registers before the slot is
// refilled, so as many tiles as slots are in flight during the compute.
// Activations are read in fragment order once per kernel (no staging area).
//
// 4-bit: 3 slots of 16 rows x RS bytes (2 KiB at K = 4096).  8-bit: a slot
// is 4 KiB at K = 4096, so 2 slots, and the partial-tile buffers keep only
// rows 0..7 (M <= 8, a separate instantiation, MH) to fit 160 KiB of LDS.
template <int DT, int BITS, int GS, int KPW, bool VEC, bool MULTI, bool MH>
__host__ __device__ constexpr bool reg_dma() {
    return MULTI && VEC && (BITS == 4 || (BITS == 8 && MH));
}
template <int BITS>
__host__ __device__ constexpr int dma_slots() {
    return BITS == 4 ? 3 : 2;
}
// per wavefront: the two partial-tile buffers (all 16 rows, or rows 0..7)
__host__ __device__ constexpr int dma_wave_lds(bool mh) { return mh ? 1024 : 2048; }
// bytes of one slot: 16 rows x the wavefront's KPW k-blocks
template <int DT, int BITS, int GS, int KPW>
__host__ __device__ constexpr int dma_slot_bytes() {
    return 16 * KPW * Fmt<DT, BITS, GS>::KBLK * BITS / 8;
}
// Scale/bias blocks of the DMA form, one more than the slots (a block is read
// by every wavefront, so it is refilled only after the next barrier): the
// tile's 16 rows of scales then of biases, rows of 2G bytes (unpadded) whose
// 16-byte pieces are swizzled like the weight slots.
__host__ __device__ inline int64_t dma_sb_block_bytes(int64_t G) { return 2 * 16 * 2 * G; }

// One direct global-to-LDS load: 16 bytes per active lane, lane q to
// lds_dst + 16 q, non-temporal.  Written as assembly on purpose: for a
// global-to-LDS load the compiler knows of, it waits for every such load
// before any later LDS read, which would drain the prefetch ring each tile.
// Callers wait explicitly (s_waitcnt vmcnt, in-order retirement).  M0 (the
// LDS address) is used by nothing else in these kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// base: a 64-bit address, the same in every lane (moved to scalar
// registers here); voff: this lane's byte offset from it; m0: the LDS byte
// address of lane 0's 16 bytes (the same in every lane).
//
// NT: non-temporal (each weight line is read once).  Without it (row-block
// grids) L2 keeps the line for the other row blocks of the same column slot.
template <bool NT = true>
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t m0) {
    // (readfirstlane returns a signed int: each half goes through uint32_t so
    // that widening cannot sign-extend the low word over the high one)
    const uint64_t b = reinterpret_cast<uintptr_t>(base);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b)));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32)));
    const uint64_t sb = (static_cast<uint64_t>(hi) << 32) | lo;
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                     :
                     : "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(voff), "s"(sb)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :
                     : "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(voff), "s"(sb)
                     : "memory", "m0");
}
#pragma clang diagnostic pop

// W wavefronts per workgroup; wavefront w owns the KPW consecutive k-blocks
// [w*KPW, (w+1)*KPW) of K.  One workgroup owns a tile of 16 columns at a
// time and walks tiles blockIdx.x, blockIdx.x + gridDim.x, ...; the loads of
// the next tile are in flight while a tile is computed (two register buffers
// used in turn).
//
// The tile loop is written so that no wait on a load can be forced early:
// loaded registers are not touched in the iteration that issues them (the
// memory counter retires in order, so an early use would also wait for every
// later load), prefetches are unconditional (past the workgroup's last tile
// they re-read its current tile, which was just fetched) and pinned ahead of
// the compute, and nothing on the weight side is masked: positions beyond K
// read valid addresses and meet zero activations.
//
// K split (SPLIT, weights-through-LDS form only): slice blockIdx.y covers K
// positions [s K, (s + 1) K) of rows ldk long, and the workgroup leaves an
// fp32 partial output in part[s][M][N] instead of y; a second kernel adds
// the slices in order.  Unsplit: ldk = K, part unused.
//
// Row blocks (ROWS, not with SPLIT): M up to 64, workgroup (., ., z)
// computes rows [16 z, 16 z + 16) -- its own activation rows -- of every
// column tile of its slot (LDS-ring form) or of its one tile (single-tile
// form).  The row blocks of a column slot or tile have linear workgroup ids
// congruent mod 8, so they run on one XCD: a tile's weights come from HBM
// once and from that XCD's L2 for the others (cached loads, not streamed).
//
// Sub-slices (V > 1, single-tile forms only): a wavefront does the work of V
// wavefronts of the W*V-wavefront form -- V consecutive runs of KPW / V
// k-blocks, each with its own unit sums, unit product and partial tile --
// and the partials are combined in the same order, so the results are
// bit-identical to that form (and to its multi-tile, batched and row-block
// relatives) with fewer, longer wavefronts.
template <int DT, int BITS, int GS, int W, int KPW, bool VEC, bool MULTI, bool MH, bool SPLIT, bool ROWS, int V = 1,
          bool WLT = false>
__global__ __launch_bounds__(64 * W, (64 * W >= 1024 ? 4 : 2)) void mfma_reg_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, uint16_t* __restrict__ y, int M, int64_t N, int64_t K, int64_t ldk,
    float* __restrict__ part) {
    using F = Fmt<DT, BITS, GS>;
    constexpr int LA = reg_lead<DT, BITS, GS, KPW, VEC>();
    constexpr bool COOP = MULTI && reg_coop<DT, BITS, GS, KPW, VEC>();
    constexpr int NG = (KPW * F::KBLK + GS - 1) / GS;  // groups touched by one wavefront (vector form)
    constexpr int NGW = NG >= 2 ? NG / 2 : 1;            // 32-bit words holding NG 16-bit values
    constexpr int NU = KPW * F::PORTIONS / V;            // units (portions) per sub-slice
    static_assert(NU <= 8, "the unit products use the first k-slot quarter only");
    static_assert(V == 1 || (V == 2 && !MULTI && !SPLIT && KPW % 2 == 0), "sub-slices: single-tile forms");
    constexpr int KPH = KPW / V;                         // k-blocks per sub-slice
    using Regs = TileRegs<VEC, NGW, KPW, F::SEG_WORDS, F::PORTIONS>;
    extern __shared__ __align__(16) uint8_t lds[];
    constexpr int XS_ROW = xs_row_elems(KPW, F::KBLK);
    constexpr bool DMA = reg_dma<DT, BITS, GS, KPW, VEC, MULTI, MH>();
    constexpr int DMA_SLOTS = dma_slots<BITS>();
    // partial-tile buffers: lanes stored per row quarter (rows 0..7 only: 32)
    constexpr int PL = DMA && MH ? 32 : 64;
    static_assert(!DMA || COOP, "the weight ring carries the cooperative scale/bias blocks");
    // (row blocks: sized for a whole block, the same in every workgroup)
    const int wave_lds = DMA ? dma_wave_lds(MH) : reg_wave_lds<BITS, MULTI, VEC>(ROWS ? 16 : M, KPW, F::KBLK);
    // (the whole-line form is its own instantiation, launched where it pays:
    // one block of at most 8 rows; with more rows the activation staging
    // keeps the LDS busy and the fragment loads are faster.  The LDS is
    // sized for it in either instantiation.)
    constexpr bool WL = reg_wl<BITS, MULTI, VEC>() && WLT && !ROWS;
    static_assert(!WL || (F::SEG_WORDS == 4 && F::SEG * BITS / 8 == 16 && F::KBLK * BITS / 8 == 64),
                  "whole-line staging: 64-byte k-blocks of four 16-byte quarters");

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane & 15;   // tile column of this lane's B operand / D output, row of its A operand
    const int jj = lane >> 4;  // k-slot quarter
    static_assert(!SPLIT || reg_dma<DT, BITS, GS, KPW, VEC, MULTI, MH>(), "the K split runs the LDS-ring form");
    static_assert(!ROWS || ((reg_dma<DT, BITS, GS, KPW, VEC, MULTI, MH>() || !MULTI) && !MH),
                  "row blocks run the LDS-ring form or one tile per workgroup, all 16 rows");
    const int m_all = M;  // rows of x and y (of each partial output when split)
    if constexpr (!SPLIT) {
        // batch entry blockIdx.y: dense [batch][...] arrays
        const int64_t be = blockIdx.y;
        x += be * m_all * K;
        wq += be * N * (K * BITS / 32);
        scales += be * N * (K / GS);
        biases += be * N * (K / GS);
        y += be * m_all * N;
    }
    int r0 = 0;           // first row of this workgroup's block
    if constexpr (ROWS) {
        r0 = 16 * static_cast<int>(blockIdx.z);
        x += static_cast<int64_t>(r0) * ldk;
        y += static_cast<int64_t>(r0) * N;
        M = M - r0 < 16 ? M - r0 : 16;
    }
    if constexpr (SPLIT) {
        const int64_t sk = static_cast<int64_t>(blockIdx.y) * K;
        x += sk;
        wq += sk * BITS / 32;
        scales += sk / GS;
        biases += sk / GS;
    }
    if constexpr (!SPLIT) ldk = K;  // (unsplit: the same value, known to the compiler as K)
    const int64_t row_words = ldk * BITS / 32;
    const int64_t G = K / GS;     // groups of a row within the K range (the LDS block layout)
    const int64_t Gf = ldk / GS;  // scale/bias row stride
    const int64_t ntiles = (N + 15) / 16;
    const int64_t kb0 = static_cast<int64_t>(wave) * KPW;

    // Tile addressing: a uniform base (scalar registers) plus a per-lane
    // offset fixed for the whole kernel.  The last tile of a ragged N is
    // shifted back to end at column N, so no lane ever reads past the last
    // row; the columns it shares with the previous tile are recomputed and
    // stored again with bit-identical values.  (N < 16: lanes clamp instead.)
    const int64_t row_bytes = row_words * 4;
    const bool narrow = N < 16;
    const uint32_t lane_row = narrow ? static_cast<uint32_t>(min(static_cast<int64_t>(c), N - 1)) : c;
    const uint32_t w_off = lane_row * static_cast<uint32_t>(row_bytes) +
                           static_cast<uint32_t>((kb0 * F::KBLK + jj * F::SEG) * BITS / 8);
    const uint32_t s_off = lane_row * static_cast<uint32_t>(G) + static_cast<uint32_t>(kb0 * F::KBLK / GS);
    // whole-line form: load j, lane l takes 16-byte piece (64 j + l) of the
    // wavefront's range, row-major over the tile's 16 rows (PPR pieces a row)
    constexpr int PPR = KPW * F::KBLK * BITS / 128;
    uint32_t wl_off[KPW];
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
        const int pc = 64 * j + lane;
        const int64_t row = narrow ? min(static_cast<int64_t>(pc / PPR), N - 1) : static_cast<int64_t>(pc / PPR);
        wl_off[j] = static_cast<uint32_t>(row) * static_cast<uint32_t>(row_bytes) +
                    static_cast<uint32_t>(kb0 * F::KBLK * BITS / 8 + (pc % PPR) * 16);
    }
    auto tile_col0 = [&](int64_t tile) -> int64_t {
        const int64_t c0 = tile * 16;
        return (narrow || c0 + 16 <= N) ? c0 : N - 16;
    };

    // this lane's chunk of the cooperative block: array, row in the tile,
    // 16-byte chunk in the row (chunks per wavefront <= 64)
    uint8_t* const sblk = lds + static_cast<int64_t>(W) * wave_lds;
    const int64_t sb_row = sb_row_bytes(G);
    const int sc_cpw = COOP ? static_cast<int>(4 * G / W) : 0;
    const bool sc_on = lane < sc_cpw;
    const int sc_q = wave * sc_cpw + lane;
    const int sc_arr = COOP ? sc_q / static_cast<int>(2 * G) : 0;
    const int sc_row = COOP ? (sc_q % static_cast<int>(2 * G)) / static_cast<int>(G / 8) : 0;
    const int sc_cc = COOP ? (sc_q % static_cast<int>(2 * G)) % static_cast<int>(G / 8) : 0;
    const uint16_t* const sc_src = sc_arr ? biases : scales;
    auto stage_scales = [&](uint4 chunk, int par) __attribute__((always_inline)) {
        if (sc_on)
            *reinterpret_cast<uint4*>(sblk + ((par * 2 + sc_arr) * 16 + sc_row) * sb_row + sc_cc * 16) = chunk;
    };

    // Weight ring (DMA form): slot s of this wavefront holds its slice of one
    // tile, 16 rows x RS bytes, as 16-byte pieces at position
    // row * NP + (piece ^ swz(row)); the swizzle spreads the 16 rows that
    // one fragment read touches over distinct banks.  Load instruction i
    // fills positions 64 i .. 64 i + 63, lane q position 64 i + q, so each
    // row's consecutive lanes read that row's slice -- whole lines.
    constexpr int RS = KPW * F::KBLK * BITS / 8;  // bytes of a row in this wavefront's slice
    constexpr int NP = RS / 16;                    // 16-byte pieces per row of the slice
    constexpr int NI = DMA ? 16 * NP / 64 : 1;     // load instructions per slot
    constexpr int SLOT = dma_slot_bytes<DT, BITS, GS, KPW>();
    static_assert(!DMA || (NP >= 4 && 16 * NP % 64 == 0 && F::SEG * BITS / 8 == 16),
                  "a slot is whole load instructions; a lane's segment is one piece");
    auto swz = [](int row) { return ((row * NP) >> 4) & (NP - 1); };
    const int64_t sb_blk = dma_sb_block_bytes(G);
    const int PR = static_cast<int>(G / 8);  // 16-byte pieces per scale row
    auto sb_swz = [PR](int row) { return ((row * PR) >> 4) & (PR - 1); };
    uint8_t* const ring = lds + static_cast<int64_t>(W) * wave_lds +
                          (DMA ? (DMA_SLOTS + 1) * sb_blk : COOP ? sb_lds_bytes(G) : 0) +
                          static_cast<int64_t>(wave) * DMA_SLOTS * SLOT;
    // DMA addressing: per lane a 32-bit byte offset fixed for the kernel, per
    // tile a uniform base (scalar registers).  (These kernels run only when N
    // spans many tiles, so a tile's 16 rows never pass N.)
    uint32_t dma_off[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int p = 64 * i + lane;
        const int row = p / NP, piece = (p % NP) ^ swz(p / NP);
        dma_off[i] = static_cast<uint32_t>(row) * static_cast<uint32_t>(row_bytes) +
                     static_cast<uint32_t>(kb0 * F::KBLK * BITS / 8 + piece * 16);
    }
    // this wavefront's chunks all lie in one array (2G / sc_cpw = W / 2
    // wavefronts per array): scales for the first half, biases for the rest
    const uint8_t* const sb_arr = reinterpret_cast<const uint8_t*>(wave < W / 2 ? scales : biases);
    const uint32_t ch_off = static_cast<uint32_t>(sc_row * 2 * Gf + (sc_cc ^ sb_swz(sc_row)) * 16);
    // LDS byte addresses (M0) of this wavefront's slot 0 and of its chunk
    // position in block 0
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t*)(lds))));
    const uint32_t m0_ring = lds0 + __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(ring - lds));
    const uint32_t m0_sb = lds0 + __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(sblk - lds + 16 * wave * sc_cpw));
    const int nfull = static_cast<int>(N / 16);     // tiles that end at or before column N
    const int lastc = static_cast<int>(N - 16);    // first column of the shifted last tile

    // coop: the scale/bias chunk first (so that waiting for it does not wait
    // for the weights), else per-lane scale/bias words after the weights
    auto load_chunk = [&](int64_t tile, uint4& dst) __attribute__((always_inline)) {
        if (sc_on) {
            const int64_t col0 = tile_col0(tile);
            const int64_t srow = col0 + sc_row < N ? col0 + sc_row : N - 1;
            dst = *reinterpret_cast<const uint4*>(sc_src + srow * G + sc_cc * 8);
        }
    };
    // DMA form: 1 + NI load instructions per tile, in this order: this
    // wavefront's chunks of the scale/bias block (position sc_q of block
    // `blk`), then its weight slice (slot `slot`)
    auto dma_col0 = [&](int tile) -> int { return tile < nfull ? tile * 16 : lastc; };
    // Past the workgroup's last tile the ring still issues its loads (the
    // waits count them), from the first KiB of the workgroup's first tile
    // instead: inside the array (these forms run only where N spans many
    // 16-row tiles, and a tile's 16 rows hold at least 1 KiB) and a
    // different line per workgroup -- one KiB shared by every workgroup made
    // a hot spot of their last iterations.  Those slots are never read.
    const uint32_t dummy_off = static_cast<uint32_t>(lane) * 16;
    const uint8_t* const dummy_src =
        reinterpret_cast<const uint8_t*>(wq) + static_cast<int64_t>(dma_col0(static_cast<int>(blockIdx.x))) * row_bytes;
    // (two branches on a uniform condition, not selects: a select between
    // the offsets makes the compiler index a stack copy of dma_off)
    auto dma_tile = [&](int tile, int slot, int blk) __attribute__((always_inline)) {
        const uint32_t m0w = m0_ring + static_cast<uint32_t>(slot * SLOT);
        const uint32_t m0s = m0_sb + static_cast<uint32_t>(blk * sb_blk);
        if (tile < static_cast<int>(ntiles)) {
            const int64_t col0 = dma_col0(tile);
            if (sc_on) dma16<!ROWS>(sb_arr + col0 * Gf * 2, ch_off, m0s);
            const uint8_t* wt = reinterpret_cast<const uint8_t*>(wq) + col0 * row_bytes;
#pragma unroll
            for (int i = 0; i < NI; ++i) dma16<!ROWS>(wt, dma_off[i], m0w + 1024 * i);
        } else {
            if (sc_on) dma16(dummy_src, dummy_off, m0s);
#pragma unroll
            for (int i = 0; i < NI; ++i) dma16(dummy_src, dummy_off, m0w + 1024 * i);
        }
    };
    auto load_tile = [&](int64_t tile, Regs& r, int slot, auto coop_tag) __attribute__((always_inline)) {
        constexpr bool coop = decltype(coop_tag)::value;
        const int64_t col0 = tile_col0(tile);
        if constexpr (coop && LA == 2) load_chunk(tile, r.sch);
        const uint8_t* wbase = reinterpret_cast<const uint8_t*>(wq) + col0 * row_bytes;
#pragma unroll
        for (int i = 0; i < KPW; ++i) {
            if constexpr (WL) {
                load_segment<BITS, F::SEG_WORDS, !ROWS>(reinterpret_cast<const uint32_t*>(wbase + wl_off[i]), r.w[i]);
            } else if constexpr (VEC) {
                // VEC: the k-blocks cover K exactly
                load_segment<BITS, F::SEG_WORDS, !ROWS>(
                    reinterpret_cast<const uint32_t*>(wbase + w_off + i * (F::KBLK * BITS / 8)), r.w[i]);
            } else {
                int64_t code0 = (kb0 + i) * F::KBLK + jj * F::SEG;
                code0 = code0 < K ? code0 : K - F::SEG;
                load_segment<BITS, F::SEG_WORDS, !ROWS>(
                    reinterpret_cast<const uint32_t*>(wbase + lane_row * row_bytes + code0 * BITS / 8), r.w[i]);
            }
        }
        if constexpr (coop) {
        } else if constexpr (VEC) {
            const uint16_t* sbase = scales + col0 * G;
            const uint16_t* bbase = biases + col0 * G;
            load_words<NGW>(sbase + s_off, r.sb.s);
            load_words<NGW>(bbase + s_off, r.sb.b);
        } else {
#pragma unroll
            for (int i = 0; i < KPW; ++i)
#pragma unroll
                for (int p = 0; p < F::PORTIONS; ++p) {
                    int64_t g = ((kb0 + i) * F::KBLK + static_cast<int64_t>(p) * F::PC) / GS;
                    g = g < G ? g : G - 1;
                    r.sb.s[i][p] = scales[(col0 + lane_row) * G + g];
                    r.sb.b[i][p] = biases[(col0 + lane_row) * G + g];
                }
        }
    };

    // MULTI: workgroups walk several tiles (prefetch, cooperative scale/bias
    // blocks where the form allows); otherwise each owns exactly one tile
    // (the grid covers N) and loads its scales per lane.  Separate kernels,
    // so that each has straight-line loads and its own register allocation.
    const int64_t step = gridDim.x;
    auto body = [&](auto coop_tag) __attribute__((always_inline)) {
        constexpr bool coop = decltype(coop_tag)::value;
        Regs buf[LA + 1];
        int64_t tile = blockIdx.x;
        uint4 xraw[KPW][F::STEPS];
        if constexpr (DMA) {
            // ---- prologue (weight ring).  The first tile goes to slot (and
            // block) 0, then the activations are read straight in fragment
            // order (once per kernel, from L2 after the first workgroups).
            // The next tiles are issued once the activations are in: the
            // wait for them would otherwise also wait for those tiles.
            dma_tile(static_cast<int>(blockIdx.x), 0, 0);
            // every lane loads (rows past M re-read row M - 1 and are zeroed
            // after the conversion below): a conditional load merged with a
            // zero makes the compiler wait for it right away
            const int64_t crow = c < M ? c : M - 1;
    #pragma unroll
            for (int i = 0; i < KPW; ++i)
    #pragma unroll
                for (int s = 0; s < F::STEPS; ++s) {
                    const int kk = i * F::KBLK + F::src_lane(s, jj) * F::SEG + F::src_slot(s, jj) * 8;
                    xraw[i][s] = *reinterpret_cast<const uint4*>(x + crow * ldk + kb0 * F::KBLK + kk);
                }
        } else {
            // ---- prologue.  This wavefront's activation rows [0, M) x its part of
            // K are read with coalesced 16-byte loads (whole lines, every lane busy)
            // ahead of the first tile's weights, then staged through its own LDS
            // region and read back in fragment order.  Positions >= K are zero.
            //
            // Four wavefronts share a SIMD here and all of them run this
            // prologue before their weight loads go out, so its vector
            // instructions are kept few: load j covers rows RPJ j .. RPJ j +
            // RPJ - 1 (a uniform branch skips loads wholly past row M - 1),
            // addressed as a uniform base plus a 32-bit lane offset; nothing
            // is zero-filled that no later step reads.
            constexpr int CPR = KPW * F::KBLK / 8;  // 16-byte chunks per row of the slice
            static_assert(64 % CPR == 0, "a load instruction covers whole rows of the slice");
            constexpr int RPJ = 64 / CPR;           // rows per load instruction
            constexpr int XG = 16 / RPJ;
            const int lrow = lane / CPR, piece = lane % CPR;
            u32x4_t xg[XG];
            if constexpr (VEC) {
                // (the k-blocks cover K exactly; an element not loaded is
                // never read, so it starts as whatever its register holds)
                const uint32_t xoff = static_cast<uint32_t>(
                    (static_cast<int64_t>(lrow) * K + kb0 * F::KBLK + piece * 8) * 2);
    #pragma unroll
                for (int j = 0; j < XG; ++j) {
                    xg[j] = __builtin_nondeterministic_value(xg[0]);
                    if (RPJ * j < M) {
                        const uint8_t* xb = reinterpret_cast<const uint8_t*>(x) + static_cast<int64_t>(RPJ * j) * K * 2;
                        if (RPJ * j + lrow < M) xg[j] = *reinterpret_cast<const u32x4_t*>(xb + xoff);
                    }
                }
            } else {
                const int64_t k = kb0 * F::KBLK + piece * 8;
    #pragma unroll
                for (int j = 0; j < XG; ++j) {
                    const int row = RPJ * j + lrow;
                    xg[j] = u32x4_t{0u, 0u, 0u, 0u};
                    if (row < M && k < K) xg[j] = *reinterpret_cast<const u32x4_t*>(x + static_cast<int64_t>(row) * K + k);
                }
            }
            load_tile(tile, buf[0], 0, coop_tag);
            __builtin_amdgcn_sched_barrier(0);

            uint16_t* xs = reinterpret_cast<uint16_t*>(lds + wave * wave_lds);
    #pragma unroll
            for (int j = 0; j < XG; ++j) {
                if (RPJ * j < M) {
                    if (RPJ * j + lrow < M) *reinterpret_cast<u32x4_t*>(xs + (RPJ * j + lrow) * XS_ROW + piece * 8) = xg[j];
                }
            }
            // Rows past M - 1 re-read row M - 1: the matrix-core products keep
            // rows apart, and those output rows are never stored.
            const int xrow = c < M ? c : M - 1;
    #pragma unroll
            for (int i = 0; i < KPW; ++i)
    #pragma unroll
                for (int s = 0; s < F::STEPS; ++s) {
                    const int kk = i * F::KBLK + F::src_lane(s, jj) * F::SEG + F::src_slot(s, jj) * 8;
                    xraw[i][s] = *reinterpret_cast<const uint4*>(xs + xrow * XS_ROW + kk);
                }
        }

        Frag xa[KPW][F::STEPS];
    #pragma unroll
        for (int i = 0; i < KPW; ++i)
    #pragma unroll
            for (int s = 0; s < F::STEPS; ++s) {
                xa[i][s] = x_frag<BITS, DT>(xraw[i][s]);
                if constexpr (DMA) {
                    if (c >= M)
    #pragma unroll
                        for (int v = 0; v < 4; ++v) xa[i][s].v[v] = 0u;
                }
            }

        // Unit sums X_u = sum x and O_u = sum x*off of row c over each unit of
        // this wavefront, on the matrix cores: with B = the activation fragment
        // of a step (B[k][c] = x[c][k], the same register that serves as A) and
        // A = a pattern with row u all ones and row 8 + u holding the offsets of
        // the k-slots (u = the step's unit), one product per step accumulates
        // D[u][c] = X_u[c] and D[8 + u][c] = O_u[c].  A lane (column c, quarter
        // jj) receives rows 4jj..4jj+3: X_0..3, X_4..7, O_0..3, O_4..7 for
        // jj = 0..3.
        //
        // Both unit products then fold into one matrix-core step with 32 k-slots
        // (8 per quarter): the A operand "xo" of lane (row c, quarter q) holds
        // units 0..7 of X_hi (q = 0), O_hi (q = 1), X_lo (q = 2), O_lo (q = 3),
        // where hi + lo splits an fp32 sum into two 16-bit values; the matching
        // B operand holds b_u in the even quarters and -s_u in the odd ones.
        //
        // fp16 (largest finite value 65504): O_u reaches 65504 already for a
        // unit sum of 64 in the activations, so the sums of row c are scaled
        // by a power of two 2^-e_c (per row, over this wavefront's units)
        // that puts the largest |X_u|, |O_u| in [2^14, 2^15) before the
        // split; the step's result for row r is then multiplied back by
        // 2^e_r (ufac, exact).  bf16 has fp32's exponent range: no scaling.
        Frag xo[V];
        float ufac[V][4];  // fp16: 2^e of output rows 4jj..4jj+3
    #pragma unroll
        for (int h = 0; h < V; ++h) {
            const int arow = lane & 15;  // A-operand row this lane supplies
            float4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
    #pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int i = h * KPH + u / F::PORTIONS, p = u % F::PORTIONS;
                Frag e;
    #pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const uint32_t ones = DtBits<DT>::one * 0x10001u;
                    const uint32_t offs = DtBits<DT>::of(slot_off<DT, BITS, GS>(2 * v)) |
                                          (DtBits<DT>::of(slot_off<DT, BITS, GS>(2 * v + 1)) << 16);
                    e.v[v] = arow == u ? ones : (arow == 8 + u ? offs : 0u);
                }
    #pragma unroll
                for (int st = 0; st < F::STEPS_PER_PORTION; ++st) d = mfma<DT>(e, xa[i][p * F::STEPS_PER_PORTION + st], d);
            }
            const int src = (jj & 1) ? 32 : 0;  // X rows (lanes 0..31) or O rows (lanes 32..63)
            float v8[8];
    #pragma unroll
            for (int r = 0; r < 4; ++r) {
                v8[r] = __shfl(d[r], (lane & 15) + src, 64);
                v8[4 + r] = __shfl(d[r], (lane & 15) + src + 16, 64);
            }
            float vscale = 1.0f;
    #pragma unroll
            for (int r = 0; r < 4; ++r) ufac[h][r] = 1.0f;
            if constexpr (DT == DT_F16) {
                // lanes c, c + 32 hold X of row c, lanes c + 16, c + 48 its O
                float m = 0.0f;
    #pragma unroll
                for (int u = 0; u < NU; ++u) m = fmaxf(m, fabsf(v8[u]));
                m = fmaxf(m, __shfl_xor(m, 16, 64));
                int ex = 0;
                (void)frexpf(m, &ex);  // m in [2^(ex-1), 2^ex) (ex = 0 for m = 0)
                vscale = ldexpf(1.0f, 15 - ex);
                const float inv = ldexpf(1.0f, ex - 15);
    #pragma unroll
                for (int r = 0; r < 4; ++r) ufac[h][r] = __shfl(inv, 4 * jj + r, 64);
            }
            const bool lo_part = jj >= 2;
    #pragma unroll
            for (int e = 0; e < 8; e += 2) {
                uint32_t h16[2];
    #pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int u = e + t;
                    const float v = u < NU ? v8[u] * vscale : 0.0f;
                    const uint32_t hi = DtOps<DT>::rne(v);
                    const uint32_t lo = DtOps<DT>::rne(v - DtOps<DT>::to_f32(static_cast<uint16_t>(hi)));
                    h16[t] = lo_part ? lo : hi;
                }
                xo[h].v[e / 2] = h16[0] | (h16[1] << 16);
            }
        }
        const UnpackConsts uk = unpack_consts<DT>();

        // 16-bit scale or bias of unit (portion p of k-block i) of this wavefront
        auto unit_value = [&](const Regs& r, bool want_scale, int i, int p) -> uint32_t {
            if constexpr (VEC) {
                const int gi = (i * F::KBLK + p * F::PC) / GS;  // compile-time after unrolling
                const uint32_t w = want_scale ? r.sb.s[gi >> 1] : r.sb.b[gi >> 1];
                return (w >> (16 * (gi & 1))) & 0xFFFFu;
            } else {
                return (want_scale ? r.sb.s[i][p] : r.sb.b[i][p]) & 0xFFFFu;
            }
        };
        // B operand of the folded unit product of sub-slice h: lane (column c,
        // quarter q) holds b_u (q even) or -s_u (q odd) of its units
        // 0..NU-1 (zero beyond NU; -s is exact: a sign flip).
        auto unit_frag = [&](const Regs& r, int h) -> Frag {
            Frag f;
            const bool odd = (jj & 1) != 0;
    #pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int u0 = 2 * v, u1 = u0 + 1;
                const int i0 = h * KPH + u0 / F::PORTIONS, i1 = h * KPH + u1 / F::PORTIONS;
                const uint32_t b0 = u0 < NU ? unit_value(r, false, i0, u0 % F::PORTIONS) : 0u;
                const uint32_t b1 = u1 < NU ? unit_value(r, false, i1, u1 % F::PORTIONS) : 0u;
                const uint32_t s0 = u0 < NU ? unit_value(r, true, i0, u0 % F::PORTIONS) : 0u;
                const uint32_t s1 = u1 < NU ? unit_value(r, true, i1, u1 % F::PORTIONS) : 0u;
                const uint32_t bias = b0 | (b1 << 16);
                const uint32_t nscale = (s0 | (s1 << 16)) ^ 0x80008000u;
                f.v[v] = odd ? nscale : bias;
            }
            return f;
        };

        int parity = 0;
        auto compute_store = [&](int64_t col0, Regs& r, int slot, uint4 next_chunk, auto coop_tag) __attribute__((always_inline)) {
            constexpr bool coop = decltype(coop_tag)::value;
            if constexpr (coop && !DMA) {
                // this wavefront's scales and biases of tile t, from the block in LDS
                r.sb.from_lds(sblk + (parity * 2 * 16 + c) * sb_row + (kb0 * F::KBLK / GS) * 2, 16 * sb_row);
            }
            if constexpr (WL) {
                // whole lines -> this wavefront's LDS region -> fragment order
                // (lane (c, jj) of k-block i: row c, bytes 64 i + 16 jj)
                constexpr int WRS = wl_row_bytes(KPW, F::KBLK * BITS / 8);
                uint8_t* ws = lds + wave * wave_lds;
    #pragma unroll
                for (int j = 0; j < KPW; ++j) {
                    const int pc = 64 * j + lane;
                    *reinterpret_cast<uint4*>(ws + (pc / PPR) * WRS + (pc % PPR) * 16) =
                        make_uint4(r.w[j][0], r.w[j][1], r.w[j][2], r.w[j][3]);
                }
    #pragma unroll
                for (int i = 0; i < KPW; ++i) {
                    const uint4 v = *reinterpret_cast<const uint4*>(ws + c * WRS + i * (F::KBLK * BITS / 8) + jj * 16);
                    r.w[i][0] = v.x; r.w[i][1] = v.y; r.w[i][2] = v.z; r.w[i][3] = v.w;
                }
            }
            float4_t yacc[V];
    #pragma unroll
            for (int h = 0; h < V; ++h) yacc[h] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    #pragma unroll
            for (int i = 0; i < KPW; ++i) {
                const int h = i / KPH;
                Frag bw[F::STEPS];
                segment_frags<DT, BITS, GS>(r.w[i], bw, uk);
    #pragma unroll
                for (int p = 0; p < F::PORTIONS; ++p) {
                    float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    #pragma unroll
                    for (int st = 0; st < F::STEPS_PER_PORTION; ++st) {
                        const int s = p * F::STEPS_PER_PORTION + st;
                        acc = mfma<DT>(xa[i][s], bw[s], acc);
                    }
                    const float sc = DtOps<DT>::to_f32(static_cast<uint16_t>(unit_value(r, true, i, p)));
    #pragma unroll
                    for (int q = 0; q < 4; ++q) yacc[h][q] = __fmaf_rn(sc, acc[q], yacc[h][q]);
                }
            }
            // unit products: + sum_u b_u X_u - sum_u s_u O_u, one step per
            // sub-slice (fp16: on the scaled sums, then scaled back per row)
    #pragma unroll
            for (int h = 0; h < V; ++h) {
                if constexpr (DT == DT_F16) {
                    const float4_t t = mfma<DT>(xo[h], unit_frag(r, h), float4_t{0.0f, 0.0f, 0.0f, 0.0f});
    #pragma unroll
                    for (int q = 0; q < 4; ++q) yacc[h][q] = __fmaf_rn(ufac[h][q], t[q], yacc[h][q]);
                } else {
                    yacc[h] = mfma<DT>(xo[h], unit_frag(r, h), yacc[h]);
                }
            }
            // the next tile's scale/bias block to the other parity; the barrier
            // below publishes it.  That buffer was last read in the previous
            // tile, before the previous barrier.
            if constexpr (coop && !DMA) stage_scales(next_chunk, parity ^ 1);
            // Combine the wavefronts' partial sums: every wavefront writes its
            // partial to the buffer of this tile's parity at the start of its own
            // LDS region (over its staged activations, which it has read by then;
            // layout [q][lane], conflict-free); after one barrier wavefronts 0..3
            // each sum one of the four D rows a lane holds and store it.  The
            // next tile writes the other buffer, and the tile after that can only
            // write this one after passing the next barrier, which the reducing
            // wavefronts reach only after reading.  Cooperative scale/bias blocks
            // follow the same parity.  (Sub-slices, single tile: partial h
            // in buffer h, read in the order of the wavefronts they stand for.)
            float* rb = reinterpret_cast<float*>(lds + wave * wave_lds) + parity * 4 * PL;
            if (lane < PL) {
    #pragma unroll
                for (int h = 0; h < V; ++h)
    #pragma unroll
                    for (int q = 0; q < 4; ++q) rb[h * 4 * PL + q * PL + lane] = yacc[h][q];
            }
            if constexpr (DMA) {
                // (after the partial's stores, so after the compute) this
                // wavefront's chunks of the next tile's block have landed: after
                // them come its weight slice and the DMA_SLOTS - 1 tiles after,
                // NI + (DMA_SLOTS - 1) (1 + NI) loads.  The barrier publishes
                // the block.
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NI + (DMA_SLOTS - 1) * (1 + NI)) : "memory");
            }
            __syncthreads();
            if (wave < 4 && lane < PL) {
                const int q = wave;
                float v = 0.0f;
    #pragma unroll
                for (int w = 0; w < W; ++w)
    #pragma unroll
                    for (int h = 0; h < V; ++h)
                        v += reinterpret_cast<const float*>(lds + w * wave_lds)[(parity + h) * 4 * PL + q * PL + lane];
                const int64_t col = col0 + c;
                const int row = 4 * jj + q;
                if (col < N && row < M) {
                    if constexpr (SPLIT)
                        part[(static_cast<int64_t>(blockIdx.y) * m_all + r0 + row) * N + col] = v;
                    else
                        y[static_cast<int64_t>(row) * N + col] = DtOps<DT>::rne(v);
                }
            }
            parity ^= 1;
        };

        if constexpr (!MULTI) {  // a single tile: nothing to prefetch
            compute_store(tile_col0(tile), buf[0], 0, buf[0].sch, coop_tag);
            return;
        }
        if constexpr (DMA) {
            // tiles 1 .. DMA_SLOTS - 1 to their slots; then the first tile has
            // landed once only their loads may be outstanding (the
            // activations, issued after it, were already waited for), and
            // the barrier publishes its scale/bias block.  Each later block
            // is published by the loop, one tile ahead.
    #pragma unroll
            for (int a = 1; a < DMA_SLOTS; ++a)
                dma_tile(static_cast<int>(blockIdx.x) + a * static_cast<int>(gridDim.x), a, a);
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"((DMA_SLOTS - 1) * (1 + NI)) : "memory");
            __syncthreads();
            const int nt = static_cast<int>(ntiles), stp = static_cast<int>(gridDim.x);
            int t = static_cast<int>(blockIdx.x);
            int blk = 0;  // scale/bias block of the current tile
            while (t < nt) {
    #pragma unroll
                for (int u = 0; u < DMA_SLOTS; ++u) {
                    // Tile t (slot u) has landed once every load but those of
                    // the DMA_SLOTS - 1 tiles after it has retired (the counter
                    // retires loads in order; the compiler does not track these,
                    // hence the explicit waits, which also keep the LDS reads
                    // below from moving above them).
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((DMA_SLOTS - 1) * (1 + NI)) : "memory");
                    Regs& r = buf[0];
                    const uint8_t* sl = ring + u * SLOT;
    #pragma unroll
                    for (int i = 0; i < KPW; ++i) {
                        const int piece = (i * F::KBLK + jj * F::SEG) * BITS / 128;
                        const uint4 v = *reinterpret_cast<const uint4*>(sl + 16 * (c * NP + (piece ^ swz(c))));
                        r.w[i][0] = v.x; r.w[i][1] = v.y; r.w[i][2] = v.z; r.w[i][3] = v.w;
                    }
                    // this wavefront's NG scales and biases of tile t (2 NG bytes
                    // inside one piece of row c)
                    static_assert(2 * NG <= 16, "a wavefront's groups lie in one piece");
                    const int gb = static_cast<int>(kb0 * F::KBLK / GS) * 2;  // byte offset in the row
                    r.sb.from_lds(sblk + blk * sb_blk + c * 2 * G + ((gb >> 4) ^ sb_swz(c)) * 16 + (gb & 15), 32 * G);
                    // the slot is refilled only after its reads have completed
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                    dma_tile(t + DMA_SLOTS * stp, u, blk == 0 ? DMA_SLOTS : blk - 1);  // (blk + DMA_SLOTS) mod (DMA_SLOTS + 1)
                    __builtin_amdgcn_sched_barrier(0);
                    compute_store(dma_col0(t), r, u, r.sch, coop_tag);
                    blk = blk == DMA_SLOTS ? 0 : blk + 1;
                    t += stp;
                    if (t >= nt) break;
                }
            }
            // no global-to-LDS load may still be in flight when the
            // workgroup's LDS is released
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            return;
        }
        // the tiles after the first up to the prefetch distance (buf[0] holds
        // the first); past the workgroup's last tile these re-read the first
    #pragma unroll
        for (int a = 1; a < LA; ++a) {
            const int64_t t_a = tile + a * step;
            load_tile(t_a < ntiles ? t_a : tile, buf[a], a, coop_tag);
        }
        // distance 1: the chunks of the first two tiles (then two ahead)
        uint4 sch2[2];
        if constexpr (coop && LA == 1) {
            load_chunk(tile, sch2[0]);
            load_chunk(tile + step < ntiles ? tile + step : tile, sch2[1]);
        }
        // the first tile's scale/bias block, published before the tile loop
        if constexpr (coop) {
            stage_scales(LA == 2 ? buf[0].sch : sch2[0], 0);
            __syncthreads();
        }
        // buffers rotate: tile t + a*step lives in buf[(u + a) % (LA + 1)]
        while (tile < ntiles) {
    #pragma unroll
            for (int u = 0; u <= LA; ++u) {
                // past the last tile of this workgroup the prefetch re-reads the
                // tile just loaded (cache hits) instead of another workgroup's
                const int64_t next = tile + LA * step;
                if constexpr (coop && LA == 1) {
                    // slot u held this tile's chunk, staged an iteration ago
                    const int64_t next2 = tile + 2 * step;
                    load_chunk(next2 < ntiles ? next2 : tile, sch2[u]);
                }
                load_tile(next < ntiles ? next : tile, buf[(u + LA) % (LA + 1)], (u + LA) % (LA + 1), coop_tag);
                // keep the prefetch ahead of the compute: left alone, the
                // scheduler sinks these loads past it to shorten live ranges
                __builtin_amdgcn_sched_barrier(0);
                compute_store(tile_col0(tile), buf[u], u, LA == 2 ? buf[(u + 1) % (LA + 1)].sch : sch2[(u + 1) % 2], coop_tag);
                tile += step;
                if (tile >= ntiles) break;
            }
        }
    };
    body(std::integral_constant<bool, COOP>{});

}

// The lane-quarter and step parts of a fragment's source position must be
// separable for the fixed-offset LDS reads above.
template <int DT, int BITS, int GS>
constexpr bool separable_sources() {
    using F = Fmt<DT, BITS, GS>;
    for (int jj = 0; jj < 4; ++jj)
        for (int s = 0; s < F::STEPS; ++s) {
            const int full = F::src_lane(s, jj) * F::SEG + F::src_slot(s, jj) * 8;
            const int split = F::src_lane(0, jj) * F::SEG + F::src_slot(0, jj) * 8 +
                              (F::src_lane(s, 0) - F::src_lane(0, 0)) * F::SEG +
                              (F::src_slot(s, 0) - F::src_slot(0, 0)) * 8;
            if (full != split) return false;
        }
    return true;
}
static_assert(separable_sources<0, 4, 32>() && separable_sources<0, 4, 64>() && separable_sources<0, 4, 128>() &&
                  separable_sources<0, 6, 32>() && separable_sources<0, 6, 64>() && separable_sources<0, 8, 32>() &&
                  separable_sources<0, 8, 128>(),
              "fragment source positions must be separable");

// Launch shape: waves per workgroup and k-blocks per wavefront (W*KPW
// k-blocks cover K), and whether the scale/bias vectors can be loaded whole.
// The activation fragments of KPW k-blocks live in registers, so KPW stays
// small: 16 wavefronts cover K = 4096 at two (4-bit) or four (6/8-bit)
// k-blocks each.
struct RegShape {
    int W, KPW;
    bool vec;
};

inline int64_t kblk_of(int bits) { return bits == 4 ? 128 : 64; }

inline bool pick_shape(int bits, int gs, int64_t K, RegShape& s) {
    const int64_t kblk = kblk_of(bits);
    const int64_t nkb = (K + kblk - 1) / kblk;
    static const int shapes[][2] = {{4, 1}, {8, 1}, {16, 1}, {16, 2}, {16, 4}};
    for (const auto& sh : shapes) {
        const int W = sh[0], KPW = sh[1];
        if (bits == 4 && KPW > 2) continue;  // 4-bit fragments of 4 k-blocks exceed the register budget
        if (static_cast<int64_t>(W) * KPW < nkb) continue;
        const int64_t portions = kblk / gs > 1 ? kblk / gs : 1;
        if (KPW * portions > 8) continue;  // unit products: at most 8 units per wavefront
        const int64_t G = K / gs;
        const int64_t ng = (KPW * kblk + gs - 1) / gs;
        const int64_t vec_vals = ng >= 8 ? 8 : ng;  // 16-bit values per vector load
        s = {W, KPW, W * KPW == nkb && KPW * kblk % gs == 0 && G % vec_vals == 0 && ng % 2 == 0 && G % 8 == 0 &&
                         4 * G <= 64 * W};
        return true;
    }
    return false;
}

// workgroups resident at once on 256 CUs (16 wavefronts per CU); each walks
// ntiles / grid tiles
inline int64_t reg_grid(int64_t ntiles, int W) {
    const int64_t resident = 256 * (16 / W);
    return ntiles < resident ? ntiles : resident;
}
// row-block grids: column slots per row block, a multiple of 8 so that the
// row blocks of a slot (linear ids slot + k * slots) share an XCD
inline int64_t reg_rows_grid(int rb) { return (256 / rb) / 8 * 8; }

// Row blocks (M 17..64): the LDS-ring form (4-bit, vector form, 16
// wavefronts) with more column tiles than slots.
inline bool reg_rows_shape(int bits, int gs, int64_t M, int64_t N, int64_t K, RegShape& s) {
    if (bits != 4 || M <= 16 || M > 64) return false;
    if (!pick_shape(bits, gs, K, s) || !s.vec || s.W != 16) return false;
    return (N + 15) / 16 > reg_rows_grid(static_cast<int>((M + 15) / 16));
}

// Row blocks, one tile per workgroup (M 17..64, any width, vector form, 16
// wavefronts): where the shape at 16 rows is single-tile (no more column
// tiles than resident workgroups) and the LDS-ring row blocks do not apply;
// the grid is tiles x blocks.
inline bool reg_rows1_shape(int bits, int gs, int64_t M, int64_t N, int64_t K, RegShape& s) {
    if (M <= 16 || M > 64 || reg_rows_shape(bits, gs, M, N, K, s)) return false;
    if (!pick_shape(bits, gs, K, s) || !s.vec || s.W != 16) return false;
    const int64_t ntiles = (N + 15) / 16;
    return ntiles <= reg_grid(ntiles, s.W);
}

// dynamic LDS bytes of one workgroup
template <int DT, int BITS, int GS, int W, int KPW, bool VEC, bool MULTI, bool MH>
size_t reg_lds_bytes(int64_t M, int64_t K) {
    constexpr bool dma = reg_dma<DT, BITS, GS, KPW, VEC, MULTI, MH>();
    constexpr size_t DMA_SLOTS = static_cast<size_t>(dma_slots<BITS>());
    const size_t wave_lds =
        dma ? dma_wave_lds(MH) : reg_wave_lds<BITS, MULTI, VEC>(static_cast<int>(M), KPW, Fmt<DT, BITS, GS>::KBLK);
    return static_cast<size_t>(W) * wave_lds +
           (dma ? (DMA_SLOTS + 1) * static_cast<size_t>(dma_sb_block_bytes(K / GS))
            : MULTI && reg_coop<DT, BITS, GS, KPW, VEC>() ? static_cast<size_t>(sb_lds_bytes(K / GS))
                                                           : 0) +
           (dma ? static_cast<size_t>(W) * DMA_SLOTS * dma_slot_bytes<DT, BITS, GS, KPW>() : 0);
}

// Launch over K range kr of rows a.K long: kr = a.K unsplit, a.K / S split
// S ways (grid.y = S, each slice with its share of the resident workgroups).
template <int DT, int BITS, int GS, int W, int KPW, bool VEC, bool MULTI, bool MH, bool SPLIT = false,
          bool ROWS = false, int V = 1, bool WLT = false>
hipError_t launch_shape_m(const MatmulArgs& a, int64_t kr) {
    const int S = SPLIT ? a.split : 1;
    const int RB = ROWS ? static_cast<int>((a.M + 15) / 16) : 1;
    const int64_t ntiles = (a.N + 15) / 16;
    // batch entries (grid.y, unsplit) share the resident workgroups of a
    // multi-tile grid
    const int64_t nb = SPLIT ? 1 : a.batch;
    int64_t grid = SPLIT  ? 256 * (16 / W) / (S * RB)
                   : ROWS ? (MULTI ? reg_rows_grid(RB) : ntiles)
                          : reg_grid(ntiles, W);
    if (MULTI && !SPLIT && nb > 1) {
        if (ROWS) {
            // the row blocks of a slot share an XCD when slots x entries is a
            // multiple of 8 (linear ids then congruent mod 8): the most slots
            // per entry within the resident workgroups that keep that
            grid = (256 / RB) / nb;
            while (grid > 1 && grid * nb % 8 != 0) --grid;
            if (grid < 1) grid = 1;
        } else {
            grid = 256 * (16 / W) / nb;
            if (grid < 1) grid = 1;
            if (grid > ntiles) grid = ntiles;
        }
    }
    if (MULTI && a.N < 16) return hipErrorInvalidValue;  // (the shifted last tile)
    // (the LDS-ring row blocks need more column tiles than column slots: the
    // unsplit grid's slots, or a split's share of the resident workgroups,
    // as reg_rows_shape / reg_split_shape require)
    if (ROWS && (a.M <= 16 || a.M > 64 ||
                 (MULTI ? ntiles <= (SPLIT ? grid : reg_rows_grid(RB)) : ntiles > reg_grid(ntiles, W))))
        return hipErrorInvalidValue;
    if (nb < 1 || nb > 65535 || (SPLIT && a.batch != 1)) return hipErrorInvalidValue;
    if (MH && a.M > 8) return hipErrorInvalidValue;  // partial tiles keep rows 0..7 only
    if (SPLIT && (grid < 1 || S < 2 || kr * S != a.K || a.part == nullptr)) return hipErrorInvalidValue;
    const size_t lds = reg_lds_bytes<DT, BITS, GS, W, KPW, VEC, MULTI, MH>(ROWS ? 16 : a.M, kr);
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    if (lds > 65536) {
        // above the default dynamic-LDS limit: raise it once per kernel and device
        static std::atomic<uint64_t> raised{0};
        if (hipError_t e = raise_lds_limit(
                reinterpret_cast<const void*>(&mfma_reg_kernel<DT, BITS, GS, W, KPW, VEC, MULTI, MH, SPLIT, ROWS, V, WLT>),
                raised);
            e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((mfma_reg_kernel<DT, BITS, GS, W, KPW, VEC, MULTI, MH, SPLIT, ROWS, V, WLT>),
                       dim3(static_cast<unsigned>(grid), static_cast<unsigned>(SPLIT ? S : nb),
                            static_cast<unsigned>(RB)),
                       dim3(64 * W), lds, a.stream,
                       static_cast<const uint16_t*>(a.x), a.wq, static_cast<const uint16_t*>(a.scales),
                       static_cast<const uint16_t*>(a.biases), static_cast<uint16_t*>(a.y), static_cast<int>(a.M), a.N,
                       kr, a.K, a.part);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    if constexpr (SPLIT) return launch_reduce_partials(DT, a.part, a.y, S, a.M * a.N, a.stream);
    return hipSuccess;
}

template <int DT, int BITS, int GS, int W, int KPW, bool VEC>
hipError_t launch_shape(const MatmulArgs& a) {
    // the tiles of every batch entry against the resident workgroups (the
    // multi-tile forms shift a ragged last tile back to end at column N, so
    // entries narrower than a tile stay single-tile)
    const int64_t ntiles = (a.N + 15) / 16 * (a.N >= 16 ? a.batch : 1);
    if (ntiles > reg_grid(ntiles, W)) {
        // 8-bit vector form at M <= 8: weights through LDS (partial tiles of
        // rows 0..7) where that fits in LDS (not gs32 at K = 4096); otherwise
        // the register-prefetch form
        if constexpr (BITS == 8 && VEC)
            if (a.M <= 8 && reg_lds_bytes<DT, BITS, GS, W, KPW, VEC, true, true>(a.M, a.K) <= 160 * 1024)
                return launch_shape_m<DT, BITS, GS, W, KPW, VEC, true, true>(a, a.K);
        return launch_shape_m<DT, BITS, GS, W, KPW, VEC, true, false>(a, a.K);
    }
    if constexpr (reg_wl<BITS, false, VEC>())
        if (a.M <= 8) return launch_shape_m<DT, BITS, GS, W, KPW, VEC, false, false, false, false, 1, true>(a, a.K);
    return launch_shape_m<DT, BITS, GS, W, KPW, VEC, false, false>(a, a.K);
}

// K split: the LDS-ring form (4-bit, vector form, 16 wavefronts) on slices
// of K / split (and, above 16 rows, 16-row blocks), each (slice, row block)
// with 256 / (split x blocks) workgroups walking more column tiles than that.
inline bool reg_split_shape(int bits, int gs, int64_t M, int64_t N, int64_t K, int split, RegShape& s) {
    if (bits != 4 || M < 1 || M > 64 || split < 2 || K % split != 0) return false;
    if (!pick_shape(bits, gs, K / split, s) || !s.vec || s.W != 16) return false;
    const int64_t ntiles = (N + 15) / 16;
    const int64_t per = 256 * (16 / s.W) / (split * ((M + 15) / 16));  // resident workgroups per (slice, block)
    return per >= 1 && ntiles > per;
}

// One tile per workgroup (single-tile forms, alone or on 16-row blocks): 8
// wavefronts of two sub-slices each instead of 16 wavefronts of kpw
// k-blocks, bit-identical to them.  A wavefront's per-lane scale/bias
// gathers touch one line per tile row whatever its share of K, so halving
// the wavefronts halves those requests.  Measured over every format at
// N = 1024 / 4096, K = 2048 / 4096, M = 6 / 16: faster for groups of 64 and
// 128 (up to 0.7 us at 16 rows); groups of 32, with twice the unit sums per
// sub-slice, lose at 6 rows and keep 16 wavefronts.
template <int DT, int BITS, int GS, bool ROWS>
hipError_t launch_single_halved(const MatmulArgs& a, int kpw) {
    // (4/8-bit, one block of at most 8 rows: the whole-line instantiation)
    if constexpr (reg_wl<BITS, false, true>() && !ROWS)
        if (a.M <= 8) {
            if (kpw == 1) return launch_shape_m<DT, BITS, GS, 8, 2, true, false, false, false, false, 2, true>(a, a.K);
            if (kpw == 2) return launch_shape_m<DT, BITS, GS, 8, 4, true, false, false, false, false, 2, true>(a, a.K);
            if constexpr (BITS != 4)
                if (kpw == 4) return launch_shape_m<DT, BITS, GS, 8, 8, true, false, false, false, false, 2, true>(a, a.K);
        }
    if (kpw == 1) return launch_shape_m<DT, BITS, GS, 8, 2, true, false, false, false, ROWS, 2>(a, a.K);
    if (kpw == 2) return launch_shape_m<DT, BITS, GS, 8, 4, true, false, false, false, ROWS, 2>(a, a.K);
    if constexpr (BITS != 4)
        if (kpw == 4) return launch_shape_m<DT, BITS, GS, 8, 8, true, false, false, false, ROWS, 2>(a, a.K);
    return hipErrorInvalidValue;
}

template <int DT, int BITS, int GS>
hipError_t launch_reg_t(const MatmulArgs& a) {
    RegShape s;
    if (a.M > 16 && a.split > 1) {
        if (!reg_split_shape(BITS, GS, a.M, a.N, a.K, a.split, s)) return hipErrorInvalidValue;
        if constexpr (BITS == 4) {
            const int64_t kr = a.K / a.split;
            if (s.KPW == 1) return launch_shape_m<DT, BITS, GS, 16, 1, true, true, false, true, true>(a, kr);
            if (s.KPW == 2) return launch_shape_m<DT, BITS, GS, 16, 2, true, true, false, true, true>(a, kr);
        }
        return hipErrorInvalidValue;
    }
    if (a.M > 16) {
        if (reg_rows_shape(BITS, GS, a.M, a.N, a.K, s)) {
            if constexpr (BITS == 4) {
                if (s.KPW == 1) return launch_shape_m<DT, BITS, GS, 16, 1, true, true, false, false, true>(a, a.K);
                if (s.KPW == 2) return launch_shape_m<DT, BITS, GS, 16, 2, true, true, false, false, true>(a, a.K);
            }
            return hipErrorInvalidValue;
        }
        if (!reg_rows1_shape(BITS, GS, a.M, a.N, a.K, s)) return hipErrorInvalidValue;
        if constexpr (GS >= 64) return launch_single_halved<DT, BITS, GS, true>(a, s.KPW);
        if (s.KPW == 1) return launch_shape_m<DT, BITS, GS, 16, 1, true, false, false, false, true>(a, a.K);
        if (s.KPW == 2) return launch_shape_m<DT, BITS, GS, 16, 2, true, false, false, false, true>(a, a.K);
        if constexpr (BITS != 4)
            if (s.KPW == 4) return launch_shape_m<DT, BITS, GS, 16, 4, true, false, false, false, true>(a, a.K);
        return hipErrorInvalidValue;
    }
    if (a.split > 1) {
        if (!reg_split_shape(BITS, GS, a.M, a.N, a.K, a.split, s)) return hipErrorInvalidValue;
        if constexpr (BITS == 4) {
            const int64_t kr = a.K / a.split;
            if (s.KPW == 1) return launch_shape_m<DT, BITS, GS, 16, 1, true, true, false, true>(a, kr);
            if (s.KPW == 2) return launch_shape_m<DT, BITS, GS, 16, 2, true, true, false, true>(a, kr);
        }
        return hipErrorInvalidValue;
    }
    if (!pick_shape(BITS, GS, a.K, s)) return hipErrorInvalidValue;
    if constexpr (GS >= 64) {
        const int64_t nt = (a.N + 15) / 16 * (a.N >= 16 ? a.batch : 1);
        if (s.W == 16 && s.vec && nt <= reg_grid(nt, 16)) return launch_single_halved<DT, BITS, GS, false>(a, s.KPW);
    }
    switch (s.W * 100 + s.KPW * 2 + (s.vec ? 1 : 0)) {
        case 402: return launch_shape<DT, BITS, GS, 4, 1, false>(a);
        case 403: return launch_shape<DT, BITS, GS, 4, 1, true>(a);
        case 802: return launch_shape<DT, BITS, GS, 8, 1, false>(a);
        case 803: return launch_shape<DT, BITS, GS, 8, 1, true>(a);
        case 1602: return launch_shape<DT, BITS, GS, 16, 1, false>(a);
        case 1603: return launch_shape<DT, BITS, GS, 16, 1, true>(a);
        case 1604: return launch_shape<DT, BITS, GS, 16, 2, false>(a);
        case 1605: return launch_shape<DT, BITS, GS, 16, 2, true>(a);
        case 1608:
            if constexpr (BITS != 4) return launch_shape<DT, BITS, GS, 16, 4, false>(a);
            return hipErrorInvalidValue;
        case 1609:
            if constexpr (BITS != 4) return launch_shape<DT, BITS, GS, 16, 4, true>(a);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Launch for one activation dtype and code width (every group size); each
// is compiled in a translation unit of its own (qmm_mfma_reg_<dt>_<bits>.hip)
// so that the library's largest kernel family builds in parallel.
hipError_t launch_mfma_reg_f16_4(const MatmulArgs& a);
hipError_t launch_mfma_reg_f16_6(const MatmulArgs& a);
hipError_t launch_mfma_reg_f16_8(const MatmulArgs& a);
hipError_t launch_mfma_reg_bf16_4(const MatmulArgs& a);
hipError_t launch_mfma_reg_bf16_6(const MatmulArgs& a);
hipError_t launch_mfma_reg_bf16_8(const MatmulArgs& a);

// Body of those launchers: the group size picks the instantiation.
#define QMM_REG_FMT_LAUNCHER(NAME, DTV, BITSV)                \
    hipError_t NAME(const MatmulArgs& a) {                    \
        switch (a.gs) {                                       \
            case 32: return launch_reg_t<DTV, BITSV, 32>(a);  \
            case 64: return launch_reg_t<DTV, BITSV, 64>(a);  \
            case 128: return launch_reg_t<DTV, BITSV, 128>(a); \
            default: return hipErrorInvalidValue;             \
        }                                                     \
    }

}  // namespace qmm
