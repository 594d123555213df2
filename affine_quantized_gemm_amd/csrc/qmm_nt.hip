// Non-transposed product: y[M, N] = x[M, K] . dequant(W)[K, N], with W
// stored [K, N] and quantized along N -- row k of W is a packed bitstream of
// N codes with one scale and bias per group of gs consecutive columns
// (scales, biases [K, N/gs]).  This is the other orientation of the call in
// MLX issue #4720, "Describe the bug" (there: transposed weights).
//
// Here the reduction runs down the rows of W, so a column's codes are not
// contiguous.  One workgroup owns 16 output columns (inside one group, since
// gs >= 32) for all of K; its 16 wavefronts take 32-row steps in turn:
//   * a lane loads the 8 codes of row k0 + l/2, columns 8 (l % 2) .. + 8
//     (4 / 6 / 8 bytes), and widens 6/8-bit codes to bytes;
//   * an 8 x 8 transpose among the 8 lanes of equal (l / 16, l % 2) (three
//     swizzle-and-merge stages, no LDS; on nibbles in one word for 4-bit
//     codes, on bytes in two words otherwise) leaves lane l with the codes
//     of rows k0 + 8 (l / 16) .. + 8 of one column: the MFMA B operand.  The
//     column a lane holds is c(p) = 8 (p % 2) + p / 2 for p = l % 16, a fixed
//     relabeling undone at the store;
//   * the lane dequantizes them, w = s q + b (the scale and bias of each of
//     its 8 rows): fp16 with packed fp16 arithmetic, rounded once; bf16 in
//     fp32 to hi = RNE_bf16(w), the dequantizer's value, and
//     lo = RNE_bf16(w - hi): with
//     bf16's 8-bit significand one rounding of w and one of y could together
//     exceed the accepted error, hi + lo carries w to about u^2;
//   * partial 16 x 16 tiles of the wavefronts are added through LDS and
//     rounded once.
// The scales and biases of the workgroup's group are staged in LDS for up
// to 4096 rows at a time.  Column blocks that share 128-byte weight lines
// run on one XCD (block ids congruent mod 8), so the lines come from HBM once.
#include "qmm.h"
#include "qmm_internal.hpp"
#include "qmm_mfma_frag.hpp"

namespace qmm {
namespace {

using mf::Frag;
using mf::float4_t;

constexpr int NT_W = 16;     // wavefronts per workgroup
constexpr int NT_KC = 4096;  // rows of scales and biases staged at a time

// partner value for the transpose: lane l ^ D (D < 32)
template <int D>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(v), (D << 10) | 0x1F));
}

// The 8 codes of this lane's row and column half, as bytes (lo: columns
// 0..3, hi: 4..7 of the half).
template <int BITS>
__device__ __forceinline__ void load_codes(const uint32_t* __restrict__ row, int64_t n0, int h, uint32_t& lo,
                                           uint32_t& hi) {
    if constexpr (BITS == 4) {  // (kept as nibbles: transposed as such)
        lo = row[n0 / 8 + h];
        hi = 0u;
    } else if constexpr (BITS == 8) {
        lo = row[n0 / 4 + 2 * h];
        hi = row[n0 / 4 + 2 * h + 1];
    } else {
        // 16 columns = 3 words; this half's 48 bits start at bit 48 h
        const int64_t base = n0 / 16 * 3 + h;
        const uint64_t u = (static_cast<uint64_t>(row[base + 1]) << 32 | row[base]) >> (16 * h);
        uint32_t b[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) b[c] = static_cast<uint32_t>(u >> (6 * c)) & 63u;
        lo = b[0] | b[1] << 8 | b[2] << 16 | b[3] << 24;
        hi = b[4] | b[5] << 8 | b[6] << 16 | b[7] << 24;
    }
}

// The same as two parts: the words holding the codes (loaded ahead), then
// the widening to bytes.
template <int BITS>
__device__ __forceinline__ void load_words(const uint32_t* __restrict__ row, int64_t n0, int h, uint32_t& a,
                                           uint32_t& b) {
    if constexpr (BITS == 4) {
        a = row[n0 / 8 + h];
        b = 0u;
    } else if constexpr (BITS == 8) {
        a = row[n0 / 4 + 2 * h];
        b = row[n0 / 4 + 2 * h + 1];
    } else {
        a = row[n0 / 16 * 3 + h];
        b = row[n0 / 16 * 3 + h + 1];
    }
}

template <int BITS>
__device__ __forceinline__ void widen_words(uint32_t a, uint32_t b, int h, uint32_t& lo, uint32_t& hi) {
    if constexpr (BITS == 4) {  // (kept as nibbles: transposed as such)
        lo = a;
        hi = 0u;
    } else if constexpr (BITS == 8) {
        lo = a;
        hi = b;
    } else {
        const uint64_t u = (static_cast<uint64_t>(b) << 32 | a) >> (16 * h);
        uint32_t c8[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) c8[c] = static_cast<uint32_t>(u >> (6 * c)) & 63u;
        lo = c8[0] | c8[1] << 8 | c8[2] << 16 | c8[3] << 24;
        hi = c8[4] | c8[5] << 8 | c8[6] << 16 | c8[7] << 24;
    }
}

// one merge stage of the transpose on one word: lanes whose row bit is
// clear keep their low part and take the partner's low part shifted up;
// the others take the partner's high part shifted down and keep their own
template <int LANE_DIST, uint32_t MASK, int SHIFT>
__device__ __forceinline__ uint32_t merge(uint32_t v, bool upper) {
    const uint32_t p = xor_lane<LANE_DIST>(v);
    return upper ? ((p >> SHIFT) & MASK) | (v & ~MASK) : (v & MASK) | ((p & MASK) << SHIFT);
}

// The 8 x 8 transpose of a lane group's codes: afterwards lane r holds rows
// 0..7 of column r.  Bytes (6/8-bit, widened) in two words, lo = columns /
// rows 0..3 and hi = 4..7; 4-bit codes as nibbles in one word, row i at
// bits 4 i (three stages on one word instead of widening first).
template <int BITS>
__device__ __forceinline__ void transpose_codes(uint32_t& lo, uint32_t& hi, int r) {
    if constexpr (BITS == 4) {
        lo = merge<8, 0x0000FFFFu, 16>(lo, (r & 4) != 0);
        lo = merge<4, 0x00FF00FFu, 8>(lo, (r & 2) != 0);
        lo = merge<2, 0x0F0F0F0Fu, 4>(lo, (r & 1) != 0);
    } else {
        // rows r, r ^ 4 (lanes 8 apart): swap the 4-column halves
        const uint32_t plo = xor_lane<8>(lo), phi = xor_lane<8>(hi);
        if (r & 4) lo = phi;
        else hi = plo;
        lo = merge<4, 0x0000FFFFu, 16>(lo, (r & 2) != 0);
        hi = merge<4, 0x0000FFFFu, 16>(hi, (r & 2) != 0);
        lo = merge<2, 0x00FF00FFu, 8>(lo, (r & 1) != 0);
        hi = merge<2, 0x00FF00FFu, 8>(hi, (r & 1) != 0);
    }
}

// 8 codes (bytes, rows e = 0..7) -> the dequantized weights w = s q + b in
// fp32 (s, b: 8 packed dt values each), as MFMA operands: hi = RNE_dt(w)
// (the dequantizer's value) and, for bf16, lo = RNE_dt(w - hi), so that
// hi + lo carries w to about u^2
template <int DT, int BITS>
__device__ __forceinline__ void dequant_frags(uint32_t lo8, uint32_t hi8, const uint32_t (&sw)[4],
                                              const uint32_t (&bw)[4], Frag& fh, Frag& fl) {
    if constexpr (BITS == 4 && DT == DT_F16) {
        // nibbles: 1024 + q for rows 2i, 2i + 1 from bits 8 i .. 8 i + 7
        typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
        const half2_t off = {static_cast<_Float16>(1024.0f), static_cast<_Float16>(1024.0f)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t a = lo8 >> (8 * i);
            const uint32_t d = 0x64006400u | (a & 0xFu) | ((a << 12) & 0xF0000u);
            const half2_t q = __builtin_bit_cast(half2_t, d) - off;
            const half2_t v = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, sw[i]), q,
                                                        __builtin_bit_cast(half2_t, bw[i]));
            fh.v[i] = __builtin_bit_cast(uint32_t, v);
            fl.v[i] = 0u;
        }
        return;
    }
    if constexpr (BITS == 4) {  // bf16: nibbles to bytes, then as below
        auto spread = [](uint32_t t) {
            return (t & 0xFu) | ((t & 0xF0u) << 4) | ((t & 0xF00u) << 8) | ((t & 0xF000u) << 12);
        };
        const uint32_t w = lo8;
        lo8 = spread(w & 0xFFFFu);
        hi8 = spread(w >> 16);
    }
    if constexpr (DT == DT_F16) {
        // packed fp16: two codes at a time become 1024 + q (a byte permute
        // under the exponent byte 0x64), minus 1024 gives q exactly, and one
        // fused multiply-add with the (already packed) scale and bias pair
        // rounds s q + b once to fp16 -- within one fp16 rounding of w, as
        // the fp32 route is
        typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
        const half2_t off = {static_cast<_Float16>(1024.0f), static_cast<_Float16>(1024.0f)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = i < 2 ? lo8 : hi8;
            const uint32_t b0 = 2u * static_cast<uint32_t>(i & 1);
            const uint32_t sel = b0 | (4u << 8) | ((b0 + 1u) << 16) | (4u << 24);
            const half2_t q = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, w, sel)) - off;
            const half2_t v = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, sw[i]), q,
                                                        __builtin_bit_cast(half2_t, bw[i]));
            fh.v[i] = __builtin_bit_cast(uint32_t, v);
            fl.v[i] = 0u;
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w = i < 2 ? lo8 : hi8;
        uint32_t hh = 0, ll = 0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float q = static_cast<float>((w >> (8 * (2 * (i & 1) + e))) & 0xFFu);
            const float v = __fmaf_rn(DtOps<DT>::to_f32(static_cast<uint16_t>(sw[i] >> (16 * e))), q,
                                      DtOps<DT>::to_f32(static_cast<uint16_t>(bw[i] >> (16 * e))));
            const uint16_t vh = DtOps<DT>::rne(v);
            hh |= static_cast<uint32_t>(vh) << (16 * e);
            if constexpr (DT == DT_BF16)
                ll |= static_cast<uint32_t>(DtOps<DT>::rne(v - DtOps<DT>::to_f32(vh))) << (16 * e);
        }
        fh.v[i] = hh;
        fl.v[i] = ll;
    }
}

template <int DT, int BITS, int RB>
__global__ __launch_bounds__(64 * NT_W, 4) void nt_kernel(const uint16_t* __restrict__ x,
                                                          const uint32_t* __restrict__ wq,
                                                          const uint16_t* __restrict__ scales,
                                                          const uint16_t* __restrict__ biases,
                                                          uint16_t* __restrict__ y, int M, int64_t N, int64_t K,
                                                          int gs) {
    extern __shared__ __align__(16) uint8_t lds[];
    uint16_t* const s_lds = reinterpret_cast<uint16_t*>(lds);
    uint16_t* const b_lds = s_lds + NT_KC;
    float* const red = reinterpret_cast<float*>(lds);  // (after the last step)

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nblk = static_cast<int>(N / 16);
    // column blocks sharing weight lines on one XCD
    const int bid = static_cast<int>(blockIdx.x);
    const int cb = nblk % 8 == 0 ? (bid % 8) * (nblk / 8) + bid / 8 : bid;
    const int64_t n0 = 16 * static_cast<int64_t>(cb);
    const int64_t G = N / gs;
    const int64_t g = n0 / gs;
    const int64_t row_words = N * BITS / 32;

    const int h = lane & 1;           // column half of this lane's load
    const int kk = lane >> 1;         // row of this lane's load in the step
    const int r = kk & 7;             // its row inside the 8 x 8 transpose
    const int p = lane & 15;          // MFMA column slot (column c(p))
    const int jq = lane >> 4;         // k-slot quarter / D row quarter

    float4_t acc[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) acc[b] = {0.0f, 0.0f, 0.0f, 0.0f};

    for (int64_t kc0 = 0; kc0 < K; kc0 += NT_KC) {
        const int kc = static_cast<int>(K - kc0 < NT_KC ? K - kc0 : NT_KC);
        for (int t = threadIdx.x; t < kc; t += 64 * NT_W) {
            s_lds[t] = scales[(kc0 + t) * G + g];
            b_lds[t] = biases[(kc0 + t) * G + g];
        }
        __syncthreads();
        for (int step = wave; step < kc / 32; step += NT_W) {
            const int64_t k0 = kc0 + 32 * static_cast<int64_t>(step);
            uint32_t lo, hi;
            load_codes<BITS>(wq + (k0 + kk) * row_words, n0, h, lo, hi);
            transpose_codes<BITS>(lo, hi, r);
            // this lane's 8 rows: scales and biases, and the dequantized weights
            const int kl = static_cast<int>(k0 - kc0) + 8 * jq;
            const uint4 sv = *reinterpret_cast<const uint4*>(s_lds + kl);
            const uint4 bv = *reinterpret_cast<const uint4*>(b_lds + kl);
            const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
            const uint32_t bw[4] = {bv.x, bv.y, bv.z, bv.w};
            Frag wh, wl;
            dequant_frags<DT, BITS>(lo, hi, sw, bw, wh, wl);
#pragma unroll
            for (int b = 0; b < RB; ++b) {
                const int m = 16 * b + p;
                uint4 xv = make_uint4(0u, 0u, 0u, 0u);
                if (m < M) xv = *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(m) * K + k0 + 8 * jq);
                Frag xf;
                xf.v[0] = xv.x; xf.v[1] = xv.y; xf.v[2] = xv.z; xf.v[3] = xv.w;
                acc[b] = mf::mfma<DT>(xf, wh, acc[b]);
                if constexpr (DT == DT_BF16) acc[b] = mf::mfma<DT>(xf, wl, acc[b]);
            }
        }
        __syncthreads();  // (the staged scales are overwritten next, or the buffer reused below)
    }

    // add the wavefronts' partial tiles: red[((w RB + b) 4 + q) 64 + lane]
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) red[((wave * RB + b) * 4 + q) * 64 + lane] = acc[b][q];
    __syncthreads();
    for (int t = threadIdx.x; t < RB * 4 * 64; t += 64 * NT_W) {
        const int ln = t & 63, q = (t >> 6) & 3, b = t >> 8;
        float v = 0.0f;
        for (int w = 0; w < NT_W; ++w) v += red[((w * RB + b) * 4 + q) * 64 + ln];
        const int m = 16 * b + 4 * (ln >> 4) + q;
        const int pp = ln & 15;
        const int64_t n = n0 + 8 * (pp & 1) + (pp >> 1);
        if (m < M) y[static_cast<int64_t>(m) * N + n] = DtOps<DT>::rne(v);
    }
}

// Wide form: one workgroup owns 128 columns (8 tiles of 16, 2 wavefronts
// per tile taking the steps in turn) of one slice of K (blockIdx.y), so that
// the 8 tiles' wavefronts share each 64-byte sector of 4-bit rows through the
// CU's L1 instead of 8 CUs each fetching it.  With more than one slice the
// workgroup leaves fp32 partial outputs part[slice][M][N], added in slice
// order by a second kernel.  Per chunk of 512 rows a wavefront issues all 8
// of its weight loads before computing, and the workgroup stages the
// chunk's activation rows in LDS, so that a chunk waits about one memory
// latency.
constexpr int NTW_TILES = 8;
constexpr int NTW_KW = NT_W / NTW_TILES;
constexpr int NTW_STEPS = 8;                       // 32-row steps of a wavefront per chunk
constexpr int NTW_KC = 32 * NTW_KW * NTW_STEPS;    // rows per chunk (512)
constexpr int NTW_XS = NTW_KC + 8;                 // activation row stride in LDS (16 bytes of padding)
constexpr int NTW_GMAX = 128 / 32;  // groups 128 columns span at most

template <int DT, int BITS, int RB, bool PART>
__global__ __launch_bounds__(64 * NT_W, 4) void nt_wide_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, uint16_t* __restrict__ y, float* __restrict__ part, int M, int64_t N,
    int64_t K, int gs, int64_t ks) {
    extern __shared__ __align__(16) uint8_t lds[];
    uint16_t* const s_lds = reinterpret_cast<uint16_t*>(lds);  // [NTW_GMAX][NTW_KC]
    uint16_t* const b_lds = s_lds + NTW_GMAX * NTW_KC;
    uint16_t* const x_lds = b_lds + NTW_GMAX * NTW_KC;        // [M][NTW_XS]
    float* const red = reinterpret_cast<float*>(lds);  // (after the last step)

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int tile = wave % NTW_TILES;
    const int kw = wave / NTW_TILES;
    const int64_t n0g = 128 * static_cast<int64_t>(blockIdx.x);
    const int64_t n0 = n0g + 16 * tile;
    const bool live = n0 < N;  // (uniform per wavefront: the last workgroup may hold 64 columns)
    const int64_t G = N / gs;
    const int64_t g0 = n0g / gs;
    const int wcols = static_cast<int>(N - n0g < 128 ? N - n0g : 128);
    const int gcount = (wcols + gs - 1) / gs;  // groups the workgroup's columns span
    const int gi = 16 * tile / gs;
    const int64_t row_words = N * BITS / 32;
    const int64_t kbeg = static_cast<int64_t>(blockIdx.y) * ks;
    const int64_t kend = kbeg + ks < K ? kbeg + ks : K;

    const int h = lane & 1;
    const int kk = lane >> 1;
    const int r = kk & 7;
    const int p = lane & 15;
    const int jq = lane >> 4;

    float4_t acc[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) acc[b] = {0.0f, 0.0f, 0.0f, 0.0f};

    for (int64_t kc0 = kbeg; kc0 < kend; kc0 += NTW_KC) {
        const int kc = static_cast<int>(kend - kc0 < NTW_KC ? kend - kc0 : NTW_KC);
        // this wavefront's weight loads of the chunk first (steps kw, kw + 2,
        // ...), all in flight together; then the chunk's activation rows and
        // scales and biases, staged in LDS by the whole workgroup
        const int nst = live ? (kc / 32 - kw + NTW_KW - 1) / NTW_KW : 0;
        uint32_t wa[NTW_STEPS], wb[NTW_STEPS];
#pragma unroll
        for (int i = 0; i < NTW_STEPS; ++i) {
            wa[i] = wb[i] = 0u;
            if (i < nst)
                load_words<BITS>(wq + (kc0 + 32 * static_cast<int64_t>(kw + i * NTW_KW) + kk) * row_words, n0, h,
                                 wa[i], wb[i]);
        }
        const int cpr = kc / 8;  // 16-byte pieces per activation row of the chunk
        for (int t = threadIdx.x; t < M * cpr; t += 64 * NT_W) {
            const int m = t / cpr, c8 = t % cpr;
            *reinterpret_cast<uint4*>(x_lds + m * NTW_XS + 8 * c8) =
                *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(m) * K + kc0 + 8 * c8);
        }
        for (int t = threadIdx.x; t < gcount * kc; t += 64 * NT_W) {
            const int gg = t / kc, k = t % kc;
            s_lds[gg * NTW_KC + k] = scales[(kc0 + k) * G + g0 + gg];
            b_lds[gg * NTW_KC + k] = biases[(kc0 + k) * G + g0 + gg];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NTW_STEPS; ++i) {
            if (i >= nst) break;
            const int kl0 = 32 * (kw + i * NTW_KW);  // step's first row in the chunk
            uint32_t lo, hi;
            widen_words<BITS>(wa[i], wb[i], h, lo, hi);
            transpose_codes<BITS>(lo, hi, r);
            const int kl = kl0 + 8 * jq;
            const uint4 sv = *reinterpret_cast<const uint4*>(s_lds + gi * NTW_KC + kl);
            const uint4 bv = *reinterpret_cast<const uint4*>(b_lds + gi * NTW_KC + kl);
            const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
            const uint32_t bw[4] = {bv.x, bv.y, bv.z, bv.w};
            Frag wh, wl;
            dequant_frags<DT, BITS>(lo, hi, sw, bw, wh, wl);
#pragma unroll
            for (int b = 0; b < RB; ++b) {
                const int m = 16 * b + p;
                uint4 xv = make_uint4(0u, 0u, 0u, 0u);
                if (m < M) xv = *reinterpret_cast<const uint4*>(x_lds + m * NTW_XS + kl);
                Frag xf;
                xf.v[0] = xv.x; xf.v[1] = xv.y; xf.v[2] = xv.z; xf.v[3] = xv.w;
                acc[b] = mf::mfma<DT>(xf, wh, acc[b]);
                if constexpr (DT == DT_BF16) acc[b] = mf::mfma<DT>(xf, wl, acc[b]);
            }
        }
        __syncthreads();
    }

    // the 2 wavefronts of each tile: red[((w RB + b) 4 + q) 64 + lane], w = kw * 8 + tile
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) red[((wave * RB + b) * 4 + q) * 64 + lane] = acc[b][q];
    __syncthreads();
    for (int t = threadIdx.x; t < NTW_TILES * RB * 4 * 64; t += 64 * NT_W) {
        const int ln = t & 63, q = (t >> 6) & 3, b = (t >> 8) % RB, tl = t / (256 * RB);
        const int64_t tn0 = n0g + 16 * tl;
        if (tn0 >= N) continue;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < NTW_KW; ++w) v += red[(((w * NTW_TILES + tl) * RB + b) * 4 + q) * 64 + ln];
        const int m = 16 * b + 4 * (ln >> 4) + q;
        const int pp = ln & 15;
        const int64_t n = tn0 + 8 * (pp & 1) + (pp >> 1);
        if (m < M) {
            if constexpr (PART)
                part[(static_cast<int64_t>(blockIdx.y) * M + m) * N + n] = v;
            else
                y[static_cast<int64_t>(m) * N + n] = DtOps<DT>::rne(v);
        }
    }
}

template <int DT, int BITS, int RB, bool PART>
hipError_t launch_nt_wide_t(const MatmulArgs& a, int split, int64_t ks) {
    const size_t lds_sb = 2 * NTW_GMAX * NTW_KC * sizeof(uint16_t) + 16 * RB * NTW_XS * sizeof(uint16_t);
    const size_t lds_red = static_cast<size_t>(NT_W) * RB * 4 * 64 * sizeof(float);
    const size_t lds = lds_sb > lds_red ? lds_sb : lds_red;
    if (lds > 65536) {
        // above the default dynamic-LDS limit: raise it once per kernel and device
        static std::atomic<uint64_t> raised{0};
        if (hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(&nt_wide_kernel<DT, BITS, RB, PART>), raised);
            e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((nt_wide_kernel<DT, BITS, RB, PART>),
                       dim3(static_cast<unsigned>((a.N + 127) / 128), static_cast<unsigned>(split)), dim3(64 * NT_W),
                       lds, a.stream, static_cast<const uint16_t*>(a.x), a.wq,
                       static_cast<const uint16_t*>(a.scales), static_cast<const uint16_t*>(a.biases),
                       static_cast<uint16_t*>(a.y), a.part, static_cast<int>(a.M), a.N, a.K, a.gs, ks);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    if constexpr (PART) return launch_reduce_partials(DT, a.part, a.y, split, a.M * a.N, a.stream);
    return hipSuccess;
}

template <int DT, int BITS, int RB>
hipError_t launch_nt_wide_r(const MatmulArgs& a, int split, int64_t ks) {
    return split > 1 ? launch_nt_wide_t<DT, BITS, RB, true>(a, split, ks)
                     : launch_nt_wide_t<DT, BITS, RB, false>(a, split, ks);
}

template <int DT, int BITS>
hipError_t launch_nt_wide_b(const MatmulArgs& a, int split, int64_t ks) {
    switch ((a.M + 15) / 16) {
        case 1: return launch_nt_wide_r<DT, BITS, 1>(a, split, ks);
        case 2: return launch_nt_wide_r<DT, BITS, 2>(a, split, ks);
        case 3: return launch_nt_wide_r<DT, BITS, 3>(a, split, ks);
        case 4: return launch_nt_wide_r<DT, BITS, 4>(a, split, ks);
        default: return hipErrorInvalidValue;
    }
}

template <int DT, int BITS, int RB>
hipError_t launch_nt_t(const MatmulArgs& a) {
    const size_t lds_sb = 2 * NT_KC * sizeof(uint16_t);
    const size_t lds_red = static_cast<size_t>(NT_W) * RB * 4 * 64 * sizeof(float);
    const size_t lds = lds_sb > lds_red ? lds_sb : lds_red;
    hipLaunchKernelGGL((nt_kernel<DT, BITS, RB>), dim3(static_cast<unsigned>(a.N / 16)), dim3(64 * NT_W), lds,
                       a.stream, static_cast<const uint16_t*>(a.x), a.wq, static_cast<const uint16_t*>(a.scales),
                       static_cast<const uint16_t*>(a.biases), static_cast<uint16_t*>(a.y), static_cast<int>(a.M),
                       a.N, a.K, a.gs);
    return hipGetLastError();
}

template <int DT, int BITS>
hipError_t launch_nt_b(const MatmulArgs& a) {
    switch ((a.M + 15) / 16) {
        case 1: return launch_nt_t<DT, BITS, 1>(a);
        case 2: return launch_nt_t<DT, BITS, 2>(a);
        case 3: return launch_nt_t<DT, BITS, 3>(a);
        case 4: return launch_nt_t<DT, BITS, 4>(a);
        default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------------------
// Transpose-read form (4- and 8-bit codes).  gfx950's LDS transpose reads
// deliver exactly the operand the matrix cores want from rows of packed codes:
// within each group of 16 lanes, ds_read_b64_tr_b4 gives lane i nibble i of
// the 8-byte blocks the 16 lanes address (lane i receives 16 codes of one
// column from 16 rows), and ds_read_b64_tr_b8 gives lane i byte i % 8 of the
// blocks of lanes 2j + i / 8, j = 0..7 (8 rows of one column when lanes 2j,
// 2j + 1 address the two 8-column halves of row j).  (Layouts checked on the
// hardware.)  So the weights go global -> LDS as whole row pieces with
// 16-byte coalesced loads, and each 16-column tile's B operand comes out of
// LDS already transposed: no cross-lane shuffles at all.
//
// Workgroup: 8 wavefronts own a block of 256 columns (16 tiles, 2 per
// wavefront) and one slice of K (blockIdx.y), walked in chunks of 16 KiB of
// weights (128 rows at 4 bits, 64 at 8; 8 KiB where a slice holds at most two
// 16 KiB chunks, so that its loads and compute still overlap) staged in LDS;
// the next chunk's
// weights, activations and scales are loaded into registers while the
// current one is computed.  A wavefront's tiles are its own for the whole
// slice, so there is no combine: it stores fp32 partials part[slice][M][N]
// (several slices; a second kernel adds them in slice order) or, with one
// slice, rounds and stores y.
//
// Rows past the end of the slice inside the last 64-row (32-row) block keep
// whatever codes the LDS holds but get scale and bias 0 (so w = 0) and zero
// activations.
// (256 columns: a 4-bit row piece is a whole 128-byte line, and each row's
// scale/bias gather serves twice the columns of a 128-column block -- those
// per-row gathers, one line per row per workgroup, outnumbered the weight
// requests two to one at 128 columns)
constexpr int NTT_BN = 256;        // columns per workgroup
constexpr int NTT_THREADS = 512;   // 8 wavefronts, 2 tiles each
constexpr int NTT_CHUNK_BYTES = 16384;  // weights per chunk (the short-slice form: half)
constexpr int NTT_GMAX = NTT_BN / 32;  // groups a block spans at most

template <int BITS, int CB = NTT_CHUNK_BYTES>
struct NttFmt {
    static_assert(CB == NTT_CHUNK_BYTES || CB == NTT_CHUNK_BYTES / 2, "16 or 8 KiB chunks");
    static constexpr int RP = NTT_BN * BITS / 8;              // bytes of a row piece (128 / 256)
    static constexpr int KC = CB / RP;                        // rows per chunk (128 / 64; 8 KiB: 64 / 32)
    static constexpr int BLK = BITS == 4 ? 64 : 32;           // rows per transpose read (16 / 8 per lane group)
    static constexpr int CPR = RP / 16;                       // 16-byte pieces per row
    static constexpr int WPT = CB / 16 / NTT_THREADS;         // weight pieces per thread (2; 8 KiB: 1)
    static constexpr int XS = KC + 8;                         // activation row stride in LDS (elements)
    // LDS position of 16-byte piece c of row r (swizzled so that the
    // transpose reads of 16 consecutive rows spread over the banks)
    __device__ static constexpr int swz(int r) { return r & 7; }
};

template <int DT, int BITS, int RB, bool PART, int SBW, int CB>
__global__ __launch_bounds__(NTT_THREADS, 2) void nt_tr_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, uint16_t* __restrict__ y, float* __restrict__ part, int M, int64_t N,
    int64_t K, int gs, int64_t kr) {
    using F = NttFmt<BITS, CB>;
    constexpr int KC = F::KC, XS = F::XS, BLK = F::BLK;
    extern __shared__ __align__(16) uint8_t lds[];
    uint8_t* const w_lds = lds;                                                       // [KC][RP], swizzled
    uint16_t* const x_lds = reinterpret_cast<uint16_t*>(lds + CB);                     // [16 RB][XS]
    uint16_t* const s_lds = x_lds + 16 * RB * XS;                                      // [GMAX][KC]
    uint16_t* const b_lds = s_lds + NTT_GMAX * KC;                                     // [GMAX][KC]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, q = lane >> 4;
    // (a block's row piece is whole 128-byte lines: no two workgroups share one)
    const int bx = static_cast<int>(blockIdx.x), by = static_cast<int>(blockIdx.y);
    const int64_t n0 = static_cast<int64_t>(bx) * NTT_BN;
    const int ncols = static_cast<int>(N - n0 < NTT_BN ? N - n0 : NTT_BN);  // a multiple of 64, <= 256
    const int64_t k_lo = static_cast<int64_t>(by) * kr;
    const int64_t k_hi = k_lo + kr < K ? k_lo + kr : K;
    const int64_t G = N / gs;
    const int64_t g0 = n0 / gs;
    const int gw = (ncols + gs - 1) / gs;  // groups of this block (1..8)
    // SBW > 0: every block spans SBW groups (N a multiple of the block
    // width), and a row's SBW scales load as one 4-, 8- or 16-byte run
    static_assert(SBW == 0 || SBW == 2 || SBW == 4 || SBW == 8, "scale run of 2, 4 or 8 values");
    constexpr bool vec_sb = SBW > 0;
    const int64_t row_bytes = N * BITS / 8;
    const uint8_t* const wbase = reinterpret_cast<const uint8_t*>(wq) + n0 * BITS / 8;

    // activation rows M .. 16 RB - 1 stay zero for the whole kernel
    for (int i = tid; i < (16 * RB - M) * XS; i += NTT_THREADS) x_lds[M * XS + i] = 0;

    // register prefetch, two chunks deep: a chunk's weights, activations
    // and scales in one buffer
    constexpr int XPT = (16 * RB * KC / 8 + NTT_THREADS - 1) / NTT_THREADS;  // activation pieces per thread
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));  // (a native vector: stays in registers)
    struct ChunkRegs {
        v4u wv[F::WPT];
        v4u xv[XPT];
        uint32_t sv[NTT_GMAX], bv[NTT_GMAX];  // packed pairs (vec_sb) or one value each
    };
    ChunkRegs cr0, cr1;
    auto load_chunk = [&](int64_t kc0, ChunkRegs& cb) __attribute__((always_inline)) {
        auto& wv = cb.wv;
        auto& xv = cb.xv;
        auto& sv = cb.sv;
        auto& bv = cb.bv;
        // Every lane issues every load, from a clamped address where its
        // piece lies past the slice, past M or past the block (the counter
        // then counts the same loads on every path, so each wait is exact;
        // a load skipped on some path makes every later wait drain the
        // queue).  What such a load brings is never used: rows past the
        // slice get scale and bias 0 and meet activations read from valid
        // rows, activation rows past M and columns past the block are never
        // staged or computed.  A chunk past the slice (the prefetch of the
        // last steps) is never staged: its loads all read the first 16
        // bytes of each array (one line).
        const bool past = kc0 >= k_hi;
        if (past) kc0 = k_lo;
        const int rows = static_cast<int>(k_hi - kc0 < KC ? k_hi - kc0 : KC);
#pragma unroll
        for (int i = 0; i < F::WPT; ++i) {
            const int p = tid + NTT_THREADS * i;
            const int r = p / F::CPR, c = (p % F::CPR) ^ F::swz(r);
            const int rr = r < rows ? r : rows - 1;
            const int cc = c * 16 * 8 / BITS < ncols ? c : 0;
            const int64_t wo = past ? 0 : (kc0 + rr) * row_bytes + cc * 16;
            wv[i] = *reinterpret_cast<const v4u*>(wbase + wo);
        }
        const int cpr = KC / 8;  // activation pieces per row
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int p = tid + NTT_THREADS * i;
            const int m = p / cpr, c = p % cpr;
            const int mm = m < M ? m : M - 1;
            const int ccx = 8 * c < rows ? c : 0;
            const int64_t xo = past ? 0 : static_cast<int64_t>(mm) * K + kc0 + 8 * ccx;
            xv[i] = *reinterpret_cast<const v4u*>(x + xo);
        }
        {
            // this row's run of gw scales (biases): one load where it is an
            // aligned run of 2, 4 or 8 (a separate kernel), kept packed until
            // staged; nothing is written to these registers but the loads
            // (a later write to a register a load targets waits for every
            // load before it).  Lanes past KC load the first line of the
            // arrays (never staged); rows past the slice are staged as 0.
            const int r = tid < rows ? tid : rows - 1;
            const int64_t o = past || tid >= KC ? 0 : (kc0 + r) * G + g0;
            if constexpr (SBW == 2) {
                sv[0] = *reinterpret_cast<const uint32_t*>(scales + o);
                bv[0] = *reinterpret_cast<const uint32_t*>(biases + o);
            } else if constexpr (SBW == 4) {
                const uint2 s4 = *reinterpret_cast<const uint2*>(scales + o);
                const uint2 b4 = *reinterpret_cast<const uint2*>(biases + o);
                sv[0] = s4.x; sv[1] = s4.y; bv[0] = b4.x; bv[1] = b4.y;
            } else if constexpr (SBW == 8) {
                const uint4 s8 = *reinterpret_cast<const uint4*>(scales + o);
                const uint4 b8 = *reinterpret_cast<const uint4*>(biases + o);
                sv[0] = s8.x; sv[1] = s8.y; sv[2] = s8.z; sv[3] = s8.w;
                bv[0] = b8.x; bv[1] = b8.y; bv[2] = b8.z; bv[3] = b8.w;
            } else {
#pragma unroll
                for (int g = 0; g < NTT_GMAX; ++g) {
                    const int gg = g < gw ? g : gw - 1;
                    sv[g] = scales[o + gg];
                    bv[g] = biases[o + gg];
                }
            }
        }
    };
    auto stage_chunk = [&](int64_t kc0, const ChunkRegs& cb) __attribute__((always_inline)) {
        const int srows = static_cast<int>(k_hi - kc0 < KC ? k_hi - kc0 : KC);
        const auto& wv = cb.wv;
        const auto& xv = cb.xv;
        const auto& sv = cb.sv;
        const auto& bv = cb.bv;
#pragma unroll
        for (int i = 0; i < F::WPT; ++i) *reinterpret_cast<v4u*>(w_lds + 16 * (tid + NTT_THREADS * i)) = wv[i];
        const int cpr = KC / 8;
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int p = tid + NTT_THREADS * i;
            const int m = p / cpr, c = p % cpr;
            if (m < M) *reinterpret_cast<v4u*>(x_lds + m * XS + 8 * c) = xv[i];
        }
        if (tid < KC) {
            // (groups past gw stage whatever the registers hold: never read)
#pragma unroll
            for (int g = 0; g < NTT_GMAX; ++g) {
                const uint32_t sg = vec_sb ? sv[g >> 1] >> (16 * (g & 1)) : sv[g];
                const uint32_t bg = vec_sb ? bv[g >> 1] >> (16 * (g & 1)) : bv[g];
                s_lds[g * KC + tid] = static_cast<uint16_t>(tid < srows ? sg : 0u);
                b_lds[g * KC + tid] = static_cast<uint16_t>(tid < srows ? bg : 0u);
            }
        }
    };

    float4_t acc[2][RB];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int b = 0; b < RB; ++b) acc[t][b] = {0.0f, 0.0f, 0.0f, 0.0f};
    const int t0 = 2 * wave;                      // this wavefront's tiles: t0, t0 + 1
    const bool live = 16 * t0 < ncols;            // (uniform: a 64-column block has tiles 0..3)
    const int gt = 16 * t0 / gs;                  // the two tiles' group (gs >= 32)

    auto compute_chunk = [&](int64_t kc0) __attribute__((always_inline)) {
        const int rows = static_cast<int>(k_hi - kc0 < KC ? k_hi - kc0 : KC);
        if (live) {
            for (int blk = 0; blk < rows; blk += BLK) {
                // scales and biases of this lane's rows (quarter q), for the tiles' group
                constexpr int SUB = BLK / 32;  // MFMA steps per transpose read (2 at 4 bits, 1 at 8)
                uint32_t sw[SUB][4], bw[SUB][4];
#pragma unroll
                for (int st = 0; st < SUB; ++st) {
                    const int r0 = blk + (BITS == 4 ? 16 * q + 8 * st : 8 * q);
                    const uint4 s4 = *reinterpret_cast<const uint4*>(s_lds + gt * KC + r0);
                    const uint4 b4 = *reinterpret_cast<const uint4*>(b_lds + gt * KC + r0);
                    sw[st][0] = s4.x; sw[st][1] = s4.y; sw[st][2] = s4.z; sw[st][3] = s4.w;
                    bw[st][0] = b4.x; bw[st][1] = b4.y; bw[st][2] = b4.z; bw[st][3] = b4.w;
                }
                // activation fragments: rows 16 b + li, the same k positions
                Frag xa[SUB][RB];
#pragma unroll
                for (int st = 0; st < SUB; ++st)
#pragma unroll
                    for (int b = 0; b < RB; ++b) {
                        const int k = blk + (BITS == 4 ? 16 * q + 8 * st : 8 * q);
                        const uint4 v = *reinterpret_cast<const uint4*>(x_lds + (16 * b + li) * XS + k);
                        xa[st][b].v[0] = v.x; xa[st][b].v[1] = v.y; xa[st][b].v[2] = v.z; xa[st][b].v[3] = v.w;
                    }
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const int t = t0 + tt;
                    // transpose read: lane (q, li) addresses one 8-byte block
                    int r, off;
                    if constexpr (BITS == 4) {
                        r = blk + 16 * q + li;                               // 16 rows per lane group
                        off = ((t >> 1) ^ F::swz(r)) * 16 + (t & 1) * 8;     // tile t's 8 bytes (16 codes)
                    } else {
                        r = blk + 8 * q + (li >> 1);                         // 8 rows, two halves each
                        off = (t ^ F::swz(r)) * 16 + (li & 1) * 8;
                    }
                    typedef int v2i_t __attribute__((ext_vector_type(2)));
                    auto* pa = reinterpret_cast<__attribute__((address_space(3))) v2i_t*>(
                        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t*)(w_lds)) + r * F::RP + off);
                    v2i_t tr;
                    if constexpr (BITS == 4)
                        tr = __builtin_amdgcn_ds_read_tr4_b64_v2i32(pa);
                    else
                        tr = __builtin_amdgcn_ds_read_tr8_b64_v2i32(pa);
#pragma unroll
                    for (int st = 0; st < SUB; ++st) {
                        Frag wh, wl;
                        if constexpr (BITS == 4)  // nibbles of rows 8 st .. 8 st + 7 (of this quarter's 16)
                            dequant_frags<DT, 4>(static_cast<uint32_t>(tr[st]), 0u, sw[st], bw[st], wh, wl);
                        else                      // bytes of rows 0..3 and 4..7
                            dequant_frags<DT, 8>(static_cast<uint32_t>(tr[0]), static_cast<uint32_t>(tr[1]), sw[st],
                                                 bw[st], wh, wl);
#pragma unroll
                        for (int b = 0; b < RB; ++b) {
                            acc[tt][b] = mf::mfma<DT>(xa[st][b], wh, acc[tt][b]);
                            if constexpr (DT == DT_BF16) acc[tt][b] = mf::mfma<DT>(xa[st][b], wl, acc[tt][b]);
                        }
                    }
                }
            }
        }
    };
    // chunk c is staged from buffer c % 2, whose next load (chunk c + 2) is
    // then in flight during the compute of chunks c and c + 1
    // (every step issues its prefetch, past the slice too: the same loads
    // on every path keep the compiler's waits to "this buffer's loads")
    auto step = [&](int64_t kc0, ChunkRegs& cb) __attribute__((always_inline)) {
        const bool in = kc0 < k_hi;
        if (in) stage_chunk(kc0, cb);
        __syncthreads();
        load_chunk(kc0 + 2 * KC, cb);
        if (in) compute_chunk(kc0);
        __syncthreads();  // the chunk's LDS is overwritten next
    };
    load_chunk(k_lo, cr0);
    load_chunk(k_lo + KC, cr1);
    for (int64_t kc0 = k_lo; kc0 < k_hi; kc0 += 2 * KC) {
        step(kc0, cr0);
        step(kc0 + KC, cr1);
    }

    if (!live) return;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int b = 0; b < RB; ++b)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int m = 16 * b + 4 * q + rr;
                const int64_t n = n0 + 16 * (t0 + tt) + li;
                if (m < M) {
                    if constexpr (PART)
                        part[(static_cast<int64_t>(by) * M + m) * N + n] = acc[tt][b][rr];
                    else
                        y[static_cast<int64_t>(m) * N + n] = DtOps<DT>::rne(acc[tt][b][rr]);
                }
            }
}

template <int BITS, int RB, int CB>
constexpr size_t ntt_lds_bytes() {
    return CB + 2 * (16 * RB * NttFmt<BITS, CB>::XS + 2 * NTT_GMAX * NttFmt<BITS, CB>::KC);
}

template <int DT, int BITS, int RB, bool PART, int SBW, int CB>
hipError_t launch_nt_tr_c(const MatmulArgs& a, int split, int64_t kr) {
    constexpr size_t lds = ntt_lds_bytes<BITS, RB, CB>();
    if (lds > 65536) {
        static std::atomic<uint64_t> raised{0};
        if (hipError_t e =
                raise_lds_limit(reinterpret_cast<const void*>(&nt_tr_kernel<DT, BITS, RB, PART, SBW, CB>), raised);
            e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((nt_tr_kernel<DT, BITS, RB, PART, SBW, CB>),
                       dim3(static_cast<unsigned>((a.N + NTT_BN - 1) / NTT_BN), static_cast<unsigned>(split)),
                       dim3(NTT_THREADS), lds, a.stream, static_cast<const uint16_t*>(a.x), a.wq,
                       static_cast<const uint16_t*>(a.scales), static_cast<const uint16_t*>(a.biases),
                       static_cast<uint16_t*>(a.y), a.part, static_cast<int>(a.M), a.N, a.K, a.gs, kr);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    if constexpr (PART) return launch_reduce_partials(DT, a.part, a.y, split, a.M * a.N, a.stream);
    return hipSuccess;
}

// The chunk size: slices of at most two 16 KiB chunks (K = 4096 on 16
// slices at 4 bits) go in 8 KiB chunks, so that a chunk's compute overlaps
// the next chunk's loads; longer slices keep 16 KiB.  Measured at M = 6:
// 4096 x 4096 (two chunks per slice) 9.9 vs 10.4 us; down 4096 x 14336 and
// gate/up 14336 x 4096 (eight) 20.1 / 20.0 vs 19.4 / 19.5 us in 8 KiB chunks.
template <int DT, int BITS, int RB, bool PART, int SBW>
hipError_t launch_nt_tr_s(const MatmulArgs& a, int split, int64_t kr) {
    if constexpr (PART)
        if (kr <= 2 * NttFmt<BITS>::KC) return launch_nt_tr_c<DT, BITS, RB, PART, SBW, NTT_CHUNK_BYTES / 2>(a, split, kr);
    return launch_nt_tr_c<DT, BITS, RB, PART, SBW, NTT_CHUNK_BYTES>(a, split, kr);
}

// the scale-run width: every block whole (N a multiple of 256) and 2, 4 or 8
// groups per block, else values one by one
template <int DT, int BITS, int RB, bool PART>
hipError_t launch_nt_tr_t(const MatmulArgs& a, int split, int64_t kr) {
    if (a.N % NTT_BN == 0) {
        if (a.gs == NTT_BN / 2) return launch_nt_tr_s<DT, BITS, RB, PART, 2>(a, split, kr);
        if (a.gs == NTT_BN / 4) return launch_nt_tr_s<DT, BITS, RB, PART, 4>(a, split, kr);
        if (a.gs == NTT_BN / 8) return launch_nt_tr_s<DT, BITS, RB, PART, 8>(a, split, kr);
    }
    return launch_nt_tr_s<DT, BITS, RB, PART, 0>(a, split, kr);
}

template <int DT, int BITS>
hipError_t launch_nt_tr_b(const MatmulArgs& a, int split, int64_t kr) {
    const bool p = split > 1;
    switch ((a.M + 15) / 16) {
        case 1: return p ? launch_nt_tr_t<DT, BITS, 1, true>(a, split, kr) : launch_nt_tr_t<DT, BITS, 1, false>(a, split, kr);
        case 2: return p ? launch_nt_tr_t<DT, BITS, 2, true>(a, split, kr) : launch_nt_tr_t<DT, BITS, 2, false>(a, split, kr);
        case 3: return p ? launch_nt_tr_t<DT, BITS, 3, true>(a, split, kr) : launch_nt_tr_t<DT, BITS, 3, false>(a, split, kr);
        case 4: return p ? launch_nt_tr_t<DT, BITS, 4, true>(a, split, kr) : launch_nt_tr_t<DT, BITS, 4, false>(a, split, kr);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_nt_tr(const MatmulArgs& a, int split, int64_t kr) {
    switch (a.dt * 10 + a.bits) {
        case 4: return launch_nt_tr_b<DT_F16, 4>(a, split, kr);
        case 8: return launch_nt_tr_b<DT_F16, 8>(a, split, kr);
        case 14: return launch_nt_tr_b<DT_BF16, 4>(a, split, kr);
        case 18: return launch_nt_tr_b<DT_BF16, 8>(a, split, kr);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// K split of the workspace entry point: 128-column workgroups, slices enough
// for about 256 workgroups (at most 16, at least 2 steps of 32 rows each);
// wide N (>= 128 such workgroups) runs unsplit.
NtPlan nt_plan(int bits, int64_t M, int64_t N, int64_t K) {
    (void)M;
    const int64_t groups = (N + 127) / 128;  // 128-column workgroups of the 16-wavefront form
    if (bits != 6 && groups >= 32) {
        // transpose-read form (256-column workgroups): the fewest slices of
        // whole 16 KiB chunks (128 rows at 4 bits, 64 at 8) that divide K and
        // give at least 224 workgroups (7/8 of the CUs: longer slices keep
        // more chunks in the prefetch pipeline), at most 512; otherwise
        // whole chunks and at least 224.  Measured at M = 6: 4096 x 4096 on
        // 16 slices of 256 rows 11.0 us (8 / 32 slices: 12.3 / 13.3);
        // gate/up (56 blocks) on 4 slices 19.8 us (8 / 16 / 32: 22.0 / 24.9
        // / 34.1); down (K = 14336) on 14 slices of 1024 rows 22.4 us (8 /
        // 16 / 28: 28.6 / 22.0 / 25.8).
        const int64_t blocks = (N + 255) / 256;
        const int64_t kc = bits == 4 ? 128 : 64;
        if (blocks >= 256 || K < 2 * kc) return NtPlan{true, 1, K, true};
        for (int64_t s = 2; s <= 32; ++s)
            if (K % s == 0 && (K / s) % kc == 0 && blocks * s >= 224 && blocks * s <= 512)
                return NtPlan{true, static_cast<int>(s), K / s, true};
        for (int64_t s = 2; s <= 32; ++s) {
            const int64_t ks = ((K + s - 1) / s + kc - 1) / kc * kc;
            const int64_t se = (K + ks - 1) / ks;
            if (blocks * se >= 224 || s == 32 || ks == kc)
                return se < 2 ? NtPlan{true, 1, K, true} : NtPlan{true, static_cast<int>(se), ks, true};
        }
    }
    NtPlan p{false, 1, K, false};
    if (groups >= 128) return NtPlan{true, 1, K, false};  // wide N: enough workgroups unsplit
    int64_t split = 256 / groups;
    if (split > 16) split = 16;
    if (split > K / 64) split = K / 64;
    if (split < 2) return p;
    const int64_t ks = ((K + split - 1) / split + 31) / 32 * 32;  // rows per slice, whole 32-row steps
    return NtPlan{true, static_cast<int>((K + ks - 1) / ks), ks, false};
}

namespace {
bool nt_shape_ok(const MatmulArgs& a) {
    return a.M >= 1 && a.M <= 64 && a.N >= 64 && a.N % 64 == 0 && a.gs >= 32 && a.N % a.gs == 0 && a.K >= 32 &&
           a.K % 32 == 0;
}
}  // namespace

hipError_t launch_nt(const MatmulArgs& a) {
    // shapes the kernels assume (validated by the caller)
    if (!nt_shape_ok(a)) return hipErrorInvalidValue;
    // wide N: the transpose-read form (4/8-bit) unsplit
    if (a.bits != 6 && (a.N + 127) / 128 >= 256) return launch_nt_tr(a, 1, a.K);
    if ((a.N + 127) / 128 >= 128) {  // wide N: the 128-column form, unsplit
        switch (a.dt * 10 + a.bits) {
            case 4: return launch_nt_wide_b<DT_F16, 4>(a, 1, a.K);
            case 6: return launch_nt_wide_b<DT_F16, 6>(a, 1, a.K);
            case 8: return launch_nt_wide_b<DT_F16, 8>(a, 1, a.K);
            case 14: return launch_nt_wide_b<DT_BF16, 4>(a, 1, a.K);
            case 16: return launch_nt_wide_b<DT_BF16, 6>(a, 1, a.K);
            case 18: return launch_nt_wide_b<DT_BF16, 8>(a, 1, a.K);
            default: return hipErrorInvalidValue;
        }
    }
    switch (a.dt * 10 + a.bits) {
        case 4: return launch_nt_b<DT_F16, 4>(a);
        case 6: return launch_nt_b<DT_F16, 6>(a);
        case 8: return launch_nt_b<DT_F16, 8>(a);
        case 14: return launch_nt_b<DT_BF16, 4>(a);
        case 16: return launch_nt_b<DT_BF16, 6>(a);
        case 18: return launch_nt_b<DT_BF16, 8>(a);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_nt_split(const MatmulArgs& a) {
    if (!nt_shape_ok(a)) return hipErrorInvalidValue;
    const NtPlan p = nt_plan(a.bits, a.M, a.N, a.K);
    if (p.split < 2) return launch_nt(a);
    if (a.part == nullptr) return hipErrorInvalidValue;
    if (p.tr) return launch_nt_tr(a, p.split, p.ks);
    switch (a.dt * 10 + a.bits) {
        case 4: return launch_nt_wide_b<DT_F16, 4>(a, p.split, p.ks);
        case 6: return launch_nt_wide_b<DT_F16, 6>(a, p.split, p.ks);
        case 8: return launch_nt_wide_b<DT_F16, 8>(a, p.split, p.ks);
        case 14: return launch_nt_wide_b<DT_BF16, 4>(a, p.split, p.ks);
        case 16: return launch_nt_wide_b<DT_BF16, 6>(a, p.split, p.ks);
        case 18: return launch_nt_wide_b<DT_BF16, 8>(a, p.split, p.ks);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
