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
//   * the workgroup's 4..8 wavefronts split K among themselves so that each
//     SIMD streams a distinct part of the tile, and their partial sums are
//     combined once through LDS at the end of the tile;
//   * the activation rows stay in registers for the whole kernel while the
//     workgroup walks over column tiles (persistent grid), so x is read once
//     per workgroup, not once per tile.
//
// Arithmetic (exact up to fp32 rounding).  Codes become fp16/bf16 values
// q + OFF with the "magic number" trick (OFF = 1024 for fp16, 128 for bf16
// at 4/6 bits; 8-bit bf16 converts exactly with OFF = 0).  Per column n and
// group g the matrix cores produce P = sum x*(q + OFF) and X = sum x, and
//   y += s*P + (b - OFF*s)*X        (fp32 FMAs, one pair per group portion)
// which equals sum_k x_k * (s*q_k + b) without rounding the dequantized
// weight to the activation dtype.
//
// Operand layout of v_mfma_f32_16x16x32 (verified on the hardware): lane l
// supplies A[l%16][8*(l/16)+e] and B[8*(l/16)+e][l%16] for e = 0..7 and
// receives D[4*(l/16)+r][l%16], r = 0..3.  A lane thus serves row i = l%16 of
// x and column c = l%16 of the tile, in k-slot quarter jj = l/16.
#include "qmm_device.hpp"
#include "qmm_internal.hpp"

namespace qmm {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

struct Frag {  // 8 packed 16-bit values = one MFMA operand of one lane
    uint32_t v[4];
};

template <int DT>
__device__ __forceinline__ float4_t mfma(const Frag& a, const Frag& b, float4_t c) {
    if constexpr (DT == DT_F16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b),
                                                      c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
}

__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}

// Per-format constants.  A lane loads one "segment" of SEG codes of its
// column per k-block; the four k-slot quarters (jj) of a column load four
// consecutive segments, so a k-block holds KBLK = 4*SEG codes and feeds
// STEPS = SEG/8 MFMA steps.
template <int DT, int BITS, int GS>
struct Fmt {
    static constexpr int SEG = BITS == 4 ? 32 : 16;      // codes per lane load
    static constexpr int SEG_WORDS = SEG * BITS / 32;    // 4, 3 or 4 words (16, 12, 16 bytes)
    static constexpr int STEPS = SEG / 8;                // MFMA steps per k-block
    static constexpr int KBLK = 4 * SEG;                 // codes per k-block
    static constexpr int PORTIONS = (KBLK / GS) > 1 ? (KBLK / GS) : 1;  // group portions per k-block
    static constexpr int STEPS_PER_PORTION = STEPS / PORTIONS;
    static constexpr float OFF = (DT == DT_F16) ? 1024.0f : (BITS == 8 ? 0.0f : 128.0f);
    static constexpr uint32_t ONES = (DT == DT_F16) ? 0x3C003C00u : 0x3F803F80u;
    // Step s, quarter jj reads its 8 codes from segment SRC_LANE of the
    // k-block, sub-block SRC_SLOT (after the lane swaps that make every step
    // lie inside one quantization group).
    __host__ __device__ static constexpr int src_lane(int s, int jj) {
        if constexpr (BITS == 4 && GS == 64) return (jj & 1) + 2 * (s >> 1);
        if constexpr (BITS == 4 && GS == 32) return s;
        if constexpr (BITS != 4 && GS == 32) return (jj & 1) + 2 * s;
        return jj;
    }
    __host__ __device__ static constexpr int src_slot(int s, int jj) {
        if constexpr (BITS == 4 && GS == 64) return (s & 1) + 2 * (jj >> 1);
        if constexpr (BITS == 4 && GS == 32) return jj;
        if constexpr (BITS != 4 && GS == 32) return jj >> 1;
        return s;
    }
};

// x fragment: 8 consecutive values (natural order, 16 bytes) rearranged into
// the order the weight unpack produces.
template <int BITS, int DT>
__device__ __forceinline__ Frag x_frag(uint4 u) {
    Frag f;
    if constexpr (BITS == 4) {          // order 0,4,1,5,2,6,3,7
        f.v[0] = __builtin_amdgcn_perm(u.z, u.x, 0x05040100u);
        f.v[1] = __builtin_amdgcn_perm(u.z, u.x, 0x07060302u);
        f.v[2] = __builtin_amdgcn_perm(u.w, u.y, 0x05040100u);
        f.v[3] = __builtin_amdgcn_perm(u.w, u.y, 0x07060302u);
    } else if constexpr (BITS == 6) {   // order 0,2,1,3,4,6,5,7
        f.v[0] = __builtin_amdgcn_perm(u.y, u.x, 0x05040100u);
        f.v[1] = __builtin_amdgcn_perm(u.y, u.x, 0x07060302u);
        f.v[2] = __builtin_amdgcn_perm(u.w, u.z, 0x05040100u);
        f.v[3] = __builtin_amdgcn_perm(u.w, u.z, 0x07060302u);
    } else {                            // natural order
        f.v[0] = u.x; f.v[1] = u.y; f.v[2] = u.z; f.v[3] = u.w;
    }
    return f;
}

// (a & m) | o.  gfx9 VOP3 encodings take no literal constant, so m and o are
// kept in VGPRs (see unpack_consts); the compiler then selects a single
// v_and_or_b32 instead of a VOP2 and plus a VOP2 or.  Written in plain C so
// that the compiler sees the instruction and inserts the wait states a VALU
// result needs before a matrix-core instruction may read it.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) { return (a & m) | o; }

// Constants of the unpack, kept in VGPRs for and_or().
struct UnpackConsts {
    uint32_t nib;    // 0x000F000F
    uint32_t six;    // 0x0000003F
    uint32_t six_hi; // 0x003F0000
    uint32_t magic;  // q + OFF pattern: 0x6400 (fp16) / 0x4300 (bf16) in both halves
};

template <int DT>
__device__ __forceinline__ UnpackConsts unpack_consts() {
    UnpackConsts k;
    k.nib = 0x000F000Fu;
    k.six = 0x3Fu;
    k.six_hi = 0x3F0000u;
    k.magic = (DT == DT_F16) ? 0x64006400u : 0x43004300u;
    // keep them in registers (not folded back into literals)
    asm volatile("" : "+v"(k.nib), "+v"(k.six), "+v"(k.six_hi), "+v"(k.magic));
    return k;
}

// 4-bit: one word (8 codes) -> q + OFF in order 0,4,1,5,2,6,3,7.
__device__ __forceinline__ Frag unpack4(uint32_t w, const UnpackConsts& k) {
    Frag f;
    f.v[0] = and_or(w, k.nib, k.magic);
    f.v[1] = and_or(w >> 4, k.nib, k.magic);
    f.v[2] = and_or(w >> 8, k.nib, k.magic);
    f.v[3] = and_or(w >> 12, k.nib, k.magic);
    return f;
}

// 6-bit: one 24-bit unit (4 codes) -> two packed pairs, order 0,2 | 1,3.
__device__ __forceinline__ void unpack6_unit(uint32_t u, const UnpackConsts& k, uint32_t& p02, uint32_t& p13) {
    p02 = and_or(u << 4, k.six_hi, and_or(u, k.six, k.magic));
    const uint32_t t = u >> 6;
    p13 = and_or(t << 4, k.six_hi, and_or(t, k.six, k.magic));
}

// 8-bit: two words (8 codes) -> values in natural order.
template <int DT>
__device__ __forceinline__ Frag unpack8(uint32_t w0, uint32_t w1) {
    Frag f;
    if constexpr (DT == DT_F16) {
        // bytes b | 0x64 << 8 = 1024 + b, exact for every byte value
        f.v[0] = __builtin_amdgcn_perm(0x64646464u, w0, 0x04010400u);
        f.v[1] = __builtin_amdgcn_perm(0x64646464u, w0, 0x04030402u);
        f.v[2] = __builtin_amdgcn_perm(0x64646464u, w1, 0x04010400u);
        f.v[3] = __builtin_amdgcn_perm(0x64646464u, w1, 0x04030402u);
    } else {
        // bf16 has 8 significant bits, so an integer below 256 is exactly the
        // top half of its fp32 value
        const uint32_t w[2] = {w0, w1};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t f0 = __builtin_bit_cast(uint32_t, static_cast<float>(w[h] & 0xFFu));
            const uint32_t f1 = __builtin_bit_cast(uint32_t, static_cast<float>((w[h] >> 8) & 0xFFu));
            const uint32_t f2 = __builtin_bit_cast(uint32_t, static_cast<float>((w[h] >> 16) & 0xFFu));
            const uint32_t f3 = __builtin_bit_cast(uint32_t, static_cast<float>(w[h] >> 24));
            f.v[2 * h] = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
            f.v[2 * h + 1] = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
        }
    }
    return f;
}

// Segment words -> STEPS weight fragments, with the lane swaps applied.
template <int DT, int BITS, int GS, int NW, int NS>
__device__ __forceinline__ void segment_frags(uint32_t (&w)[NW], Frag (&b)[NS], const UnpackConsts& k) {
    static_assert(NW == Fmt<DT, BITS, GS>::SEG_WORDS && NS == Fmt<DT, BITS, GS>::STEPS, "segment shape");
    if constexpr (BITS == 4) {
        if constexpr (GS == 64 || GS == 32) {
            swap32(w[0], w[2]);
            swap32(w[1], w[3]);
        }
        if constexpr (GS == 32) {
            swap16(w[0], w[1]);
            swap16(w[2], w[3]);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) b[s] = unpack4(w[s], k);
    } else if constexpr (BITS == 8) {
        if constexpr (GS == 32) {
            swap32(w[0], w[2]);
            swap32(w[1], w[3]);
        }
        b[0] = unpack8<DT>(w[0], w[1]);
        b[1] = unpack8<DT>(w[2], w[3]);
    } else {  // 6-bit: 16 codes in 3 words = 4 units of 24 bits
        const uint32_t u0 = w[0];
        const uint32_t u1 = __builtin_amdgcn_alignbit(w[1], w[0], 24);
        const uint32_t u2 = __builtin_amdgcn_alignbit(w[2], w[1], 16);
        const uint32_t u3 = w[2] >> 8;
        unpack6_unit(u0, k, b[0].v[0], b[0].v[1]);
        unpack6_unit(u1, k, b[0].v[2], b[0].v[3]);
        unpack6_unit(u2, k, b[1].v[0], b[1].v[1]);
        unpack6_unit(u3, k, b[1].v[2], b[1].v[3]);
        if constexpr (GS == 32) {
#pragma unroll
            for (int v = 0; v < 4; ++v) swap32(b[0].v[v], b[1].v[v]);
        }
    }
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int BITS, int NW>
__device__ __forceinline__ void load_segment(const uint32_t* __restrict__ p, uint32_t (&w)[NW]) {
    if constexpr (NW == 4) {
        // streamed once: non-temporal hint keeps the weights from displacing x
        const u32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
        w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
    } else {
        const uint3 a = *reinterpret_cast<const uint3*>(p);
        w[0] = a.x; w[1] = a.y; w[2] = a.z;
    }
}

// Scale/bias words of one tile for one lane.  Vector form (VEC): the
// wavefront's NG consecutive groups as NG/2 words (two 16-bit values per
// word) of scales and of biases.  Scalar form: one value per group portion.
template <bool VEC, int NGW, int KPW, int NP>
struct ScaleRegs;
template <int NGW, int KPW, int NP>
struct ScaleRegs<true, NGW, KPW, NP> {
    uint32_t s[NGW], b[NGW];
};
template <int NGW, int KPW, int NP>
struct ScaleRegs<false, NGW, KPW, NP> {
    uint32_t s[KPW][NP], b[KPW][NP];
};

// Weight words and raw scale/bias values of one tile for one lane.
template <bool VEC, int NGW, int KPW, int NW, int NP>
struct TileRegs {
    uint32_t w[KPW][NW];
    ScaleRegs<VEC, NGW, KPW, NP> sb;
};

template <int NWORDS>
__device__ __forceinline__ void load_words(const uint16_t* __restrict__ p, uint32_t (&d)[NWORDS]) {
    if constexpr (NWORDS == 8) {
        const uint4 a = reinterpret_cast<const uint4*>(p)[0];
        const uint4 b = reinterpret_cast<const uint4*>(p)[1];
        d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w; d[4] = b.x; d[5] = b.y; d[6] = b.z; d[7] = b.w;
    } else if constexpr (NWORDS == 4) {
        const uint4 a = *reinterpret_cast<const uint4*>(p);
        d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w;
    } else if constexpr (NWORDS == 2) {
        const uint2 a = *reinterpret_cast<const uint2*>(p);
        d[0] = a.x; d[1] = a.y;
    } else {
        d[0] = *reinterpret_cast<const uint32_t*>(p);
    }
}

// LDS layout of the staged activations: rows 0..M-1 of x and one zero row
// (read by the lanes of rows >= M), each row holding the KC = W*KPW*KBLK
// positions the wavefronts cover (zero beyond K) with every run of 8 values
// already in the order the weight unpack produces.  Row stride KC + 8 values:
// the 16-byte pad rotates rows across LDS banks.  Then two buffers of
// per-wavefront partial sums (one per tile parity).
__host__ __device__ constexpr int64_t x_stride(int64_t KC) { return KC + 8; }
__host__ __device__ inline int64_t lds_x_bytes(int64_t M, int64_t KC) { return (M + 1) * x_stride(KC) * 2; }
__host__ __device__ inline int64_t lds_red_bytes(int W) { return 2LL * W * 64 * 4 * 4; }

// W wavefronts per workgroup; wavefront w owns the KPW consecutive k-blocks
// [w*KPW, (w+1)*KPW) of K.  One workgroup owns a tile of 16 columns at a
// time and walks tiles blockIdx.x, blockIdx.x + gridDim.x, ...; the loads of
// the next LA tiles are in flight while a tile is computed (LA+1 register
// buffers used in turn).  x is staged once per workgroup in LDS; each MFMA
// step reads its 8-value A fragment with one 16-byte LDS read at a fixed
// offset from a per-lane base.
//
// The tile loop is written so that no wait on a load can be forced early:
// loaded registers are not touched in the iteration that issues them (the
// memory counter retires in order, so an early use would also wait for every
// later load), prefetches are unconditional (the last ones re-read the final
// tile), and nothing on the weight side is masked: positions beyond K read
// valid addresses and meet zero activations.
template <int DT, int BITS, int GS, int W, int KPW, bool VEC, int LA>
__global__ __launch_bounds__(64 * W, (KPW <= 4 ? 4 : 2)) void mfma_reg_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, uint16_t* __restrict__ y, int M, int64_t N, int64_t K) {
    using F = Fmt<DT, BITS, GS>;
    constexpr int NG = (KPW * F::KBLK + GS - 1) / GS;  // groups touched by one wavefront (vector form)
    constexpr int NGW = NG >= 2 ? NG / 2 : 1;            // 32-bit words holding NG 16-bit values
    constexpr int64_t KC = static_cast<int64_t>(W) * KPW * F::KBLK;
    using Regs = TileRegs<VEC, NGW, KPW, F::SEG_WORDS, F::PORTIONS>;
    extern __shared__ __align__(16) uint8_t lds[];
    uint16_t* xs_lds = reinterpret_cast<uint16_t*>(lds);
    float* red = reinterpret_cast<float*>(lds + lds_x_bytes(M, KC));

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane & 15;   // tile column of this lane's B operand / D output
    const int jj = lane >> 4;  // k-slot quarter
    const int64_t row_words = K * BITS / 32;
    const int64_t G = K / GS;
    const int64_t ntiles = (N + 15) / 16;
    const int64_t kb0 = static_cast<int64_t>(wave) * KPW;
    constexpr int64_t xstride = x_stride(KC);

    auto load_tile = [&](int64_t tile, Regs& r) {
        const int64_t n = min(tile * 16 + c, N - 1);  // tail columns re-read the last row
        const uint32_t* wrow = wq + n * row_words;
#pragma unroll
        for (int i = 0; i < KPW; ++i) {
            int64_t code0 = (kb0 + i) * F::KBLK + jj * F::SEG;
            if constexpr (!VEC) code0 = code0 < K ? code0 : K - F::SEG;  // VEC: the k-blocks cover K exactly
            load_segment<BITS, F::SEG_WORDS>(wrow + code0 * BITS / 32, r.w[i]);
        }
        if constexpr (VEC) {
            const int64_t g0 = kb0 * F::KBLK / GS;
            load_words<NGW>(scales + n * G + g0, r.sb.s);
            load_words<NGW>(biases + n * G + g0, r.sb.b);
        } else {
#pragma unroll
            for (int i = 0; i < KPW; ++i)
#pragma unroll
                for (int p = 0; p < F::PORTIONS; ++p) {
                    int64_t g = ((kb0 + i) * F::KBLK + static_cast<int64_t>(p) * (F::KBLK / F::PORTIONS)) / GS;
                    g = g < G ? g : G - 1;
                    r.sb.s[i][p] = scales[n * G + g];
                    r.sb.b[i][p] = biases[n * G + g];
                }
        }
    };

    // ---- prologue: first tiles' loads in flight, then x staged in LDS
    Regs buf[LA + 1];
    const int64_t step = gridDim.x;
    int64_t tile = blockIdx.x;
#pragma unroll
    for (int a = 0; a < LA; ++a) load_tile(min(tile + a * step, ntiles - 1), buf[a]);
    {
        constexpr int64_t runs = KC / 8;  // 16-byte runs per staged row
        const int64_t units = static_cast<int64_t>(M + 1) * runs;
        for (int64_t u = threadIdx.x; u < units; u += 64 * W) {
            const int64_t m = u / runs;
            const int64_t k8 = u - m * runs;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (m < M && k8 * 8 < K) v = *reinterpret_cast<const uint4*>(x + m * K + k8 * 8);
            const Frag f = x_frag<BITS, DT>(v);
            *reinterpret_cast<uint4*>(xs_lds + m * xstride + k8 * 8) = make_uint4(f.v[0], f.v[1], f.v[2], f.v[3]);
        }
        __syncthreads();
    }
    // A fragment of k-block i, step s: base + i*KBLK + step_off(s); the
    // per-quarter and per-step parts of the source position are separable.
    const uint16_t* a_base =
        xs_lds + static_cast<int64_t>(c < M ? c : M) * xstride + kb0 * F::KBLK + F::src_lane(0, jj) * F::SEG +
        F::src_slot(0, jj) * 8;
    auto a_frag = [&](int i, int s) -> Frag {
        const int off = i * F::KBLK + (F::src_lane(s, 0) - F::src_lane(0, 0)) * F::SEG +
                        (F::src_slot(s, 0) - F::src_slot(0, 0)) * 8;
        const uint4 v = *reinterpret_cast<const uint4*>(a_base + off);
        return Frag{{v.x, v.y, v.z, v.w}};
    };
    const Frag ones = {{F::ONES, F::ONES, F::ONES, F::ONES}};
    const UnpackConsts uk = unpack_consts<DT>();

    auto scale_bias = [&](const Regs& r, int i, int p, float& sc, float& bi) {
        uint32_t sv, bv;
        if constexpr (VEC) {
            const int gi = (i * F::KBLK + p * (F::KBLK / F::PORTIONS)) / GS;  // compile-time after unrolling
            sv = r.sb.s[gi >> 1] >> (16 * (gi & 1));
            bv = r.sb.b[gi >> 1] >> (16 * (gi & 1));
        } else {
            sv = r.sb.s[i][p];
            bv = r.sb.b[i][p];
        }
        sc = DtOps<DT>::to_f32(static_cast<uint16_t>(sv));
        bi = DtOps<DT>::to_f32(static_cast<uint16_t>(bv));
    };

    int parity = 0;
    auto compute_store = [&](int64_t t, Regs& r) {
        float4_t yacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < KPW; ++i) {
            Frag bw[F::STEPS];
            segment_frags<DT, BITS, GS>(r.w[i], bw, uk);
#pragma unroll
            for (int p = 0; p < F::PORTIONS; ++p) {
                float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
                float4_t xsum = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int st = 0; st < F::STEPS_PER_PORTION; ++st) {
                    const int s = p * F::STEPS_PER_PORTION + st;
                    const Frag xa = a_frag(i, s);
                    acc = mfma<DT>(xa, bw[s], acc);
                    xsum = mfma<DT>(xa, ones, xsum);
                }
                float sc, bi;
                scale_bias(r, i, p, sc, bi);
                const float bp = __fmaf_rn(-F::OFF, sc, bi);
#pragma unroll
                for (int q = 0; q < 4; ++q) yacc[q] = __fmaf_rn(sc, acc[q], __fmaf_rn(bp, xsum[q], yacc[q]));
            }
        }
        // Combine the wavefronts' partial sums: every wavefront writes its
        // partial to the buffer of this tile's parity; after one barrier
        // wavefronts 0..3 each sum one of the four D rows a lane holds and
        // store it.  The next tile writes the other buffer, and the tile
        // after that can only write this one after passing the next
        // barrier, which the reducing wavefronts reach only after reading.
        float* rb = red + parity * (W * 64 * 4);
        *reinterpret_cast<float4_t*>(rb + (wave * 64 + lane) * 4) = yacc;
        __syncthreads();
        if (wave < 4) {
            const int q = wave;
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < W; ++w) v += rb[(w * 64 + lane) * 4 + q];
            const int64_t col = t * 16 + c;
            const int row = 4 * jj + q;
            if (col < N && row < M) y[static_cast<int64_t>(row) * N + col] = DtOps<DT>::rne(v);
        }
        parity ^= 1;
    };

    // buffers rotate: tile t + a*step lives in buf[(u + a) % (LA + 1)]
    while (tile < ntiles) {
#pragma unroll
        for (int u = 0; u <= LA; ++u) {
            load_tile(min(tile + LA * step, ntiles - 1), buf[(u + LA) % (LA + 1)]);
            compute_store(tile, buf[u]);
            tile += step;
            if (tile >= ntiles) break;
        }
    }
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

// Launch shape: waves per workgroup, k-blocks per wavefront (W*KPW k-blocks
// cover K), whether the scale/bias vectors can be loaded whole.
struct RegShape {
    int W, KPW;
    bool vec;
};

inline int64_t kblk_of(int bits) { return bits == 4 ? 128 : 64; }

inline bool pick_shape(int bits, int gs, int64_t K, RegShape& s) {
    const int64_t kblk = kblk_of(bits);
    const int64_t nkb = (K + kblk - 1) / kblk;
    // 8 wavefronts (two per SIMD); the smallest KPW that covers K.  The x
    // fragments of a wavefront's k-blocks stay in registers, which bounds K.
    for (int KPW : {1, 2, 4, 8}) {
        if (8 * KPW >= nkb) {
            const int64_t G = K / gs;
            const int64_t ng = (KPW * kblk + gs - 1) / gs;
            const int64_t vec_vals = ng >= 8 ? 8 : ng;  // 16-bit values per vector load
            s = {8, KPW, 8 * KPW == nkb && KPW * kblk % gs == 0 && G % vec_vals == 0 && ng % 2 == 0};
            return true;
        }
    }
    return false;
}

template <int DT, int BITS, int GS, int W, int KPW, bool VEC>
hipError_t launch_shape(const MatmulArgs& a) {
    const int64_t ntiles = (a.N + 15) / 16;
    const int64_t KC = static_cast<int64_t>(W) * KPW * (BITS == 4 ? 128 : 64);
    const size_t lds = static_cast<size_t>(lds_x_bytes(a.M, KC) + lds_red_bytes(W));
    // up to two resident workgroups per CU on 256 CUs; each walks several tiles
    const int64_t grid = ntiles < 512 ? ntiles : 512;
    constexpr int LA = 1;
    hipLaunchKernelGGL((mfma_reg_kernel<DT, BITS, GS, W, KPW, VEC, LA>), dim3(static_cast<unsigned>(grid)),
                       dim3(64 * W), lds, a.stream, static_cast<const uint16_t*>(a.x), a.wq,
                       static_cast<const uint16_t*>(a.scales), static_cast<const uint16_t*>(a.biases),
                       static_cast<uint16_t*>(a.y), static_cast<int>(a.M), a.N, a.K);
    return hipGetLastError();
}

template <int DT, int BITS, int GS>
hipError_t launch_reg_t(const MatmulArgs& a) {
    RegShape s;
    if (!pick_shape(BITS, GS, a.K, s)) return hipErrorInvalidValue;
    switch (s.KPW * 2 + (s.vec ? 1 : 0)) {
        case 2: return launch_shape<DT, BITS, GS, 8, 1, false>(a);
        case 3: return launch_shape<DT, BITS, GS, 8, 1, true>(a);
        case 4: return launch_shape<DT, BITS, GS, 8, 2, false>(a);
        case 5: return launch_shape<DT, BITS, GS, 8, 2, true>(a);
        case 8: return launch_shape<DT, BITS, GS, 8, 4, false>(a);
        case 9: return launch_shape<DT, BITS, GS, 8, 4, true>(a);
        case 16: return launch_shape<DT, BITS, GS, 8, 8, false>(a);
        case 17: return launch_shape<DT, BITS, GS, 8, 8, true>(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool mfma_reg_supports(int bits, int64_t M, int64_t K) {
    if (M > 16) return false;
    RegShape s;
    if (!pick_shape(bits, 128, K, s)) return false;
    // staged activations plus the reduction buffers must fit the 160 KiB of LDS
    const int64_t KC = static_cast<int64_t>(s.W) * s.KPW * kblk_of(bits);
    return lds_x_bytes(M, KC) + lds_red_bytes(s.W) <= 160 * 1024;
}

hipError_t launch_mfma_reg(const MatmulArgs& a) {
#define RCALL(D, B, G) launch_reg_t<D, B, G>(a)
    switch (a.dt * 100 + a.bits * 10 + a.gs / 32) {
        case 41: return RCALL(0, 4, 32);   case 42: return RCALL(0, 4, 64);   case 44: return RCALL(0, 4, 128);
        case 61: return RCALL(0, 6, 32);   case 62: return RCALL(0, 6, 64);   case 64: return RCALL(0, 6, 128);
        case 81: return RCALL(0, 8, 32);   case 82: return RCALL(0, 8, 64);   case 84: return RCALL(0, 8, 128);
        case 141: return RCALL(1, 4, 32);  case 142: return RCALL(1, 4, 64);  case 144: return RCALL(1, 4, 128);
        case 161: return RCALL(1, 6, 32);  case 162: return RCALL(1, 6, 64);  case 164: return RCALL(1, 6, 128);
        case 181: return RCALL(1, 8, 32);  case 182: return RCALL(1, 8, 64);  case 184: return RCALL(1, 8, 128);
        default: return hipErrorInvalidValue;
    }
#undef RCALL
}

}  // namespace qmm
