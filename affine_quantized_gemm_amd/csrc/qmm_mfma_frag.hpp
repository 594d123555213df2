// Matrix-core fragment helpers shared by the MFMA small-M kernels (gfx950).
//
// A wavefront computes 16x16 output tiles with v_mfma_f32_16x16x32_{f16,bf16}
// (operand layout verified on the hardware: lane l supplies A[l%16][8*(l/16)+e]
// and B[8*(l/16)+e][l%16] for e = 0..7 and receives D[4*(l/16)+r][l%16],
// r = 0..3).  The weight operand is built in registers from packed codes: a
// lane loads one "segment" of its column's codes, lane swaps make every
// matrix step lie inside one quantization group, and the "magic number"
// unpack turns codes into exact fp16/bf16 values q + off.  The activation
// operand is permuted to the order that unpack produces.
#pragma once

#include "qmm_device.hpp"

namespace qmm {
namespace mf {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

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

// Exchange of 32-lane halves / odd and even 16-lane rows between two
// registers (gfx950 permlane swaps; semantics checked on the hardware).
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
// STEPS = SEG/8 MFMA steps.  A k-block splits into PORTIONS runs of PC
// codes, each inside one quantization group; a portion is the "unit" of the
// scale step.
template <int DT, int BITS, int GS>
struct Fmt {
    static constexpr int SEG = BITS == 4 ? 32 : 16;      // codes per lane load
    static constexpr int SEG_WORDS = SEG * BITS / 32;    // 4, 3 or 4 words (16, 12, 16 bytes)
    static constexpr int STEPS = SEG / 8;                // MFMA steps per k-block
    static constexpr int KBLK = 4 * SEG;                 // codes per k-block
    static constexpr int PORTIONS = (KBLK / GS) > 1 ? (KBLK / GS) : 1;
    static constexpr int STEPS_PER_PORTION = STEPS / PORTIONS;
    static constexpr int PC = KBLK / PORTIONS;           // codes per portion
    // offset carried by the code at natural position t of an 8-code run
    __host__ __device__ static constexpr float off(int t) {
        if (DT == DT_F16 && BITS == 4) return (t & 1) ? 64.0f : 1024.0f;
        if (DT == DT_F16) return 1024.0f;
        if (BITS == 8) return 0.0f;
        return 128.0f;
    }
    static constexpr bool HAS_OFF = !(DT == DT_BF16 && BITS == 8);
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
    uint32_t nib;     // 0x000F000F
    uint32_t nib_hi;  // 0x00F000F0
    uint32_t six;     // 0x0000003F
    uint32_t six_hi;  // 0x003F0000
    uint32_t magic;   // q + off pattern: 0x6400 (fp16, 1024) / 0x4300 (bf16, 128) in both halves
    uint32_t magic4;  // fp16 with the code in mantissa bits 4..7: 0x5400 = 64, step 1/16
};

template <int DT>
__device__ __forceinline__ UnpackConsts unpack_consts() {
    UnpackConsts k;
    k.nib = 0x000F000Fu;
    k.nib_hi = 0x00F000F0u;
    k.six = 0x3Fu;
    k.six_hi = 0x3F0000u;
    k.magic = (DT == DT_F16) ? 0x64006400u : 0x43004300u;
    k.magic4 = 0x54005400u;
    // keep them in registers (not folded back into literals)
    asm volatile("" : "+v"(k.nib), "+v"(k.nib_hi), "+v"(k.six), "+v"(k.six_hi), "+v"(k.magic), "+v"(k.magic4));
    return k;
}

// 4-bit: one word (8 codes) -> q + off in order 0,4,1,5,2,6,3,7.  fp16 takes
// the odd nibbles in place (64 + q, via magic4), bf16 shifts them down
// (its 7 mantissa bits cannot hold a code at bits 4..7).
// UNI: every code carries the same offset (fp16 shifts the odd nibbles
// down too, two more operations per word).
template <int DT, bool UNI = false>
__device__ __forceinline__ Frag unpack4(uint32_t w, const UnpackConsts& k) {
    Frag f;
    const uint32_t w8 = w >> 8;
    f.v[0] = and_or(w, k.nib, k.magic);
    f.v[2] = and_or(w8, k.nib, k.magic);
    if constexpr (DT == DT_F16 && !UNI) {
        f.v[1] = and_or(w, k.nib_hi, k.magic4);
        f.v[3] = and_or(w8, k.nib_hi, k.magic4);
    } else {
        f.v[1] = and_or(w >> 4, k.nib, k.magic);
        f.v[3] = and_or(w >> 12, k.nib, k.magic);
    }
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
template <int DT, int BITS, int GS, int NW, int NS, bool UNI = false>
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
        for (int s = 0; s < 4; ++s) b[s] = unpack4<DT, UNI>(w[s], k);
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

template <int BITS, int NW, bool NT = true>
__device__ __forceinline__ void load_segment(const uint32_t* __restrict__ p, uint32_t (&w)[NW]) {
    if constexpr (NW == 4) {
        // streamed once: the non-temporal hint keeps the weights from
        // displacing reused data in the caches (NT = false: read again by
        // other workgroups, so kept in L2)
        u32x4_t a;
        if constexpr (NT)
            a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
        else
            a = *reinterpret_cast<const u32x4_t*>(p);
        w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
    } else {
        const uint3 a = *reinterpret_cast<const uint3*>(p);
        w[0] = a.x; w[1] = a.y; w[2] = a.z;
    }
}

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

// Offset carried by the value in slot e of an activation fragment (the
// fragment holds its 8 codes in the order the weight unpack produces).
template <int DT, int BITS, int GS>
__host__ __device__ constexpr float slot_off(int e) {
    using F = Fmt<DT, BITS, GS>;
    if constexpr (BITS == 4) {
        constexpr int perm[8] = {0, 4, 1, 5, 2, 6, 3, 7};
        return F::off(perm[e]);
    } else if constexpr (BITS == 6) {
        constexpr int perm[8] = {0, 2, 1, 3, 4, 6, 5, 7};
        return F::off(perm[e]);
    } else {
        return F::off(e);
    }
}

// 16-bit patterns of the few exact constants the unit sums use (1 and the
// code offsets 0, 64, 128, 1024).
template <int DT>
struct DtBits;
template <>
struct DtBits<DT_F16> {
    static constexpr uint32_t one = 0x3C00u;
    __host__ __device__ static constexpr uint32_t of(float v) {
        return v == 1024.0f ? 0x6400u : v == 64.0f ? 0x5400u : v == 128.0f ? 0x5800u : v == 1.0f ? 0x3C00u : 0u;
    }
};
template <>
struct DtBits<DT_BF16> {
    static constexpr uint32_t one = 0x3F80u;
    __host__ __device__ static constexpr uint32_t of(float v) {
        return v == 1024.0f ? 0x4480u : v == 64.0f ? 0x4280u : v == 128.0f ? 0x4300u : v == 1.0f ? 0x3F80u : 0u;
    }
};


}  // namespace mf
}  // namespace qmm
