// Device helpers shared by the libqmm kernels (gfx950, wave64).
//
// Values of the activation dtype travel as raw 16-bit patterns (uint16_t);
// DtOps<DT> converts them.  Code extraction follows the packed layout of the
// library boundary: each weight row is a little-endian bitstream with code k
// at bits [BITS*k, BITS*k + BITS) of consecutive little-endian uint32 words.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

enum : int { DT_F16 = 0, DT_BF16 = 1 };

template <int DT>
struct DtOps;

template <>
struct DtOps<DT_F16> {
    __device__ __forceinline__ static float to_f32(uint16_t h) {
        return static_cast<float>(__builtin_bit_cast(_Float16, h));
    }
    // Nearest-even (the hardware conversion in the default rounding mode).
    __device__ __forceinline__ static uint16_t rne(float f) {
        return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
    }
};

template <>
struct DtOps<DT_BF16> {
    __device__ __forceinline__ static float to_f32(uint16_t h) {
        return __builtin_bit_cast(float, static_cast<uint32_t>(h) << 16);
    }
    // Nearest-even on the bit pattern (finite inputs).
    __device__ __forceinline__ static uint16_t rne(float f) {
        uint32_t u = __builtin_bit_cast(uint32_t, f);
        u += 0x7FFFu + ((u >> 16) & 1u);
        return static_cast<uint16_t>(u >> 16);
    }
};

// Toward +infinity for f >= 0: nearest-even, then one step up if that
// landed below f (for a non-negative pattern the next pattern is the next
// larger value).
template <int DT>
__device__ __forceinline__ uint16_t round_up_nonneg(float f) {
    uint16_t r = DtOps<DT>::rne(f);
    if (DtOps<DT>::to_f32(r) < f) r = static_cast<uint16_t>(r + 1u);
    return r;
}

// Code t (0 <= t < 32) of a 32-code chunk whose BITS words start at w[0].
// All indices are compile-time constants after unrolling.
template <int BITS>
__device__ __forceinline__ uint32_t chunk_code(const uint32_t* w, int t) {
    constexpr uint32_t mask = (1u << BITS) - 1u;
    const int pos = BITS * t;
    const int wi = pos >> 5;
    const int off = pos & 31;
    uint32_t v = w[wi] >> off;
    if (off + BITS > 32) v |= w[wi + 1] << (32 - off);
    return v & mask;
}

// Load the BITS words (16, 24 or 32 bytes) of one 32-code chunk.
template <int BITS>
__device__ __forceinline__ void load_chunk_words(const uint32_t* __restrict__ p, uint32_t (&w)[BITS]) {
    if constexpr (BITS == 4) {
        const uint4 a = *reinterpret_cast<const uint4*>(p);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    } else if constexpr (BITS == 8) {
        const uint4 a = *reinterpret_cast<const uint4*>(p);
        const uint4 b = *reinterpret_cast<const uint4*>(p + 4);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else {
        // 24 bytes, 8-byte aligned (chunk offset is a multiple of 24 bytes)
        const uint2 a = *reinterpret_cast<const uint2*>(p);
        const uint2 b = *reinterpret_cast<const uint2*>(p + 2);
        const uint2 c = *reinterpret_cast<const uint2*>(p + 4);
        w[0] = a.x; w[1] = a.y; w[2] = b.x; w[3] = b.y; w[4] = c.x; w[5] = c.y;
    }
}

}  // namespace qmm
