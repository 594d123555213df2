// Quantize and dequantize kernels (bit-exact; not on the timed path).
//
// Format: affine codes of 4, 6 or 8 bits with one scale and one bias per
// group of 32, 64 or 128 consecutive K elements, fp16/bf16 values ("What Are
// NAX Verify Kernels and When Is the Turbo Profile Activated in MTPLX?",
// "Supported Data Formats and Quantization Schemes"); quantize returns
// (wq, scales, biases) as in MLX issue #4720, "To Reproduce".
//
// Quantizer (the min/max affine reading; every step IEEE fp32 with explicit
// round-to-nearest-even intrinsics so that no contraction or fast division
// can change a bit):
//   lo = min, hi = max of the group (exact dtype values; a zero minimum is +0)
//   s  = round_up_dt(fl32(fl32(hi - lo) / (2^BITS - 1))),  b = lo
//   q  = s == 0 ? 0 : clamp(rint(fl32(fl32(w - b) / s)), 0, 2^BITS - 1)
// Dequantize: RNE_dt(fma(s, q, b)); s*q is exact in fp32, so the fused and
// unfused forms agree bit for bit.
#include "qmm_device.hpp"
#include "qmm_internal.hpp"

namespace qmm {

// One thread per (row, group).  The group's GS values are read with 16-byte
// loads; its GS*BITS/32 packed words are assembled in registers.
template <int DT, int BITS, int GS>
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ w,
                                                       uint32_t* __restrict__ wq,
                                                       uint16_t* __restrict__ scales,
                                                       uint16_t* __restrict__ biases,
                                                       int64_t N, int64_t K) {
    const int64_t G = K / GS;
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (gid >= N * G) return;
    const int64_t n = gid / G;
    const int64_t g = gid - n * G;

    float v[GS];
    const uint4* src = reinterpret_cast<const uint4*>(w + n * K + g * GS);
#pragma unroll
    for (int i = 0; i < GS / 8; ++i) {
        const uint4 u = src[i];
        const uint32_t p[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[8 * i + 2 * j] = DtOps<DT>::to_f32(static_cast<uint16_t>(p[j] & 0xFFFFu));
            v[8 * i + 2 * j + 1] = DtOps<DT>::to_f32(static_cast<uint16_t>(p[j] >> 16));
        }
    }
    float lo = v[0], hi = v[0];
#pragma unroll
    for (int k = 1; k < GS; ++k) {
        lo = fminf(lo, v[k]);
        hi = fmaxf(hi, v[k]);
    }
    lo = __fadd_rn(lo, 0.0f);  // -0 -> +0 so the bias of a zero minimum is +0

    constexpr float Q = static_cast<float>((1 << BITS) - 1);
    const float s32 = __fdiv_rn(__fsub_rn(hi, lo), Q);
    const uint16_t s_bits = round_up_nonneg<DT>(s32);
    const float s = DtOps<DT>::to_f32(s_bits);

    constexpr int NW = GS * BITS / 32;
    uint32_t words[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) words[i] = 0u;
#pragma unroll
    for (int k = 0; k < GS; ++k) {
        uint32_t q = 0u;
        if (s != 0.0f) {
            const float t = __fdiv_rn(__fsub_rn(v[k], lo), s);
            q = static_cast<uint32_t>(fminf(fmaxf(rintf(t), 0.0f), Q));
        }
        const int pos = BITS * k;
        words[pos >> 5] |= q << (pos & 31);
        if ((pos & 31) + BITS > 32) words[(pos >> 5) + 1] |= q >> (32 - (pos & 31));
    }
    uint32_t* dst = wq + n * (K * BITS / 32) + g * NW;
#pragma unroll
    for (int i = 0; i < NW; ++i) dst[i] = words[i];
    scales[n * G + g] = s_bits;
    biases[n * G + g] = DtOps<DT>::rne(lo);
}

// One thread per 32-code chunk (a chunk never straddles a group since
// GS is a multiple of 32): BITS words in, 64 bytes out.
template <int DT, int BITS, int GS>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint32_t* __restrict__ wq,
                                                         const uint16_t* __restrict__ scales,
                                                         const uint16_t* __restrict__ biases,
                                                         uint16_t* __restrict__ out,
                                                         int64_t N, int64_t K) {
    const int64_t chunks = K / 32;
    const int64_t id = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (id >= N * chunks) return;
    const int64_t n = id / chunks;
    const int64_t c = id - n * chunks;
    uint32_t w[BITS];
    load_chunk_words<BITS>(wq + n * (K * BITS / 32) + c * BITS, w);
    const int64_t gi = n * (K / GS) + (c * 32) / GS;
    const float s = DtOps<DT>::to_f32(scales[gi]);
    const float b = DtOps<DT>::to_f32(biases[gi]);
    uint32_t o[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const float lo_v = __fmaf_rn(s, static_cast<float>(chunk_code<BITS>(w, 2 * t)), b);
        const float hi_v = __fmaf_rn(s, static_cast<float>(chunk_code<BITS>(w, 2 * t + 1)), b);
        o[t] = static_cast<uint32_t>(DtOps<DT>::rne(lo_v)) | (static_cast<uint32_t>(DtOps<DT>::rne(hi_v)) << 16);
    }
    uint4* dst = reinterpret_cast<uint4*>(out + n * K + c * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
}

template <int DT, int BITS, int GS>
static hipError_t launch_quantize_t(const void* w, uint32_t* wq, void* s, void* b, int64_t N, int64_t K,
                                    hipStream_t st) {
    const int64_t total = N * (K / GS);
    const int block = 256;
    const int64_t grid = (total + block - 1) / block;
    hipLaunchKernelGGL((quantize_kernel<DT, BITS, GS>), dim3(static_cast<unsigned>(grid)), dim3(block), 0, st,
                       static_cast<const uint16_t*>(w), wq, static_cast<uint16_t*>(s),
                       static_cast<uint16_t*>(b), N, K);
    return hipGetLastError();
}

template <int DT, int BITS, int GS>
static hipError_t launch_dequantize_t(const uint32_t* wq, const void* s, const void* b, void* out, int64_t N,
                                      int64_t K, hipStream_t st) {
    const int64_t total = N * (K / 32);
    const int block = 256;
    const int64_t grid = (total + block - 1) / block;
    hipLaunchKernelGGL((dequantize_kernel<DT, BITS, GS>), dim3(static_cast<unsigned>(grid)), dim3(block), 0, st,
                       wq, static_cast<const uint16_t*>(s), static_cast<const uint16_t*>(b),
                       static_cast<uint16_t*>(out), N, K);
    return hipGetLastError();
}

#define QMM_FORMAT_SWITCH(DTV, BITSV, GSV, CALL)                                   \
    switch ((DTV) * 100 + (BITSV) * 10 + (GSV) / 32) {                             \
        case 41: return CALL(0, 4, 32);   case 42: return CALL(0, 4, 64);           \
        case 44: return CALL(0, 4, 128);  case 61: return CALL(0, 6, 32);           \
        case 62: return CALL(0, 6, 64);   case 64: return CALL(0, 6, 128);          \
        case 81: return CALL(0, 8, 32);   case 82: return CALL(0, 8, 64);           \
        case 84: return CALL(0, 8, 128);  case 141: return CALL(1, 4, 32);          \
        case 142: return CALL(1, 4, 64);  case 144: return CALL(1, 4, 128);         \
        case 161: return CALL(1, 6, 32);  case 162: return CALL(1, 6, 64);          \
        case 164: return CALL(1, 6, 128); case 181: return CALL(1, 8, 32);          \
        case 182: return CALL(1, 8, 64);  case 184: return CALL(1, 8, 128);         \
        default: return hipErrorInvalidValue;                                      \
    }

hipError_t launch_quantize(int dt, int bits, int gs, const void* w, uint32_t* wq, void* s, void* b,
                           int64_t N, int64_t K, hipStream_t st) {
#define QCALL(D, B, G) launch_quantize_t<D, B, G>(w, wq, s, b, N, K, st)
    QMM_FORMAT_SWITCH(dt, bits, gs, QCALL)
#undef QCALL
}

hipError_t launch_dequantize(int dt, int bits, int gs, const uint32_t* wq, const void* s, const void* b,
                             void* out, int64_t N, int64_t K, hipStream_t st) {
#define DCALL(D, B, G) launch_dequantize_t<D, B, G>(wq, s, b, out, N, K, st)
    QMM_FORMAT_SWITCH(dt, bits, gs, DCALL)
#undef DCALL
}

}  // namespace qmm
