// Launchers shared between the libqmm translation units (host side).
#pragma once

#include <atomic>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

hipError_t launch_quantize(int dt, int bits, int gs, const void* w, uint32_t* wq, void* s, void* b,
                           int64_t N, int64_t K, hipStream_t st);
hipError_t launch_dequantize(int dt, int bits, int gs, const uint32_t* wq, const void* s, const void* b,
                             void* out, int64_t N, int64_t K, hipStream_t st);

// Arguments of one small-M matmul call (validated by the ABI layer).
struct MatmulArgs {
    int dt, bits, gs;
    int64_t M, N, K;
    const void* x;
    const uint32_t* wq;
    const void* scales;
    const void* biases;
    void* y;
    hipStream_t stream;
    // K split across workgroups (tile kernels only): `split` fp32 partial
    // outputs [split][M][N] in `part`, added in order by a second kernel.
    // split < 2: no split, `part` unused.
    float* part;
    int split;
    // Batch entries (register kernel only; the others are launched once per
    // entry): entry b reads x, wq, scales, biases and writes y at b times the
    // dense size of one entry's array.
    int64_t batch = 1;
};

// Raise a kernel's dynamic-LDS limit to the CU's 160 KiB on the current
// device, once per device (the attribute is a per-device setting; `done`
// holds one bit per device id below 64, beyond that the call is repeated).
inline hipError_t raise_lds_limit(const void* kernel, std::atomic<uint64_t>& done) {
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t{1} << dev : 0;
    if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

hipError_t launch_valu(const MatmulArgs& a);
hipError_t launch_mfma_reg(const MatmulArgs& a);
hipError_t launch_mfma_pass(const MatmulArgs& a);
// tile kernel shapes (columns per workgroup tile)
enum { TILE_CFG_16 = 0, TILE_CFG_64 = 1 };
hipError_t launch_mfma_tile(const MatmulArgs& a, int cfg);
// non-transposed weights (W [K, N], quantized along N): y = x . dequant(W)
hipError_t launch_nt(const MatmulArgs& a);
// ... with K split across 128-column workgroups where the plan splits
// (fp32 partials [split][M][N] in a.part); otherwise as launch_nt
struct NtPlan {
    bool wide;   // 128-column workgroups
    int split;   // K slices (1: unsplit, no workspace)
    int64_t ks;  // rows per slice (a multiple of 32)
    bool tr;     // the transpose-read form (4- and 8-bit codes)
};
NtPlan nt_plan(int bits, int64_t M, int64_t N, int64_t K);
hipError_t launch_nt_split(const MatmulArgs& a);
// M <= 16: every format where the k-blocks fit; M 17..64, on 16-row blocks
// (vector form, 16 wavefronts): 4-bit LDS-ring grids on shapes with more
// 16-column tiles than column slots, else any width where 16 rows take one
// tile per workgroup.
bool mfma_reg_supports(int bits, int gs, int64_t M, int64_t N, int64_t K);
// the second of those (one tile per workgroup, 16-row blocks)
bool mfma_reg_single_tile_rows(int bits, int gs, int64_t M, int64_t N, int64_t K);
// The register kernel's K split (4-bit LDS-ring form): K a whole number
// `split` of slices that form covers, with more column tiles than
// workgroups per slice.
bool mfma_reg_split_supports(int bits, int gs, int64_t M, int64_t N, int64_t K, int split);
// y[i] = sum over s < split of part[s * mn + i], in that order, rounded once
// to dt (the second kernel of every K split).
hipError_t launch_reduce_partials(int dt, const float* part, void* y, int split, int64_t mn, hipStream_t st);
bool mfma_tile_supports(int bits, int64_t M, int64_t K, int cfg);
// weights dequantized into LDS (64-column tiles, whole K chunks)
bool mfma_dqlds_supports(int bits, int64_t M, int64_t N, int64_t K);
hipError_t launch_mfma_dqlds(const MatmulArgs& a);
// A split count made valid for the tile kernel (every split gets at least
// one pass); the workspace holds that many partial outputs.
int tile_split(int bits, int64_t K, int cfg, int split);

}  // namespace qmm
