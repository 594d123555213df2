// extern "C" boundary of libqmm: argument validation, kernel selection and
// launches on the caller's stream.  Declarations and contracts: qmm.h.
//
// Unsupported formats are an explicit error here.  The pages' own wrapper
// silently falls back to a stock kernel when given unsupported parameters
// ("What Are NAX Verify Kernels and When Is the Turbo Profile Activated in
// MTPLX?", "Frequently Asked Questions"); this library has one code path per
// variant and reports QMM_ERR_UNSUPPORTED instead.
#include <algorithm>
#include <cstdint>
#include <stdint.h>

#include <initializer_list>

#include "qmm.h"
#include "qmm_internal.hpp"
#include "qmm_dispatch.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_format(int dt, int bits, int gs, int64_t N, int64_t K) {
    if (N < 0 || K < 0) return QMM_ERR_INVALID_ARG;
    if (dt != QMM_F16 && dt != QMM_BF16) return QMM_ERR_UNSUPPORTED;
    if (bits != 4 && bits != 6 && bits != 8) return QMM_ERR_UNSUPPORTED;
    if (gs != 32 && gs != 64 && gs != 128) return QMM_ERR_UNSUPPORTED;
    if (K < 64 || K % 64 != 0 || K % gs != 0) return QMM_ERR_UNSUPPORTED;
    // grid-size limits of the launchers (N*K/32 threads in a 32-bit grid)
    if (N > INT32_MAX || K > INT32_MAX) return QMM_ERR_UNSUPPORTED;
    if ((N * (K / 32) + 255) / 256 > INT32_MAX) return QMM_ERR_UNSUPPORTED;
    return QMM_OK;
}

int check_ptrs(std::initializer_list<const void*> ps) {
    for (const void* p : ps)
        if (p == nullptr) return QMM_ERR_INVALID_ARG;
    for (const void* p : ps)
        if (!aligned16(p)) return QMM_ERR_MISALIGNED;
    return QMM_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? QMM_OK : QMM_ERR_HIP; }

int check_matmul(int dt, int bits, int gs, int64_t M, int64_t N, int64_t K, const void* x, const uint32_t* wq,
                 const void* scales, const void* biases, void* y) {
    if (M < 0) return QMM_ERR_INVALID_ARG;
    int st = check_format(dt, bits, gs, N, K);
    if (st != QMM_OK) return st;
    if (M > 64) return QMM_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return QMM_OK;
    return check_ptrs({x, wq, scales, biases, y});
}

}  // namespace

extern "C" {

int qmm_quantize(int dt, int bits, int group_size, int64_t N, int64_t K, const void* w, uint32_t* wq, void* scales,
                 void* biases, void* stream) {
    int st = check_format(dt, bits, group_size, N, K);
    if (st != QMM_OK) return st;
    if (N == 0) return QMM_OK;
    st = check_ptrs({w, wq, scales, biases});
    if (st != QMM_OK) return st;
    return hip_status(qmm::launch_quantize(dt, bits, group_size, w, wq, scales, biases, N, K,
                                           static_cast<hipStream_t>(stream)));
}

int qmm_dequantize(int dt, int bits, int group_size, int64_t N, int64_t K, const uint32_t* wq, const void* scales,
                   const void* biases, void* w_out, void* stream) {
    int st = check_format(dt, bits, group_size, N, K);
    if (st != QMM_OK) return st;
    if (N == 0) return QMM_OK;
    st = check_ptrs({wq, scales, biases, w_out});
    if (st != QMM_OK) return st;
    return hip_status(qmm::launch_dequantize(dt, bits, group_size, wq, scales, biases, w_out, N, K,
                                             static_cast<hipStream_t>(stream)));
}

int qmm_select_kernel(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K) {
    if (M < 0) return QMM_ERR_INVALID_ARG;
    int st = check_format(dt, bits, group_size, N, K);
    if (st != QMM_OK) return st;
    if (M > 64) return QMM_ERR_UNSUPPORTED;
    return qmm::select_kernel(dt, bits, group_size, M, N, K);
}

int qmm_kernel_supported(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K, int kernel_id) {
    if (M < 0) return QMM_ERR_INVALID_ARG;
    int st = check_format(dt, bits, group_size, N, K);
    if (st != QMM_OK) return st;
    if (M > 64) return QMM_ERR_UNSUPPORTED;
    return qmm::kernel_supports(kernel_id, dt, bits, group_size, M, N, K) ? 1 : 0;
}

int qmm_small_m_forced(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K, const void* x,
                       const uint32_t* wq, const void* scales, const void* biases, void* y, void* stream,
                       int kernel_id) {
    int st = check_matmul(dt, bits, group_size, M, N, K, x, wq, scales, biases, y);
    if (st != QMM_OK) return st;
    if (!qmm::kernel_supports(kernel_id, dt, bits, group_size, M, N, K)) return QMM_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return QMM_OK;
    qmm::MatmulArgs a{dt, bits, group_size, M, N, K, x, wq, scales, biases, y, static_cast<hipStream_t>(stream)};
    return hip_status(qmm::launch_kernel(kernel_id, a));
}

int qmm_small_m(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K, const void* x,
                const uint32_t* wq, const void* scales, const void* biases, void* y, void* stream) {
    int st = check_matmul(dt, bits, group_size, M, N, K, x, wq, scales, biases, y);
    if (st != QMM_OK) return st;
    if (M == 0 || N == 0) return QMM_OK;
    const int kid = qmm::select_kernel(dt, bits, group_size, M, N, K);
    qmm::MatmulArgs a{dt, bits, group_size, M, N, K, x, wq, scales, biases, y, static_cast<hipStream_t>(stream)};
    return hip_status(qmm::launch_kernel(kid, a));
}

int qmm_small_m_batched(int dt, int bits, int group_size, int64_t batch, int64_t M, int64_t N, int64_t K,
                        const void* x, const uint32_t* wq, const void* scales, const void* biases, void* y,
                        void* stream) {
    if (batch < 0 || M < 0) return QMM_ERR_INVALID_ARG;
    int st = check_format(dt, bits, group_size, N, K);
    if (st != QMM_OK) return st;
    if (M > 64) return QMM_ERR_UNSUPPORTED;
    if (batch == 0 || M == 0 || N == 0) return QMM_OK;
    st = check_ptrs({x, wq, scales, biases, y});
    if (st != QMM_OK) return st;
    // bytes of one entry's array; every entry starts 16-byte aligned
    const int64_t sx = M * K * 2, sw = N * (K * bits / 8), ss = N * (K / group_size) * 2, sy = M * N * 2;
    const int64_t smax = std::max(std::max(sx, sw), std::max(ss, sy));
    if (batch > INT64_MAX / smax) return QMM_ERR_INVALID_ARG;
    if (batch > 1 && ((sx | sw | ss | sy) & 15) != 0) return QMM_ERR_MISALIGNED;
    const int kid = qmm::select_kernel(dt, bits, group_size, M, N, K);
    auto at = [](const void* p, int64_t off) { return static_cast<const void*>(static_cast<const char*>(p) + off); };
    // the register kernel takes up to 65535 entries per launch (grid.y); the
    // others one launch per entry
    const int64_t per = kid == QMM_KERNEL_MFMA_REG ? 65535 : 1;
    for (int64_t b0 = 0; b0 < batch; b0 += per) {
        qmm::MatmulArgs a{dt, bits, group_size, M, N, K, at(x, b0 * sx),
                          static_cast<const uint32_t*>(at(wq, b0 * sw)), at(scales, b0 * ss), at(biases, b0 * ss),
                          const_cast<void*>(at(y, b0 * sy)), static_cast<hipStream_t>(stream)};
        a.batch = std::min(per, batch - b0);
        st = hip_status(qmm::launch_kernel(kid, a));
        if (st != QMM_OK) return st;
    }
    return QMM_OK;
}

int qmm_small_m_nt(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K, const void* x,
                   const uint32_t* wq, const void* scales, const void* biases, void* y, void* stream) {
    if (M < 0 || K < 0) return QMM_ERR_INVALID_ARG;
    // the quantized axis is N here: it obeys the rules K obeys in the transposed layout
    int st = check_format(dt, bits, group_size, K, N);
    if (st != QMM_OK) return st;
    if (M > 64 || K < 32 || K % 32 != 0) return QMM_ERR_UNSUPPORTED;
    if (M == 0) return QMM_OK;
    st = check_ptrs({x, wq, scales, biases, y});
    if (st != QMM_OK) return st;
    qmm::MatmulArgs a{dt, bits, group_size, M, N, K, x, wq, scales, biases, y, static_cast<hipStream_t>(stream)};
    return hip_status(qmm::launch_nt(a));
}

int64_t qmm_small_m_nt_workspace_bytes(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K) {
    if (M < 0 || K < 0) return QMM_ERR_INVALID_ARG;
    int st = check_format(dt, bits, group_size, K, N);
    if (st != QMM_OK) return st;
    if (M > 64 || K < 32 || K % 32 != 0) return QMM_ERR_UNSUPPORTED;
    const qmm::NtPlan p = qmm::nt_plan(bits, M, N, K);
    return p.split > 1 ? static_cast<int64_t>(p.split) * M * N * 4 : 0;
}

int qmm_small_m_nt_ws(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K, const void* x,
                      const uint32_t* wq, const void* scales, const void* biases, void* y, void* workspace,
                      int64_t workspace_bytes, void* stream) {
    const int64_t need = qmm_small_m_nt_workspace_bytes(dt, bits, group_size, M, N, K);
    if (need < 0) return static_cast<int>(need);
    if (workspace_bytes < 0) return QMM_ERR_INVALID_ARG;
    if (M == 0) return QMM_OK;
    int st = check_ptrs({x, wq, scales, biases, y});
    if (st != QMM_OK) return st;
    if (need > 0) {
        if (workspace == nullptr || workspace_bytes < need) return QMM_ERR_INVALID_ARG;
        if (!aligned16(workspace)) return QMM_ERR_MISALIGNED;
    }
    qmm::MatmulArgs a{dt, bits, group_size, M, N, K, x, wq, scales, biases, y, static_cast<hipStream_t>(stream)};
    a.part = static_cast<float*>(workspace);
    return hip_status(qmm::launch_nt_split(a));
}

int qmm_split_plan(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K, int* kernel_id, int* split) {
    if (M < 0 || kernel_id == nullptr || split == nullptr) return QMM_ERR_INVALID_ARG;
    int st = check_format(dt, bits, group_size, N, K);
    if (st != QMM_OK) return st;
    if (M > 64) return QMM_ERR_UNSUPPORTED;
    const qmm::SplitPlan p = qmm::plan_split(dt, bits, group_size, M, N, K);
    *kernel_id = p.kernel;
    *split = p.split;
    return QMM_OK;
}

int64_t qmm_small_m_workspace_bytes(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K) {
    if (M < 0) return QMM_ERR_INVALID_ARG;
    int st = check_format(dt, bits, group_size, N, K);
    if (st != QMM_OK) return st;
    if (M > 64) return QMM_ERR_UNSUPPORTED;
    const qmm::SplitPlan p = qmm::plan_split(dt, bits, group_size, M, N, K);
    return p.split > 1 ? static_cast<int64_t>(p.split) * M * N * 4 : 0;
}

int qmm_small_m_split_forced(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K, const void* x,
                             const uint32_t* wq, const void* scales, const void* biases, void* y,
                             void* workspace, int64_t workspace_bytes, void* stream, int kernel_id, int split) {
    int st = check_matmul(dt, bits, group_size, M, N, K, x, wq, scales, biases, y);
    if (st != QMM_OK) return st;
    if (split < 1 || workspace_bytes < 0) return QMM_ERR_INVALID_ARG;
    const int cfg = kernel_id == QMM_KERNEL_MFMA_TILE16  ? qmm::TILE_CFG_16
                    : kernel_id == QMM_KERNEL_MFMA_TILE64 ? qmm::TILE_CFG_64
                                                          : -1;
    int eff = 1;
    if (split > 1 && kernel_id == QMM_KERNEL_MFMA_REG) {
        // the register kernel splits K into exactly `split` slices it covers
        // (it cannot run K that deep split-free)
        if (!qmm::mfma_reg_split_supports(bits, group_size, M, N, K, split)) return QMM_ERR_UNSUPPORTED;
        eff = split;
    } else {
        if (!qmm::kernel_supports(kernel_id, dt, bits, group_size, M, N, K)) return QMM_ERR_UNSUPPORTED;
        if (split > 1 && cfg < 0) return QMM_ERR_UNSUPPORTED;
        eff = split > 1 ? qmm::tile_split(bits, K, cfg, split) : 1;
    }
    if (M == 0 || N == 0) return QMM_OK;
    if (eff > 1) {
        if (workspace == nullptr || workspace_bytes < static_cast<int64_t>(eff) * M * N * 4)
            return QMM_ERR_INVALID_ARG;
        if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0) return QMM_ERR_MISALIGNED;
    }
    qmm::MatmulArgs a{dt, bits, group_size, M, N, K, x, wq, scales, biases, y, static_cast<hipStream_t>(stream),
                      static_cast<float*>(workspace), eff};
    return hip_status(qmm::launch_kernel(kernel_id, a));
}

int qmm_small_m_ws(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K, const void* x,
                   const uint32_t* wq, const void* scales, const void* biases, void* y, void* workspace,
                   int64_t workspace_bytes, void* stream) {
    int st = check_matmul(dt, bits, group_size, M, N, K, x, wq, scales, biases, y);
    if (st != QMM_OK) return st;
    if (workspace_bytes < 0) return QMM_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return QMM_OK;
    const qmm::SplitPlan p = qmm::plan_split(dt, bits, group_size, M, N, K);
    return qmm_small_m_split_forced(dt, bits, group_size, M, N, K, x, wq, scales, biases, y, workspace,
                                    workspace_bytes, stream, p.kernel, p.split);
}

int64_t qmm_packed_words(int bits, int64_t K) {
    if (bits != 4 && bits != 6 && bits != 8) return -1;
    if (K < 0 || (K * bits) % 32 != 0) return -1;
    return K * bits / 32;
}

// The build passes the digest of the sources this library was compiled from
// (every csrc/ and include/ file); the binding compares it with the sources
// beside the library before using it.
#ifndef QMM_SOURCE_DIGEST
#define QMM_SOURCE_DIGEST "unknown"
#endif
const char* qmm_build_digest(void) { return QMM_SOURCE_DIGEST; }

const char* qmm_strerror(int status) {
    switch (status) {
        case QMM_OK: return "ok";
        case QMM_ERR_INVALID_ARG: return "invalid argument (negative size or null pointer)";
        case QMM_ERR_UNSUPPORTED: return "unsupported format or shape";
        case QMM_ERR_MISALIGNED: return "array base pointer not 16-byte aligned";
        case QMM_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

const char* qmm_kernel_name(int kernel_id) {
    switch (kernel_id) {
        case QMM_KERNEL_VALU: return "valu_splitfree";
        case QMM_KERNEL_MFMA_REG: return "mfma_splitfree_reg";
        case QMM_KERNEL_MFMA_PASS: return "mfma_splitfree_pass";
        case QMM_KERNEL_MFMA_TILE16: return "mfma_splitfree_tile16";
        case QMM_KERNEL_MFMA_TILE64: return "mfma_splitfree_tile64";
        case QMM_KERNEL_MFMA_DQLDS: return "mfma_splitfree_dqlds";
        default: return "?";
    }
}

}  // extern "C"
