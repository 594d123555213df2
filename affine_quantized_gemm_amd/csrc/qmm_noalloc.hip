// qmm_small_m_noalloc: qmm_small_m_ws with its workspace in a fixed,
// library-owned device array instead of a caller buffer, for callers that
// cannot allocate (code under stream capture, serving loops that forbid
// allocation).  Contract: qmm.h.
//
// The array lives in this file as a static __device__ object: the loader
// gives every GPU the library runs on its own copy, held until the process
// ends.  On the host its name is only a stand-in, so host code never passes
// it to a kernel or a copy; the device address is looked up once per device
// with hipGetSymbolAddress (with that device current, at the first call on
// it) and kept.  What the array holds is each K-split's fp32 partial
// outputs, which the split kernels overwrite in full before the reduction
// reads them, so nothing needs clearing between calls; calls that overlap
// on one GPU share the array and race.
#include <mutex>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "qmm.h"

namespace {

static __device__ __align__(256) unsigned char scratch[QMM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this GPU's copy of `scratch` (set up on first use).
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return QMM_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return QMM_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return QMM_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return QMM_OK;
}

}  // namespace

extern "C" int qmm_small_m_noalloc(int dt, int bits, int group_size, int64_t M, int64_t N, int64_t K,
                                   const void* x, const uint32_t* wq, const void* scales, const void* biases,
                                   void* y, void* stream) {
    // all validation is host logic and comes first: the planned workspace
    // (0 when the plan does not split K) against the array's size
    const int64_t need = qmm_small_m_workspace_bytes(dt, bits, group_size, M, N, K);
    if (need < 0) return static_cast<int>(need);
    if (need > QMM_NOALLOC_SCRATCH_BYTES) return QMM_ERR_UNSUPPORTED;
    if (M == 0 || N == 0 || need == 0)
        return qmm_small_m_ws(dt, bits, group_size, M, N, K, x, wq, scales, biases, y, nullptr, 0, stream);
    // (pointer checks before the one-time set-up, so that a rejected call
    // makes no HIP call at all)
    const void* ps[] = {x, wq, scales, biases, y};
    for (const void* p : ps) {
        if (p == nullptr) return QMM_ERR_INVALID_ARG;
    }
    for (const void* p : ps) {
        if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0) return QMM_ERR_MISALIGNED;
    }
    void* ws = nullptr;
    if (const int st = scratch_address(&ws); st != QMM_OK) return st;
    return qmm_small_m_ws(dt, bits, group_size, M, N, K, x, wq, scales, biases, y, ws, need, stream);
}
