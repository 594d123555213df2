// Kernel selection for qmm_small_m (host logic, no HIP calls).
#pragma once

#include <stdint.h>

#include "qmm_internal.hpp"

namespace qmm {

// Whether variant `kid` can run this (already validated) problem.
bool kernel_supports(int kid, int dt, int bits, int gs, int64_t M, int64_t N, int64_t K);

// The variant qmm_small_m uses: a table of crossovers measured on MI355X.
int select_kernel(int dt, int bits, int gs, int64_t M, int64_t N, int64_t K);

hipError_t launch_kernel(int kid, const MatmulArgs& a);

// The variant and K split qmm_small_m_ws uses (split 1: what qmm_small_m
// does, no workspace).
struct SplitPlan {
    int kernel;
    int split;
};
SplitPlan plan_split(int dt, int bits, int gs, int64_t M, int64_t N, int64_t K);

}  // namespace qmm
