// splitk.hpp -- the product with k split across workgroups (host side).
//
// C[b] <- alpha * sum_p A[b] B[b] (+ C[b]) as P partial products over
// consecutive k partitions, each written to a caller-owned workspace, then
// one reduction that adds the partials in partition order and applies the
// epilogue (StaleyNET "GPU Implementation", section "The matrix product":
// the product, optionally plus C).  This serves products whose output has
// too few tiles to occupy the chip and whose k is long: one tile per
// workgroup leaves most CUs idle however the k loop is organised inside a
// workgroup.
//
// Phase 1 is an ordinary launch of the tiled or wavefront kernels: the
// partitions are an inner batch level (inner stride kc along k for A and
// B, m*n in the workspace), plus one more launch when the last partition is
// shorter.  The partials use alpha = 1 and no C; the reduction forms
// alpha * S (+ C_old) with the same rounding as the other kernels'
// epilogue.  The partition order is fixed, so results are reproducible bit
// for bit (they differ from the unsplit product's bits: the k sum is
// grouped differently).
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <string>

#include "plan.hpp"

namespace sgemm {

struct SplitPlan {
    int splits = 1;                 // k partitions; 1 runs `whole` (no workspace used)
    int64_t kc = 0;                 // k of each partition but possibly the last
    int64_t k_last = 0;             // k of the last partition
    int full = 0;                   // partitions of exactly kc (launched together in `parts`)
    Plan whole, parts, tail;        // tail: the last partition when it is shorter
    int64_t workspace_floats = 0;   // splits * batch * m * n
    double cost = 0.0;              // cost model estimate (cycles), reduction included
};

// Partial-sum layout in the workspace: partition q of batch entry b at
// W + (b * splits + q) * m * n, rows of n floats.
// Chooses the split (1 when splitting does not pay or the workspace holds
// none) for validated arguments `a`: `workspace` may be 0 for a size query
// (a 256-byte aligned address is assumed), `workspace_floats` caps the
// partials (< 0: no cap).  Returns kOk or a status with `why`.
int make_split_plan(const GemmArgs &a, int num_cus, uintptr_t workspace, int64_t workspace_floats,
                    SplitPlan &sp, std::string &why);

// Enqueues the split plan's launches (phase 1, then the reduction) on `stream`.
int launch_split_plan(const GemmArgs &a, const SplitPlan &sp, uintptr_t workspace, hipStream_t stream,
                      std::string &why);

// The reduction: C[b,i,j] <- epilogue(alpha, sum_q W[b,q,i,j], C_old) for
// b < batch, i < m, j < n (kernels.hip / splitk_kernel.hip).
struct SplitReduceArgs {
    const float *W;
    float *C;
    long long batch, m, n;
    int splits;
    float alpha;
    int accumulate;
    long long sC_b, sC_m, sC_n;
    int vec4;   // n % 4 == 0, C rows contiguous and 16-byte aligned: 4 outputs per thread
};
void launch_split_reduce(const SplitReduceArgs &r, hipStream_t stream);

}  // namespace sgemm
