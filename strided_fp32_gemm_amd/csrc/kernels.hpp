// kernels.hpp -- kernel argument blocks and the launch entry used by the ABI.
#pragma once

#include <hip/hip_runtime_api.h>

#include <string>

#include "plan.hpp"

namespace sgemm {

// Arguments of the MFMA kernels (kernel terms: A m x k, B k x n, C m x n).
// 64-bit strides place each workgroup's base; offsets inside a workgroup's
// slice fit 32 bits (checked by the planner).
struct MfmaArgs {
    const float *A;
    const float *B;
    float *C;
    long long sA_b, sA_m, sA_k;
    long long sB_b, sB_k, sB_n;
    long long sC_b, sC_m, sC_n;
    int m, n, k;
    int tiles_m, tiles_n;
    int vec_a, vec_b;
    float alpha;
};

// Arguments of the generic kernel: everything 64-bit.
struct GenericArgs {
    const float *A;
    const float *B;
    float *C;
    long long sA_b, sA_m, sA_k;
    long long sB_b, sB_k, sB_n;
    long long sC_b, sC_m, sC_n;
    long long m, n, k, batch;
    long long tiles_m, tiles_n;
    float alpha;
    int accumulate;
};

// Enqueues the plan on `stream`.  Returns kOk, or kErrHip with `why` set when
// the runtime rejects the launch.
int launch_plan(const Plan &p, hipStream_t stream, std::string &why);

}  // namespace sgemm
