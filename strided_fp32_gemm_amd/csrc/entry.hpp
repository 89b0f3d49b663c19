// entry.hpp -- library-internal pieces of the C ABI shared between abi.cpp
// and the allocation-free entry point in scratch.hip.
#pragma once

#include <cstdint>
#include <string>

namespace sgemm {

// Where the distance product keeps its two norm vectors: the caller's
// workspace (`fixed_floats` == 0), or a fixed device array of `fixed_floats`
// floats whose address `fixed_address` looks up for the current device (it
// is asked only after every argument check has passed).
typedef int (*ScratchAddressFn)(float **address, std::string &why);

int pairwise_sqdist(int64_t batch, int64_t m, int64_t n, int64_t k, const float *X, int64_t sX_batch,
                    int64_t sX_row, int64_t sX_col, const float *Y, int64_t sY_batch, int64_t sY_row,
                    int64_t sY_col, float *D, int64_t sD_batch, int64_t sD_row, int64_t sD_col,
                    float *workspace, int64_t workspace_floats, int64_t fixed_floats,
                    ScratchAddressFn fixed_address, void *stream);

}  // namespace sgemm
