// epilogue.hpp -- the value every kernel writes to C (device code only).
//
// C <- alpha * (A*B) + beta * C_old + row[i] + col[j] (the general epilogue;
// "optionally plus C" of StaleyNET "GPU Implementation", section "The matrix
// product", is beta = 1 with no vector terms).
#pragma once

#include <hip/hip_runtime.h>

namespace sgemm {

// The stored value for a product `acc`: alpha * acc when nothing is added,
// else one fused multiply-add onto t = beta * c_old (only when C is read) +
// r (row term) + c (column term), summed in that order.  With beta = 1 and no
// vector terms this is fma(alpha, acc, c_old), the accumulate mode's bits.
__device__ __forceinline__ float epilogue_value(float alpha, float acc, bool read_c, float beta,
                                                float c_old, bool has_row, float r, bool has_col,
                                                float c) {
    if (!read_c && !has_row && !has_col) return alpha * acc;
    float t = read_c ? beta * c_old : 0.0f;
    if (has_row) t += r;
    if (has_col) t += c;
    return __builtin_fmaf(alpha, acc, t);
}

}  // namespace sgemm
