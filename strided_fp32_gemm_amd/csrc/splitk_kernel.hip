// splitk_kernel.hip -- the reduction of the split-k product.
//
// Adds the partition partials of each output in a fixed order and writes
// alpha * S (+ C_old) with the same rounding as every other kernel's
// epilogue.  HBM-bound, and with few outputs latency-bound: eight threads
// share each group of 4 (or 1) outputs, thread t summing the t-th run of
// consecutive partitions (in partition order), and the first of them adding
// the eight run sums in run order.  The order depends only on the number of
// partitions, so the bits are reproducible; with at most 8 partitions it is
// plain partition order.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "epilogue.hpp"
#include "splitk.hpp"

namespace sgemm {

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kRuns = 8;                    // threads per output group
constexpr int kGroups = 256 / kRuns;        // output groups per workgroup

template <typename T>
__device__ __forceinline__ T load_part(const float *p) {
    return *reinterpret_cast<const T *>(p);
}

// Output group g of a workgroup, run t: threads tid = t * kGroups + g, so
// the 32 threads of one run read 32 consecutive groups (coalesced).
template <typename T, int W>
__device__ void reduce_groups(const SplitReduceArgs &r, T (&runs)[kRuns][kGroups]) {
    const long long per_row = r.n / W;
    const long long total = r.batch * r.m * per_row;
    const long long mn = r.m * r.n;
    const bool acc = r.accumulate != 0;
    const int tid = threadIdx.x, g = tid % kGroups, t = tid / kGroups;
    const int per_run = (r.splits + kRuns - 1) / kRuns;
    const int q0 = min(t * per_run, r.splits), q1 = min(q0 + per_run, r.splits);
    for (long long base = (long long)blockIdx.x * kGroups; base < total; base += (long long)gridDim.x * kGroups) {
        const long long e = base + g;
        const bool live = e < total;
        const long long row = live ? e / per_row : 0;   // b * m + i
        const long long j = (live ? e - row * per_row : 0) * W;
        const long long b = row / r.m, i = row - b * r.m;
        const float *w = r.W + b * r.splits * mn + i * r.n + j;
        T s{};
        if (live && q0 < q1) {
            // Loads of up to four partitions go out before their sum.
            s = load_part<T>(w + q0 * mn);
            int q = q0 + 1;
            for (; q + 4 <= q1; q += 4) {
                const T v0 = load_part<T>(w + q * mn), v1 = load_part<T>(w + (q + 1) * mn);
                const T v2 = load_part<T>(w + (q + 2) * mn), v3 = load_part<T>(w + (q + 3) * mn);
                s += v0;
                s += v1;
                s += v2;
                s += v3;
            }
            for (; q < q1; ++q) s += load_part<T>(w + q * mn);
        }
        runs[t][g] = s;
        __syncthreads();
        if (t == 0 && live) {
            T sum = runs[0][g];
            for (int u = 1; u < kRuns && u * per_run < r.splits; ++u) sum += runs[u][g];
            float *c = r.C + b * r.sC_b + i * r.sC_m + j * r.sC_n;
            if constexpr (W == 4) {
                const f4 old = acc ? *reinterpret_cast<const f4 *>(c) : f4{0.0f, 0.0f, 0.0f, 0.0f};
                f4 o;
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    o[x] = epilogue_value(r.alpha, sum[x], acc, 1.0f, old[x], false, 0.0f, false, 0.0f);
                *reinterpret_cast<f4 *>(c) = o;
            } else {
                const float old = acc ? c[0] : 0.0f;
                c[0] = epilogue_value(r.alpha, sum, acc, 1.0f, old, false, 0.0f, false, 0.0f);
            }
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void sgemm_splitk_reduce4(SplitReduceArgs r) {
    __shared__ f4 runs[kRuns][kGroups];
    reduce_groups<f4, 4>(r, runs);
}

__global__ __launch_bounds__(256) void sgemm_splitk_reduce1(SplitReduceArgs r) {
    __shared__ float runs[kRuns][kGroups];
    reduce_groups<float, 1>(r, runs);
}

}  // namespace

void launch_split_reduce(const SplitReduceArgs &r, hipStream_t stream) {
    const long long total = r.batch * r.m * (r.vec4 ? r.n / 4 : r.n);
    const long long blocks = std::min<long long>((total + kGroups - 1) / kGroups, 16384);
    if (r.vec4)
        hipLaunchKernelGGL(sgemm_splitk_reduce4, dim3(unsigned(blocks)), dim3(256), 0, stream, r);
    else
        hipLaunchKernelGGL(sgemm_splitk_reduce1, dim3(unsigned(blocks)), dim3(256), 0, stream, r);
}

}  // namespace sgemm
