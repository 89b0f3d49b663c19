// kernels.hip -- the generic kernel and the launch dispatch.
//
// C[b,i,j] <- alpha * sum_p A[b,i,p] B[b,p,j] (+ beta C[b,i,j] + row[b,i] +
// col[b,j], the general epilogue of epilogue.hpp); operands are
// addressed through (batch, row, col) element strides (StaleyNET "GPU
// Implementation", section "The matrix product").  The matrix-core kernels
// live in mfma_kernel.hpp (LDS-tiled) and wave_kernel.hpp (direct
// wavefront); this file holds the generic kernel, which serves layouts whose
// offsets exceed the 32-bit buffer range, and launch_plan().
#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>

#include "epilogue.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace sgemm {

// ---------------------------------------------------------------------------
// Generic kernel: any strides, 64-bit addressing.  64 x 64 tile, 256
// threads, each thread a 4 x 4 block (rows ty + 16*r, columns tx + 16*c);
// 16-deep k slices staged through LDS; grid-stride loop over tiles.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void sgemm_generic(GenericArgs p) {
    __shared__ float As[16][64 + 1];
    __shared__ float Bs[16][64 + 1];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const long long per_batch = p.tiles_m * p.tiles_n;
    const long long total = p.batch * per_batch;
    for (long long tile = blockIdx.x; tile < total; tile += gridDim.x) {
        const long long b = tile / per_batch, t = tile - b * per_batch;
        const long long i0 = (t / p.tiles_n) * 64, j0 = (t % p.tiles_n) * 64;
        const long long bo = b / p.inner, bi = b - bo * p.inner;
        const float *A = p.A + bo * p.sA_b + (bi / p.gA) * p.sA_i;
        const float *B = p.B + bo * p.sB_b + (bi / p.gB) * p.sB_i;
        float acc[4][4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[r][c] = 0.0f;
        for (long long k0 = 0; k0 < p.k; k0 += 16) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int e = tid + 256 * q;
                const int x = e & 63, kk = e >> 6;
                const long long kg = k0 + kk;
                const long long i = i0 + x, j = j0 + x;
                As[kk][x] = (i < p.m && kg < p.k) ? A[i * p.sA_m + kg * p.sA_k] : 0.0f;
                Bs[kk][x] = (j < p.n && kg < p.k) ? B[kg * p.sB_k + j * p.sB_n] : 0.0f;
            }
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) {
                float av[4], bv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) av[r] = As[kk][ty + 16 * r];
#pragma unroll
                for (int c = 0; c < 4; ++c) bv[c] = Bs[kk][tx + 16 * c];
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[r][c] = __builtin_fmaf(av[r], bv[c], acc[r][c]);
            }
            __syncthreads();
        }
        float *C = p.C + bo * p.sC_b + bi * p.sC_i;
        const Epilogue &e = p.epi;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const long long i = i0 + ty + 16 * r;
            if (i >= p.m) continue;
            const float rv = e.has_row ? e.row[b * e.sR_b + i * e.sR_m] : 0.0f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const long long j = j0 + tx + 16 * c;
                if (j >= p.n) continue;
                float *dst = C + i * p.sC_m + j * p.sC_n;
                const float cv = e.has_col ? e.col[b * e.sL_b + j * e.sL_n] : 0.0f;
                const float old = p.accumulate ? *dst : 0.0f;
                *dst = epilogue_value(p.alpha, acc[r][c], p.accumulate != 0, e.beta, old, e.has_row != 0,
                                      rv, e.has_col != 0, cv);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Squared norms out[b,i] = sum_p X[b,i,p]^2 (the terms a distance table adds
// to its product).  Vectors whose elements are contiguous: one wavefront per
// vector, lanes striding by 64 elements, then a fixed butterfly over the
// wavefront.  Otherwise one thread per vector, elements in order, so that
// neighbouring threads read neighbouring items.  fp32 sums in a fixed order
// either way: the same bits on every run.  Grid-stride loops, 64-bit
// addressing; every loop bound is uniform across a wavefront.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void sqnorms_contiguous(const float *X, long long sX_b, long long sX_i,
                                                          float *out, long long sO_b, long long sO_i,
                                                          long long batch, long long count, long long len) {
    const int lane = threadIdx.x & 63;
    const long long total = batch * count;
    for (long long v = (long long)blockIdx.x * 4 + (threadIdx.x >> 6); v < total;
         v += (long long)gridDim.x * 4) {
        const long long b = v / count, i = v - b * count;
        const float *x = X + b * sX_b + i * sX_i;
        float sq = 0.0f;
        for (long long e = lane; e < len; e += 64) {
            const float t = x[e];
            sq = __builtin_fmaf(t, t, sq);
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off, 64);
        if (lane == 0) out[b * sO_b + i * sO_i] = sq;
    }
}

__global__ __launch_bounds__(256) void sqnorms_strided(const float *X, long long sX_b, long long sX_i,
                                                       long long sX_e, float *out, long long sO_b,
                                                       long long sO_i, long long batch, long long count,
                                                       long long len) {
    const long long total = batch * count;
    for (long long v = (long long)blockIdx.x * 256 + threadIdx.x; v < total; v += (long long)gridDim.x * 256) {
        const long long b = v / count, i = v - b * count;
        const float *x = X + b * sX_b + i * sX_i;
        float sq = 0.0f;
        for (long long e = 0; e < len; ++e) {
            const float t = x[e * sX_e];
            sq = __builtin_fmaf(t, t, sq);
        }
        out[b * sO_b + i * sO_i] = sq;
    }
}

int launch_sqnorms(long long batch, long long count, long long len, const float *X, long long sX_b,
                   long long sX_i, long long sX_e, float *out, long long sO_b, long long sO_i,
                   hipStream_t stream, std::string &why) {
    const long long total = batch * count;
    if (total == 0) return kOk;
    (void)hipGetLastError();
    if (sX_e == 1 && len >= 64) {
        const long long grid = std::min<long long>((total + 3) / 4, 65536);
        hipLaunchKernelGGL(sqnorms_contiguous, dim3(unsigned(grid)), dim3(256), 0, stream, X, sX_b, sX_i,
                           out, sO_b, sO_i, batch, count, len);
    } else {
        const long long grid = std::min<long long>((total + 255) / 256, 65536);
        hipLaunchKernelGGL(sqnorms_strided, dim3(unsigned(grid)), dim3(256), 0, stream, X, sX_b, sX_i,
                           sX_e, out, sO_b, sO_i, batch, count, len);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        why = std::string("kernel launch failed: ") + hipGetErrorString(e);
        return kErrHip;
    }
    return kOk;
}

namespace {

const MfmaTable &table() {
    static const MfmaTable t = [] {
        MfmaTable tab{};
        fill_tile_0(tab);
        fill_tile_1(tab);
        fill_tile_2(tab);
        fill_tile_3(tab);
        fill_tile_4(tab);
        fill_tile_5(tab);
        fill_tile_6(tab);
        fill_tile_7(tab);
        fill_tile_8(tab);
        fill_tile_9(tab);
        fill_tile_10(tab);
        fill_tile_11(tab);
        fill_tile_12(tab);
        static_assert(kNumTiles == 13, "launch table covers every tile");
        return tab;
    }();
    return t;
}

const WaveTable &wave_table() {
    static const WaveTable t = [] {
        WaveTable tab{};
        fill_wave_0(tab);
        fill_wave_1(tab);
        fill_wave_2(tab);
        fill_wave_3(tab);
        fill_wave_4(tab);
        fill_wave_5(tab);
        fill_wave_6(tab);
        fill_wave_7(tab);
        static_assert(kNumWaveTiles == 8, "launch table covers every wave tile");
        return tab;
    }();
    return t;
}

const PersistTable &persist_table() {
    static const PersistTable t = [] {
        PersistTable tab{};
        fill_persist_0(tab);
        fill_persist_1(tab);
        fill_persist_2(tab);
        static_assert(kNumPersistTiles == 3, "launch table covers every persistent tile");
        return tab;
    }();
    return t;
}

}  // namespace

Epilogue make_epilogue(const Plan &p) {
    Epilogue e;
    e.beta = p.beta;
    e.row = reinterpret_cast<const float *>(p.row_add);
    e.col = reinterpret_cast<const float *>(p.col_add);
    e.sR_b = p.sR_b; e.sR_m = p.sR_m; e.sL_b = p.sL_b; e.sL_n = p.sL_n;
    e.has_row = p.row_add ? 1 : 0;
    e.has_col = p.col_add ? 1 : 0;
    e.col_vec4 = p.col_vec4 ? 1 : 0;
    return e;
}

int launch_plan(const Plan &p, hipStream_t stream, std::string &why) {
    if (p.empty) return kOk;
    (void)hipGetLastError();  // clear a stale error left by unrelated work
    if (p.family == Family::Generic) {
        GenericArgs g;
        g.A = reinterpret_cast<const float *>(p.A);
        g.B = reinterpret_cast<const float *>(p.B);
        g.C = reinterpret_cast<float *>(p.C);
        g.sA_b = p.sA_b; g.sA_m = p.sA_m; g.sA_k = p.sA_k;
        g.sB_b = p.sB_b; g.sB_k = p.sB_k; g.sB_n = p.sB_n;
        g.sC_b = p.sC_b; g.sC_m = p.sC_m; g.sC_n = p.sC_n;
        g.m = p.m; g.n = p.n; g.k = p.k; g.batch = p.batch;
        g.tiles_m = p.tiles_m; g.tiles_n = p.tiles_n;
        g.alpha = p.alpha; g.accumulate = p.accumulate;
        g.epi = make_epilogue(p);
        g.inner = p.inner; g.gA = p.gA; g.gB = p.gB;
        g.sA_i = p.sA_i; g.sB_i = p.sB_i; g.sC_i = p.sC_i;
        hipLaunchKernelGGL(sgemm_generic, dim3(unsigned(p.workgroups)), dim3(256), 0, stream, g);
    } else {
        MfmaArgs a;
        a.A = reinterpret_cast<const float *>(p.A);
        a.B = reinterpret_cast<const float *>(p.B);
        a.C = reinterpret_cast<float *>(p.C);
        a.sA_b = p.sA_b; a.sA_m = p.sA_m; a.sA_k = p.sA_k;
        a.sB_b = p.sB_b; a.sB_k = p.sB_k; a.sB_n = p.sB_n;
        a.sC_b = p.sC_b; a.sC_m = p.sC_m; a.sC_n = p.sC_n;
        a.m = int(p.m); a.n = int(p.n); a.k = int(p.k);
        a.tiles_m = int(p.tiles_m); a.tiles_n = int(p.tiles_n);
        a.total_tiles = int(p.batch * p.tiles_m * p.tiles_n);
        a.map = make_tile_map(p.batch, p.tiles_m, p.tiles_n);
        a.split = make_batch_split(p.inner, p.gA, p.gB);
        a.sA_i = p.sA_i; a.sB_i = p.sB_i; a.sC_i = p.sC_i;
        a.accumulate = p.accumulate;
        a.c_vec4 = p.c_vec4 ? 1 : 0;
        a.alpha = p.alpha;
        a.epi = make_epilogue(p);
        a.ksplit = p.ksplit;
        if (p.persist)
            persist_table().f[p.tile][p.a_kfast][p.b_kfast][p.accumulate != 0](
                a, unsigned(p.workgroups), stream);
        else if (p.strip)
            launch_strip(a, p.tile, p.accumulate != 0, unsigned(p.workgroups), stream);
        else if (p.family == Family::Wave)
            wave_table().f[p.tile][p.a_kfast][p.b_kfast][p.vec_a == 4][p.vec_b == 4](
                a, unsigned(p.workgroups), stream);
        else {
            const MfmaLaunch fn =
                table().f[p.tile][p.a_kfast][p.b_kfast][width_index(p.vec_a)][width_index(p.vec_b)][p.fixed_offsets];
            if (!fn) {
                why = "no tiled kernel instance for load widths " + std::to_string(p.vec_a) + "/" +
                      std::to_string(p.vec_b) + (p.fixed_offsets ? " with" : " without") + " fixed offsets";
                return kErrUnsupported;
            }
            fn(a, unsigned(p.workgroups), stream);
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        why = std::string("kernel launch failed: ") + hipGetErrorString(e);
        return kErrHip;
    }
    return kOk;
}

}  // namespace sgemm
