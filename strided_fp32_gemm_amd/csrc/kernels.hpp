// kernels.hpp -- kernel argument blocks and the launch entry used by the ABI.
#pragma once

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <string>

#include "plan.hpp"

namespace sgemm {

// Raises kernel `fn`'s dynamic LDS limit to `bytes` on the current device,
// once per device: `done` holds one bit per device id below 64 (a larger id
// sets the attribute on every launch).  A failure leaves the bit clear; the
// launch then fails and reports through hipGetLastError.
inline void allow_dynamic_lds(const void *fn, int bytes, std::atomic<unsigned long long> &done) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return;
    const unsigned long long bit = dev >= 0 && dev < 64 ? 1ull << dev : 0ull;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return;
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess && bit)
        done.fetch_or(bit, std::memory_order_acq_rel);
}

// The general epilogue's extra terms: C <- alpha*acc + beta*C_old + row[i] +
// col[j], the vectors at row + b*sR_b + i*sR_m and col + b*sL_b + j*sL_n.
struct Epilogue {
    float beta;
    const float *row;
    const float *col;
    long long sR_b, sR_m, sL_b, sL_n;
    int has_row, has_col;
    int col_vec4;   // col is contiguous and 16-byte aligned per row quad (one 16-byte load)
};

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
    int total_tiles;   // batch * tiles_m * tiles_n (the persistent kernel's loop bound)
    TileMap map;       // tile id -> (batch, tile row, tile column)
    BatchSplit split;  // flat batch index -> (outer, inner) entries of A, B, C
    long long sA_i, sB_i, sC_i;   // inner-level batch strides
    int accumulate;   // beta != 0: C is read
    int c_vec4;   // C rows take 16-byte stores (n-contiguous, aligned, n % 4 == 0)
    float alpha;
    Epilogue epi;
    int ksplit;   // wavefront kernel: wavefronts per workgroup sharing one tile's k (1: no split)
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
    Epilogue epi;
    long long inner, gA, gB, sA_i, sB_i, sC_i;   // two batch levels (see BatchSplit)
};

// Launchers indexed [tile][A k-fast][B k-fast][A 16-byte loads]
// [B 16-byte loads]; the LDS-tiled kernel's table is indexed by load width
// (0: element, 1: 8-byte, 2: 16-byte; see width_index) and [fixed slot
// offsets].  Each tile's row is filled by its own translation unit
// (mfma_t<tile>.hip, wave_w<tile>.hip) so the instantiations compile in
// parallel.
using MfmaLaunch = void (*)(const MfmaArgs &, unsigned, hipStream_t);
struct MfmaTable {
    MfmaLaunch f[kNumTiles][2][2][3][3][2];
};
constexpr int width_index(int floats) { return floats == 4 ? 2 : floats == 2 ? 1 : 0; }
struct WaveTable {
    MfmaLaunch f[kNumWaveTiles][2][2][2][2];
};
// Persistent kernel: [tile][A k-fast][B k-fast][accumulate] (16-byte loads only).
struct PersistTable {
    MfmaLaunch f[kNumPersistTiles][2][2][2];
};
void fill_tile_0(MfmaTable &);
void fill_tile_1(MfmaTable &);
void fill_tile_2(MfmaTable &);
void fill_tile_3(MfmaTable &);
void fill_tile_4(MfmaTable &);
void fill_tile_5(MfmaTable &);
void fill_tile_6(MfmaTable &);
void fill_tile_7(MfmaTable &);
void fill_tile_8(MfmaTable &);
void fill_tile_9(MfmaTable &);
void fill_tile_10(MfmaTable &);
void fill_tile_11(MfmaTable &);
void fill_tile_12(MfmaTable &);
void fill_wave_0(WaveTable &);
void fill_wave_1(WaveTable &);
void fill_wave_2(WaveTable &);
void fill_wave_3(WaveTable &);
void fill_wave_4(WaveTable &);
void fill_wave_5(WaveTable &);
void fill_wave_6(WaveTable &);
void fill_wave_7(WaveTable &);
void fill_persist_0(PersistTable &);
void fill_persist_1(PersistTable &);
void fill_persist_2(PersistTable &);

// Strip kernel (kStripTiles[tile]); a.map has one tile column per batch entry.
void launch_strip(const MfmaArgs &a, int tile, bool accumulate, unsigned grid, hipStream_t stream);

// Squared norms of batch x count vectors of length len (see sgemm_sqnorms).
int launch_sqnorms(long long batch, long long count, long long len, const float *X, long long sX_b,
                   long long sX_i, long long sX_e, float *out, long long sO_b, long long sO_i,
                   hipStream_t stream, std::string &why);

// Enqueues the plan on `stream`.  Returns kOk, or kErrHip with `why` set when
// the runtime rejects the launch.
int launch_plan(const Plan &p, hipStream_t stream, std::string &why);

}  // namespace sgemm
