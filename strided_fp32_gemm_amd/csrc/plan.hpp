// plan.hpp -- host-side validation and planning for the strided batched fp32
// product.  Pure C++ (no HIP headers): every decision the library makes
// before a launch lives here, so it can be checked without a GPU.
#pragma once

#include <cstdint>
#include <string>

namespace sgemm {

// Arguments in the ABI's own terms (pointers only as integers: the planner
// reads their alignment, never their memory).
struct GemmArgs {
    int64_t batch, m, n, k;
    float alpha;
    uintptr_t A; int64_t sA_batch, sA_row, sA_col;
    uintptr_t B; int64_t sB_batch, sB_row, sB_col;
    int accumulate;
    uintptr_t C; int64_t sC_batch, sC_row, sC_col;
};

enum class Family : int { Auto = 0, Mfma = 1, Wave = 2, Generic = 3 };

// One LDS-tiled MFMA configuration.  Tiles are BM x BN outputs with BK-deep
// k steps; WGM x WGN wavefronts each own a (BM/WGM) x (BN/WGN) sub-tile made
// of MF x MF matrix-core blocks (MF = 32: v_mfma_f32_32x32x2_f32, MF = 16:
// v_mfma_f32_16x16x4_f32).
struct TileCfg {
    int bm, bn, bk;
    int wgm, wgn;
    int mf;
    int pf;   // k slices of A and B in flight ahead of the one being multiplied (1 or 2)
    const char *name;
    // Fraction of the matrix-core peak a CU sustains on this tile when it
    // is full (fitted to tile sweeps on MI355X).
    double rate;
    constexpr int waves() const { return wgm * wgn; }
    // Padding of an LDS tile row: 4 floats on a k-fast tile; on an m- or
    // n-fast tile 8 (32-wide blocks) or 4 (16-wide blocks), which spreads the
    // lane groups that read different k rows over distinct banks.
    constexpr int pad(bool kfast) const { return kfast ? 4 : (mf == 32 ? 8 : 4); }
    // LDS bytes of one buffer of the A and B tiles, each stored
    // [slow][fast + pad]; the main loop double-buffers them unless the whole
    // k extent fits one slice.
    constexpr int buffer_lds_bytes(bool a_kfast, bool b_kfast) const {
        return 4 * ((a_kfast ? bm * (bk + pad(true)) : bk * (bm + pad(false))) +
                    (b_kfast ? bn * (bk + pad(true)) : bk * (bn + pad(false))));
    }
    // LDS bytes of the staged epilogue: every wavefront's (bm/wgm) x (bn/wgn)
    // sub-tile of C, rows padded by 4 floats.
    constexpr int epilogue_lds_bytes() const { return 4 * waves() * (bm / wgm) * (bn / wgn + 4); }
    // LDS a launch allocates for k-slice count `slices` (dynamic shared memory).
    constexpr int lds_bytes(bool a_kfast, bool b_kfast, long long slices) const {
        int loop = buffer_lds_bytes(a_kfast, b_kfast) * (slices > 1 ? 2 : 1);
        return loop > epilogue_lds_bytes() ? loop : epilogue_lds_bytes();
    }
};

// The LDS-tiled (MFMA family) tile table.  Kernel instantiations are
// generated from the same indices (one translation unit per tile), so the
// order is part of the contract between planner and kernels.
constexpr int kNumTiles = 12;
inline constexpr TileCfg kTiles[kNumTiles] = {
    {128, 128, 32, 2, 2, 32, 2, "t128x128", 0.83},
    {128, 64, 32, 2, 2, 32, 2, "t128x64", 0.80},
    {64, 128, 32, 2, 2, 32, 2, "t64x128", 0.84},
    {64, 64, 32, 2, 2, 32, 2, "t64x64", 0.88},
    {256, 128, 32, 2, 2, 32, 2, "t256x128", 0.77},
    {128, 160, 32, 4, 1, 32, 2, "t128x160", 0.74},
    {128, 80, 32, 4, 1, 16, 2, "t128x80m16", 0.71},
    {64, 176, 32, 4, 1, 16, 2, "t64x176m16", 0.59},
    {64, 64, 32, 2, 2, 16, 2, "t64x64m16", 0.97},
    {128, 128, 32, 2, 2, 16, 2, "t128x128m16", 0.83},
    {128, 64, 32, 2, 2, 16, 2, "t128x64m16", 0.86},
    {64, 128, 32, 2, 2, 16, 2, "t64x128m16", 0.96},
};

// One tile of the direct wavefront kernel (WAVE family): a single
// wavefront owns bm x bn outputs in 16 x 16 matrix-core blocks and reads its
// operands straight from global memory.
struct WaveCfg {
    int bm, bn;
    int waves_per_simd;  // resident wavefronts per SIMD (register-limited, from the compiled code)
    const char *name;
    double rate;         // sustained fraction of peak on a full CU (fitted)
};

constexpr int kNumWaveTiles = 4;
inline constexpr WaveCfg kWaveTiles[kNumWaveTiles] = {
    {32, 32, 5, "w32x32", 0.55},
    {32, 64, 3, "w32x64", 0.60},
    {64, 32, 3, "w64x32", 0.60},
    {64, 64, 2, "w64x64", 0.65},
};


// Everything a launch needs, in kernel terms: A is m x k, B is k x n, C is
// m x n, each with a batch stride, and "fast" names the contiguous axis.
struct Plan {
    bool empty = false;        // batch*m*n == 0: nothing to enqueue
    bool transposed = false;   // solved as C^T = B^T A^T
    Family family = Family::Generic;
    int tile = -1;             // index into kTiles (MFMA) or kWaveTiles (WAVE)
    bool a_kfast = true, b_kfast = false;
    int vec_a = 1, vec_b = 1;
    bool c_vec4 = false;       // C rows take 16-byte stores
    int64_t batch = 0, m = 0, n = 0, k = 0;
    float alpha = 1.0f;
    int accumulate = 0;
    uintptr_t A = 0, B = 0, C = 0;
    int64_t sA_b = 0, sA_m = 0, sA_k = 0;
    int64_t sB_b = 0, sB_k = 0, sB_n = 0;
    int64_t sC_b = 0, sC_m = 0, sC_n = 0;
    int64_t tiles_m = 0, tiles_n = 0, workgroups = 0;
    std::string kernel_name;
};

// Status codes (mirrors enum sgemm_status of the public header).
constexpr int kOk = 0, kErrSize = -1, kErrStride = -2, kErrNull = -3, kErrAlias = -4,
              kErrUnsupported = -5, kErrHip = -6, kErrPath = -7;

// Checks sizes, strides, pointers, overflow and aliasing; on failure fills
// `why` and returns the status.
int validate(const GemmArgs &a, std::string &why);

// Builds the launch plan for validated arguments.  `family` may force a
// kernel family; one that cannot serve the arguments falls back to Generic.
int make_plan(const GemmArgs &a, Family family, int num_cus, Plan &plan, std::string &why);

}  // namespace sgemm
