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
    const char *name;
    // Fraction of the matrix-core peak a CU sustains on this tile when k is
    // long and the CU is full (measured on MI355X, 4 x 4096^3).
    double rate;
    constexpr int waves() const { return wgm * wgn; }
    // Padding of an LDS tile row: 4 floats on a k-fast tile; on an m- or
    // n-fast tile 8 (32-wide blocks) or 4 (16-wide blocks), which spreads the
    // lane groups that read different k rows over distinct banks.
    constexpr int pad(bool kfast) const { return kfast ? 4 : (mf == 32 ? 8 : 4); }
    // LDS bytes of the kernel's carve-up: two buffers of the A and B tiles,
    // each stored [slow][fast + pad].
    constexpr int lds_bytes(bool a_kfast, bool b_kfast) const {
        return 2 * 4 * ((a_kfast ? bm * (bk + pad(true)) : bk * (bm + pad(false))) +
                        (b_kfast ? bn * (bk + pad(true)) : bk * (bn + pad(false))));
    }
};

// The MFMA tile table.  Kernel instantiations are generated from the same
// indices (one translation unit per tile), so the order is part of the
// contract between planner and kernels.  Index kWaveTile is the
// one-wavefront tile of the WAVE family.
constexpr int kNumTiles = 10;
constexpr int kWaveTile = 5;
inline constexpr TileCfg kTiles[kNumTiles] = {
    {128, 128, 32, 2, 2, 32, "t128x128", 0.83},
    {128, 64, 32, 2, 2, 32, "t128x64", 0.80},
    {64, 128, 32, 2, 2, 32, "t64x128", 0.81},
    {64, 64, 32, 2, 2, 32, "t64x64", 0.77},
    {256, 128, 32, 2, 2, 32, "t256x128", 0.74},
    {32, 32, 32, 1, 1, 32, "wave32x32", 0.64},
    {128, 160, 32, 4, 1, 32, "t128x160", 0.81},
    {128, 80, 32, 4, 1, 16, "t128x80m16", 0.76},
    {64, 176, 32, 4, 1, 16, "t64x176m16", 0.71},
    {64, 64, 32, 2, 2, 16, "t64x64m16", 0.82},
};

// Everything a launch needs, in kernel terms: A is m x k, B is k x n, C is
// m x n, each with a batch stride, and "fast" names the contiguous axis.
struct Plan {
    bool empty = false;        // batch*m*n == 0: nothing to enqueue
    bool transposed = false;   // solved as C^T = B^T A^T
    Family family = Family::Generic;
    int tile = -1;             // index into kTiles (MFMA / WAVE)
    bool a_kfast = true, b_kfast = false;
    int vec_a = 1, vec_b = 1;
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
