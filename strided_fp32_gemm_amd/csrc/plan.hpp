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
    int accumulate;            // beta != 0
    uintptr_t C; int64_t sC_batch, sC_row, sC_col;
    // General epilogue: C <- alpha*A*B + beta*C + row_add[b,i] + col_add[b,j];
    // a zero vector pointer drops its term.
    float beta = 0.0f;
    uintptr_t row_add = 0; int64_t sR_batch = 0, sR_row = 0;
    uintptr_t col_add = 0; int64_t sL_batch = 0, sL_col = 0;
    // Two batch levels: batch = outer * inner, flat index b = o*inner + i.
    // Operand X of batch entry (o, i) starts at X + o*sX_batch + (i/gX)*sX_inner
    // (gC = 1).  inner = 1 is the single-level product.
    int64_t inner = 1;
    int64_t sA_inner = 0, gA = 1;
    int64_t sB_inner = 0, gB = 1;
    int64_t sC_inner = 0;
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
    // Fraction of the matrix-core peak a CU sustains on this tile when it
    // is full (fitted to tile sweeps on MI355X).
    double rate;
    constexpr int waves() const { return wgm * wgn; }
    // Padding (floats) of an LDS tile row, chosen so that the fragment reads
    // and the staging writes meet no bank conflict.  gfx950's LDS has 64
    // banks of 4 bytes; a 16-byte read serves the lanes in four groups of
    // 16, {0-3, 12-15, 20-23, 24-27}, {4-11, 16-19, 28-31} and the same two
    // shifted by 32; 8- and 4-byte reads serve 32 consecutive lanes, 16-byte
    // writes 8 (measured per lane pair with the bank-conflict counter).
    // `blocks` is the operand's count of MF-wide blocks per wavefront.
    //  * 32-wide blocks: 4 on a k-fast tile, 8 on an m- or n-fast one (lane
    //    halves 4 rows apart land 32 banks apart).
    //  * 16-wide blocks, k-fast: 8, so the 16 rows a read group touches
    //    start on distinct 4-bank quads.
    //  * 16-wide blocks, m- or n-fast, read 4 (2) blocks per 16-byte (8-byte)
    //    load: 0 (8), so the lane quarters 4 rows apart stay on the same
    //    (opposite) half of the banks; single-float reads: 4.
    constexpr int pad(bool kfast, int blocks) const {
        if (mf == 32) return kfast ? 4 : 8;
        if (kfast) return 8;
        return blocks == 4 ? 0 : blocks == 2 ? 8 : 4;
    }
    constexpr int a_blocks() const { return bm / wgm / mf; }
    constexpr int b_blocks() const { return bn / wgn / mf; }
    // LDS bytes of one buffer of the A and B tiles, each stored
    // [slow][fast + pad]; the main loop double-buffers them unless the whole
    // k extent fits one slice.
    constexpr int buffer_lds_bytes(bool a_kfast, bool b_kfast) const {
        return 4 * ((a_kfast ? bm * (bk + pad(true, a_blocks())) : bk * (bm + pad(false, a_blocks()))) +
                    (b_kfast ? bn * (bk + pad(true, b_blocks())) : bk * (bn + pad(false, b_blocks()))));
    }
    // Row pitch (floats) of the staged epilogue, where each wavefront parks
    // its (bm/wgm) x (bn/wgn) sub-tile of C before storing whole rows.  The
    // row stores read it back with 16-byte LDS reads, 16 lanes per cycle in
    // the groups above; with rows of 32 or 64 floats and no padding those
    // groups cover 64 distinct banks.  The accumulators go in with 16- or
    // 8-byte writes (four or two 16-wide blocks side by side: an n-fast B
    // tile with 4 or 2 blocks per wavefront; 8 and 16 consecutive lanes per
    // cycle, all on one row) or, on 32-wide blocks, with single-float writes
    // of 32 consecutive columns: all free of conflicts at that pitch.  The
    // single-float writes of the other 16-wide-block tiles put lane quarters
    // 4 rows apart in one 32-lane cycle, so their rows keep 4 floats of
    // padding.
    constexpr int epi_pitch(bool b_kfast) const {
        const int wn = bn / wgn;
        return (mf == 32 || (!b_kfast && (b_blocks() == 4 || b_blocks() == 2))) ? wn : wn + 4;
    }
    // LDS bytes of the staged epilogue: every wavefront's sub-tile of C.
    constexpr int epilogue_lds_bytes(bool b_kfast) const { return 4 * waves() * (bm / wgm) * epi_pitch(b_kfast); }
    // LDS a launch allocates for k-slice count `slices` (dynamic shared memory).
    constexpr int lds_bytes(bool a_kfast, bool b_kfast, long long slices) const {
        int loop = buffer_lds_bytes(a_kfast, b_kfast) * (slices > 1 ? 2 : 1);
        return loop > epilogue_lds_bytes(b_kfast) ? loop : epilogue_lds_bytes(b_kfast);
    }
};

// The LDS-tiled (MFMA family) tile table.  Kernel instantiations are
// generated from the same indices (one translation unit per tile), so the
// order is part of the contract between planner and kernels.
constexpr int kNumTiles = 13;
inline constexpr TileCfg kTiles[kNumTiles] = {
    {128, 128, 32, 2, 2, 32, "t128x128", 0.897},
    {128, 64, 32, 2, 2, 32, "t128x64", 0.860},
    {64, 128, 32, 2, 2, 32, "t64x128", 0.847},
    {64, 64, 32, 2, 2, 32, "t64x64", 0.837},
    {256, 128, 32, 2, 2, 32, "t256x128", 0.919},
    {128, 160, 32, 4, 1, 32, "t128x160", 0.934},
    {128, 80, 32, 4, 1, 16, "t128x80m16", 0.805},
    {64, 176, 32, 4, 1, 16, "t64x176m16", 0.796},
    {64, 64, 32, 2, 2, 16, "t64x64m16", 0.896},
    {128, 128, 32, 2, 2, 16, "t128x128m16", 0.936},
    {128, 64, 32, 2, 2, 16, "t128x64m16", 0.824},
    {64, 128, 32, 2, 2, 16, "t64x128m16", 0.931},
    {64, 32, 32, 4, 1, 16, "t64x32m16", 0.830},
};

// One tile of the direct wavefront kernel (WAVE family): a wavefront owns
// bm x bn outputs in 16 x 16 matrix-core blocks and reads its operands
// straight from global memory.  Up to max_split wavefronts of one workgroup
// may share a tile, each taking a share of k.
struct WaveCfg {
    int bm, bn;
    int waves_per_simd;  // resident wavefronts per SIMD (register-limited, from the compiled code)
    const char *name;
    double rate;         // sustained fraction of peak on a full CU (fitted)
    int max_split;       // most wavefronts per workgroup in the split variant
};

constexpr int kNumWaveTiles = 8;
// Largest split of a wave tile's k over the wavefronts of a workgroup.
constexpr int kWaveMaxSplit = 16;
inline constexpr WaveCfg kWaveTiles[kNumWaveTiles] = {
    {32, 32, 5, "w32x32", 0.58, 16},
    {32, 64, 3, "w32x64", 0.75, 8},
    {64, 32, 3, "w64x32", 0.76, 8},
    {64, 64, 2, "w64x64", 0.77, 8},
    {16, 32, 7, "w16x32", 0.41, 16},
    {16, 64, 4, "w16x64", 0.48, 16},
    {32, 16, 7, "w32x16", 0.36, 16},
    {64, 16, 4, "w64x16", 0.41, 16},
};

// One tile of the persistent short-k kernel (MFMA family): a fixed grid of
// wgm x wgn-wavefront workgroups loops over bm x bn output tiles whose whole
// k extent (k <= kmax) sits in one LDS slab; two slabs alternate.  Served
// only with 16-byte loads of both operands and 16-byte C rows.
struct PersistCfg {
    int bm, bn, kmax;
    int wgm, wgn;
    const char *name;
    double rate;   // sustained fraction of the matrix-core peak (fitted)
    constexpr int waves() const { return wgm * wgn; }
    // Row padding (floats) of a slab: 8 on a k-fast operand (its 16-byte
    // fragment reads of 16 rows then start on distinct bank quads within
    // each of gfx950's 16-lane read groups), 4 on an m- or n-fast one (its
    // single-float reads, 32 lanes at a time, land on distinct banks).
    static constexpr int pad(bool kfast) { return kfast ? 8 : 4; }
    // LDS bytes of one slab: A and B stored [slow][fast + pad].
    constexpr int slab_bytes(bool a_kfast, bool b_kfast) const {
        return 4 * ((a_kfast ? bm * (kmax + pad(true)) : kmax * (bm + pad(false))) +
                    (b_kfast ? bn * (kmax + pad(true)) : kmax * (bn + pad(false))));
    }
};

constexpr int kNumPersistTiles = 3;
inline constexpr PersistCfg kPersistTiles[kNumPersistTiles] = {
    {64, 64, 64, 2, 2, "p64x64k64", 0.59},
    {128, 64, 64, 4, 2, "p128x64k64", 0.59},
    {64, 128, 64, 2, 4, "p64x128k64", 0.59},
};

// Short-k strip kernel: a workgroup of `waves` wavefronts owns `rows` = 16 *
// waves * (1 or 2) rows of C across all n columns; each wavefront keeps its rows of A
// (k <= kmax, k-contiguous) in registers and streams B (k-contiguous) in
// 64-column blocks through LDS.
struct StripCfg {
    int rows, waves, kmax;
    const char *name;
    double rate;   // sustained fraction of the matrix-core peak (fitted)
    static constexpr int kBlockCols = 64;
    static constexpr int lds_bytes() { return 2 * kBlockCols * (64 + 8) * 4; }
};

constexpr int kNumStripTiles = 4;
inline constexpr StripCfg kStripTiles[kNumStripTiles] = {
    {64, 4, 64, "s64k64", 0.67},
    {128, 8, 64, "s128k64", 0.71},
    {128, 4, 64, "s128r2k64", 0.63},   // two 16-row sub-strips per wavefront
    {64, 2, 64, "s64r2k64", 0.62},
};

// Division by a launch constant as a multiply and a shift (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994):
// for 1 <= d < 2^31 take l = ceil(log2 d) and m = ceil(2^(31+l) / d), which
// lies in [2^31, 2^32).  For 0 <= n < 2^31, n*m / 2^(31+l) exceeds n/d by
// less than n / 2^(31+l) < 2^-l <= 1/d, which never reaches the next
// integer, so (n*m) >> (31+l) == floor(n/d).  On the GPU this is a 64-bit
// scalar product and a shift instead of a ~40-instruction division.
struct Divisor {
    uint32_t d, m, s;
};

constexpr Divisor make_divisor(uint32_t d) {
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    const uint64_t num = uint64_t(1) << (31 + l);
    return Divisor{d, uint32_t((num + d - 1) / d), 31 + l};
}

constexpr uint32_t divide(uint32_t n, Divisor v) { return uint32_t((uint64_t(n) * v.m) >> v.s); }

// Order in which a launch visits its batch * tiles_m * tiles_n output tiles.
// Workgroup ids reach the 8 XCDs round-robin; when the tile count is a
// multiple of 8, id w is remapped to (w % 8) * (count / 8) + w / 8, so that
// each XCD (and its L2) works through one contiguous range.  Within a batch
// entry, tiles go in groups of kGroupRows tile rows, column by column inside
// a group, so neighbouring ids share B columns and nearby A rows.
constexpr int kGroupRows = 8;

struct TileMap {
    int tiles_m, tiles_n;
    int per_xcd;          // count / 8 if count % 8 == 0, else 0 (no remap)
    Divisor per_batch;    // tiles_m * tiles_n
    Divisor group;        // kGroupRows * tiles_n
    Divisor last_rows;    // tile rows of the last group (tiles_m % kGroupRows, or kGroupRows)
};

constexpr TileMap make_tile_map(int64_t batch, int64_t tiles_m, int64_t tiles_n) {
    const int64_t count = batch * tiles_m * tiles_n;
    const int64_t rem = tiles_m % kGroupRows;
    return TileMap{int(tiles_m), int(tiles_n), count % 8 == 0 ? int(count / 8) : 0,
                   make_divisor(uint32_t(tiles_m * tiles_n)), make_divisor(uint32_t(kGroupRows * tiles_n)),
                   make_divisor(uint32_t(rem ? rem : kGroupRows))};
}

// Tile id w (0 <= w < count) -> batch entry b, tile row tm, tile column tn.
constexpr void tile_coords(const TileMap &map, int w, int &b, int &tm, int &tn) {
    if (map.per_xcd) w = (w & 7) * map.per_xcd + (w >> 3);
    const uint32_t uw = uint32_t(w);
    const uint32_t ub = divide(uw, map.per_batch);
    const uint32_t t = uw - ub * map.per_batch.d;
    const uint32_t group = divide(t, map.group);
    const uint32_t in = t - group * map.group.d;
    const int first = int(group) * kGroupRows;
    const bool full = first + kGroupRows <= map.tiles_m;
    const uint32_t col = full ? in / uint32_t(kGroupRows) : divide(in, map.last_rows);
    const uint32_t row = in - col * (full ? uint32_t(kGroupRows) : map.last_rows.d);
    b = int(ub);
    tm = first + int(row);
    tn = int(col);
}

// Two batch levels: flat batch index b = o*inner + i; operand X of entry b
// starts at o*sX_outer + (i / gX)*sX_inner (gC = 1).  ia / ib are the inner
// indices of A's and B's entries, ic = i that of C's.
struct BatchSplit {
    Divisor inner, gA, gB;
};

constexpr BatchSplit make_batch_split(int64_t inner, int64_t gA, int64_t gB) {
    return BatchSplit{make_divisor(uint32_t(inner)), make_divisor(uint32_t(gA)), make_divisor(uint32_t(gB))};
}

constexpr void batch_entry(const BatchSplit &s, uint32_t b, uint32_t &o, uint32_t &ia, uint32_t &ib,
                           uint32_t &ic) {
    o = divide(b, s.inner);
    ic = b - o * s.inner.d;
    ia = divide(ic, s.gA);
    ib = divide(ic, s.gB);
}

// Everything a launch needs, in kernel terms: A is m x k, B is k x n, C is
// m x n, each with a batch stride, and "fast" names the contiguous axis.
struct Plan {
    bool empty = false;        // batch*m*n == 0: nothing to enqueue
    bool transposed = false;   // solved as C^T = B^T A^T
    Family family = Family::Generic;
    int tile = -1;             // index into kTiles / kPersistTiles (MFMA) or kWaveTiles (WAVE)
    bool persist = false;      // MFMA family, persistent short-k kernel (tile indexes kPersistTiles)
    bool strip = false;        // MFMA family, short-k strip kernel (tile indexes kStripTiles)
    bool a_kfast = true, b_kfast = false;
    int vec_a = 1, vec_b = 1;
    bool fixed_offsets = false;  // LDS-tiled kernel: load offsets fixed over the k loop (see make_plan)
    bool c_vec4 = false;       // C rows take 16-byte stores
    int64_t batch = 0, m = 0, n = 0, k = 0;
    float alpha = 1.0f;
    int accumulate = 0;        // beta != 0: C is read
    float beta = 0.0f;
    uintptr_t row_add = 0, col_add = 0;   // per-row / per-column terms (kernel terms, after any rewrite)
    int64_t sR_b = 0, sR_m = 0, sL_b = 0, sL_n = 0;
    bool col_vec4 = false;     // column term read 4 at a time (with c_vec4)
    int64_t inner = 1;         // second batch level (kernel terms, after any rewrite)
    int64_t sA_i = 0, gA = 1, sB_i = 0, gB = 1, sC_i = 0;
    uintptr_t A = 0, B = 0, C = 0;
    int64_t sA_b = 0, sA_m = 0, sA_k = 0;
    int64_t sB_b = 0, sB_k = 0, sB_n = 0;
    int64_t sC_b = 0, sC_m = 0, sC_n = 0;
    int64_t tiles_m = 0, tiles_n = 0, workgroups = 0;  // workgroups < tiles for the persistent kernel
    int ksplit = 1;            // WAVE family: wavefronts per workgroup sharing one tile's k
    double cost = 0.0;         // the cost model's estimate for the chosen kernel (cycles)
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
