// plan.cpp -- validation, layout classification and tile choice.
//
// Semantics follow StaleyNET "GPU Implementation", section "The matrix
// product": C <- alpha*A*B (optionally + C) over a batch, every operand
// described by strides, a transposed operand being the same memory with its
// row and column strides exchanged.  The safety rule of the same page
// (section "Safety": check every size a kernel depends on, then launch) is
// what validate() and the buffer-range checks below implement.
#include "plan.hpp"
#include "extent.hpp"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

namespace sgemm {

namespace {

// Width (in floats) of the global loads along an operand's fast axis: 4
// (16-byte loads) when the fast axis is contiguous, its extent a multiple of
// 4 and every tile base 16-byte aligned; otherwise 1 (element loads, any
// stride and alignment).
int vector_width(uintptr_t base, int64_t fast_stride, int64_t fast_extent,
                 int64_t slow_stride, int64_t batch_stride, int64_t batch) {
    if (fast_stride != 1) return 1;
    for (int w : {4, 2}) {
        if (fast_extent % w || base % (4 * w) || slow_stride % w || (batch > 1 && batch_stride % w)) continue;
        return w;
    }
    return 1;
}

// Which axis of a rows x cols operand is contiguous: returns true if the
// column axis (cols) is the fast one.
bool cols_fast(int64_t rows, int64_t s_row, int64_t cols, int64_t s_col) {
    bool c1 = (s_col == 1), r1 = (s_row == 1);
    if (c1 && r1) return cols >= rows;
    if (c1) return true;
    if (r1) return false;
    if (cols == 1) return false;
    if (rows == 1) return true;
    return s_col <= s_row;
}

// Bytes a workgroup may address from its base, for the 32-bit buffer range.
constexpr int64_t kBufferLimit = (int64_t(1) << 31) - 64;

bool fits_buffer(int64_t span_rows, int64_t s_rows, int64_t span_cols, int64_t s_cols) {
    int64_t off = last_offset(1, 0, std::max<int64_t>(span_rows, 1), s_rows,
                              std::max<int64_t>(span_cols, 1), s_cols);
    if (off < 0) return false;
    int64_t bytes;
    if (!mul64(off + 4, 4, bytes)) return false;
    return bytes < kBufferLimit;
}

}  // namespace

int validate(const GemmArgs &a, std::string &why) {
    if (a.batch < 0 || a.m < 0 || a.n < 0 || a.k < 0) {
        why = "negative size (batch, m, n, k must be >= 0)";
        return kErrSize;
    }
    if (a.inner < 1 || a.gA < 1 || a.gB < 1 || (a.batch > 0 && a.batch % a.inner != 0)) {
        why = "inner batch count and groups must be >= 1, and the inner count must divide the batch";
        return kErrSize;
    }
    const int64_t strides[12] = {a.sA_batch, a.sA_row, a.sA_col, a.sB_batch, a.sB_row, a.sB_col,
                                 a.sC_batch, a.sC_row, a.sC_col, a.sA_inner, a.sB_inner, a.sC_inner};
    static const char *names[12] = {"sA_batch", "sA_row", "sA_col", "sB_batch", "sB_row", "sB_col",
                                    "sC_batch", "sC_row", "sC_col", "sA_inner", "sB_inner", "sC_inner"};
    for (int i = 0; i < 12; ++i)
        if (strides[i] < 0) {
            why = std::string("negative stride ") + names[i];
            return kErrStride;
        }
    if ((a.row_add && (a.sR_batch < 0 || a.sR_row < 0)) || (a.col_add && (a.sL_batch < 0 || a.sL_col < 0))) {
        why = "negative stride of row_add or col_add";
        return kErrStride;
    }
    int64_t bm, work;
    if (!mul64(a.batch, a.m, bm) || !mul64(bm, a.n, work)) {
        why = "batch*m*n overflows int64";
        return kErrUnsupported;
    }
    if (work == 0) return kOk;
    if (!a.C) {
        why = "C is NULL";
        return kErrNull;
    }
    if (a.k > 0 && (!a.A || !a.B)) {
        why = a.A ? "B is NULL" : "A is NULL";
        return kErrNull;
    }
    const int64_t outer = a.batch / a.inner;
    int64_t lastC = last_offset4(outer, a.sC_batch, a.inner, a.sC_inner, a.m, a.sC_row, a.n, a.sC_col);
    int64_t lastA = 0, lastB = 0;
    if (a.k > 0) {
        lastA = last_offset4(outer, a.sA_batch, (a.inner + a.gA - 1) / a.gA, a.sA_inner, a.m, a.sA_row,
                             a.k, a.sA_col);
        lastB = last_offset4(outer, a.sB_batch, (a.inner + a.gB - 1) / a.gB, a.sB_inner, a.k, a.sB_row,
                             a.n, a.sB_col);
    }
    int64_t lastR = a.row_add ? last_offset(a.batch, a.sR_batch, a.m, a.sR_row, 1, 0) : 0;
    int64_t lastL = a.col_add ? last_offset(a.batch, a.sL_batch, a.n, a.sL_col, 1, 0) : 0;
    int64_t bytes;
    if (lastC < 0 || lastA < 0 || lastB < 0 || lastR < 0 || lastL < 0 ||
        !mul64(std::max({lastA, lastB, lastC, lastR, lastL}) + 1, 4, bytes)) {
        why = "an operand's extent times its strides overflows int64";
        return kErrUnsupported;
    }
    // C must address every output at its own element.
    const int64_t c_ext[4] = {outer, a.inner, a.m, a.n};
    const int64_t c_str[4] = {a.sC_batch, a.sC_inner, a.sC_row, a.sC_col};
    if (!distinct_axes(c_ext, c_str)) {
        why = "C's strides map two outputs to the same element";
        return kErrAlias;
    }
    if (a.k > 0 && (ranges_overlap(a.C, lastC, a.A, lastA) || ranges_overlap(a.C, lastC, a.B, lastB))) {
        why = "C's address range overlaps A or B";
        return kErrAlias;
    }
    if ((a.row_add && ranges_overlap(a.C, lastC, a.row_add, lastR)) ||
        (a.col_add && ranges_overlap(a.C, lastC, a.col_add, lastL))) {
        why = "C's address range overlaps row_add or col_add";
        return kErrAlias;
    }
    return kOk;
}

namespace {

bool tile_fits(const Plan &p, int bm, int bn) {
    // Buffer offsets are 32-bit from a per-workgroup base: the workgroup's
    // slice of each operand has to lie within 2 GiB of that base.  (A fetch
    // may run up to two k slices past the end; those lanes are out of range
    // and their offsets are never formed from valid rows.)
    int64_t kspan = p.k;
    return fits_buffer(bm, p.sA_m, kspan, p.sA_k) && fits_buffer(kspan, p.sB_k, bn, p.sB_n) &&
           fits_buffer(bm, p.sC_m, bn, p.sC_n) && (!p.row_add || fits_buffer(bm, p.sR_m, 1, 0)) &&
           (!p.col_add || fits_buffer(1, 0, bn, p.sL_n));
}

// No launch streams faster than HBM: ~2700 bytes per cycle across the chip,
// and ~15 per cycle into one CU (measured: with few workgroups only their
// CUs fetch).  Each distinct operand is read once (a zero batch stride
// shares it) and C written once (read too when accumulating).  Streaming
// and compute overlap imperfectly: a quarter of the smaller of the two
// shows, which also ranks launches that all sit at the HBM floor.
double stream_floor(const Plan &p, double cost, double workgroups, int num_cus) {
    const double kHbmBytesPerCycle = 2700.0, kCuStreamBytesPerCycle = 15.0, kOverlapLoss = 0.25;
    const double a_elems = double(p.sA_b == 0 && p.sA_i == 0 ? 1 : p.batch) * double(p.m) * double(p.k);
    const double b_elems = double(p.sB_b == 0 && p.sB_i == 0 ? 1 : p.batch) * double(p.k) * double(p.n);
    const double c_elems = double(p.batch) * double(p.m) * double(p.n) * (p.accumulate ? 2.0 : 1.0);
    const double bytes = 4.0 * (a_elems + b_elems + c_elems);
    const double cus = std::min(std::max(workgroups, 1.0), double(std::max(num_cus, 1)));
    const double fetch = std::max(bytes / kHbmBytesPerCycle, bytes / (cus * kCuStreamBytesPerCycle));
    return std::max(cost, fetch) + kOverlapLoss * std::min(cost, fetch);
}

// Estimated cycles of an LDS-tiled launch.  The dispatcher hands a CU its
// next workgroup as soon as one finishes, so the busiest CU runs
// ceil(tiles / CUs) tiles; each costs the larger of its matrix-core work at
// the tile's sustained rate and its operand reads through L2, plus its C
// traffic.  With fewer than two workgroups resident per CU (LDS-bound, or
// too few tiles) a CU's matrix cores idle more, so the rate drops by up to
// kLowOccupancy.  The first two slices' memory latency is not hidden.  Rates
// and constants were fitted to tile sweeps on MI355X (the benchmark
// workloads and twelve other shapes; mean regret 0.5%); the single-slice term
// for 16x16 tiles to a sweep of every tile on 270 random products.
double tile_cost(const Plan &p, const TileCfg &t, int num_cus) {
    const double kFlopPerCuCycle = 256.0, kOperandBytesPerCycle = 64.0, kStoreBytesPerCycle = 11.0;
    const double kLdsBytes = 160.0 * 1024.0, kSliceLatency = 368.0, kLowOccupancy = 0.05, kShortK16 = 0.1;
    const long long slices = (p.k + t.bk - 1) / t.bk;
    const double tiles = double(p.batch) * double((p.m + t.bm - 1) / t.bm) * double((p.n + t.bn - 1) / t.bn);
    const double cus = double(std::max(num_cus, 1));
    const double per_cu = std::ceil(tiles / cus);
    const double fit = std::max(1.0, std::min(8.0, std::floor(kLdsBytes / t.lds_bytes(p.a_kfast, p.b_kfast, slices))));
    const double resident = std::min(fit, tiles / cus);
    const double rate = t.rate * (1.0 - kLowOccupancy * std::max(0.0, 2.0 - resident) / 2.0);
    const double kpad = double(slices) * t.bk;
    const double compute = double(t.bm) * t.bn * 2.0 * kpad / kFlopPerCuCycle / rate;
    const double operands = double(t.bm + t.bn) * kpad * 4.0 / kOperandBytesPerCycle;
    const double epilogue = double(t.bm) * t.bn * 4.0 * (p.accumulate ? 2.0 : 1.0) / kStoreBytesPerCycle;
    // With a single k slice the 16x16 tiles' longer fragment bookkeeping is
    // not amortised: there the 32x32 tiles measured 10-21% faster.
    const double short_k = t.mf == 16 && slices <= 1 ? kShortK16 * t.bm * t.bn : 0.0;
    return stream_floor(p, per_cu * (std::max(compute, operands) + epilogue + short_k) +
                               kSliceLatency * std::min<double>(double(slices), 2.0), tiles, num_cus);
}

// Estimated cycles of a direct-wavefront launch whose workgroups hold
// `splits` wavefronts sharing one tile's k.  Workgroups are spread over the
// CUs and up to `occ` of them run concurrently on one CU (bounded by
// registers, and by how many each CU receives).  A CU's four SIMDs share its
// wavefronts; with fewer than four, SIMDs idle and each wavefront runs at
// one SIMD's pace.  A round costs the larger of the busiest SIMD's
// matrix-core work at the tile's sustained rate and the CU's operand reads
// through L2 (~64 bytes per cycle), plus the epilogue traffic of C (read and
// written when accumulating, ~11 bytes per cycle per CU), the fixed-order sum
// of the split partials through LDS, and memory latency the round cannot
// hide (a SIMD with a single wavefront hides less of it: kLoneWave); then
// the HBM floor.  Rates and constants were fitted to tile and split sweeps
// on MI355X; every tile competes on every shape (the 16-wide tiles too: on
// 270 random shapes with m or n above 16 they were often the fastest), and
// the narrow-contiguous factor was set on those sweeps (mean regret against
// the fastest tile and split 10.4% -> 6.9% on 120 shapes not used to set it).
double wave_cost(const Plan &p, const WaveCfg &t, int splits, int num_cus) {
    const double kFlopPerSimdCycle = 64.0, kOperandBytesPerCycle = 64.0, kStoreBytesPerCycle = 11.0;
    const double kLdsBytesPerCycle = 128.0, kLatency = 2720.0, kLoneWave = 0.8, kNarrowContiguous = 0.85;
    const double tiles = double(p.batch) * double((p.m + t.bm - 1) / t.bm) * double((p.n + t.bn - 1) / t.bn);
    const double cus = double(std::max(num_cus, 1));
    const double fit = std::max(1.0, std::floor(4.0 * t.waves_per_simd / splits));
    const double occ = std::max(1.0, std::min(fit, std::ceil(tiles / cus)));
    const double rounds = std::ceil(tiles / (cus * occ));
    const double groups = double((p.k + 15) / 16);
    const double kwave = std::ceil(groups / splits) * 16.0;   // k of one wavefront
    const double per_simd = std::max(1.0, occ * splits / 4.0);
    // A 16-wide tile along an operand's contiguous axis (A m-fast with 16
    // rows, B n-fast with 16 columns) reads that operand in short segments.
    const double narrow = (!p.a_kfast && t.bm == 16 ? kNarrowContiguous : 1.0) *
                          (!p.b_kfast && t.bn == 16 ? kNarrowContiguous : 1.0);
    const double rate = t.rate * narrow * (occ * splits <= 4.0 ? kLoneWave : 1.0);
    const double compute = per_simd * t.bm * t.bn * 2.0 * kwave / kFlopPerSimdCycle / rate;
    const double operands = occ * double(t.bm + t.bn) * groups * 16.0 * 4.0 / kOperandBytesPerCycle;
    const double epilogue = occ * t.bm * t.bn * 4.0 * (p.accumulate ? 2.0 : 1.0) / kStoreBytesPerCycle;
    const double reduce = splits > 1 ? occ * (splits - 1) * t.bm * t.bn * 4.0 / kLdsBytesPerCycle : 0.0;
    return stream_floor(p, rounds * (std::max(compute, operands) + epilogue + reduce + kLatency), tiles, num_cus);
}


// Workgroups of a persistent launch: as many as the CUs hold at once (LDS
// bound, two slabs each), at most one per tile.  When the tile count is a
// multiple of 8 the grid is too, so that every workgroup's tiles stay on the
// XCD its id maps to.  SGEMM_PERSIST_WGS=<n> caps the grid (tuning sweeps,
// and tests that need many tiles per workgroup on small shapes).
int64_t persist_grid(const Plan &p, const PersistCfg &t, int num_cus, int64_t tiles) {
    const int lds = 2 * t.slab_bytes(p.a_kfast, p.b_kfast);
    int64_t per_cu = std::max(1, std::min(8, int(160 * 1024 / lds)));
    int64_t grid = std::min<int64_t>(tiles, int64_t(std::max(num_cus, 1)) * per_cu);
    if (const char *cap = std::getenv("SGEMM_PERSIST_WGS")) {
        long long v = std::atoll(cap);
        if (v > 0) grid = std::min<int64_t>(grid, v);
    }
    if (tiles % 8 == 0 && grid >= 8) grid -= grid % 8;
    return grid;
}

// Persistent launch: each CU holds grid/num_cus workgroups, and a workgroup's
// tiles follow one another with the next operands already loaded, so per
// tile the CU pays the larger of its matrix-core work, operand reads and C
// traffic rather than their sum; the pipeline's fill is paid once.
double persist_cost(const Plan &p, const PersistCfg &t, int num_cus, int64_t grid) {
    const double kFlopPerCuCycle = 256.0, kOperandBytesPerCycle = 64.0, kStoreBytesPerCycle = 11.0;
    const double kFill = 5350.0;
    int64_t tm = (p.m + t.bm - 1) / t.bm, tn = (p.n + t.bn - 1) / t.bn;
    double tiles = double(p.batch) * double(tm) * double(tn);
    double cus = double(std::max(num_cus, 1));
    double occ = std::max(1.0, std::ceil(double(grid) / cus));
    double iters = std::ceil(tiles / double(grid));
    double kpad = double((p.k + 15) / 16) * 16.0;
    double compute = occ * t.bm * t.bn * 2.0 * kpad / kFlopPerCuCycle / t.rate;
    double operands = occ * double(t.bm + t.bn) * kpad * 4.0 / kOperandBytesPerCycle;
    double epilogue = occ * t.bm * t.bn * 4.0 * (p.accumulate ? 2.0 : 1.0) / kStoreBytesPerCycle;
    return stream_floor(p, iters * std::max({compute, operands, epilogue}) + kFill, double(grid), num_cus);
}

bool persist_serves(const Plan &p, const PersistCfg &t) {
    return p.vec_a == 4 && p.vec_b == 4 && p.c_vec4 && p.k >= 1 && p.k <= t.kmax && !p.row_add &&
           !p.col_add;
}

// The strip kernel needs A and B contiguous along k with 16-byte loads,
// 16-byte C stores, k <= 64 and no vector terms; offsets within one batch
// entry are 32-bit (the whole of A's, B's and C's slices from one base).
bool strip_serves(const Plan &p, const StripCfg &t) {
    return p.a_kfast && p.b_kfast && p.vec_a == 4 && p.vec_b == 4 && p.c_vec4 && p.k >= 1 &&
           p.k <= t.kmax && !p.row_add && !p.col_add && fits_buffer(p.m, p.sA_m, p.k, 1) &&
           fits_buffer(p.n, p.sB_n, p.k, 1) && fits_buffer(p.m, p.sC_m, p.n, 1);
}

// Strip launch: batch * ceil(m / rows) workgroups, each multiplying its rows
// by all of B (k padded to 64) and writing its rows of C; a CU holds as many
// as LDS and its 32 wavefront slots allow.
double strip_cost(const Plan &p, const StripCfg &t, int num_cus) {
    const double kFlopPerCuCycle = 256.0, kStoreBytesPerCycle = 11.0, kFill = 3000.0;
    double wgs = double(p.batch) * double((p.m + t.rows - 1) / t.rows);
    double cus = double(std::max(num_cus, 1));
    double slots = std::min(std::floor(160.0 * 1024.0 / StripCfg::lds_bytes()), std::floor(32.0 / t.waves));
    double occ = std::max(1.0, std::min(slots, std::ceil(wgs / cus)));
    double rounds = std::ceil(wgs / (cus * occ));
    double npad = double((p.n + StripCfg::kBlockCols - 1) / StripCfg::kBlockCols) * StripCfg::kBlockCols;
    double compute = occ * t.rows * npad * 2.0 * t.kmax / kFlopPerCuCycle / t.rate;
    double epilogue = occ * t.rows * double(p.n) * 4.0 * (p.accumulate ? 2.0 : 1.0) / kStoreBytesPerCycle;
    return stream_floor(p, rounds * std::max(compute, epilogue) + kFill, wgs, num_cus);
}

}  // namespace

int make_plan(const GemmArgs &a, Family family, int num_cus, Plan &p, std::string &why) {
    int st = validate(a, why);
    if (st != kOk) return st;
    p = Plan();
    p.batch = a.batch; p.m = a.m; p.n = a.n; p.k = a.k;
    p.alpha = a.alpha; p.beta = a.beta; p.accumulate = a.beta != 0.0f ? 1 : 0;
    p.row_add = a.row_add; p.sR_b = a.sR_batch; p.sR_m = a.sR_row;
    p.col_add = a.col_add; p.sL_b = a.sL_batch; p.sL_n = a.sL_col;
    if (a.batch == 0 || a.m == 0 || a.n == 0) {
        p.empty = true;
        p.kernel_name = "none";
        return kOk;
    }
    // Kernel terms: A is m x k with strides (m, k), B is k x n with (k, n).
    p.A = a.A; p.sA_b = a.sA_batch; p.sA_m = a.sA_row; p.sA_k = a.sA_col;
    p.B = a.B; p.sB_b = a.sB_batch; p.sB_k = a.sB_row; p.sB_n = a.sB_col;
    p.C = a.C; p.sC_b = a.sC_batch; p.sC_m = a.sC_row; p.sC_n = a.sC_col;
    p.inner = a.inner;
    // A group at least as large as the inner count maps every inner entry to
    // the first, as a group of exactly that size does; this keeps it in 32 bits.
    p.sA_i = a.sA_inner; p.gA = std::min(a.gA, a.inner);
    p.sB_i = a.sB_inner; p.gB = std::min(a.gB, a.inner);
    p.sC_i = a.sC_inner;
    // Outputs are written row segments at a time; a column-major C is served
    // as C^T = B^T A^T (kael book ch. 09, section "cuBLAS": the same bytes
    // read in the other order are the transpose), which only exchanges roles
    // and strides.
    bool c_nfast = (p.n == 1 || p.sC_n == 1);
    bool c_mfast = (p.m == 1 || p.sC_m == 1);
    if (!c_nfast && c_mfast && p.m > 1) {
        p.transposed = true;
        std::swap(p.m, p.n);
        uintptr_t A0 = p.A;
        int64_t a_b = p.sA_b, a_m = p.sA_m, a_k = p.sA_k;
        p.A = p.B; p.sA_b = p.sB_b; p.sA_m = p.sB_n; p.sA_k = p.sB_k;
        p.B = A0; p.sB_b = a_b; p.sB_k = a_k; p.sB_n = a_m;
        std::swap(p.sC_m, p.sC_n);
        std::swap(p.sA_i, p.sB_i);
        std::swap(p.gA, p.gB);
        // Rows of C^T are the columns of C: the two vector terms trade places.
        std::swap(p.row_add, p.col_add);
        std::swap(p.sR_b, p.sL_b);
        std::swap(p.sR_m, p.sL_n);
    }
    // Broadcast strides of extent-1 axes never matter; zero them so that
    // alignment checks see only strides that are used.
    if (p.batch == 1) { p.sA_b = 0; p.sB_b = 0; p.sC_b = 0; p.sR_b = 0; p.sL_b = 0; }
    if (p.inner == 1) { p.sA_i = 0; p.sB_i = 0; p.sC_i = 0; p.gA = 1; p.gB = 1; }
    if (p.batch == p.inner) { p.sA_b = 0; p.sB_b = 0; p.sC_b = 0; }  // one outer entry

    p.a_kfast = cols_fast(p.m, p.sA_m, p.k, p.sA_k);
    p.b_kfast = !cols_fast(p.k, p.sB_k, p.n, p.sB_n);
    p.vec_a = p.a_kfast ? vector_width(p.A, p.sA_k, p.k, p.sA_m, p.sA_b, p.batch)
                        : vector_width(p.A, p.sA_m, p.m, p.sA_k, p.sA_b, p.batch);
    p.vec_b = p.b_kfast ? vector_width(p.B, p.sB_k, p.k, p.sB_n, p.sB_b, p.batch)
                        : vector_width(p.B, p.sB_n, p.n, p.sB_k, p.sB_b, p.batch);
    // The inner batch stride moves every tile base as well.
    while (p.vec_a > 1 && p.sA_i % p.vec_a) p.vec_a /= 2;
    while (p.vec_b > 1 && p.sB_i % p.vec_b) p.vec_b /= 2;

    p.c_vec4 = p.sC_n == 1 && p.n % 4 == 0 && p.C % 16 == 0 && p.sC_m % 4 == 0 &&
               (p.batch == 1 || p.sC_b % 4 == 0) && p.sC_i % 4 == 0;
    p.col_vec4 = p.c_vec4 && p.col_add && p.sL_n == 1 && p.col_add % 16 == 0 &&
                 (p.batch == 1 || p.sL_b % 4 == 0);

    const int64_t i32max = (int64_t(1) << 31) - 1;
    bool small_enough = p.m <= i32max && p.n <= i32max && p.k <= i32max && p.batch <= i32max;

    // SGEMM_FORCE_TILE=<tile name> restricts the choice to that tile (of
    // either family) when it can serve the call (for tuning sweeps);
    // otherwise it is ignored.
    const char *force = std::getenv("SGEMM_FORCE_TILE");
    auto allowed = [&](const char *name) { return !force || std::strcmp(force, name) == 0; };
    bool force_known = false;
    if (force) {
        for (int t = 0; t < kNumTiles; ++t)
            if (std::strcmp(force, kTiles[t].name) == 0 && tile_fits(p, kTiles[t].bm, kTiles[t].bn))
                force_known = true;
        for (int t = 0; t < kNumWaveTiles; ++t)
            if (std::strcmp(force, kWaveTiles[t].name) == 0 && tile_fits(p, kWaveTiles[t].bm, kWaveTiles[t].bn))
                force_known = true;
        for (int t = 0; t < kNumPersistTiles; ++t)
            if (std::strcmp(force, kPersistTiles[t].name) == 0 && persist_serves(p, kPersistTiles[t]) &&
                tile_fits(p, kPersistTiles[t].bm, kPersistTiles[t].bn))
                force_known = true;
        for (int t = 0; t < kNumStripTiles; ++t)
            if (std::strcmp(force, kStripTiles[t].name) == 0 && strip_serves(p, kStripTiles[t]))
                force_known = true;
        if (!force_known || family != Family::Auto) force = nullptr;
    }

    int best = -1, best_split = 1;
    bool best_wave = false, best_persist = false, best_strip = false;
    double best_cost = 0;
    auto consider = [&](int t, bool wave, bool persist, int bm, int bn, double cost, int split = 1) {
        int64_t wgs = p.batch * ((p.m + bm - 1) / bm) * ((p.n + bn - 1) / bn);
        if (wgs > i32max || !tile_fits(p, bm, bn)) return;
        if (best < 0 || cost < best_cost) {
            best = t; best_wave = wave; best_persist = persist; best_strip = false; best_cost = cost;
            best_split = split;
        }
    };
    if (small_enough && family != Family::Generic) {
        if (family != Family::Wave) {
            for (int t = 0; t < kNumTiles; ++t)
                if (allowed(kTiles[t].name))
                    consider(t, false, false, kTiles[t].bm, kTiles[t].bn, tile_cost(p, kTiles[t], num_cus));
            for (int t = 0; t < kNumPersistTiles; ++t) {
                const PersistCfg &c = kPersistTiles[t];
                if (!allowed(c.name) || !persist_serves(p, c)) continue;
                int64_t tiles = p.batch * ((p.m + c.bm - 1) / c.bm) * ((p.n + c.bn - 1) / c.bn);
                consider(t, false, true, c.bm, c.bn, persist_cost(p, c, num_cus, persist_grid(p, c, num_cus, tiles)));
            }
            for (int t = 0; t < kNumStripTiles; ++t) {
                const StripCfg &c = kStripTiles[t];
                if (!allowed(c.name) || !strip_serves(p, c)) continue;
                const int64_t wgs = p.batch * ((p.m + c.rows - 1) / c.rows);
                const double cost = strip_cost(p, c, num_cus);
                if (wgs <= i32max && (best < 0 || cost < best_cost)) {
                    best = t; best_wave = false; best_persist = false; best_strip = true; best_cost = cost;
                }
            }
        }
        if (family != Family::Mfma) {
            // Splits of k over 1, 2, 4, ... wavefronts.  SGEMM_WAVE_SPLIT=<s>
            // fixes the split at the largest power of two <= s the tile
            // allows (tuning sweeps, and tests that force a split on small
            // shapes).
            int fixed_split = 0;
            if (const char *ks = std::getenv("SGEMM_WAVE_SPLIT")) fixed_split = std::max(1, std::atoi(ks));
            const int64_t groups = (p.k + 15) / 16;
            for (int t = 0; t < kNumWaveTiles; ++t) {
                if (!allowed(kWaveTiles[t].name)) continue;
                const int most = std::min(kWaveTiles[t].max_split, fixed_split ? fixed_split : kWaveMaxSplit);
                const int64_t tiles = p.batch * ((p.m + kWaveTiles[t].bm - 1) / kWaveTiles[t].bm) *
                                      ((p.n + kWaveTiles[t].bn - 1) / kWaveTiles[t].bn);
                for (int s = 1; s <= most; s *= 2) {
                    // Unforced, a split is for launches that leave SIMDs idle
                    // unsplit (fewer tiles than SIMDs); it must leave every
                    // wavefront at least four groups and the chip at most two
                    // wavefronts per SIMD.
                    const int64_t simds = 4 * int64_t(num_cus);
                    if (fixed_split ? 2 * s <= most
                                    : s > 1 && (tiles >= simds || groups < 4 * s || tiles * s > 2 * simds))
                        continue;
                    consider(t, true, false, kWaveTiles[t].bm, kWaveTiles[t].bn, wave_cost(p, kWaveTiles[t], s, num_cus), s);
                }
            }
        }
    }
    if (best >= 0) p.cost = best_cost;
    if (best >= 0 && best_strip) {
        const StripCfg &c = kStripTiles[best];
        p.family = Family::Mfma;
        p.tile = best;
        p.strip = true;
        p.tiles_m = (p.m + c.rows - 1) / c.rows;
        p.tiles_n = 1;
        p.workgroups = p.batch * p.tiles_m;
        p.kernel_name = std::string("strip_") + c.name + "_ak_bk" + (p.accumulate ? "_acc" : "");
    } else if (best >= 0) {
        int bm = best_wave ? kWaveTiles[best].bm : best_persist ? kPersistTiles[best].bm : kTiles[best].bm;
        int bn = best_wave ? kWaveTiles[best].bn : best_persist ? kPersistTiles[best].bn : kTiles[best].bn;
        const char *name = best_wave ? kWaveTiles[best].name
                                     : best_persist ? kPersistTiles[best].name : kTiles[best].name;
        p.family = best_wave ? Family::Wave : Family::Mfma;
        p.tile = best;
        p.persist = best_persist;
        p.tiles_m = (p.m + bm - 1) / bm;
        p.tiles_n = (p.n + bn - 1) / bn;
        p.workgroups = p.batch * p.tiles_m * p.tiles_n;
        p.ksplit = best_wave ? best_split : 1;
        if (best_persist) p.workgroups = persist_grid(p, kPersistTiles[best], num_cus, p.workgroups);
        if (!best_wave && !best_persist) {
            // The LDS-tiled kernel keeps each thread's load offsets for the
            // whole k loop when the buffer resource alone can bound k: an
            // operand read along k (tile columns along k) needs whole slices,
            // one read across k (tile rows along k) needs rows that do not
            // overlap, so that a row index past K means an offset past the
            // resource's end.
            // The size is formed in 32 bits from at most one slice of rows, so
            // that slice must stay below 2 GiB (it can exceed it only through
            // the stride of a k extent of 1, which otherwise never matters).
            const int64_t bk = kTiles[best].bk;
            auto bounded = [&](bool kfast, int64_t extent, int64_t s_fast, int64_t s_k) {
                return kfast ? p.k % bk == 0
                             : (extent - 1) * s_fast < s_k && std::min(p.k, bk) * s_k * 4 < kBufferLimit;
            };
            p.fixed_offsets = bounded(p.a_kfast, p.m, p.sA_m, p.sA_k) && bounded(p.b_kfast, p.n, p.sB_n, p.sB_k);
        }
        p.kernel_name = std::string(best_wave ? "wave_" : best_persist ? "persist_" : "mfma_") + name +
                        (p.a_kfast ? "_ak" : "_am") + (p.b_kfast ? "_bk" : "_bn") +
                        (p.accumulate ? "_acc" : "") + (p.row_add || p.col_add ? "_vec" : "") +
                        (p.ksplit > 1 ? "_s" + std::to_string(p.ksplit) : "");
    } else {
        p.family = Family::Generic;
        p.tile = -1;
        p.vec_a = p.vec_b = 1;
        p.tiles_m = (p.m + 63) / 64;
        p.tiles_n = (p.n + 63) / 64;
        int64_t tiles = p.batch * p.tiles_m * p.tiles_n;
        p.workgroups = std::min<int64_t>(tiles, 65536);
        // Plain fp32 FMA at a fifth of the vector peak (256 FLOP per CU cycle).
        p.cost = 2.0 * double(p.batch) * double(p.m) * double(p.n) * double(std::max<int64_t>(p.k, 1)) /
                 (256.0 * 0.2 * double(std::max(num_cus, 1)));
        p.kernel_name = std::string("generic_t64x64") + (p.accumulate ? "_acc" : "") +
                        (p.row_add || p.col_add ? "_vec" : "");
    }
    // 8-byte loads exist only in the LDS-tiled kernel with fixed offsets;
    // every other kernel reads such an operand element by element.
    if (p.family != Family::Mfma || p.persist || p.strip || !p.fixed_offsets) {
        if (p.vec_a == 2) p.vec_a = 1;
        if (p.vec_b == 2) p.vec_b = 1;
    }
    return kOk;
}

}  // namespace sgemm
