// splitk.cpp -- planning and launching the split-k product (see splitk.hpp).
#include "splitk.hpp"

#include <algorithm>
#include <cmath>
#include <cstdlib>

#include "extent.hpp"
#include "kernels.hpp"

namespace sgemm {

namespace {

// Partitions are a multiple of 64 deep (two k slices of the tiled kernels,
// four groups of the wavefront kernel; 16-byte aligned partition starts for
// a k-contiguous operand) and at least 128 deep; at most 256 of them.
constexpr int64_t kPartAlign = 64, kMinPart = 128;
constexpr int kMaxSplits = 256;
// A size query plans against this stand-in address (256-byte aligned).
constexpr uintptr_t kQueryWorkspace = uintptr_t(1) << 44;
// Cycles one more dependent launch adds on a stream (measured: a phase-1
// launch followed by a reduction over 8 MB of partials took ~5 us more than
// phase 1 alone).
constexpr double kLaunchCycles = 8000.0;

int64_t ceil_div(int64_t x, int64_t y) { return (x + y - 1) / y; }

// Partitions 0 .. full-1 (each kc deep) as an inner batch level, into the
// workspace: partition q of batch entry b at W + (b * splits + q) * m * n.
GemmArgs parts_args(const GemmArgs &a, uintptr_t W, int splits, int full, int64_t kc) {
    GemmArgs p = a;
    p.alpha = 1.0f;
    p.accumulate = 0;
    p.beta = 0.0f;
    p.row_add = 0;
    p.col_add = 0;
    p.k = kc;
    p.batch = a.batch * full;
    p.inner = full;
    p.sA_inner = kc * a.sA_col; p.gA = 1;
    p.sB_inner = kc * a.sB_row; p.gB = 1;
    p.C = W;
    p.sC_batch = int64_t(splits) * a.m * a.n;
    p.sC_inner = a.m * a.n;
    p.sC_row = a.n;
    p.sC_col = 1;
    return p;
}

// The last partition, k_last deep, when it is shorter than kc.
GemmArgs tail_args(const GemmArgs &a, uintptr_t W, int splits, int full, int64_t kc, int64_t k_last) {
    GemmArgs p = a;
    p.alpha = 1.0f;
    p.accumulate = 0;
    p.beta = 0.0f;
    p.row_add = 0;
    p.col_add = 0;
    p.k = k_last;
    p.A = a.A + 4u * uintptr_t(int64_t(full) * kc * a.sA_col);
    p.B = a.B + 4u * uintptr_t(int64_t(full) * kc * a.sB_row);
    p.C = W + 4u * uintptr_t(int64_t(full) * a.m * a.n);
    p.sC_batch = int64_t(splits) * a.m * a.n;
    p.sC_row = a.n;
    p.sC_col = 1;
    return p;
}

// The reduction reads every partial once and writes C (reading it when
// accumulating): HBM-bound, ~2700 bytes per cycle, plus its launch.
double reduce_cost(const GemmArgs &a, int splits) {
    const double outputs = double(a.batch) * double(a.m) * double(a.n);
    return 4.0 * outputs * (splits + (a.accumulate ? 2.0 : 1.0)) / 2700.0 + kLaunchCycles;
}

}  // namespace

int make_split_plan(const GemmArgs &a, int num_cus, uintptr_t workspace, int64_t workspace_floats,
                    SplitPlan &sp, std::string &why) {
    sp = SplitPlan{};
    int st = make_plan(a, Family::Auto, num_cus, sp.whole, why);
    if (st != kOk) return st;
    sp.cost = sp.whole.cost;
    // The split serves the product, optionally plus C: no vector terms and
    // beta in {0, 1} (the only epilogues its entry point takes).
    if (sp.whole.empty || a.k < 2 || a.row_add || a.col_add || (a.beta != 0.0f && a.beta != 1.0f)) return kOk;
    const uintptr_t W = workspace ? workspace : kQueryWorkspace;
    int64_t outputs;
    if (!mul64(a.batch, a.m, outputs) || !mul64(outputs, a.n, outputs)) return kOk;
    // SGEMM_SPLITK=<P> plans exactly P partitions of a multiple of 64 in k
    // (or none, if the workspace cannot hold them), whatever the cost
    // (tests and sweeps; P = 1 forces the unsplit product).
    int forced = 0;
    if (const char *f = std::getenv("SGEMM_SPLITK")) forced = std::max(1, std::atoi(f));
    if (forced == 1) return kOk;
    if (forced) sp.cost = 1e300;
    for (int P = forced ? forced : 2; P <= (forced ? forced : kMaxSplits); P *= 2) {
        const int64_t kc = ceil_div(ceil_div(a.k, P), kPartAlign) * kPartAlign;
        if (kc < (forced ? kPartAlign : kMinPart)) break;
        const int64_t splits = ceil_div(a.k, kc);
        if (splits < 2) continue;
        int64_t floats;
        if (!mul64(outputs, splits, floats)) break;
        if (workspace_floats >= 0 && floats > workspace_floats) continue;
        const int full = int(a.k / kc);   // at most splits <= P
        const int64_t k_last = a.k - (splits - 1) * kc;
        int64_t flat;
        if (!mul64(a.batch, full, flat)) break;
        Plan parts, tail;
        std::string ignore;
        if (make_plan(parts_args(a, W, int(splits), full, kc), Family::Auto, num_cus, parts, ignore) != kOk)
            continue;
        double cost = parts.cost + reduce_cost(a, int(splits));
        if (full < splits) {
            if (make_plan(tail_args(a, W, int(splits), full, kc, k_last), Family::Auto, num_cus, tail, ignore) !=
                kOk)
                continue;
            cost += tail.cost + kLaunchCycles;
        }
        if (cost < sp.cost || forced) {
            sp.splits = int(splits);
            sp.kc = kc;
            sp.k_last = k_last;
            sp.full = full;
            sp.parts = parts;
            sp.tail = tail;
            sp.workspace_floats = floats;
            sp.cost = cost;
        }
    }
    if (sp.splits == 1) sp.cost = sp.whole.cost;
    return kOk;
}

int launch_split_plan(const GemmArgs &a, const SplitPlan &sp, uintptr_t workspace, hipStream_t stream,
                      std::string &why) {
    if (sp.splits <= 1) return launch_plan(sp.whole, stream, why);
    int st = launch_plan(sp.parts, stream, why);
    if (st != kOk) return st;
    if (sp.full < sp.splits) {
        st = launch_plan(sp.tail, stream, why);
        if (st != kOk) return st;
    }
    SplitReduceArgs r;
    r.W = reinterpret_cast<const float *>(workspace);
    r.C = reinterpret_cast<float *>(a.C);
    r.batch = a.batch; r.m = a.m; r.n = a.n;
    r.splits = sp.splits;
    r.alpha = a.alpha;
    r.accumulate = a.beta != 0.0f ? 1 : 0;
    r.sC_b = a.sC_batch; r.sC_m = a.sC_row; r.sC_n = a.sC_col;
    r.vec4 = a.n % 4 == 0 && a.sC_col == 1 && a.C % 16 == 0 && a.sC_row % 4 == 0 &&
             (a.batch == 1 || a.sC_batch % 4 == 0) && workspace % 16 == 0;
    launch_split_reduce(r, stream);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        why = std::string("split-k reduction launch failed: ") + hipGetErrorString(e);
        return kErrHip;
    }
    return kOk;
}

}  // namespace sgemm
