// attention.cpp -- argument checks and kernel choice for fused attention.
//
// Every size, stride and pointer the kernels depend on is checked before
// anything is enqueued (StaleyNET "GPU Implementation", section "Safety").
#include "attention.hpp"

#include <algorithm>
#include <cmath>
#include <cstdlib>

#include "extent.hpp"

namespace sgemm {

namespace {

constexpr int kAttnQueriesPerWave = 16;
constexpr int64_t kInt32Max = 0x7fffffff;
constexpr int64_t kSliceBytes = (int64_t(1) << 31) - 64;   // 32-bit buffer offsets per slice

const char *const kOperand[4] = {"Q", "K", "V", "O"};

int64_t kv_heads(const AttnCall &c) { return (c.nb_inner + c.g - 1) / c.g; }

// Largest element offset of each operand over the whole call (-1 on overflow).
void last_offsets(const AttnCall &c, int64_t last[4]) {
    const int64_t heads[4] = {c.nb_inner, kv_heads(c), kv_heads(c), c.nb_inner};
    const int64_t rows[4] = {c.tq, c.tk, c.tk, c.tq};
    const int64_t *s[4] = {c.sQ, c.sK, c.sV, c.sO};
    for (int x = 0; x < 4; ++x)
        last[x] = last_offset4(c.nb_outer, s[x][0], heads[x], s[x][1], rows[x], s[x][2], c.d, s[x][3]);
}

// One (outer, inner) slice of an operand addressed with 32-bit byte offsets.
bool slice_fits(int64_t rows, int64_t s_row, int64_t d) {
    const int64_t off = last_offset(1, 0, rows, s_row, d, 1);
    int64_t bytes;
    return off >= 0 && mul64(off + 1, 4, bytes) && bytes < kSliceBytes;
}

}  // namespace

int validate_attention(const AttnCall &c, std::string &why) {
    if (c.nb_outer < 0 || c.nb_inner < 1 || c.tq < 0 || c.tk < 0 || c.d < 0 || c.g < 1) {
        why = "sizes must be >= 0, nb_inner and g >= 1";
        return kErrSize;
    }
    const int64_t *s[4] = {c.sQ, c.sK, c.sV, c.sO};
    for (int x = 0; x < 4; ++x)
        for (int a = 0; a < 4; ++a)
            if (s[x][a] < 0) {
                why = std::string("negative stride of ") + kOperand[x];
                return kErrStride;
            }
    int64_t heads, rows;
    if (!mul64(c.nb_outer, c.nb_inner, heads) || !mul64(heads, c.tq, rows)) {
        why = "nb_outer*nb_inner*tq overflows int64";
        return kErrUnsupported;
    }
    if (rows == 0 || c.d == 0) return kOk;   // no output element
    if (c.tk == 0) {
        why = "tk = 0: a query has no key to attend to";
        return kErrSize;
    }
    if (c.causal && c.tq > c.tk) {
        why = "causal with tq > tk: the first queries would see no key";
        return kErrSize;
    }
    if (c.d > kAttnMaxDim) {
        why = "head dimension d above " + std::to_string(kAttnMaxDim);
        return kErrUnsupported;
    }
    if (c.tq > kInt32Max || c.tk > kInt32Max || c.nb_inner > kInt32Max) {
        why = "tq, tk and nb_inner must be below 2^31";
        return kErrUnsupported;
    }
    const uintptr_t ptr[4] = {c.Q, c.K, c.V, c.O};
    for (int x = 0; x < 4; ++x)
        if (!ptr[x]) {
            why = std::string(kOperand[x]) + " is NULL";
            return kErrNull;
        }
    int64_t last[4];
    last_offsets(c, last);
    int64_t bytes;
    for (int x = 0; x < 4; ++x)
        if (last[x] < 0 || !mul64(last[x] + 1, 4, bytes)) {
            why = std::string(kOperand[x]) + ": extent times strides overflows int64";
            return kErrUnsupported;
        }
    const int64_t o_ext[4] = {c.nb_outer, c.nb_inner, c.tq, c.d};
    if (!distinct_axes(o_ext, c.sO)) {
        why = "O's strides map two outputs to the same element";
        return kErrAlias;
    }
    for (int x = 0; x < 3; ++x)
        if (ranges_overlap(c.O, last[3], ptr[x], last[x])) {
            why = std::string("O's address range overlaps ") + kOperand[x];
            return kErrAlias;
        }
    return kOk;
}

namespace {

// Can the matrix-core kernel (head dimension 64, unit column strides,
// 16-byte aligned rows, 32-bit offsets inside each slice) run this call?
bool mfma_serves(const AttnCall &c, std::string &why) {
    if (c.d != 64) { why = "the matrix-core kernel needs d = 64"; return false; }
    const int64_t *s[4] = {c.sQ, c.sK, c.sV, c.sO};
    const uintptr_t ptr[4] = {c.Q, c.K, c.V, c.O};
    const int64_t rows[4] = {c.tq, c.tk, c.tk, c.tq};
    for (int x = 0; x < 4; ++x) {
        if (s[x][3] != 1) { why = "the matrix-core kernel needs unit column strides"; return false; }
        if (ptr[x] % 16 || s[x][0] % 4 || s[x][1] % 4 || s[x][2] % 4) {
            why = "the matrix-core kernel needs 16-byte aligned rows";
            return false;
        }
        if (!slice_fits(rows[x], s[x][2], c.d)) {
            why = "a slice spans more than 2 GiB";
            return false;
        }
    }
    return true;
}

}  // namespace

bool attention_overlaps(const AttnCall &c, uintptr_t p, int64_t floats) {
    if (!p || floats <= 0) return false;
    int64_t last[4];
    last_offsets(c, last);
    const uintptr_t ptr[4] = {c.Q, c.K, c.V, c.O};
    for (int x = 0; x < 4; ++x)
        if (last[x] >= 0 && ranges_overlap(p, floats - 1, ptr[x], last[x])) return true;
    return false;
}

void make_splitkv_plan(const AttnCall &c, int num_cus, uintptr_t workspace, int64_t workspace_floats,
                       SplitKvPlan &sp) {
    sp = SplitKvPlan{};
    std::string ignore;
    const int64_t g = std::min(c.g, c.nb_inner);
    if (c.nb_outer == 0 || c.tq == 0 || c.tk == 0 || c.d == 0 || !mfma_serves(c, ignore)) return;
    int64_t rows;   // query rows of a group
    if (!mul64(g, c.tq, rows) || rows > kSkvMaxRows) return;
    const int64_t row_tiles = (rows + kSkvRows - 1) / kSkvRows;
    // One group's query rows are addressed from one base with 32-bit offsets.
    const int64_t qlast = last_offset(g, c.sQ[1], c.tq, c.sQ[2], c.d, 1);
    int64_t qbytes;
    if (qlast < 0 || !mul64(qlast + 1, 4, qbytes) || qbytes >= kSliceBytes) return;
    const int64_t n_kv = kv_heads(c);
    int64_t groups;   // (outer, KV head, row tile) triples: wavefronts per chunk
    // The merge launches 16 workgroups per triple.
    if (!mul64(c.nb_outer, n_kv, groups) || !mul64(groups, row_tiles, groups) || groups > kInt32Max / kSkvRows)
        return;
    // Chunks of a whole number of 32-key blocks.  The kernel's time is taken
    // as that of the busiest CU, ceil(workgroups / CUs) workgroups of four
    // wavefronts each streaming one chunk (the dispatcher spreads them
    // evenly), plus a little merge work per chunk.  The cheapest count that
    // gives every CU a workgroup is taken; where the keys allow none, the
    // cheapest count overall.  SGEMM_ATTN_CHUNKS=<n> fixes the count (tests
    // and sweeps).
    const int64_t blocks = (c.tk + 31) / 32;
    int64_t cap = blocks;
    if (workspace_floats >= 0) cap = std::min<int64_t>(cap, workspace_floats / (groups * kSkvItemFloats));
    if (cap < 1) return;
    int64_t chunks = 0;
    if (const char *f = std::getenv("SGEMM_ATTN_CHUNKS")) {
        chunks = std::min<int64_t>(std::max(1, std::atoi(f)), cap);
    } else {
        const int64_t cus = std::max(num_cus, 1);
        int64_t fill = 0, any = 0;   // best count filling every CU, best count overall
        double fill_cost = 0.0, any_cost = 0.0;
        // b = blocks per chunk, visiting each distinct chunk count once.
        for (int64_t b = 1; b <= blocks;) {
            const int64_t n = (blocks + b - 1) / b;
            if (n <= cap) {
                const int64_t per = (blocks + n - 1) / n;   // blocks of the longest chunk
                const int64_t wgs = (groups * n + 3) / 4;
                const double cost =
                    double((wgs + cus - 1) / cus) * 4.0 * double(per) + kSkvMergePerChunk * double(n);
                if (wgs >= cus && (fill == 0 || cost < fill_cost)) {
                    fill = n;
                    fill_cost = cost;
                }
                if (any == 0 || cost < any_cost) {
                    any = n;
                    any_cost = cost;
                }
            }
            if (n == 1) break;
            b = (blocks + n - 2) / (n - 1);   // the smallest b that gives fewer chunks
        }
        chunks = fill ? fill : any;
    }
    const int64_t chunk_keys = ((c.tk + chunks - 1) / chunks + 31) / 32 * 32;
    chunks = (c.tk + chunk_keys - 1) / chunk_keys;
    int64_t items, floats;
    if (!mul64(groups, chunks, items) || !mul64(items, kSkvItemFloats, floats) || items > 4 * kInt32Max) return;

    SplitKvArgs &a = sp.args;
    a.Q = reinterpret_cast<const float *>(c.Q);
    a.K = reinterpret_cast<const float *>(c.K);
    a.V = reinterpret_cast<const float *>(c.V);
    a.O = reinterpret_cast<float *>(c.O);
    a.W = reinterpret_cast<float *>(workspace);
    a.sQ_o = c.sQ[0]; a.sQ_i = c.sQ[1]; a.sQ_r = c.sQ[2];
    a.sK_o = c.sK[0]; a.sK_i = c.sK[1]; a.sK_r = c.sK[2];
    a.sV_o = c.sV[0]; a.sV_i = c.sV[1]; a.sV_r = c.sV[2];
    a.sO_o = c.sO[0]; a.sO_i = c.sO[1]; a.sO_r = c.sO[2];
    a.nb_inner = int(c.nb_inner); a.n_kv = int(n_kv); a.g = int(g);
    a.tq = int(c.tq); a.tk = int(c.tk); a.causal = c.causal ? 1 : 0;
    a.scale_log2 = float(double(c.alpha) * 1.4426950408889634);   // alpha * log2(e)
    a.chunks = int(chunks);
    a.chunk_keys = int(chunk_keys);
    a.row_tiles = int(row_tiles);
    a.items = items;
    sp.chunks = int(chunks);
    sp.chunk_keys = int(chunk_keys);
    sp.workspace_floats = floats;
}

int make_attention_plan(const AttnCall &c, AttnPath path, AttnPlan &plan, std::string &why) {
    plan = AttnPlan{};
    int64_t rows = c.nb_outer * c.nb_inner * c.tq;
    plan.empty = rows == 0 || c.d == 0;
    if (plan.empty) return kOk;
    std::string no_mfma;
    const bool mfma = mfma_serves(c, no_mfma);
    if (path == AttnPath::Mfma && !mfma) {
        why = "matrix-core attention forced but unavailable: " + no_mfma;
        return kErrUnsupported;
    }
    plan.path = (path == AttnPath::Generic || !mfma) ? AttnPath::Generic : AttnPath::Mfma;

    AttnArgs &a = plan.args;
    a.Q = reinterpret_cast<const float *>(c.Q);
    a.K = reinterpret_cast<const float *>(c.K);
    a.V = reinterpret_cast<const float *>(c.V);
    a.O = reinterpret_cast<float *>(c.O);
    a.sQ_o = c.sQ[0]; a.sQ_i = c.sQ[1]; a.sQ_r = c.sQ[2]; a.sQ_c = c.sQ[3];
    a.sK_o = c.sK[0]; a.sK_i = c.sK[1]; a.sK_r = c.sK[2]; a.sK_c = c.sK[3];
    a.sV_o = c.sV[0]; a.sV_i = c.sV[1]; a.sV_r = c.sV[2]; a.sV_c = c.sV[3];
    a.sO_o = c.sO[0]; a.sO_i = c.sO[1]; a.sO_r = c.sO[2]; a.sO_c = c.sO[3];
    a.tq = int(c.tq); a.tk = int(c.tk); a.d = int(c.d);
    a.causal = c.causal ? 1 : 0;
    a.scale_log2 = float(double(c.alpha) * 1.4426950408889634);   // alpha * log2(e)
    const int64_t g = std::min(c.g, c.nb_inner);
    a.inner = make_divisor(uint32_t(c.nb_inner));
    a.group = make_divisor(uint32_t(g));
    a.rows = rows;
    a.nb_inner_ll = c.nb_inner;
    a.g_ll = g;

    if (plan.path == AttnPath::Mfma) {
        plan.waves = 8;
        if (const char *w = std::getenv("SGEMM_ATTN_WAVES")) {
            const int v = std::atoi(w);
            if (v == 4 || v == 8) plan.waves = v;
        }
        const int64_t bq = int64_t(plan.waves) * kAttnQueriesPerWave;
        int64_t qblocks = (c.tq + bq - 1) / bq;
        if (c.causal) {
            // Causal work grows with the query index: each workgroup pairs an
            // early block of bq/2 rows with the mirrored late one, so every
            // workgroup (and every SIMD, whose two wavefronts come one from
            // each half) sees about the same number of keys.
            const int64_t half = (c.tq + bq / 2 - 1) / (bq / 2);
            a.zigzag = 1;
            a.half_blocks = int(half);
            qblocks = (half + 1) / 2;
        }
        int64_t blocks;
        if (!mul64(c.nb_outer * c.nb_inner, qblocks, blocks) || blocks > kInt32Max) {
            why = "too many query blocks for one launch";
            return kErrUnsupported;
        }
        a.qblocks = make_divisor(uint32_t(qblocks));
        a.blocks = int(blocks);
        a.xcd_remap = blocks % 8 == 0;
        plan.workgroups = blocks;
        plan.kernel_name = std::string("attn_mfma_d64_w") + std::to_string(plan.waves) +
                           (c.causal ? "_causal" : "");
    } else {
        // One wavefront per query row, four per workgroup, grid-stride loop.
        const int64_t wgs = std::min<int64_t>((rows + 3) / 4, 65536);
        plan.workgroups = wgs;
        plan.waves = 4;
        plan.kernel_name = std::string("attn_generic") + (c.causal ? "_causal" : "");
    }
    return kOk;
}

}  // namespace sgemm
