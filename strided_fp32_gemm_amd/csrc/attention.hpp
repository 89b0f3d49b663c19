// attention.hpp -- fused scaled dot-product attention: argument checks,
// planning and the launch (host side), and the argument block the kernels
// take.
//
// For o < nb_outer, i < nb_inner and query row q < tq:
//
//     O[o,i,q,:] = sum_j softmax_j(alpha * <Q[o,i,q,:], K[o,i/g,j,:]>) V[o,i/g,j,:]
//
// over the keys j < tk that query q sees (all of them, or with `causal` the
// keys j <= q + tk - tq: the queries are the last tq positions of the
// context).  This is the three-step attention of the rvllm post (section
// "Matmuls go to cuBLAS": the scores as one strided batched product with the
// 1/sqrt(head_dim) scale in alpha, then a softmax, then the probabilities
// times V) done in one pass, so the scores never reach global memory (the
// same post, "What's basic about it", names that round trip as the cost a
// fused kernel removes).  g query heads share one key/value head.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <string>

#include "plan.hpp"

namespace sgemm {

// Largest head dimension any kernel serves.
constexpr int kAttnMaxDim = 256;

// Caller's view of one attention call (element strides, >= 0).
struct AttnCall {
    int64_t nb_outer = 0, nb_inner = 1, tq = 0, tk = 0, d = 0, g = 1;
    float alpha = 1.0f;
    int causal = 0;
    uintptr_t Q = 0, K = 0, V = 0, O = 0;
    int64_t sQ[4] = {0, 0, 0, 0};   // outer, inner, row, col
    int64_t sK[4] = {0, 0, 0, 0};
    int64_t sV[4] = {0, 0, 0, 0};
    int64_t sO[4] = {0, 0, 0, 0};
};

enum class AttnPath { Auto = 0, Mfma = 1, Generic = 3 };

// Kernel arguments.  The matrix-core kernel takes 32-bit element offsets
// from each (outer, inner) base (the planner checks they fit) and unit
// column strides; the generic kernel takes everything as 64-bit.
struct AttnArgs {
    const float *Q, *K, *V;
    float *O;
    long long sQ_o, sQ_i, sQ_r, sQ_c;
    long long sK_o, sK_i, sK_r, sK_c;
    long long sV_o, sV_i, sV_r, sV_c;
    long long sO_o, sO_i, sO_r, sO_c;
    int tq, tk, d;
    int causal;
    float scale_log2;   // alpha * log2(e): softmax weights are exp2(scale_log2 * (s - max))
    Divisor inner, group, qblocks;
    int blocks;         // nb_outer * nb_inner * qblocks
    int xcd_remap;      // blocks % 8 == 0: consecutive blocks share an XCD
    int zigzag;         // causal: a workgroup's two halves take query blocks qb and half_blocks-1-qb
    int half_blocks;    // query blocks of half a workgroup's rows (zigzag)
    long long rows;     // nb_outer * nb_inner * tq (generic kernel)
    long long nb_inner_ll, g_ll;
};

struct AttnPlan {
    AttnArgs args{};
    AttnPath path = AttnPath::Generic;
    int waves = 4;            // wavefronts per workgroup (matrix-core kernel)
    int64_t workgroups = 0;
    bool empty = true;
    std::string kernel_name;
};

// Split-KV attention (decode): the g query heads of a KV head and their tq
// queries (g * tq <= 64) stacked as the rows of up to four 16-row tiles, the
// keys cut into chunks, one wavefront per (outer, KV head, row tile, chunk)
// reading its chunk of K and V straight from memory, its partial result (the
// unnormalised output rows, their reference maxima and weight sums) written
// to a workspace; then one merge per output row over the chunks in order.
constexpr int kSkvRows = 16;                          // query rows of a wavefront's tile
constexpr int kSkvMaxRows = 4 * kSkvRows;             // rows of a group the split serves
constexpr int kSkvItemFloats = kSkvRows * 64 + 2 * kSkvRows;   // partial: O rows, m, l
// Merge cost of one more chunk, in units of one wavefront streaming one
// 32-key block on the busiest CU (fitted: about 0.06 us against 0.7 us).
constexpr double kSkvMergePerChunk = 0.1;
struct SplitKvArgs {
    const float *Q, *K, *V;
    float *O;
    float *W;                        // workspace: (o, kv, row tile, chunk) at W + index * kSkvItemFloats
    long long sQ_o, sQ_i, sQ_r;      // unit column strides (checked by the planner)
    long long sK_o, sK_i, sK_r;
    long long sV_o, sV_i, sV_r;
    long long sO_o, sO_i, sO_r;
    int nb_inner, n_kv, g, tq, tk, causal;
    float scale_log2;                // alpha * log2(e)
    int chunks, chunk_keys;
    int row_tiles;                   // 16-row tiles per group, ceil(g * tq / 16)
    long long items;                 // nb_outer * n_kv * row_tiles * chunks
};
struct SplitKvPlan {
    int chunks = 0;                  // 0: not split (the call is sgemm_attention)
    int chunk_keys = 0;
    int64_t workspace_floats = 0;
    SplitKvArgs args{};
};

// Returns kOk or a status (kErrSize, kErrStride, kErrNull, kErrAlias,
// kErrUnsupported) with `why` filled; touches no device.
int validate_attention(const AttnCall &c, std::string &why);

// Plans the split-KV form of a validated call for a workspace of at most
// `workspace_floats` floats (< 0: no cap) at `workspace` (0 for a size
// query): chunks = 0 when it does not apply (head dimension other than 64,
// non-unit column strides, unaligned rows, g * tq > 16) or no chunk fits.
void make_splitkv_plan(const AttnCall &c, int num_cus, uintptr_t workspace, int64_t workspace_floats,
                       SplitKvPlan &sp);

// True if the `floats` floats at p meet any element range of Q, K, V or O.
bool attention_overlaps(const AttnCall &c, uintptr_t p, int64_t floats);

// Enqueues the chunk launch and the merge; kErrHip on a rejected launch.
int launch_splitkv(const SplitKvPlan &sp, hipStream_t stream, std::string &why);

// Chooses the kernel.  `path` Auto picks the matrix-core kernel when it
// serves the call; forcing Mfma on a call it cannot serve is kErrUnsupported.
int make_attention_plan(const AttnCall &c, AttnPath path, AttnPlan &plan, std::string &why);

// Enqueues the plan on `stream`; kErrHip on a rejected launch.
int launch_attention(const AttnPlan &plan, hipStream_t stream, std::string &why);

}  // namespace sgemm
