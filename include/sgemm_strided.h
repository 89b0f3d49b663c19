/*
 * sgemm_strided.h -- C ABI of the strided, batched fp32 matrix product for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (StaleyNET "GPU Implementation", section "The matrix
 * product"): for a batch of matrix pairs,
 *
 *     C[b,i,j] <- alpha * sum_{p<k} A[b,i,p] * B[b,p,j]   (+ C[b,i,j] if accumulate)
 *
 * for b < batch, i < m, j < n.  Each operand X is addressed as
 *
 *     X[b,r,c] = X + b*sX_batch + r*sX_row + c*sX_col
 *
 * with strides counted in float ELEMENTS (not bytes), as signed 64-bit
 * values that must be >= 0.  A transposed input is the same pointer with its
 * row and column strides exchanged; no flag and no copy is involved.  A batch
 * stride of 0 broadcasts one matrix to every batch entry (a shared weight or
 * basis).  One call covers the whole batch in one launch, which is how all
 * heads and sequences of attention are served together.
 *
 * Memory and ownership: A, B and C are device pointers allocated by the
 * caller (e.g. by PyTorch); the library allocates nothing, keeps no
 * per-call state and never frees caller memory.  It remembers, per host
 * thread, the plans of the last few products it planned (a plan depends on
 * the arguments and the device's CU count alone), so a repeated call skips
 * validation and planning.  It may be called from several host threads on
 * different streams.
 *
 * Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL means the
 * null stream) and the call returns without synchronising.  Argument errors
 * are reported before anything is enqueued; a fault during execution shows up
 * at the caller's next synchronisation (kael book ch. 09 "CUDA backend",
 * sections "Synchronous and asynchronous work" and "Edge cases and
 * pitfalls").
 *
 * Numerics: the products are accumulated in fp32 on the matrix cores (fp32
 * MFMA; no reduced-precision input format), in an order fixed by the chosen
 * kernel, so repeated calls with the same arguments give bit-identical
 * results.  No atomics are used.  alpha scales the fresh product only; with
 * accumulate != 0 the stored C is added once per element.  With
 * accumulate == 0 the stored C is never read.
 *
 * Entry points:
 *   sgemm_strided_batched[_path]       the product (optionally + C)
 *   sgemm_strided_batched_ex[_path]    + beta*C + per-row and per-column terms
 *   sgemm_strided_batched2[_path]      two batch levels, grouped inputs (KV heads)
 *   sgemm_strided_batched_splitk       the product with k split across workgroups (caller's workspace)
 *   sgemm_sqnorms, sgemm_pairwise_sqdist   squared norms, squared distances
 *   sgemm_pairwise_sqdist_noalloc      the same distances without a workspace
 *   sgemm_attention[_path]             softmax(alpha Q K^T) V, fused, over two batch levels
 *   sgemm_attention_splitkv[_describe] the same for decode, keys split across the GPU (caller's workspace)
 *   sgemm_plan_describe[2], sgemm_splitk_describe, sgemm_attention_describe
 *                                      the launch a call would make
 *   sgemm_status_string, sgemm_last_error   status text
 * The _path variants force a kernel family (tests, sweeps).
 */
#ifndef SGEMM_STRIDED_H
#define SGEMM_STRIDED_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Every non-zero status leaves C untouched and enqueues
 * nothing, except SGEMM_ERR_HIP, which reports a failed launch.
 *
 * Why they exist: a launch whose sizes do not match what the kernel assumes
 * reads or writes memory it must not, and nothing reports it, so every size,
 * stride and pointer a kernel depends on is checked before the launch
 * (StaleyNET "GPU Implementation", section "Safety").  The individual codes
 * follow the failure modes kael book ch. 09 "CUDA backend" lists in section
 * "Edge cases and pitfalls": a zero extent returns before any launch (a grid
 * of zero blocks is itself an error), index arithmetic that would wrap is
 * refused rather than run (-5), and faults inside a running kernel are not
 * reported by the launch but by a later runtime call (-6 only covers what
 * the runtime reports at launch time). */
enum sgemm_status {
    SGEMM_OK = 0,
    SGEMM_ERR_INVALID_SIZE = -1,   /* batch, m, n or k < 0 */
    SGEMM_ERR_INVALID_STRIDE = -2, /* a stride < 0 */
    SGEMM_ERR_NULL_POINTER = -3,   /* C null with batch*m*n > 0, or A/B null with k > 0 as well */
    SGEMM_ERR_C_ALIAS = -4,        /* C's strides map two outputs to one address, or C overlaps A or B */
    SGEMM_ERR_UNSUPPORTED = -5,    /* an extent times its stride overflows int64, or no kernel fits */
    SGEMM_ERR_HIP = -6,            /* the HIP runtime rejected a query or launch; see sgemm_last_error() */
    SGEMM_ERR_INVALID_PATH = -7,   /* unknown path code */
    SGEMM_ERR_WORKSPACE = -8       /* workspace NULL or smaller than the call needs */
};

/* Kernel families the planner chooses between (for sgemm_strided_batched_path
 * and sgemm_plan_describe). */
enum sgemm_path {
    SGEMM_PATH_AUTO = 0,    /* planner's choice (what sgemm_strided_batched uses) */
    SGEMM_PATH_MFMA = 1,    /* LDS-tiled fp32 MFMA kernel, per-layout coalesced loaders */
    SGEMM_PATH_WAVE = 2,    /* one wavefront per tile, operands straight to registers: short k, few tiles */
    SGEMM_PATH_GENERIC = 3  /* any strides, 64-bit addressing, fp32 FMA */
};

/*
 * C <- alpha * A * B (+ C), batched and strided, on `stream`.
 * Sizes: batch, m, n, k >= 0.  batch, m or n == 0 returns SGEMM_OK without
 * enqueueing; k == 0 is the empty sum, so C <- alpha*0 (+ C).
 * Pointers: device pointers; A and B may be NULL when k == 0, all three may
 * be NULL when batch*m*n == 0.
 * Returns an sgemm_status.
 */
int sgemm_strided_batched(int64_t batch, int64_t m, int64_t n, int64_t k,
                          float alpha,
                          const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                          const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                          int accumulate,
                          float *C, int64_t sC_batch, int64_t sC_row, int64_t sC_col,
                          void *stream);

/*
 * Same operation with the kernel family forced (for tests that must cover
 * every path on every shape).  A family that cannot serve the arguments
 * (e.g. MFMA for offsets beyond its 32-bit buffer range) is replaced by the
 * generic path, never refused.  Returns an sgemm_status.
 */
int sgemm_strided_batched_path(int64_t batch, int64_t m, int64_t n, int64_t k,
                               float alpha,
                               const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                               const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                               int accumulate,
                               float *C, int64_t sC_batch, int64_t sC_row, int64_t sC_col,
                               int path, void *stream);

/*
 * The product with a general epilogue (the matrix-and-bias fusion of
 * "PyTorch demystified 3", section "Comparison with cuBLAS and outlook", and
 * the per-row / per-column terms of distance tables, StaleyNET "GPU
 * Implementation", section "The matrix product"):
 *
 *     C[b,i,j] <- alpha * sum_{p<k} A[b,i,p] * B[b,p,j] + beta * C[b,i,j]
 *                 + row_add[b*sR_batch + i*sR_row] + col_add[b*sL_batch + j*sL_col]
 *
 * beta == 0 never reads C (it may hold NaN).  row_add / col_add are device
 * vectors owned by the caller; NULL drops the term (its strides are then
 * ignored).  A bias over output features is col_add with sL_batch = 0.
 * Strides are in elements, >= 0; the vectors must not overlap C
 * (SGEMM_ERR_C_ALIAS).  beta = 1 with no vectors is exactly
 * sgemm_strided_batched with accumulate = 1 (same bits), beta = 0 with no
 * vectors the plain product.  Other arguments, ownership, asynchrony and
 * determinism as for sgemm_strided_batched.  Returns an sgemm_status.
 */
int sgemm_strided_batched_ex(int64_t batch, int64_t m, int64_t n, int64_t k,
                             float alpha,
                             const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                             const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                             float beta,
                             float *C, int64_t sC_batch, int64_t sC_row, int64_t sC_col,
                             const float *row_add, int64_t sR_batch, int64_t sR_row,
                             const float *col_add, int64_t sL_batch, int64_t sL_col,
                             void *stream);

/* sgemm_strided_batched_ex with the kernel family forced (as for
 * sgemm_strided_batched_path).  Returns an sgemm_status. */
int sgemm_strided_batched_ex_path(int64_t batch, int64_t m, int64_t n, int64_t k,
                                  float alpha,
                                  const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                                  const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                                  float beta,
                                  float *C, int64_t sC_batch, int64_t sC_row, int64_t sC_col,
                                  const float *row_add, int64_t sR_batch, int64_t sR_row,
                                  const float *col_add, int64_t sL_batch, int64_t sL_col,
                                  int path, void *stream);

/*
 * The product over two batch levels, with a group divisor on the inner level
 * of each input (attention scores for every sequence and every head in one
 * launch, with several query heads sharing one key/value head: the rvllm
 * post, section "Matmuls go to cuBLAS"):
 *
 *     C[o,i] <- alpha * A[o, i/gA] @ B[o, i/gB]   (+ C[o,i] when accumulate)
 *
 * for o < nb_outer, i < nb_inner, where operand X[o,j] is the matrix whose
 * element (r,c) sits at X + o*sX_outer + j*sX_inner + r*sX_row + c*sX_col
 * (C's group is 1).  A [sequence][token][head][dim] buffer is addressed as is,
 * with no transposing copy: outer = sequence, inner = head, row = token.
 * Grouped key/value heads: gB = query heads per KV head (B's inner index is
 * i/gB).  A group >= nb_inner maps every inner entry to the first.  With
 * nb_inner = 1 this is sgemm_strided_batched with batch = nb_outer, and with
 * nb_outer = 1 it is sgemm_strided_batched over the inner level when both
 * groups are 1 (same bits in both cases).  nb_outer may be 0 (nothing is
 * enqueued); nb_inner, gA, gB must be >= 1 (SGEMM_ERR_INVALID_SIZE); strides
 * are in elements, >= 0 (SGEMM_ERR_INVALID_STRIDE); C must give every
 * (o, i, r, c) its own element and must not overlap A or B
 * (SGEMM_ERR_C_ALIAS).  Other arguments, ownership, asynchrony and
 * determinism as for sgemm_strided_batched.  Returns an sgemm_status.
 */
int sgemm_strided_batched2(int64_t nb_outer, int64_t nb_inner, int64_t m, int64_t n, int64_t k,
                           float alpha,
                           const float *A, int64_t sA_outer, int64_t sA_inner, int64_t gA,
                           int64_t sA_row, int64_t sA_col,
                           const float *B, int64_t sB_outer, int64_t sB_inner, int64_t gB,
                           int64_t sB_row, int64_t sB_col,
                           int accumulate,
                           float *C, int64_t sC_outer, int64_t sC_inner, int64_t sC_row, int64_t sC_col,
                           void *stream);

/* sgemm_strided_batched2 with the kernel family forced (as for
 * sgemm_strided_batched_path).  Returns an sgemm_status. */
int sgemm_strided_batched2_path(int64_t nb_outer, int64_t nb_inner, int64_t m, int64_t n, int64_t k,
                                float alpha,
                                const float *A, int64_t sA_outer, int64_t sA_inner, int64_t gA,
                                int64_t sA_row, int64_t sA_col,
                                const float *B, int64_t sB_outer, int64_t sB_inner, int64_t gB,
                                int64_t sB_row, int64_t sB_col,
                                int accumulate,
                                float *C, int64_t sC_outer, int64_t sC_inner, int64_t sC_row,
                                int64_t sC_col, int path, void *stream);

/*
 * The product of sgemm_strided_batched (same arguments, same operation,
 * C <- alpha * A * B (+ C)) with k split across workgroups, for products
 * whose output has too few tiles to occupy the GPU and whose k is long (a
 * weight gradient over many tokens, a small output over a deep
 * contraction): StaleyNET "GPU Implementation", section "The matrix
 * product", defines the operation; splitting the sum over k is a
 * regrouping of it.
 *
 * The call enqueues, on `stream`, the partial products of P consecutive k
 * partitions into `workspace` (partition q of batch entry b at
 * workspace + (b*P + q)*m*n, rows of n floats), then one kernel that adds
 * each output's partials in partition order and writes alpha * S (+ C_old).
 * The planner picks P (1 when splitting does not pay for the extra traffic
 * and launches; then this is exactly sgemm_strided_batched, same bits) among
 * the splits whose P*batch*m*n floats fit in workspace_floats; a smaller
 * workspace gives a smaller split or none, never an error.
 * sgemm_splitk_describe tells what a call would do and how much workspace
 * the best split needs.
 *
 * Numerics: fp32 throughout, partition order fixed, so repeated calls give
 * the same bits; they differ from the unsplit product's bits (the k sum is
 * grouped differently) within the same error bound.
 * workspace: caller-owned device memory, NULL only with workspace_floats ==
 * 0 (no split); it must not overlap A, B or C (SGEMM_ERR_C_ALIAS).  Its
 * contents on entry do not matter and are left overwritten.
 * Returns an sgemm_status: SGEMM_ERR_INVALID_SIZE if workspace_floats < 0,
 * SGEMM_ERR_NULL_POINTER if workspace is NULL with workspace_floats > 0,
 * otherwise as sgemm_strided_batched.
 */
int sgemm_strided_batched_splitk(int64_t batch, int64_t m, int64_t n, int64_t k,
                                 float alpha,
                                 const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                                 const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                                 int accumulate,
                                 float *C, int64_t sC_batch, int64_t sC_row, int64_t sC_col,
                                 float *workspace, int64_t workspace_floats,
                                 void *stream);

/*
 * Squared Euclidean norms of a batch of vectors, the terms a distance table
 * adds to its product:
 *
 *     out[b*sO_batch + i*sO_item] <- sum_{p<len} X[b*sX_batch + i*sX_item + p*sX_elem]^2
 *
 * for b < batch, i < count.  Rows of a matrix are (sX_item = row stride,
 * sX_elem = 1), its columns the same storage with the two exchanged.  Sums
 * are formed in fp32 in a fixed order (reproducible bits).  X and out are
 * device pointers owned by the caller and must not overlap.  Returns an
 * sgemm_status; count or batch == 0 enqueues nothing, len == 0 writes 0.
 */
int sgemm_sqnorms(int64_t batch, int64_t count, int64_t len,
                  const float *X, int64_t sX_batch, int64_t sX_item, int64_t sX_elem,
                  float *out, int64_t sO_batch, int64_t sO_item,
                  void *stream);

/*
 * Squared Euclidean distances between the rows of X [batch][m][k] and the
 * rows of Y [batch][n][k] (sY_batch = 0 shares one Y, e.g. a codebook):
 *
 *     D[b,i,j] <- sum_p (X[b,i,p] - Y[b,j,p])^2
 *
 * computed as |x_i|^2 + |y_j|^2 - 2 x_i . y_j: two sgemm_sqnorms launches
 * into `workspace` followed by one sgemm_strided_batched_ex launch (alpha =
 * -2, beta = 0, the norms as row_add / col_add), all on `stream`.  For
 * nearly equal vectors the result may be slightly negative by rounding.
 * workspace: caller-owned device memory of at least batch*m + nY*n floats,
 * nY = (sY_batch == 0 ? 1 : batch); it must not overlap X, Y or D.
 * Returns an sgemm_status (SGEMM_ERR_WORKSPACE if workspace is NULL or
 * smaller than that).
 */
int sgemm_pairwise_sqdist(int64_t batch, int64_t m, int64_t n, int64_t k,
                          const float *X, int64_t sX_batch, int64_t sX_row, int64_t sX_col,
                          const float *Y, int64_t sY_batch, int64_t sY_row, int64_t sY_col,
                          float *D, int64_t sD_batch, int64_t sD_row, int64_t sD_col,
                          float *workspace, int64_t workspace_floats,
                          void *stream);

/*
 * sgemm_pairwise_sqdist without a workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, result bits and status
 * codes as sgemm_pairwise_sqdist, except that the two norm vectors go to a
 * device array inside the library (one per GPU, SGEMM_SCRATCH_FLOATS floats,
 * 4 MiB, held from the library's load until the process ends), so no memory
 * is allocated or freed by the call.
 *
 * Limit: batch*m + nY*n <= SGEMM_SCRATCH_FLOATS (nY = 1 when sY_batch == 0,
 * else batch); a larger call returns SGEMM_ERR_WORKSPACE before anything is
 * enqueued, with the sizes in sgemm_last_error().  Every call on one GPU uses
 * that GPU's array and leaves its norms there: calls that overlap in time on
 * one GPU (different streams or host threads without ordering) race and
 * must be serialised by the caller.  Nothing in the array needs clearing
 * between calls (each call writes every norm it reads).
 */
#define SGEMM_SCRATCH_FLOATS (1 << 20)
int sgemm_pairwise_sqdist_noalloc(int64_t batch, int64_t m, int64_t n, int64_t k,
                                  const float *X, int64_t sX_batch, int64_t sX_row, int64_t sX_col,
                                  const float *Y, int64_t sY_batch, int64_t sY_row, int64_t sY_col,
                                  float *D, int64_t sD_batch, int64_t sD_row, int64_t sD_col,
                                  void *stream);

/* What the planner would launch (filled by sgemm_plan_describe). */
typedef struct sgemm_plan_info {
    int path;            /* sgemm_path actually used (never AUTO) */
    int transposed;      /* 1 if computed as C^T = B^T A^T (C column-major) */
    int tile_m, tile_n, tile_k;
    int waves;           /* wavefronts per workgroup */
    int vec_a, vec_b;    /* global load width in floats for A and B */
    int a_kfast, b_kfast;/* 1 if the operand's contiguous axis is k */
    int launches;        /* kernels enqueued (0 for an empty product) */
    int fixed_offsets;   /* LDS-tiled kernel: load offsets computed once, k bounded by the buffer size */
    int64_t workgroups;  /* workgroups of the main launch */
    char kernel[64];     /* kernel variant name */
} sgemm_plan_info;

/* What sgemm_strided_batched_splitk would launch (sgemm_splitk_describe). */
typedef struct sgemm_splitk_info {
    int splits;               /* k partitions (1: the unsplit product, no workspace used) */
    int launches;             /* kernels enqueued: 1 unsplit; 2 or 3 split (a shorter last partition adds one) */
    int64_t kc;               /* k of each partition but the last */
    int64_t k_last;           /* k of the last partition */
    int64_t workspace_floats; /* floats of workspace the plan writes (0 unsplit) */
    sgemm_plan_info parts;    /* the launch of the partial products (of the product when unsplit) */
} sgemm_splitk_info;

/*
 * Validates the arguments as sgemm_strided_batched_splitk does and fills
 * *info with its plan, without touching the device or dereferencing any
 * pointer.  workspace_floats < 0 asks what the best split needs (no cap;
 * workspace is then ignored): info->workspace_floats is the size to pass.
 * num_cus as for sgemm_plan_describe.  Returns an sgemm_status; *info is
 * filled only on SGEMM_OK.
 */
int sgemm_splitk_describe(int64_t batch, int64_t m, int64_t n, int64_t k,
                          float alpha,
                          const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                          const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                          int accumulate,
                          float *C, int64_t sC_batch, int64_t sC_row, int64_t sC_col,
                          const float *workspace, int64_t workspace_floats, int num_cus,
                          sgemm_splitk_info *info);

/*
 * Validates the arguments exactly as sgemm_strided_batched does and fills
 * *info with the plan, without touching the device or dereferencing any
 * pointer (pointer values are used for alignment only).  num_cus is the
 * compute-unit count to plan for (256 on MI355X); 0 asks the current device.
 * Returns an sgemm_status; *info is filled only on SGEMM_OK.
 */
int sgemm_plan_describe(int64_t batch, int64_t m, int64_t n, int64_t k,
                        float alpha,
                        const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                        const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                        int accumulate,
                        float *C, int64_t sC_batch, int64_t sC_row, int64_t sC_col,
                        int path, int num_cus, sgemm_plan_info *info);

/* sgemm_plan_describe for a sgemm_strided_batched2 call (same arguments,
 * validated the same way).  Returns an sgemm_status. */
int sgemm_plan_describe2(int64_t nb_outer, int64_t nb_inner, int64_t m, int64_t n, int64_t k,
                         float alpha,
                         const float *A, int64_t sA_outer, int64_t sA_inner, int64_t gA,
                         int64_t sA_row, int64_t sA_col,
                         const float *B, int64_t sB_outer, int64_t sB_inner, int64_t gB,
                         int64_t sB_row, int64_t sB_col,
                         int accumulate,
                         float *C, int64_t sC_outer, int64_t sC_inner, int64_t sC_row,
                         int64_t sC_col, int path, int num_cus, sgemm_plan_info *info);

/*
 * Fused scaled dot-product attention over two batch levels (the three-step
 * attention of the rvllm post, section "Matmuls go to cuBLAS": scores as a
 * strided batched product with the 1/sqrt(head_dim) scale in alpha, a
 * softmax, the probabilities times V; done in one pass so the scores never
 * reach memory, the fusion its section "What's basic about it" names):
 *
 *     O[o,i,q,:] = sum_j softmax_j(alpha * <Q[o,i,q,:], K[o,i/g,j,:]>) V[o,i/g,j,:]
 *
 * for o < nb_outer, i < nb_inner (e.g. sequence and query head), q < tq,
 * over the keys j < tk, or with causal != 0 over j <= q + tk - tq (the
 * queries are the last tq positions of the context: a prefill with tq = tk
 * sees j <= q, one decode query sees every key).  Each operand X is addressed
 * as X + o*sX_outer + h*sX_inner + row*sX_row + c*sX_col, where h = i for Q
 * and O and h = i/g for K and V (g query heads share a key/value head; a g
 * at least nb_inner maps every query head to the first).  Q and O are
 * tq x d, K and V are tk x d.  A [sequence][token][head][dim] buffer is read
 * as it is (row stride = heads*dim).
 *
 * Sizes: nb_outer, tq, tk, d >= 0, nb_inner and g >= 1
 * (SGEMM_ERR_INVALID_SIZE); tk = 0 with queries to answer, or causal with
 * tq > tk, is SGEMM_ERR_INVALID_SIZE (a query would see no key); d above 256
 * is SGEMM_ERR_UNSUPPORTED.  Strides in elements, >= 0.  O must give every
 * output its own element and must not overlap Q, K or V (SGEMM_ERR_C_ALIAS).
 * Pointers are device pointers owned by the caller; no workspace, nothing is
 * allocated.  Arithmetic is fp32 (matrix cores for d = 64 with unit column
 * strides and 16-byte aligned rows, a 64-bit generic kernel otherwise); the
 * order of every sum is fixed, so results are reproducible bit for bit.
 * Enqueued on `stream` without synchronising.  Returns an sgemm_status.
 */
int sgemm_attention(int64_t nb_outer, int64_t nb_inner, int64_t tq, int64_t tk, int64_t d,
                    float alpha, int causal,
                    const float *Q, int64_t sQ_outer, int64_t sQ_inner, int64_t sQ_row, int64_t sQ_col,
                    const float *K, int64_t sK_outer, int64_t sK_inner, int64_t g,
                    int64_t sK_row, int64_t sK_col,
                    const float *V, int64_t sV_outer, int64_t sV_inner, int64_t sV_row, int64_t sV_col,
                    float *O, int64_t sO_outer, int64_t sO_inner, int64_t sO_row, int64_t sO_col,
                    void *stream);

/* sgemm_attention with the kernel forced: SGEMM_PATH_AUTO, SGEMM_PATH_MFMA
 * (SGEMM_ERR_UNSUPPORTED if the matrix-core kernel cannot serve the call) or
 * SGEMM_PATH_GENERIC; SGEMM_PATH_WAVE is SGEMM_ERR_INVALID_PATH.  Returns an
 * sgemm_status. */
int sgemm_attention_path(int64_t nb_outer, int64_t nb_inner, int64_t tq, int64_t tk, int64_t d,
                         float alpha, int causal,
                         const float *Q, int64_t sQ_outer, int64_t sQ_inner, int64_t sQ_row,
                         int64_t sQ_col,
                         const float *K, int64_t sK_outer, int64_t sK_inner, int64_t g,
                         int64_t sK_row, int64_t sK_col,
                         const float *V, int64_t sV_outer, int64_t sV_inner, int64_t sV_row,
                         int64_t sV_col,
                         float *O, int64_t sO_outer, int64_t sO_inner, int64_t sO_row, int64_t sO_col,
                         int path, void *stream);

/*
 * sgemm_attention for decode-shaped calls (few queries per head, a long KV
 * cache), with the keys split across the GPU through a caller workspace.
 * Same arguments, operation and status codes as sgemm_attention, plus the
 * workspace.  The g query heads of a KV head and their tq queries are
 * stacked as the rows of 16-row matrix-core tiles (g * tq <= 64, up to four
 * tiles; the rvllm post, "Matmuls go to cuBLAS", stacks a group's query
 * heads as rows of one product), so K and V are read once per tile rather
 * than once per query head; the keys are cut into chunks, one wavefront per
 * (outer, KV head, row tile, chunk) forms that chunk's
 * online softmax (unnormalised output rows, reference maxima, weight sums:
 * kael book ch. 09 and the rvllm post's softmax in three steps, done in one
 * pass) into `workspace`, and a second launch merges each output row's
 * chunks in chunk order: O = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c,
 * M = max_c m_c.  Results are reproducible bit for bit; they differ from
 * sgemm_attention's (the keys' sum is grouped by chunk) within the same
 * bound.
 * Chunks are whole 32-key blocks; their count is the one that keeps the
 * busiest CU's work least (its workgroups times their blocks, plus a small
 * merge cost per chunk) among the counts giving every CU a workgroup, capped
 * by the workspace.
 * Serves head dimension 64, unit column strides and 16-byte aligned rows
 * with g * tq <= 64 (g capped at nb_inner); any other call, or a workspace
 * too small for one chunk per (outer, KV head, row tile), runs as
 * sgemm_attention.
 * workspace: caller-owned device memory of workspace_floats floats, NULL
 * only with workspace_floats == 0, not overlapping Q, K, V or O
 * (SGEMM_ERR_C_ALIAS); sgemm_attention_splitkv_describe gives the size.
 * Returns an sgemm_status.
 */
int sgemm_attention_splitkv(int64_t nb_outer, int64_t nb_inner, int64_t tq, int64_t tk, int64_t d,
                            float alpha, int causal,
                            const float *Q, int64_t sQ_outer, int64_t sQ_inner, int64_t sQ_row, int64_t sQ_col,
                            const float *K, int64_t sK_outer, int64_t sK_inner, int64_t g,
                            int64_t sK_row, int64_t sK_col,
                            const float *V, int64_t sV_outer, int64_t sV_inner, int64_t sV_row, int64_t sV_col,
                            float *O, int64_t sO_outer, int64_t sO_inner, int64_t sO_row, int64_t sO_col,
                            float *workspace, int64_t workspace_floats,
                            void *stream);

/*
 * The split sgemm_attention_splitkv would make with a workspace of
 * workspace_floats floats (< 0: no cap, a size query): *chunks key chunks
 * per (outer, KV head) of *chunk_keys keys, *floats_used floats of
 * workspace (0 and 0: not split).  Validates like sgemm_attention; touches
 * no device when num_cus > 0.  Returns an sgemm_status.
 */
int sgemm_attention_splitkv_describe(int64_t nb_outer, int64_t nb_inner, int64_t tq, int64_t tk, int64_t d,
                                     float alpha, int causal,
                                     const float *Q, int64_t sQ_outer, int64_t sQ_inner, int64_t sQ_row,
                                     int64_t sQ_col,
                                     const float *K, int64_t sK_outer, int64_t sK_inner, int64_t g,
                                     int64_t sK_row, int64_t sK_col,
                                     const float *V, int64_t sV_outer, int64_t sV_inner, int64_t sV_row,
                                     int64_t sV_col,
                                     float *O, int64_t sO_outer, int64_t sO_inner, int64_t sO_row, int64_t sO_col,
                                     int64_t workspace_floats, int num_cus,
                                     int64_t *chunks, int64_t *chunk_keys, int64_t *floats_used);

/* The plan of a sgemm_attention_path call (validated the same way, no
 * device access): tile_m = query rows per workgroup.  Returns an
 * sgemm_status. */
int sgemm_attention_describe(int64_t nb_outer, int64_t nb_inner, int64_t tq, int64_t tk, int64_t d,
                             float alpha, int causal,
                             const float *Q, int64_t sQ_outer, int64_t sQ_inner, int64_t sQ_row,
                             int64_t sQ_col,
                             const float *K, int64_t sK_outer, int64_t sK_inner, int64_t g,
                             int64_t sK_row, int64_t sK_col,
                             const float *V, int64_t sV_outer, int64_t sV_inner, int64_t sV_row,
                             int64_t sV_col,
                             float *O, int64_t sO_outer, int64_t sO_inner, int64_t sO_row,
                             int64_t sO_col, int path, sgemm_plan_info *info);

/* Static description of a status code (never NULL; an unknown code gets a
 * generic text).  The checks behind the codes are those of StaleyNET "GPU
 * Implementation", section "Safety" (sizes checked before every launch). */
const char *sgemm_status_string(int status);

/* Detail of the last non-OK status returned on the calling thread ("" if
 * none): which argument failed which check, or the HIP runtime's message for
 * SGEMM_ERR_HIP.  Valid until the next call on the same thread.  It never
 * reports a fault inside a kernel that already started: such faults surface
 * at the caller's next synchronising runtime call (kael book ch. 09 "CUDA
 * backend", section "Edge cases and pitfalls", asynchronous errors). */
const char *sgemm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_STRIDED_H */
