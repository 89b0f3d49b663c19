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
 * per-call state and never frees caller memory.  It may be called from
 * several host threads on different streams.
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
 */
#ifndef SGEMM_STRIDED_H
#define SGEMM_STRIDED_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Every non-zero status leaves C untouched and enqueues
 * nothing, except SGEMM_ERR_HIP, which reports a failed launch. */
enum sgemm_status {
    SGEMM_OK = 0,
    SGEMM_ERR_INVALID_SIZE = -1,   /* batch, m, n or k < 0 */
    SGEMM_ERR_INVALID_STRIDE = -2, /* a stride < 0 */
    SGEMM_ERR_NULL_POINTER = -3,   /* C null with batch*m*n > 0, or A/B null with k > 0 as well */
    SGEMM_ERR_C_ALIAS = -4,        /* C's strides map two outputs to one address, or C overlaps A or B */
    SGEMM_ERR_UNSUPPORTED = -5,    /* an extent times its stride overflows int64, or no kernel fits */
    SGEMM_ERR_HIP = -6,            /* the HIP runtime rejected a query or launch; see sgemm_last_error() */
    SGEMM_ERR_INVALID_PATH = -7    /* unknown path code */
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

/* What the planner would launch (filled by sgemm_plan_describe). */
typedef struct sgemm_plan_info {
    int path;            /* sgemm_path actually used (never AUTO) */
    int transposed;      /* 1 if computed as C^T = B^T A^T (C column-major) */
    int tile_m, tile_n, tile_k;
    int waves;           /* wavefronts per workgroup */
    int vec_a, vec_b;    /* global load width in floats for A and B */
    int a_kfast, b_kfast;/* 1 if the operand's contiguous axis is k */
    int launches;        /* kernels enqueued (0 for an empty product) */
    int64_t workgroups;  /* workgroups of the main launch */
    char kernel[64];     /* kernel variant name */
} sgemm_plan_info;

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

/* Static description of a status code (never NULL). */
const char *sgemm_status_string(int status);

/* Detail of the last non-OK status returned on the calling thread ("" if
 * none).  Valid until the next call on the same thread. */
const char *sgemm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_STRIDED_H */
