/*
 * ref_sgemm.c -- CPU oracle for the strided, batched fp32 matrix product.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load it.  It shares no code, header or
 * constant with the HIP path.
 *
 * What it computes (StaleyNET "GPU Implementation", section "The matrix
 * product", the displayed formula and the paragraph after it): for a batch
 * of matrix pairs, C <- alpha * A * B, optionally plus the C already stored.
 * Every operand is addressed through its own strides, so a transposed input
 * is the same memory read with the row and column strides exchanged, and the
 * batch index selects the pair.  The plain-mode output is overwritten, not
 * added to (kael book ch. 09 "CUDA backend", section "Matmul": the device
 * tile is written with '=').
 *
 * Readings taken where the pages are silent:
 *   - strides are counted in float elements and are signed 64-bit values;
 *   - "optionally plus C" means C_new = C_old + alpha * (A*B): alpha scales
 *     only the fresh product;
 *   - k = 0 is the empty sum, so C <- alpha*0 (+ C_old);
 *   - arithmetic is literal IEEE: alpha = 0 does not skip the product, NaN
 *     propagates.
 *
 * Precision: each product of two fp32 values is exact in fp64 (24+24 < 53
 * significand bits), the products are summed in fp64 in ascending p, then
 * alpha is applied and C_old added in fp64, and the result is rounded to
 * fp32 once.  Every output element is computed on its own, so the order in
 * which elements are visited cannot change any bit.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Address of element (b, r, c) of an operand described by (base, strides). */
static inline int64_t elem_offset(int64_t b, int64_t r, int64_t c,
                                  int64_t s_batch, int64_t s_row, int64_t s_col)
{
    return b * s_batch + r * s_row + c * s_col;
}

/* One output element, straight from the definition. */
static float one_element(int64_t b, int64_t i, int64_t j, int64_t k, float alpha,
                         const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                         const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                         int accumulate, float c_old)
{
    double sum = 0.0;
    for (int64_t p = 0; p < k; ++p) {
        double a = (double)A[elem_offset(b, i, p, sA_batch, sA_row, sA_col)];
        double bv = (double)B[elem_offset(b, p, j, sB_batch, sB_row, sB_col)];
        sum += a * bv;
    }
    double out = (double)alpha * sum;
    if (accumulate)
        out += (double)c_old;
    return (float)out;
}

/*
 * Full product.  Same argument order and meaning as the library entry point,
 * with host pointers.  `reverse` visits the (b, i, j) elements last-to-first
 * (the order-independence check of kael's host emulation); it must not change
 * any bit.  Returns 0, or -1 for a negative size.
 */
int oracle_sgemm(int64_t batch, int64_t m, int64_t n, int64_t k, float alpha,
                 const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                 const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                 int accumulate,
                 float *C, int64_t sC_batch, int64_t sC_row, int64_t sC_col,
                 int reverse)
{
    if (batch < 0 || m < 0 || n < 0 || k < 0)
        return -1;
    int64_t rows = batch * m;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < rows; ++t) {
        int64_t row = reverse ? rows - 1 - t : t;
        int64_t b = row / m, i = row % m;
        for (int64_t jj = 0; jj < n; ++jj) {
            int64_t j = reverse ? n - 1 - jj : jj;
            float *c = C + elem_offset(b, i, j, sC_batch, sC_row, sC_col);
            float c_old = accumulate ? *c : 0.0f;
            *c = one_element(b, i, j, k, alpha, A, sA_batch, sA_row, sA_col,
                             B, sB_batch, sB_row, sB_col, accumulate, c_old);
        }
    }
    return 0;
}

/*
 * Selected elements only: for each q < count, (b, i, j) = idx[3q .. 3q+2],
 * out[q] receives what oracle_sgemm would store at C[b, i, j].  C_old is read
 * from C when accumulating; C is never written.  This is how outputs of
 * products too large for the full oracle are checked one by one.
 * Returns 0, or -1 for an index outside [0,batch) x [0,m) x [0,n).
 */
int oracle_sgemm_entries(int64_t batch, int64_t m, int64_t n, int64_t k, float alpha,
                         const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                         const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                         int accumulate,
                         const float *C, int64_t sC_batch, int64_t sC_row, int64_t sC_col,
                         int64_t count, const int64_t *idx, float *out)
{
    for (int64_t q = 0; q < count; ++q) {
        int64_t b = idx[3 * q], i = idx[3 * q + 1], j = idx[3 * q + 2];
        if (b < 0 || b >= batch || i < 0 || i >= m || j < 0 || j >= n)
            return -1;
    }
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t q = 0; q < count; ++q) {
        int64_t b = idx[3 * q], i = idx[3 * q + 1], j = idx[3 * q + 2];
        float c_old = accumulate ? C[elem_offset(b, i, j, sC_batch, sC_row, sC_col)] : 0.0f;
        out[q] = one_element(b, i, j, k, alpha, A, sA_batch, sA_row, sA_col,
                             B, sB_batch, sB_row, sB_col, accumulate, c_old);
    }
    return 0;
}

/* Number of OpenMP threads a parallel region of this library will use. */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
