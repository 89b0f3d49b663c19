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
 * The general epilogue (any beta, a per-row and a per-column term) and the
 * squared norms and distances follow the same rules: every term is formed in
 * fp64 and the element is rounded to fp32 once.  So does attention (scores,
 * softmax and the product with V, all in fp64, exp from the C library).
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared ... -lm (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Address of element (b, r, c) of an operand described by (base, strides). */
static inline int64_t elem_offset(int64_t b, int64_t r, int64_t c,
                                  int64_t s_batch, int64_t s_row, int64_t s_col)
{
    return b * s_batch + r * s_row + c * s_col;
}

/* sum_p A[b,i,p] * B[b,p,j] in fp64, ascending p (the products of two fp32
 * values are exact in fp64). */
static double dot_fp64(int64_t b, int64_t i, int64_t j, int64_t k,
                       const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                       const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col)
{
    double sum = 0.0;
    for (int64_t p = 0; p < k; ++p) {
        double a = (double)A[elem_offset(b, i, p, sA_batch, sA_row, sA_col)];
        double bv = (double)B[elem_offset(b, p, j, sB_batch, sB_row, sB_col)];
        sum += a * bv;
    }
    return sum;
}

/*
 * One output element, straight from the definition, with the epilogue in its
 * general form:
 *
 *   C[b,i,j] <- alpha * sum_p A[b,i,p] B[b,p,j] + beta * C_old[b,i,j]
 *               + row_add[b,i] + col_add[b,j]
 *
 * "Optionally plus C" is beta = 1, the plain product beta = 0.  The general
 * beta and the two vector terms serve the matrix-and-bias fusion of "PyTorch
 * demystified 3" ("Comparison with cuBLAS and outlook": a feed-forward layer's
 * product and its bias add in one kernel) and the tokenizer distances that
 * StaleyNET ("The matrix product") routes through the product.  beta == 0
 * drops the C_old term without reading it (the stored C may hold anything,
 * NaN included); a NULL row_add or col_add drops its term.  The vectors are
 * addressed as row_add[b*sR_batch + i*sR_row] and col_add[b*sL_batch +
 * j*sL_col].
 */
static float one_element(int64_t b, int64_t i, int64_t j, int64_t k, float alpha,
                         const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                         const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                         float beta, const float *c_old,
                         const float *row_add, int64_t sR_batch, int64_t sR_row,
                         const float *col_add, int64_t sL_batch, int64_t sL_col)
{
    double total = dot_fp64(b, i, j, k, A, sA_batch, sA_row, sA_col, B, sB_batch, sB_row, sB_col);
    double out = (double)alpha * total;
    if (beta != 0.0f)
        out += (double)beta * (double)*c_old;
    if (row_add)
        out += (double)row_add[b * sR_batch + i * sR_row];
    if (col_add)
        out += (double)col_add[b * sL_batch + j * sL_col];
    return (float)out;
}

/*
 * Full product with the general epilogue, host pointers.  `reverse` visits
 * the (b, i, j) elements last-to-first (the order-independence check of
 * kael's host emulation); it must not change any bit.  Returns 0, or -1 for a
 * negative size.
 */
int oracle_sgemm_ex(int64_t batch, int64_t m, int64_t n, int64_t k, float alpha,
                    const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                    const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                    float beta,
                    float *C, int64_t sC_batch, int64_t sC_row, int64_t sC_col,
                    const float *row_add, int64_t sR_batch, int64_t sR_row,
                    const float *col_add, int64_t sL_batch, int64_t sL_col,
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
            *c = one_element(b, i, j, k, alpha, A, sA_batch, sA_row, sA_col, B, sB_batch, sB_row,
                             sB_col, beta, c, row_add, sR_batch, sR_row, col_add, sL_batch, sL_col);
        }
    }
    return 0;
}

/*
 * Selected elements only: for each q < count, (b, i, j) = idx[3q .. 3q+2],
 * out[q] receives what oracle_sgemm_ex would store at C[b, i, j].  C is only
 * read (as C_old, and only when beta != 0), never written.  This is how
 * outputs of products too large for the full oracle are checked one by one.
 * Returns 0, or -1 for an index outside [0,batch) x [0,m) x [0,n).
 */
int oracle_sgemm_ex_entries(int64_t batch, int64_t m, int64_t n, int64_t k, float alpha,
                            const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                            const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                            float beta,
                            const float *C, int64_t sC_batch, int64_t sC_row, int64_t sC_col,
                            const float *row_add, int64_t sR_batch, int64_t sR_row,
                            const float *col_add, int64_t sL_batch, int64_t sL_col,
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
        out[q] = one_element(b, i, j, k, alpha, A, sA_batch, sA_row, sA_col, B, sB_batch, sB_row,
                             sB_col, beta, C + elem_offset(b, i, j, sC_batch, sC_row, sC_col),
                             row_add, sR_batch, sR_row, col_add, sL_batch, sL_col);
    }
    return 0;
}

/* "Optionally plus C" as a flag: beta = 1 when accumulating, else 0. */
static float accumulate_beta(int accumulate) { return accumulate ? 1.0f : 0.0f; }

/* The product of the pages, C <- alpha*A*B (+ C): same argument order and
 * meaning as the library entry point.  Returns 0, or -1 for a negative size. */
int oracle_sgemm(int64_t batch, int64_t m, int64_t n, int64_t k, float alpha,
                 const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                 const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                 int accumulate,
                 float *C, int64_t sC_batch, int64_t sC_row, int64_t sC_col,
                 int reverse)
{
    return oracle_sgemm_ex(batch, m, n, k, alpha, A, sA_batch, sA_row, sA_col, B, sB_batch, sB_row,
                           sB_col, accumulate_beta(accumulate), C, sC_batch, sC_row, sC_col,
                           NULL, 0, 0, NULL, 0, 0, reverse);
}

/* Selected elements of oracle_sgemm (see oracle_sgemm_ex_entries). */
int oracle_sgemm_entries(int64_t batch, int64_t m, int64_t n, int64_t k, float alpha,
                         const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                         const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                         int accumulate,
                         const float *C, int64_t sC_batch, int64_t sC_row, int64_t sC_col,
                         int64_t count, const int64_t *idx, float *out)
{
    return oracle_sgemm_ex_entries(batch, m, n, k, alpha, A, sA_batch, sA_row, sA_col, B, sB_batch,
                                   sB_row, sB_col, accumulate_beta(accumulate), C, sC_batch, sC_row,
                                   sC_col, NULL, 0, 0, NULL, 0, 0, count, idx, out);
}

/*
 * Two batch levels (outer o < nb_outer, inner i < nb_inner) with a group
 * divisor on the inner level of each input:
 *
 *   C[o,i,r,c] <- alpha * sum_p A[o, i/gA, r, p] * B[o, i/gB, p, c]  (+ C_old)
 *
 * with X[o, j, r, c] at o*sX_outer + j*sX_inner + r*sX_row + c*sX_col.  This
 * addresses attention over a [sequence][token][head][dim] buffer directly
 * (outer = sequence, inner = head) and grouped KV heads (gB = query heads per
 * KV head): the rvllm post ("Matmuls go to cuBLAS") transposes such buffers
 * with a copy kernel first and folds the query heads of a group into the
 * rows.  Each (o, i) is one product of the definition above, formed by the
 * same element function.  Returns 0, or -1 for a negative size or a group
 * below 1.
 */
int oracle_sgemm_batched2(int64_t nb_outer, int64_t nb_inner, int64_t m, int64_t n, int64_t k,
                          float alpha,
                          const float *A, int64_t sA_outer, int64_t sA_inner, int64_t gA,
                          int64_t sA_row, int64_t sA_col,
                          const float *B, int64_t sB_outer, int64_t sB_inner, int64_t gB,
                          int64_t sB_row, int64_t sB_col,
                          int accumulate,
                          float *C, int64_t sC_outer, int64_t sC_inner, int64_t sC_row, int64_t sC_col)
{
    if (nb_outer < 0 || nb_inner < 0 || m < 0 || n < 0 || k < 0 || gA < 1 || gB < 1)
        return -1;
    for (int64_t o = 0; o < nb_outer; ++o)
        for (int64_t i = 0; i < nb_inner; ++i) {
            const float *Ab = A + o * sA_outer + (i / gA) * sA_inner;
            const float *Bb = B + o * sB_outer + (i / gB) * sB_inner;
            float *Cb = C + o * sC_outer + i * sC_inner;
            oracle_sgemm_ex(1, m, n, k, alpha, Ab, 0, sA_row, sA_col, Bb, 0, sB_row, sB_col,
                            accumulate_beta(accumulate), Cb, 0, sC_row, sC_col, NULL, 0, 0, NULL, 0, 0, 0);
        }
    return 0;
}

/*
 * Scaled dot-product attention over two batch levels, one query row at a
 * time, in the three steps the rvllm post uses (sections "Matmuls go to
 * cuBLAS" and "The kernels"): scores s_j = alpha * <Q[q,:], K[j,:]> (the
 * 1/sqrt(head_dim) scale rides in alpha), a softmax over the visible keys
 * taken as max, then the sum of exp(s_j - max), then the division, and the
 * probabilities times V.  With `causal`, query q of tq sees keys
 * j <= q + (tk - tq): the queries are the last tq positions of a context of
 * tk (a prefill with tq = tk sees j <= q; one decode query sees every key);
 * this is the attention mask the post adds before its softmax.
 *
 *   O[o,i,q,c] = sum_j softmax_j(s)[j] * V[o, i/g, j, c]
 *
 * Q[o,i] and O[o,i] are tq x d, K[o, i/g] is tk x d and V[o, i/g] tk x d,
 * each addressed by (outer, inner, row, col) strides; g query heads share
 * one key/value head.  Every step runs in fp64 (exp of fp64 arguments) and
 * O is rounded to fp32 once.  Returns 0, or -1 for a negative size, a group
 * below 1, tk = 0 with queries to answer, or causal with tq > tk (a query
 * that would see no key).
 */
int oracle_attention(int64_t nb_outer, int64_t nb_inner, int64_t tq, int64_t tk, int64_t d,
                     float alpha, int causal,
                     const float *Q, int64_t sQ_outer, int64_t sQ_inner, int64_t sQ_row, int64_t sQ_col,
                     const float *K, int64_t sK_outer, int64_t sK_inner, int64_t g,
                     int64_t sK_row, int64_t sK_col,
                     const float *V, int64_t sV_outer, int64_t sV_inner, int64_t sV_row, int64_t sV_col,
                     float *O, int64_t sO_outer, int64_t sO_inner, int64_t sO_row, int64_t sO_col)
{
    if (nb_outer < 0 || nb_inner < 0 || tq < 0 || tk < 0 || d < 0 || g < 1)
        return -1;
    const int64_t rows = nb_outer * nb_inner * tq;
    if (rows == 0)
        return 0;
    if (tk == 0 || (causal && tq > tk))
        return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t w = 0; w < rows; ++w) {
        const int64_t o = w / (nb_inner * tq), i = (w / tq) % nb_inner, q = w % tq;
        const float *Qr = Q + o * sQ_outer + i * sQ_inner + q * sQ_row;
        const float *Kb = K + o * sK_outer + (i / g) * sK_inner;
        const float *Vb = V + o * sV_outer + (i / g) * sV_inner;
        float *Or = O + o * sO_outer + i * sO_inner + q * sO_row;
        const int64_t seen = causal ? q + (tk - tq) + 1 : tk;   /* keys 0 .. seen-1 */
        double *s = (double *)malloc((size_t)seen * sizeof(double));
        if (!s) {
#pragma omp atomic write
            bad = 1;
            continue;
        }
        for (int64_t j = 0; j < seen; ++j) {
            double dot = 0.0;
            for (int64_t p = 0; p < d; ++p)
                dot += (double)Qr[p * sQ_col] * (double)Kb[j * sK_row + p * sK_col];
            s[j] = (double)alpha * dot;
        }
        double mx = s[0];
        for (int64_t j = 1; j < seen; ++j)
            if (s[j] > mx) mx = s[j];
        double z = 0.0;
        for (int64_t j = 0; j < seen; ++j) {
            s[j] = exp(s[j] - mx);
            z += s[j];
        }
        for (int64_t j = 0; j < seen; ++j)
            s[j] /= z;
        for (int64_t c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int64_t j = 0; j < seen; ++j)
                acc += s[j] * (double)Vb[j * sV_row + c * sV_col];
            Or[c * sO_col] = (float)acc;
        }
        free(s);
    }
    return bad ? -1 : 0;
}

/*
 * Squared Euclidean norms of a batch of vectors: out[b,i] = sum_p X[b,i,p]^2,
 * with X[b,i,p] at b*sX_batch + i*sX_item + p*sX_elem and out[b,i] at
 * b*sO_batch + i*sO_item.  Returns 0, or -1 for a negative size.
 */
int oracle_sqnorms(int64_t batch, int64_t count, int64_t len,
                   const float *X, int64_t sX_batch, int64_t sX_item, int64_t sX_elem,
                   float *out, int64_t sO_batch, int64_t sO_item)
{
    if (batch < 0 || count < 0 || len < 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < batch * count; ++t) {
        int64_t bb = t / count, item = t % count;
        double sq = 0.0;
        for (int64_t e = 0; e < len; ++e) {
            double x = (double)X[bb * sX_batch + item * sX_item + e * sX_elem];
            sq += x * x;
        }
        out[bb * sO_batch + item * sO_item] = (float)sq;
    }
    return 0;
}

/*
 * Squared Euclidean distances between the rows of X [batch][m][k] and the
 * rows of Y [batch][n][k], straight from the definition:
 * D[b,i,j] = sum_p (X[b,i,p] - Y[b,j,p])^2 (differences and squares in fp64).
 * The tokenizer distances of StaleyNET ("The matrix product") are such a
 * table of vectors against codebook entries.  With idx == NULL the whole
 * table is written to D (strides sD_*); otherwise out[q] receives the
 * element (b, i, j) = idx[3q .. 3q+2] and D is not touched.
 * Returns 0, -1 for a negative size, -2 for an index outside the table.
 */
int oracle_sqdist(int64_t batch, int64_t m, int64_t n, int64_t k,
                  const float *X, int64_t sX_batch, int64_t sX_row, int64_t sX_col,
                  const float *Y, int64_t sY_batch, int64_t sY_row, int64_t sY_col,
                  float *D, int64_t sD_batch, int64_t sD_row, int64_t sD_col,
                  int64_t count, const int64_t *idx, float *out)
{
    if (batch < 0 || m < 0 || n < 0 || k < 0)
        return -1;
    if (idx)
        for (int64_t q = 0; q < count; ++q)
            if (idx[3 * q] < 0 || idx[3 * q] >= batch || idx[3 * q + 1] < 0 || idx[3 * q + 1] >= m ||
                idx[3 * q + 2] < 0 || idx[3 * q + 2] >= n)
                return -2;
    int64_t total = idx ? count : batch * m * n;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t q = 0; q < total; ++q) {
        int64_t bq = idx ? idx[3 * q] : q / (m * n);
        int64_t iq = idx ? idx[3 * q + 1] : (q / n) % m;
        int64_t jq = idx ? idx[3 * q + 2] : q % n;
        double d = 0.0;
        for (int64_t e = 0; e < k; ++e) {
            double diff = (double)X[bq * sX_batch + iq * sX_row + e * sX_col] -
                          (double)Y[bq * sY_batch + jq * sY_row + e * sY_col];
            d += diff * diff;
        }
        if (idx)
            out[q] = (float)d;
        else
            D[bq * sD_batch + iq * sD_row + jq * sD_col] = (float)d;
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
