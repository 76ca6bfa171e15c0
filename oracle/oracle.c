/*
 * CPU oracle for the CSR SpMM / SDDMM hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the bench's CPU-baseline leg may load this library.  The product path never
 * calls it and shares no code, header, table or helper with it.
 *
 * Source of what is computed: the summary card of "Sparse GPU Kernels for Deep
 * Learning" (Gale, Zaharia, Young, Elsen; SC 2020):
 *   - "Summary": SpMM and SDDMM kernels that work on plain CSR with unstructured
 *     sparsity, and a load-balancing scheme decoupled from the kernels;
 *   - "Interesting ideas", I3: the SDDMM form drops the element-wise scaling and
 *     takes its second operand transposed;
 *   - "Interesting ideas", I4: "row swizzle" reorders rows for balance,
 *     independently of how the work is split;
 *   - "Interesting ideas", I5: the format is standard CSR with no structural
 *     constraint.
 * The card prints no formula, so every routine here is the textbook definition
 * of its operation written out as plain loops.  Readings where the card is
 * silent (swizzle direction and tie order, overwrite rather than accumulate,
 * int32 indices) are stated at each function.
 *
 * Arithmetic: every floating-point result is accumulated in double from fp32
 * inputs.  A product of two fp32 values is exact in double, so the only error
 * of an oracle result is the double summation (and one final rounding where an
 * fp32 result is returned).  Single-threaded, no SIMD intrinsics, and built
 * without -ffast-math and with FP contraction off.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* CSR structure                                                            */
/* ------------------------------------------------------------------------ */

/* Number of set entries of a dense row-major m x k byte mask (nonzero byte =
 * structural nonzero).  Summary card, "Summary" / I5: the structure is plain
 * CSR, so nnz is the count of structural positions. */
long long orc_mask_nnz(int m, int k, const uint8_t *mask)
{
    long long count = 0;
    for (long long i = 0; i < (long long)m * k; ++i)
        if (mask[i] != 0)
            ++count;
    return count;
}

/* Standard CSR of a dense mask: rows ascending, columns ascending inside a row,
 * one entry per set mask position.  row_offsets[i] is the number of set
 * positions in rows 0..i-1.  If dense_values is non-NULL, values[p] takes the
 * dense value at the position of entry p (an explicit zero value stays an
 * entry: the structure comes from the mask alone).  I5: standard CSR. */
void orc_csr_from_dense(int m, int k, const uint8_t *mask,
                        const float *dense_values, int32_t *row_offsets,
                        int32_t *col_indices, float *values)
{
    int32_t p = 0;
    for (int i = 0; i < m; ++i) {
        row_offsets[i] = p;
        for (int j = 0; j < k; ++j) {
            long long at = (long long)i * k + j;
            if (mask[at] != 0) {
                col_indices[p] = j;
                if (dense_values != NULL && values != NULL)
                    values[p] = dense_values[at];
                ++p;
            }
        }
    }
    row_offsets[m] = p;
}

/* Row offsets of a CSR matrix whose rows have the given lengths: the exclusive
 * prefix sum, row_offsets[0] = 0 and row_offsets[i+1] = row_offsets[i] +
 * lengths[i].  Standard CSR (I5). */
void orc_csr_offsets_from_lengths(int m, const int32_t *lengths,
                                  int32_t *row_offsets)
{
    row_offsets[0] = 0;
    for (int i = 0; i < m; ++i)
        row_offsets[i + 1] = row_offsets[i] + lengths[i];
}

/* Validity of a CSR structure for an m x k matrix with nnz entries:
 *   0  valid: offsets start at 0, never decrease, end at nnz, and every row's
 *      columns lie in [0, k) and strictly increase;
 *   1  row_offsets[0] != 0;   2  offsets decrease;   3  row_offsets[m] != nnz;
 *   4  a column outside [0, k);   5  columns not strictly increasing in a row. */
int orc_csr_check(int m, int k, long long nnz, const int32_t *row_offsets,
                  const int32_t *col_indices)
{
    if (row_offsets[0] != 0)
        return 1;
    for (int i = 0; i < m; ++i)
        if (row_offsets[i + 1] < row_offsets[i])
            return 2;
    if ((long long)row_offsets[m] != nnz)
        return 3;
    for (int i = 0; i < m; ++i) {
        for (int32_t p = row_offsets[i]; p < row_offsets[i + 1]; ++p) {
            if (col_indices[p] < 0 || col_indices[p] >= k)
                return 4;
            if (p > row_offsets[i] && col_indices[p] <= col_indices[p - 1])
                return 5;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* 16-bit operand formats (mixed precision: 16-bit storage, products and     */
/* sums in wider arithmetic)                                                 */
/* ------------------------------------------------------------------------ */

/* Value of an IEEE 754 binary16 bit pattern: sign bit 15, exponent bits 14-10
 * (bias 15), fraction bits 9-0.  Exponent 0 encodes zero and the subnormals
 * f * 2^-24; exponent 31 encodes infinity (f = 0) or NaN; otherwise the value
 * is (1024 + f) * 2^(e - 25). */
double orc_f16_value(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int e = (bits >> 10) & 0x1f;
    int f = bits & 0x3ff;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -24);
    else if (e == 31)
        mag = f == 0 ? INFINITY : NAN;
    else
        mag = ldexp((double)(1024 + f), e - 25);
    return sign ? -mag : mag;
}

/* Value of a bfloat16 bit pattern (the upper half of a binary32): sign bit
 * 15, exponent bits 14-7 (bias 127), fraction bits 6-0.  Exponent 0: f *
 * 2^-133 (zero and subnormals); 255: infinity or NaN; otherwise
 * (128 + f) * 2^(e - 134). */
double orc_bf16_value(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int e = (bits >> 7) & 0xff;
    int f = bits & 0x7f;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -133);
    else if (e == 255)
        mag = f == 0 ? INFINITY : NAN;
    else
        mag = ldexp((double)(128 + f), e - 134);
    return sign ? -mag : mag;
}

/* out[i] = value of bits[i]; kind 1 = binary16, 2 = bfloat16. */
void orc_decode16(int kind, long long count, const uint16_t *bits, double *out)
{
    for (long long i = 0; i < count; ++i)
        out[i] = kind == 1 ? orc_f16_value(bits[i]) : orc_bf16_value(bits[i]);
}

/* ------------------------------------------------------------------------ */
/* Row swizzle                                                              */
/* ------------------------------------------------------------------------ */

struct orc_row_key {
    int32_t length;
    int32_t row;
};

static int orc_row_key_order(const void *pa, const void *pb)
{
    const struct orc_row_key *a = (const struct orc_row_key *)pa;
    const struct orc_row_key *b = (const struct orc_row_key *)pb;
    if (a->length != b->length)
        return a->length > b->length ? -1 : 1; /* longer rows first */
    return a->row < b->row ? -1 : (a->row > b->row ? 1 : 0);
}

/* Row swizzle (I4): the order in which rows are handed to workers, by nonzero
 * count.  Reading taken where the card is silent: longest row first, and rows
 * of equal length in ascending row index, so the order is unique.
 * row_indices[r] is the row handled r-th.  The keys (length, row) are
 * distinct, so the library sort's own tie behaviour never matters. */
void orc_row_swizzle(int m, const int32_t *row_offsets, int32_t *row_indices)
{
    struct orc_row_key *keys =
        (struct orc_row_key *)malloc(sizeof(struct orc_row_key) * (size_t)(m > 0 ? m : 1));
    for (int i = 0; i < m; ++i) {
        keys[i].length = row_offsets[i + 1] - row_offsets[i];
        keys[i].row = i;
    }
    qsort(keys, (size_t)m, sizeof(struct orc_row_key), orc_row_key_order);
    for (int r = 0; r < m; ++r)
        row_indices[r] = keys[r].row;
    free(keys);
}

/* ------------------------------------------------------------------------ */
/* SpMM                                                                     */
/* ------------------------------------------------------------------------ */

/* One output row of C = A * B (see orc_spmm). */
static void orc_spmm_one_row(int i, int n, const int32_t *row_offsets,
                             const int32_t *col_indices, const float *values,
                             const float *b, double *c_row, double *abs_row)
{
    for (int j = 0; j < n; ++j) {
        c_row[j] = 0.0;
        abs_row[j] = 0.0;
    }
    for (int32_t p = row_offsets[i]; p < row_offsets[i + 1]; ++p) {
        double a = (double)values[p];
        const float *b_row = b + (long long)col_indices[p] * n;
        for (int j = 0; j < n; ++j) {
            double term = a * (double)b_row[j];
            c_row[j] += term;
            abs_row[j] += fabs(term);
        }
    }
}

/* SpMM ("Summary"): C = A * B with A (m x k) in CSR and B (k x n) dense,
 *   C[i][j] = sum over entries p of row i of values[p] * B[col_indices[p]][j],
 * summed with p ascending.  B and C are dense row-major; C is overwritten
 * (reading: the card speaks of the product only, not of accumulation into C).
 * c receives the sum in double; abs_sum receives sum |values[p] * B[..][j]|,
 * the scale the fp32 error tolerance is stated against.  k only bounds the
 * column indices. */
void orc_spmm(int m, int k, int n, const int32_t *row_offsets,
              const int32_t *col_indices, const float *values, const float *b,
              double *c, double *abs_sum)
{
    (void)k;
    for (int i = 0; i < m; ++i)
        orc_spmm_one_row(i, n, row_offsets, col_indices, values, b,
                         c + (long long)i * n, abs_sum + (long long)i * n);
}

/* orc_spmm restricted to the listed rows: output row r is row rows[r] of C.
 * Used to check sampled rows of products too large to recompute whole. */
void orc_spmm_rows(int nrows, const int32_t *rows, int n,
                   const int32_t *row_offsets, const int32_t *col_indices,
                   const float *values, const float *b, double *c_rows,
                   double *abs_rows)
{
    for (int r = 0; r < nrows; ++r)
        orc_spmm_one_row(rows[r], n, row_offsets, col_indices, values, b,
                         c_rows + (long long)r * n, abs_rows + (long long)r * n);
}

/* ------------------------------------------------------------------------ */
/* Transpose and the transposed product (the backward pass of a sparse      */
/* layer: the card's "Summary" speaks of training, and the input gradient   */
/* of C = A B is dB = A^T dC)                                               */
/* ------------------------------------------------------------------------ */

/* CSR of A^T (k x m) from the CSR of A (m x k): row j of A^T lists the rows i
 * of A that hold an entry in column j, ascending, each with that entry's
 * value -- so the result is again standard CSR.  A counting sort by column:
 * count the entries of each column, take the exclusive prefix sum as the row
 * offsets of A^T, then visit A's entries in order (rows ascending) and append
 * each to its column's list.  t_perm[q] (if non-NULL) is the index in A's
 * arrays of the entry that became entry q of A^T; t_values may be NULL. */
void orc_csr_transpose(int m, int k, const int32_t *row_offsets,
                       const int32_t *col_indices, const float *values,
                       int32_t *t_row_offsets, int32_t *t_col_indices,
                       float *t_values, int32_t *t_perm)
{
    int32_t *next = (int32_t *)malloc(sizeof(int32_t) * (size_t)(k > 0 ? k : 1));
    for (int j = 0; j <= k; ++j)
        t_row_offsets[j] = 0;
    for (int32_t p = 0; p < row_offsets[m]; ++p)
        t_row_offsets[col_indices[p] + 1] += 1;
    for (int j = 0; j < k; ++j)
        t_row_offsets[j + 1] += t_row_offsets[j];
    for (int j = 0; j < k; ++j)
        next[j] = t_row_offsets[j];
    for (int i = 0; i < m; ++i) {
        for (int32_t p = row_offsets[i]; p < row_offsets[i + 1]; ++p) {
            int32_t q = next[col_indices[p]]++;
            t_col_indices[q] = i;
            if (t_values != NULL)
                t_values[q] = values[p];
            if (t_perm != NULL)
                t_perm[q] = p;
        }
    }
    free(next);
}

/* dX = A^T dY for A (m x k) in CSR and dY (m x n) dense: dX is k x n with
 *   dX[j][l] = sum over entries p = (i, j) of A, rows i ascending, of
 *              values[p] * dY[i][l],
 * written from A's own structure without forming A^T (each entry adds its
 * product to the row of dX named by its column).  abs_sum is the matching sum
 * of |values[p] * dY[i][l]|.  dX is overwritten. */
void orc_spmm_transposed(int m, int k, int n, const int32_t *row_offsets,
                         const int32_t *col_indices, const float *values,
                         const float *dy, double *dx, double *abs_sum)
{
    for (long long e = 0; e < (long long)k * n; ++e) {
        dx[e] = 0.0;
        abs_sum[e] = 0.0;
    }
    for (int i = 0; i < m; ++i) {
        for (int32_t p = row_offsets[i]; p < row_offsets[i + 1]; ++p) {
            double a = (double)values[p];
            double *dx_row = dx + (long long)col_indices[p] * n;
            double *abs_row = abs_sum + (long long)col_indices[p] * n;
            for (int l = 0; l < n; ++l) {
                double term = a * (double)dy[(long long)i * n + l];
                dx_row[l] += term;
                abs_row[l] += fabs(term);
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* SDDMM                                                                    */
/* ------------------------------------------------------------------------ */

/* SDDMM in the specialised form of I3: the dense product X * Y^T evaluated only
 * at the mask's entries, with no scaling by the mask's values, and the second
 * operand given transposed, i.e. Y stored k x d row-major:
 *   out[p] = sum over l < d of X[i][l] * Y[col_indices[p]][l]   (p in row i),
 * summed with l ascending.  X is m x d row-major.  out is overwritten and
 * abs_sum[p] = sum over l of |X[i][l] * Y[col][l]|. */
void orc_sddmm(int m, int k, int d, const int32_t *row_offsets,
               const int32_t *col_indices, const float *x, const float *y,
               double *out, double *abs_sum)
{
    (void)k;
    for (int i = 0; i < m; ++i) {
        const float *x_row = x + (long long)i * d;
        for (int32_t p = row_offsets[i]; p < row_offsets[i + 1]; ++p) {
            const float *y_row = y + (long long)col_indices[p] * d;
            double acc = 0.0, mag = 0.0;
            for (int l = 0; l < d; ++l) {
                double term = (double)x_row[l] * (double)y_row[l];
                acc += term;
                mag += fabs(term);
            }
            out[p] = acc;
            abs_sum[p] = mag;
        }
    }
}

/* General SDDMM: the form I3 says is easy to add back -- scaling by the
 * mask's values, either layout of the second operand, and accumulation:
 *   out[p] = alpha * v_p * sum over l < d of X[i][l] * Yop(col_indices[p], l)
 *            + beta * out_in[p]
 * for each entry p of row i, where v_p = mask_values[p] (1 when mask_values is
 * NULL) and Yop(c, l) = Y[c][l] with Y stored k x d (y_layout 0) or Y[l][c]
 * with Y stored d x k (y_layout 1).  With beta == 0, out_in is not read.
 * abs_sum[p] = |alpha * v_p| * sum |X[i][l] * Yop(c, l)| + |beta * out_in[p]|,
 * the scale of the fp32 tolerance.  Double arithmetic throughout. */
void orc_sddmm_general(int m, int k, int d, const int32_t *row_offsets,
                       const int32_t *col_indices, const float *mask_values,
                       const float *x, const float *y, int y_layout, double alpha,
                       double beta, const float *out_in, double *out, double *abs_sum)
{
    for (int i = 0; i < m; ++i) {
        for (int32_t p = row_offsets[i]; p < row_offsets[i + 1]; ++p) {
            const int c = col_indices[p];
            double acc = 0.0, mag = 0.0;
            for (int l = 0; l < d; ++l) {
                double yv = y_layout == 0 ? (double)y[(long long)c * d + l]
                                          : (double)y[(long long)l * k + c];
                double term = (double)x[(long long)i * d + l] * yv;
                acc += term;
                mag += fabs(term);
            }
            double scale = alpha * (mask_values != NULL ? (double)mask_values[p] : 1.0);
            double prior = beta != 0.0 ? beta * (double)out_in[p] : 0.0;
            out[p] = scale * acc + prior;
            abs_sum[p] = fabs(scale) * mag + fabs(prior);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Row softmax over CSR entries (the step between SDDMM and SpMM in sparse   */
/* attention, I3)                                                            */
/* ------------------------------------------------------------------------ */

/* For each row i with entries p in [row_offsets[i], row_offsets[i+1]):
 *   mx = max_p s[p];  e_p = exp(s[p] - mx);  p_out[p] = e_p / sum_q e_q.
 * Computed in double.  An empty row produces nothing.  Subtracting the row
 * maximum changes nothing mathematically and keeps exp() in range. */
void orc_softmax_rows(int m, const int32_t *row_offsets, const float *s,
                      double *p_out)
{
    for (int i = 0; i < m; ++i) {
        int32_t p0 = row_offsets[i], p1 = row_offsets[i + 1];
        if (p1 <= p0)
            continue;
        double mx = (double)s[p0];
        for (int32_t p = p0 + 1; p < p1; ++p)
            if ((double)s[p] > mx)
                mx = (double)s[p];
        double total = 0.0;
        for (int32_t p = p0; p < p1; ++p) {
            p_out[p] = exp((double)s[p] - mx);
            total += p_out[p];
        }
        for (int32_t p = p0; p < p1; ++p)
            p_out[p] /= total;
    }
}
