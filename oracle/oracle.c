/*
 * CPU oracle for sparse matrix-vector multiply-accumulate, y <- A*x + y.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file.  No product code path calls
 * it, and it shares no code, header or table with the GPU library.
 *
 * Plain single-threaded C.  Each function restates its definition from the
 * source pages:
 *   [P1] PMPP notes ch.14, "Sparse Matrices and Basic Formats (COO & CSR)"
 *   [P2] PMPP notes ch.14, "Regularized Formats (ELL, Hybrid ELL-COO, JDS)"
 *   [P3] "SpMV storage-format choice and performance comparison" (CUDA tuning
 *        article), numbered sections
 *   [P5] SpGEMM/AIA article, section 5.3 "common problems" (input checks)
 *   [INTRO] "Introduction to sparse computing and locating performance
 *        bottlenecks" article, sections on the three core challenges and on
 *        building the overall picture (irregular x gathers, memory and
 *        parallel efficiency)
 *
 * Arithmetic: products of two fp32 numbers are exact in fp64 (24+24 < 53
 * significand bits); sums are taken in fp64 in row order.  Values are moved by
 * the builders as raw 32-bit patterns, never re-rounded.
 *
 * Readings of points the pages leave open (each listed in the design notes):
 *   - SpMV accumulates (y += A x), as the P1 background and kernels define it.
 *   - ELL padding: value +0.0f (bit pattern 0), column index 0.
 *   - HYB tail: entries past position K of each row, rows in order, positions
 *     in order; ELL part of width min(K, W).
 *   - JDS: rows sorted by length, longest first, ties by ascending original row.
 *   - Sectioned ELL: sections of S consecutive sorted rows (the last one may be
 *     shorter), each padded to its own longest row, column-major inside the
 *     section.
 *   - The selector's comparison operators (lost from P3 4.3) are restored as
 *     W*R <= 2*nnz -> ELL; nnz < 10*R -> COO; W*R > 5*nnz -> HYB; else CSR,
 *     with the HYB width/budget extension described at orc_select().
 *   - ELL with x tiles, blocked COO and the automatic build's storage rules
 *     are encodings and build-time rules, not formulas of the pages: each is
 *     written out as a definition at orc_csr_to_ell_xtile(), orc_coo_blocked(),
 *     orc_bc_chunk_entries(), orc_bc_block_rows() and orc_select_build().
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Status numbers: the same values the library documents for its C ABI. */
enum {
    ORC_OK = 0,
    ORC_ERR_INVALID_ARG = 1,
    ORC_ERR_BAD_ROWPTRS = 2,
    ORC_ERR_BAD_COLIDX = 3,
    ORC_ERR_BAD_ROWIDX = 4,
    ORC_ERR_TOO_LARGE = 5,
};

/* Format numbers for the selector's answer (same values as the C ABI). */
enum {
    ORC_FMT_COO_ATOMIC = 1,
    ORC_FMT_COO_SEGMENTED = 2,
    ORC_FMT_CSR_SCALAR = 3,
    ORC_FMT_CSR_VECTOR = 4,
    ORC_FMT_ELL = 5,
    ORC_FMT_HYB = 6,
    ORC_FMT_JDS = 7,
    ORC_FMT_CSR_MERGE = 8,
    ORC_FMT_SELL = 9,
};

#define ORC_INT32_MAX 2147483647LL

/* ------------------------------------------------------------------------ */
/* Input checks [P1 CSR section: rowPtrs[numRows] = nnz; P5 5.3: row_ptr    */
/* monotone, every column index below the column count, value length = nnz] */
/* ------------------------------------------------------------------------ */

int orc_validate_csr(int64_t R, int64_t C, int64_t nnz, const int32_t *row_ptrs,
                     const int32_t *col_idx)
{
    if (R < 0 || C < 0 || nnz < 0 || R > ORC_INT32_MAX || C > ORC_INT32_MAX ||
        nnz > ORC_INT32_MAX || row_ptrs == NULL || (nnz > 0 && col_idx == NULL))
        return ORC_ERR_INVALID_ARG;
    if (row_ptrs[0] != 0)
        return ORC_ERR_BAD_ROWPTRS;
    for (int64_t r = 0; r < R; ++r)
        if (row_ptrs[r + 1] < row_ptrs[r])
            return ORC_ERR_BAD_ROWPTRS;
    if ((int64_t)row_ptrs[R] != nnz)
        return ORC_ERR_BAD_ROWPTRS;
    for (int64_t i = 0; i < nnz; ++i)
        if (col_idx[i] < 0 || (int64_t)col_idx[i] >= C)
            return ORC_ERR_BAD_COLIDX;
    return ORC_OK;
}

int orc_validate_coo(int64_t R, int64_t C, int64_t nnz, const int32_t *row_idx,
                     const int32_t *col_idx)
{
    if (R < 0 || C < 0 || nnz < 0 || R > ORC_INT32_MAX || C > ORC_INT32_MAX ||
        nnz > ORC_INT32_MAX || (nnz > 0 && (row_idx == NULL || col_idx == NULL)))
        return ORC_ERR_INVALID_ARG;
    for (int64_t i = 0; i < nnz; ++i)
        if (row_idx[i] < 0 || (int64_t)row_idx[i] >= R)
            return ORC_ERR_BAD_ROWIDX;
    for (int64_t i = 0; i < nnz; ++i)
        if (col_idx[i] < 0 || (int64_t)col_idx[i] >= C)
            return ORC_ERR_BAD_COLIDX;
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* SpMV by definition [P1 background: SpMV computes A*X + Y; P1 CSR section:*/
/* row r holds value/colIdx[rowPtrs[r] .. rowPtrs[r+1]-1]]                  */
/*                                                                          */
/*   y_ref[r] = y[r] + sum_i value[i] * x[colIdx[i]]                        */
/*   bound[r] = |y[r]| + sum_i |value[i] * x[colIdx[i]]|                    */
/* ------------------------------------------------------------------------ */

void orc_spmv_csr(int64_t R, const int32_t *row_ptrs, const int32_t *col_idx,
                  const float *values, const float *x, const float *y_in,
                  double *y_ref, double *bound)
{
    for (int64_t r = 0; r < R; ++r) {
        double s = (double)y_in[r];
        double b = fabs((double)y_in[r]);
        for (int64_t i = row_ptrs[r]; i < row_ptrs[r + 1]; ++i) {
            double p = (double)values[i] * (double)x[col_idx[i]];
            s += p;
            b += fabs(p);
        }
        y_ref[r] = s;
        if (bound)
            bound[r] = b;
    }
}

/* The same definition over COO triples (no grouping needed): used to check
 * that COO input and its CSR conversion describe the same matrix. */
void orc_spmv_coo(int64_t R, int64_t nnz, const int32_t *row_idx, const int32_t *col_idx,
                  const float *values, const float *x, const float *y_in,
                  double *y_ref, double *bound)
{
    for (int64_t r = 0; r < R; ++r) {
        y_ref[r] = (double)y_in[r];
        if (bound)
            bound[r] = fabs((double)y_in[r]);
    }
    for (int64_t i = 0; i < nnz; ++i) {
        double p = (double)values[i] * (double)x[col_idx[i]];
        y_ref[row_idx[i]] += p;
        if (bound)
            bound[row_idx[i]] += fabs(p);
    }
}

/* Row-wise acceptance test: |y_gpu - y_ref| <= rtol * bound, and y_gpu finite
 * wherever y_ref is.  Where y_ref is not finite, y_gpu must not be finite
 * either (and an infinity must carry the same sign).  Returns the number of
 * failing rows; *first_bad is the first such row (or -1); *worst is the
 * largest |y_gpu - y_ref| / bound over rows with a nonzero bound. */
int64_t orc_check(int64_t R, const float *y_gpu, const double *y_ref, const double *bound,
                  double rtol, int64_t *first_bad, double *worst)
{
    int64_t bad = 0;
    double w = 0.0;
    if (first_bad)
        *first_bad = -1;
    for (int64_t r = 0; r < R; ++r) {
        double g = (double)y_gpu[r];
        double ref = y_ref[r];
        int ok;
        if (isfinite(ref)) {
            double err = fabs(g - ref);
            ok = isfinite(g) && err <= rtol * bound[r];
            if (bound[r] > 0.0 && isfinite(g) && err / bound[r] > w)
                w = err / bound[r];
        } else if (isnan(ref)) {
            ok = isnan(g);
        } else {
            ok = isinf(g) && (signbit(g) == signbit(ref));
        }
        if (!ok) {
            if (bad == 0 && first_bad)
                *first_bad = r;
            ++bad;
        }
    }
    if (worst)
        *worst = w;
    return bad;
}

/* ------------------------------------------------------------------------ */
/* COO -> CSR [P1 COO section: one (row, col, value) per nonzero; P1 CSR    */
/* section: nonzeros grouped by row, rowPtrs[r] = offset of row r's first   */
/* nonzero, rowPtrs[numRows] = nnz].  Count per row, prefix sum of the      */
/* counts, then place entries in input order, so each row keeps the order   */
/* its entries had in the COO input.                                        */
/* ------------------------------------------------------------------------ */

int orc_coo_to_csr(int64_t R, int64_t nnz, const int32_t *row_idx, const int32_t *col_idx,
                   const uint32_t *values, int32_t *row_ptrs, int32_t *csr_col,
                   uint32_t *csr_val)
{
    int64_t *next = (int64_t *)calloc((size_t)R + 1, sizeof(int64_t));
    if (!next)
        return ORC_ERR_INVALID_ARG;
    for (int64_t i = 0; i < nnz; ++i)
        next[row_idx[i] + 1] += 1;                      /* counts, shifted by one */
    for (int64_t r = 0; r < R; ++r)
        next[r + 1] += next[r];                         /* running total */
    for (int64_t r = 0; r <= R; ++r)
        row_ptrs[r] = (int32_t)next[r];
    for (int64_t i = 0; i < nnz; ++i) {
        int64_t p = next[row_idx[i]]++;
        csr_col[p] = col_idx[i];
        csr_val[p] = values[i];
    }
    free(next);
    return ORC_OK;
}

/* CSR -> COO: the row index of every nonzero. */
void orc_csr_to_coo(int64_t R, const int32_t *row_ptrs, int32_t *row_idx)
{
    for (int64_t r = 0; r < R; ++r)
        for (int64_t i = row_ptrs[r]; i < row_ptrs[r + 1]; ++i)
            row_idx[i] = (int32_t)r;
}

/* ------------------------------------------------------------------------ */
/* Row-length statistics [P3 4.1: nonzero-per-row histogram and row-length  */
/* variance; P3 4.3: mean and max row length; "Introduction to sparse       */
/* computing", parallel-efficiency check: max/mean of the work per worker]. */
/* out[0] = W (max length), out[1] = sum len, out[2] = sum len^2,           */
/* out[3] = number of empty rows.                                           */
/* ------------------------------------------------------------------------ */

void orc_row_stats(int64_t R, const int32_t *row_ptrs, int64_t *out)
{
    int64_t W = 0, s1 = 0, s2 = 0, empty = 0;
    for (int64_t r = 0; r < R; ++r) {
        int64_t len = (int64_t)row_ptrs[r + 1] - row_ptrs[r];
        if (len > W)
            W = len;
        s1 += len;
        s2 += len * len;
        if (len == 0)
            ++empty;
    }
    out[0] = W;
    out[1] = s1;
    out[2] = s2;
    out[3] = empty;
}

/* hist[l] = number of rows of length l, l = 0..W. */
void orc_len_hist(int64_t R, const int32_t *row_ptrs, int64_t W, int64_t *hist)
{
    for (int64_t l = 0; l <= W; ++l)
        hist[l] = 0;
    for (int64_t r = 0; r < R; ++r)
        hist[row_ptrs[r + 1] - row_ptrs[r]] += 1;
}

/* ------------------------------------------------------------------------ */
/* ELL [P2 ELL section]: (1) pad every row with zeros to the longest row's  */
/* length W (column indices padded as well), (2) store the padded R x W     */
/* array column-major, so slot t of row r sits at i = t*R + r.  nnzPerRow   */
/* keeps each row's true length.  Refused when R*W exceeds int32 range.     */
/*                                                                          */
/* HYB [P2 hybrid ELL-COO section]: before building the ELL part, the       */
/* entries of a row beyond position K go to a separate COO list; the ELL    */
/* part then has width min(K, W).  This builder with K >= W is plain ELL.   */
/* ------------------------------------------------------------------------ */

int64_t orc_hyb_tail_count(int64_t R, const int32_t *row_ptrs, int64_t K)
{
    int64_t n = 0;
    for (int64_t r = 0; r < R; ++r) {
        int64_t len = (int64_t)row_ptrs[r + 1] - row_ptrs[r];
        if (len > K)
            n += len - K;
    }
    return n;
}

int orc_csr_to_hyb(int64_t R, const int32_t *row_ptrs, const int32_t *col_idx,
                   const uint32_t *values, int64_t Kw, int32_t *ell_col, uint32_t *ell_val,
                   int32_t *ell_nnz, int32_t *tail_row, int32_t *tail_col, uint32_t *tail_val)
{
    if (Kw < 0)
        return ORC_ERR_INVALID_ARG;
    if (R * Kw > ORC_INT32_MAX)
        return ORC_ERR_TOO_LARGE;
    /* padded slots: value +0.0f, column 0 */
    for (int64_t i = 0; i < R * Kw; ++i) {
        ell_col[i] = 0;
        ell_val[i] = 0u;
    }
    int64_t tail = 0;
    for (int64_t r = 0; r < R; ++r) {
        int64_t start = row_ptrs[r];
        int64_t len = (int64_t)row_ptrs[r + 1] - start;
        int64_t in_ell = len < Kw ? len : Kw;
        for (int64_t t = 0; t < in_ell; ++t) {
            ell_col[t * R + r] = col_idx[start + t];
            ell_val[t * R + r] = values[start + t];
        }
        ell_nnz[r] = (int32_t)in_ell;
        for (int64_t t = in_ell; t < len; ++t) {
            tail_row[tail] = (int32_t)r;
            tail_col[tail] = col_idx[start + t];
            tail_val[tail] = values[start + t];
            ++tail;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* JDS [P2 JDS section]: (1) group by row, (2) sort rows by nonzero count,  */
/* longest first, recording each sorted row's original index, (3) store the */
/* sorted rows column-major without padding, (4) iterPtr[t] marks where     */
/* iteration (jagged column) t starts.  Entry t of sorted row s lives at    */
/* iterPtr[t] + s; iterPtr[W] = nnz.                                        */
/* ------------------------------------------------------------------------ */

static const int32_t *g_sort_len;

static int orc_cmp_len_desc(const void *a, const void *b)
{
    int32_t ra = *(const int32_t *)a, rb = *(const int32_t *)b;
    int32_t la = g_sort_len[ra], lb = g_sort_len[rb];
    if (la != lb)
        return la > lb ? -1 : 1;     /* longer rows first */
    return ra < rb ? -1 : (ra > rb); /* equal lengths keep original order */
}

int orc_csr_to_jds(int64_t R, const int32_t *row_ptrs, const int32_t *col_idx,
                   const uint32_t *values, int64_t W, int32_t *perm, int32_t *jds_len,
                   int32_t *iter_ptr, int32_t *jds_col, uint32_t *jds_val)
{
    int32_t *len = (int32_t *)malloc(((size_t)R + 1) * sizeof(int32_t));
    if (!len)
        return ORC_ERR_INVALID_ARG;
    for (int64_t r = 0; r < R; ++r) {
        len[r] = row_ptrs[r + 1] - row_ptrs[r];
        perm[r] = (int32_t)r;
    }
    g_sort_len = len;
    qsort(perm, (size_t)R, sizeof(int32_t), orc_cmp_len_desc);
    for (int64_t s = 0; s < R; ++s)
        jds_len[s] = len[perm[s]];
    /* iteration t holds one entry for every sorted row longer than t */
    iter_ptr[0] = 0;
    for (int64_t t = 0; t < W; ++t) {
        int64_t rows = 0;
        for (int64_t s = 0; s < R && jds_len[s] > t; ++s)
            ++rows;
        iter_ptr[t + 1] = iter_ptr[t] + (int32_t)rows;
    }
    for (int64_t s = 0; s < R; ++s) {
        int64_t start = row_ptrs[perm[s]];
        for (int64_t t = 0; t < jds_len[s]; ++t) {
            jds_col[iter_ptr[t] + s] = col_idx[start + t];
            jds_val[iter_ptr[t] + s] = values[start + t];
        }
    }
    free(len);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Format selector [P3 4.3, automatic selection by mean and max row length; */
/* P3 4.1: HYB with ELL width 20 for rows mostly 10-20 long; P3 5.2: power- */
/* law graphs -> merge-based CSR; P3 2.2: one vector group per row].        */
/*                                                                          */
/* With mean = nnz/R, comparisons kept exact in integers:                   */
/*   W*R <= 2*nnz            -> ELL                                         */
/*   nnz <  10*R             -> COO (segmented)                             */
/*   W*R >  5*nnz            -> HYB with K = smallest k such that at least  */
/*                              99% of rows have length <= k, taken only    */
/*                              if R*K <= 1.5*nnz, else merge-based CSR     */
/*   otherwise               -> CSR vector, lanes = smallest power of two   */
/*                              >= ceil(mean), clamped to [2, 64]           */
/* A padded choice whose slot count W*R (ELL) or R*K (HYB) exceeds the      */
/* int32 index range is not taken: ELL falls through to the later rules,    */
/* HYB becomes merge-based CSR.                                             */
/* hyb_width > 0 replaces the percentile K; lanes > 0 replaces the lane     */
/* rule.  hist has W+1 entries.  out[0]=format, out[1]=K (0 if not HYB),    */
/* out[2]=lanes (0 if not CSR vector).                                      */
/* ------------------------------------------------------------------------ */

int64_t orc_hyb_width(int64_t R, int64_t W, const int64_t *hist)
{
    /* smallest k with 100 * #{len <= k} >= 99 * R */
    int64_t cum = 0;
    for (int64_t k = 0; k <= W; ++k) {
        cum += hist[k];
        if (100 * cum >= 99 * R)
            return k;
    }
    return W;
}

int64_t orc_vector_lanes(int64_t R, int64_t nnz)
{
    int64_t mean_ceil = R > 0 ? (nnz + R - 1) / R : 0;
    int64_t L = 2;
    while (L < mean_ceil && L < 64)
        L *= 2;
    return L;
}

void orc_select(int64_t R, int64_t nnz, int64_t W, const int64_t *hist, int64_t hyb_width,
                int64_t lanes, int64_t *out)
{
    out[0] = ORC_FMT_ELL;
    out[1] = 0;
    out[2] = 0;
    if (W * R <= 2 * nnz && W * R <= ORC_INT32_MAX)
        return;                                   /* ELL */
    if (nnz < 10 * R) {
        out[0] = ORC_FMT_COO_SEGMENTED;
        return;
    }
    if (W * R > 5 * nnz) {
        int64_t K = hyb_width > 0 ? hyb_width : orc_hyb_width(R, W, hist);
        if (2 * R * K <= 3 * nnz && R * K <= ORC_INT32_MAX) {   /* R*K <= 1.5*nnz */
            out[0] = ORC_FMT_HYB;
            out[1] = K;
        } else {
            out[0] = ORC_FMT_CSR_MERGE;
        }
        return;
    }
    out[0] = ORC_FMT_CSR_VECTOR;
    out[2] = lanes > 0 ? lanes : orc_vector_lanes(R, nnz);
}

/* ------------------------------------------------------------------------ */
/* Sectioned ELL, the JDS variant [REG, JDS variant section]: after the JDS */
/* sort, cut the sorted rows into sections; each section is an ELL padded   */
/* only to the longest row of that section; section pointers replace        */
/* iterPtr.  Section k holds sorted rows [k*S, k*S + m_k), m_k = min(S,     */
/* R - k*S), width w_k = its longest row; entry t of its row i sits at      */
/* sect_ptr[k] + t*m_k + i; padding is (column 0, +0.0f).                   */
/* perm and sell_len are the JDS ones.  Returns ORC_ERR_TOO_LARGE when the  */
/* padded total exceeds int32.                                              */
/* ------------------------------------------------------------------------ */

int64_t orc_sell_slots(int64_t R, const int32_t *row_ptrs, int64_t S)
{
    /* padded slots = sum over sections of m_k * (longest row in section) */
    int32_t *len = (int32_t *)malloc(((size_t)R + 1) * sizeof(int32_t));
    int32_t *perm = (int32_t *)malloc(((size_t)R + 1) * sizeof(int32_t));
    int64_t total = 0;
    for (int64_t r = 0; r < R; ++r) {
        len[r] = row_ptrs[r + 1] - row_ptrs[r];
        perm[r] = (int32_t)r;
    }
    g_sort_len = len;
    qsort(perm, (size_t)R, sizeof(int32_t), orc_cmp_len_desc);
    for (int64_t k0 = 0; k0 < R; k0 += S) {
        int64_t m = R - k0 < S ? R - k0 : S;
        total += m * (int64_t)len[perm[k0]];
    }
    free(len);
    free(perm);
    return total;
}

int orc_csr_to_sell(int64_t R, const int32_t *row_ptrs, const int32_t *col_idx,
                    const uint32_t *values, int64_t S, int32_t *perm, int32_t *sell_len,
                    int32_t *sect_ptr, int32_t *sell_col, uint32_t *sell_val)
{
    if (S <= 0)
        return ORC_ERR_INVALID_ARG;
    int32_t *len = (int32_t *)malloc(((size_t)R + 1) * sizeof(int32_t));
    if (!len)
        return ORC_ERR_INVALID_ARG;
    for (int64_t r = 0; r < R; ++r) {
        len[r] = row_ptrs[r + 1] - row_ptrs[r];
        perm[r] = (int32_t)r;
    }
    g_sort_len = len;
    qsort(perm, (size_t)R, sizeof(int32_t), orc_cmp_len_desc);
    for (int64_t s = 0; s < R; ++s)
        sell_len[s] = len[perm[s]];
    int64_t nsect = (R + S - 1) / S;
    int64_t off = 0;
    for (int64_t k = 0; k < nsect; ++k) {
        int64_t first = k * S;
        int64_t m = R - first < S ? R - first : S;
        int64_t w = sell_len[first];            /* longest row of the section */
        if (off > ORC_INT32_MAX) {
            free(len);
            return ORC_ERR_TOO_LARGE;
        }
        sect_ptr[k] = (int32_t)off;
        for (int64_t t = 0; t < w; ++t) {
            for (int64_t i = 0; i < m; ++i) {
                int64_t slot = off + t * m + i;
                int64_t s = first + i;
                if (t < sell_len[s]) {
                    int64_t src = row_ptrs[perm[s]] + t;
                    sell_col[slot] = col_idx[src];
                    sell_val[slot] = values[src];
                } else {
                    sell_col[slot] = 0;
                    sell_val[slot] = 0u;
                }
            }
        }
        off += m * w;
    }
    if (off > ORC_INT32_MAX) {
        free(len);
        return ORC_ERR_TOO_LARGE;
    }
    sect_ptr[nsect] = (int32_t)off;
    free(len);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Conjugate gradient [P1 background: for positive-definite A the iterative  */
/* method guesses X, evaluates A*X + Y, tests how close it is to zero and    */
/* corrects X along the gradient].  The system here is A x = b (Y = -b), and */
/* the correction is the conjugate-gradient one of Hestenes and Stiefel:     */
/*                                                                          */
/*   r = b - A x;  p = r                                                    */
/*   repeat:  stop if ||r|| <= rtol * ||b||  (or max_iter steps done)        */
/*            alpha = (r.r) / (p.Ap);  x = x + alpha p;  r = r - alpha Ap    */
/*            beta  = (r'.r') / (r.r); p = r' + beta p                       */
/*                                                                          */
/* Everything in fp64 (the fp32 values widened).  alpha is 0 when p.Ap = 0   */
/* and beta is 0 when r.r = 0, so an exactly solved system stays put.        */
/* out[0] = iterations run, out[1] = ||r|| / ||b|| (||r|| when b = 0).       */
/* ------------------------------------------------------------------------ */

static void orc_csr_apply(int64_t R, const int32_t *row_ptrs, const int32_t *col_idx,
                          const float *values, const double *v, double *out)
{
    for (int64_t r = 0; r < R; ++r) {
        double s = 0.0;
        for (int64_t i = row_ptrs[r]; i < row_ptrs[r + 1]; ++i)
            s += (double)values[i] * v[col_idx[i]];
        out[r] = s;
    }
}

static double orc_dot(int64_t n, const double *a, const double *b)
{
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i)
        s += a[i] * b[i];
    return s;
}

int orc_cg(int64_t R, const int32_t *row_ptrs, const int32_t *col_idx, const float *values,
           const double *b, double *x, int64_t max_iter, double rtol, double *out)
{
    double *r = (double *)malloc(sizeof(double) * (size_t)(R > 0 ? R : 1));
    double *p = (double *)malloc(sizeof(double) * (size_t)(R > 0 ? R : 1));
    double *ap = (double *)malloc(sizeof(double) * (size_t)(R > 0 ? R : 1));
    if (!r || !p || !ap) {
        free(r); free(p); free(ap);
        return ORC_ERR_INVALID_ARG;
    }
    orc_csr_apply(R, row_ptrs, col_idx, values, x, ap);
    for (int64_t i = 0; i < R; ++i) {
        r[i] = b[i] - ap[i];
        p[i] = r[i];
    }
    const double bnorm = sqrt(orc_dot(R, b, b));
    const double target = rtol * (bnorm > 0.0 ? bnorm : 1.0);
    double rr = orc_dot(R, r, r);
    int64_t k = 0;
    while (k < max_iter && sqrt(rr) > target) {
        orc_csr_apply(R, row_ptrs, col_idx, values, p, ap);
        const double pap = orc_dot(R, p, ap);
        const double alpha = pap != 0.0 ? rr / pap : 0.0;
        for (int64_t i = 0; i < R; ++i) {
            x[i] += alpha * p[i];
            r[i] -= alpha * ap[i];
        }
        const double rr_new = orc_dot(R, r, r);
        const double beta = rr != 0.0 ? rr_new / rr : 0.0;
        for (int64_t i = 0; i < R; ++i)
            p[i] = r[i] + beta * p[i];
        rr = rr_new;
        ++k;
    }
    out[0] = (double)k;
    out[1] = bnorm > 0.0 ? sqrt(rr) / bnorm : sqrt(rr);
    free(r); free(p); free(ap);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* ELL with x tiles [REG, ELL slot layout; INTRO, x blocking].  Rows in      */
/* blocks of B.  Block b's tile is the set of distinct columns of its        */
/* entries in increasing order; a run is a maximal stretch of consecutive    */
/* columns in the tile, stored as (first column, offset of that column in    */
/* the tile, length).  Slot t of row r (at t*R + r, as in ELL) holds the     */
/* tile position of the entry's column (int16) and its value; slots past     */
/* the row's length hold (0, +0.0f).  ell_nnz[r] = row length.              */
/* Refused (ORC_ERR_TOO_LARGE) when R*W > INT32_MAX or a block's columns     */
/* span more than 2^18 (greatest - least + 1) or it has more than 8192       */
/* distinct columns or more than 1024 runs.                                  */
/* With runs == NULL only *runs_total is computed (sizing call).             */
/* ------------------------------------------------------------------------ */

static int orc_cmp_i32(const void *a, const void *b)
{
    const int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

int orc_csr_to_ell_xtile(int64_t R, const int32_t *row_ptrs, const int32_t *col_idx,
                         const uint32_t *val_bits, int64_t W, int64_t B, int32_t *run_ptr,
                         int32_t *runs, int16_t *lidx, uint32_t *ell_val, int32_t *ell_nnz,
                         int64_t *runs_total)
{
    if (R * W > ORC_INT32_MAX)
        return ORC_ERR_TOO_LARGE;
    int64_t nb = (R + B - 1) / B;
    int64_t maxn = 0;
    for (int64_t b = 0; b < nb; ++b) {
        int64_t r0 = b * B, r1 = r0 + B < R ? r0 + B : R;
        int64_t n = (int64_t)row_ptrs[r1] - row_ptrs[r0];
        if (n > maxn)
            maxn = n;
    }
    int32_t *tile = (int32_t *)malloc(sizeof(int32_t) * (size_t)(maxn > 0 ? maxn : 1));
    if (!tile)
        return ORC_ERR_INVALID_ARG;
    int64_t total = 0;
    if (run_ptr)
        run_ptr[0] = 0;
    int status = ORC_OK;
    for (int64_t b = 0; b < nb && status == ORC_OK; ++b) {
        int64_t r0 = b * B, r1 = r0 + B < R ? r0 + B : R;
        int64_t s0 = row_ptrs[r0], n = (int64_t)row_ptrs[r1] - s0;
        /* the tile: sorted distinct columns */
        for (int64_t i = 0; i < n; ++i)
            tile[i] = col_idx[s0 + i];
        qsort(tile, (size_t)n, sizeof(int32_t), orc_cmp_i32);
        int64_t u = 0;
        for (int64_t i = 0; i < n; ++i)
            if (u == 0 || tile[i] != tile[u - 1])
                tile[u++] = tile[i];
        int64_t nruns = 0;
        for (int64_t i = 0; i < u; ++i)
            if (i == 0 || tile[i] != tile[i - 1] + 1)
                ++nruns;
        if (u > 0 && (int64_t)tile[u - 1] - tile[0] + 1 > (1 << 18))
            status = ORC_ERR_TOO_LARGE;
        if (u > 8192 || nruns > 1024)
            status = ORC_ERR_TOO_LARGE;
        if (status != ORC_OK)
            break;
        if (runs) {
            int64_t k = total;
            for (int64_t i = 0; i < u; ++i) {
                if (i == 0 || tile[i] != tile[i - 1] + 1) {
                    runs[3 * k] = tile[i];
                    runs[3 * k + 1] = (int32_t)i;
                    runs[3 * k + 2] = 1;
                    ++k;
                } else {
                    runs[3 * (k - 1) + 2] += 1;
                }
            }
            for (int64_t r = r0; r < r1; ++r) {
                int64_t a = row_ptrs[r], len = (int64_t)row_ptrs[r + 1] - a;
                ell_nnz[r] = (int32_t)len;
                for (int64_t t = 0; t < W; ++t) {
                    int64_t slot = t * R + r;
                    if (t < len) {
                        const int32_t *hit = (const int32_t *)bsearch(
                            &col_idx[a + t], tile, (size_t)u, sizeof(int32_t), orc_cmp_i32);
                        lidx[slot] = (int16_t)(hit - tile);
                        ell_val[slot] = val_bits[a + t];
                    } else {
                        lidx[slot] = 0;
                        ell_val[slot] = 0u;
                    }
                }
            }
        }
        total += nruns;
        if (run_ptr)
            run_ptr[b + 1] = (int32_t)total;
    }
    free(tile);
    if (runs_total)
        *runs_total = total;
    return status;
}

/* ------------------------------------------------------------------------ */
/* Blocked COO: x blocking and a split of the work by nonzeros [INTRO,      */
/* memory- and parallel-efficiency checks], with the entries of one row     */
/* that meet in a group summed as a run [P3 3.2, segmented COO].  This is   */
/* an encoding, so the oracle writes out its definition:                    */
/*   entry i of row r, column c: slice k = c / sc (sc = ceil(C/S), at least */
/*   1), row block b = r / RT, segment s = k*B + b (B = ceil(R/RT) blocks). */
/*   Entries in order of (s, c), ties in CSR order.  Chunks are runs of one */
/*   segment's entries and work items runs of chunks, chosen slice by slice */
/*   (P = 256 / S work items of a balanced slice, one per CU of its XCDs):  */
/*   - by chunk: each segment's run cut into chunks of E entries, the last  */
/*     one the remainder, which joins the chunk before it when shorter than */
/*     E/2 (integer halving); each chunk its own work item;                 */
/*   - balanced: cost of an entry of segment s, in 1/1024:                  */
/*     r_s = floor((n_s + 3*lines_s) * 1024 / n_s), n_s its entries and     */
/*     lines_s the entries that are the segment's first or whose column     */
/*     c >> 5 (128-byte line of x) differs from the entry before; total =   */
/*     sum of n_s*r_s over the slice; item w (0 <= w < P) runs from cut[w]  */
/*     to cut[w+1], cut[0] the slice's first entry, cut[P] its end, cut[w]  */
/*     the first position whose preceding entries of the slice cost at      */
/*     least floor(total*w/P); an item's entries cut at segment ends into   */
/*     chunks.                                                              */
/*   A slice is balanced when it holds at least P*max(RT/4, 64) entries and */
/*   its by-chunk chunks, each given in order to the least loaded of P      */
/*   loads (a chunk adding its entries times r_s), leave the largest load   */
/*   `most` with 8*most*P > 9*total.  Chunks and items are numbered slice   */
/*   by slice; each chunk is cut into groups of 64 entries (the last        */
/*   shorter, padded to 64 slots).                                          */
/*   Hot rows of block b: its rows with at least hot_min_len entries,       */
/*   longest first, ties by row, the first H (hot[b*H + h], -1 for unused). */
/*   The code of an entry is r - b*RT, or RT + h when r is hot row h.       */
/*   In a group the entries are reordered by code, ties kept in column      */
/*   order.  base[g] = the group's smallest column (its first in column     */
/*   order) -- unless its largest minus smallest column exceeds 65535: then */
/*   the group is wide group w (w = wide groups before it), base[g] =       */
/*   -(w+1), its slots' columns go to wide[w*64 + lane] and their offsets   */
/*   are 0.  pk = code << 16 | (column - base).  Padding: pk 0xFFFF0000,    */
/*   value bits 0, wide column 0.                                           */
/*   chunk_grp[c] = first group of chunk c (chunks+1 entries),              */
/*   chunk_blk[c] = its row block, slice_chunk[k] = first chunk of slice k  */
/*   (S+1 entries), slice_item[k] = first work item of slice k (S+1),       */
/*   item_chunk[i] = first chunk of work item i (items+1).                  */
/* sizes[0..4] = chunks, groups, wide groups, work items, balanced slices; */
/* with chunk_grp == NULL only the sizes are computed.                      */
/* ------------------------------------------------------------------------ */

static const int64_t *g_hot_len;

static int orc_cmp_hot(const void *a, const void *b)
{
    /* (block, length descending, row) for rows packed as block<<32 | row */
    const int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    const int64_t bx = x >> 32, by = y >> 32;
    if (bx != by)
        return bx < by ? -1 : 1;
    const int64_t lx = g_hot_len[x & 0xFFFFFFFF], ly = g_hot_len[y & 0xFFFFFFFF];
    if (lx != ly)
        return lx > ly ? -1 : 1;
    return (x > y) - (x < y);
}

int orc_coo_blocked(int64_t R, int64_t C, int64_t nnz, const int32_t *row_ptrs,
                    const int32_t *col_idx, const uint32_t *val_bits, int64_t S, int64_t RT,
                    int64_t E, int64_t H, int64_t hot_min_len, int64_t *sizes,
                    int32_t *chunk_grp, int32_t *chunk_blk, int32_t *slice_chunk,
                    int32_t *slice_item, int32_t *item_chunk, int32_t *hot, int32_t *base,
                    uint32_t *pk, uint32_t *val, int32_t *wide)
{
    if (R < 0 || C < 0 || nnz < 0 || S < 1 || S > 256 || RT < 1 || E < 1 || H < 0 ||
        RT + H > 0xFFFF)
        return ORC_ERR_INVALID_ARG;
    const int64_t sc = C > 0 ? (C + S - 1) / S : 1;
    const int64_t B = (R + RT - 1) / RT;
    const int64_t nseg = S * B;
    int64_t *row = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nnz > 0 ? nnz : 1));
    int64_t *by_col = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nnz > 0 ? nnz : 1));
    int64_t *order = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nnz > 0 ? nnz : 1));
    int64_t *cnt_col = (int64_t *)calloc((size_t)(C + 1), sizeof(int64_t));
    int64_t *seg_start = (int64_t *)calloc((size_t)(nseg + 1), sizeof(int64_t));
    int64_t *len = (int64_t *)malloc(sizeof(int64_t) * (size_t)(R > 0 ? R : 1));
    int64_t *code = (int64_t *)malloc(sizeof(int64_t) * (size_t)(R > 0 ? R : 1));
    int64_t *cand = (int64_t *)malloc(sizeof(int64_t) * (size_t)(R > 0 ? R : 1));
    if (!row || !by_col || !order || !cnt_col || !seg_start || !len || !code || !cand) {
        free(row); free(by_col); free(order); free(cnt_col); free(seg_start);
        free(len); free(code); free(cand);
        return ORC_ERR_INVALID_ARG;
    }
    for (int64_t r = 0; r < R; ++r) {
        len[r] = (int64_t)row_ptrs[r + 1] - row_ptrs[r];
        for (int64_t i = row_ptrs[r]; i < row_ptrs[r + 1]; ++i)
            row[i] = r;
    }
    /* stable counting sort by column, then stable counting sort by segment */
    for (int64_t i = 0; i < nnz; ++i)
        cnt_col[col_idx[i] + 1]++;
    for (int64_t c = 0; c < C; ++c)
        cnt_col[c + 1] += cnt_col[c];
    for (int64_t i = 0; i < nnz; ++i)
        by_col[cnt_col[col_idx[i]]++] = i;
    for (int64_t j = 0; j < nnz; ++j) {
        int64_t i = by_col[j];
        int64_t s = (col_idx[i] / sc) * B + row[i] / RT;
        seg_start[s + 1]++;
    }
    for (int64_t s = 0; s < nseg; ++s)
        seg_start[s + 1] += seg_start[s];
    {
        int64_t *next = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nseg > 0 ? nseg : 1));
        if (!next) {
            free(row); free(by_col); free(order); free(cnt_col); free(seg_start);
            free(len); free(code); free(cand);
            return ORC_ERR_INVALID_ARG;
        }
        for (int64_t s = 0; s < nseg; ++s)
            next[s] = seg_start[s];
        for (int64_t j = 0; j < nnz; ++j) {
            int64_t i = by_col[j];
            int64_t s = (col_idx[i] / sc) * B + row[i] / RT;
            order[next[s]++] = i;
        }
        free(next);
    }
    /* hot rows and codes */
    int64_t ncand = 0;
    for (int64_t r = 0; r < R; ++r) {
        code[r] = r % RT;
        if (len[r] >= hot_min_len)
            cand[ncand++] = ((r / RT) << 32) | r;
    }
    g_hot_len = len;
    qsort(cand, (size_t)ncand, sizeof(int64_t), orc_cmp_hot);
    if (hot)
        for (int64_t i = 0; i < B * H; ++i)
            hot[i] = -1;
    for (int64_t i = 0, h = 0; i < ncand; ++i) {
        int64_t b = cand[i] >> 32, r = cand[i] & 0xFFFFFFFF;
        h = (i > 0 && (cand[i - 1] >> 32) == b) ? h + 1 : 0;
        if (h < H) {
            code[r] = RT + h;
            if (hot)
                hot[b * H + h] = (int32_t)r;
        }
    }
    /* chunks and work items: (segment, first entry, end) of every chunk, */
    /* slice by slice, and the first chunk of every work item               */
    const int64_t P = 256 / S;
    int64_t *lines = (int64_t *)calloc((size_t)(nseg > 0 ? nseg : 1), sizeof(int64_t));
    int64_t *rate = (int64_t *)calloc((size_t)(nseg > 0 ? nseg : 1), sizeof(int64_t));
    int64_t *load = (int64_t *)calloc((size_t)P, sizeof(int64_t));
    int64_t *cut = (int64_t *)calloc((size_t)P + 1, sizeof(int64_t));
    /* chunks: by chunk at most ceil(n/E) <= n/E + 1 per segment of n entries; */
    /* balanced at most one per segment plus one per cut                       */
    int64_t cap = nnz / E + nseg + S * P + 2;
    int64_t *ch = (int64_t *)malloc(sizeof(int64_t) * 3 * (size_t)cap);
    int64_t *item_first = (int64_t *)malloc(sizeof(int64_t) * (size_t)cap);
    int64_t *slice_first_item = (int64_t *)malloc(sizeof(int64_t) * (size_t)(S + 1));
    int64_t *slice_first_chunk = (int64_t *)malloc(sizeof(int64_t) * (size_t)(S + 1));
    if (!lines || !rate || !load || !cut || !ch || !item_first || !slice_first_item ||
        !slice_first_chunk) {
        free(lines); free(rate); free(load); free(cut); free(ch); free(item_first);
        free(slice_first_item); free(slice_first_chunk);
        free(row); free(by_col); free(order); free(cnt_col); free(seg_start);
        free(len); free(code); free(cand);
        return ORC_ERR_INVALID_ARG;
    }
    for (int64_t s = 0; s < nseg; ++s) {
        const int64_t n = seg_start[s + 1] - seg_start[s];
        for (int64_t j = seg_start[s]; j < seg_start[s + 1]; ++j)
            if (j == seg_start[s] || (col_idx[order[j]] >> 5) != (col_idx[order[j - 1]] >> 5))
                lines[s]++;
        rate[s] = n > 0 ? (n + 3 * lines[s]) * 1024 / n : 0;
    }
    int64_t nch = 0, nitem = 0, nbal = 0;
    for (int64_t k = 0; k < S; ++k) {
        const int64_t first = seg_start[k * B], end = seg_start[(k + 1) * B];
        slice_first_item[k] = nitem;
        slice_first_chunk[k] = nch;
        /* the by-chunk cut, and its loads */
        int64_t total = 0, most = 0;
        for (int64_t p = 0; p < P; ++p)
            load[p] = 0;
        for (int64_t s = k * B; s < (k + 1) * B; ++s) {
            total += (seg_start[s + 1] - seg_start[s]) * rate[s];
            for (int64_t e0 = seg_start[s], e1 = 0; e0 < seg_start[s + 1]; e0 = e1) {
                /* runs of E entries; a last piece shorter than E/2 joins the run before it */
                e1 = e0 + E < seg_start[s + 1] ? e0 + E : seg_start[s + 1];
                if (seg_start[s + 1] - e1 < E / 2)
                    e1 = seg_start[s + 1];
                int64_t least = 0;
                for (int64_t p = 1; p < P; ++p)
                    if (load[p] < load[least])
                        least = p;
                load[least] += (e1 - e0) * rate[s];
                if (load[least] > most)
                    most = load[least];
                ch[3 * nch] = s;
                ch[3 * nch + 1] = e0;
                ch[3 * nch + 2] = e1;
                item_first[nitem++] = nch++;
            }
        }
        if (end - first >= P * (RT / 4 > 64 ? RT / 4 : 64) && 8 * most * P > 9 * total) {
            /* balanced: drop the by-chunk cut of this slice, cut by cost */
            ++nbal;
            nch = slice_first_chunk[k];
            nitem = slice_first_item[k];
            int64_t spent = 0, w = 1;   /* spent: cost of the entries before entry j */
            cut[0] = first;
            cut[P] = end;
            for (int64_t s = k * B; s < (k + 1) * B; ++s)
                for (int64_t j = seg_start[s]; j < seg_start[s + 1]; ++j) {
                    while (w < P && spent >= total * w / P)
                        cut[w++] = j;
                    spent += rate[s];
                }
            while (w < P)
                cut[w++] = end;
            for (int64_t i = 0; i < P; ++i) {
                item_first[nitem++] = nch;
                int64_t s = k * B;
                for (int64_t e0 = cut[i]; e0 < cut[i + 1];) {
                    while (seg_start[s + 1] <= e0)
                        ++s;
                    int64_t e1 = cut[i + 1] < seg_start[s + 1] ? cut[i + 1] : seg_start[s + 1];
                    ch[3 * nch] = s;
                    ch[3 * nch + 1] = e0;
                    ch[3 * nch + 2] = e1;
                    ++nch;
                    e0 = e1;
                }
            }
        }
    }
    slice_first_item[S] = nitem;
    slice_first_chunk[S] = nch;
    item_first[nitem] = nch;

    /* groups of every chunk */
    int64_t ngrp = 0, nwide = 0;
    if (chunk_grp)
        chunk_grp[0] = 0;
    for (int64_t c = 0; c < nch; ++c) {
        const int64_t s = ch[3 * c], e0 = ch[3 * c + 1], e1 = ch[3 * c + 2];
        for (int64_t g0 = e0; g0 < e1; g0 += 64) {
            int64_t n = e1 - g0 < 64 ? e1 - g0 : 64;
            int64_t lo = col_idx[order[g0]], hi = col_idx[order[g0 + n - 1]];
            int is_wide = hi - lo > 65535;
            if (pk) {
                /* lanes: the group's entries, stably reordered by code */
                int64_t lane_of[64];
                for (int64_t q = 0; q < n; ++q) {
                    int64_t p = q;
                    while (p > 0 && code[row[order[g0 + lane_of[p - 1]]]] >
                                        code[row[order[g0 + q]]]) {
                        lane_of[p] = lane_of[p - 1];
                        --p;
                    }
                    lane_of[p] = q;
                }
                base[ngrp] = is_wide ? (int32_t)(-(nwide + 1)) : (int32_t)lo;
                for (int64_t l = 0; l < 64; ++l) {
                    int64_t slot = ngrp * 64 + l;
                    if (l < n) {
                        int64_t i = order[g0 + lane_of[l]];
                        int64_t off = is_wide ? 0 : col_idx[i] - lo;
                        pk[slot] = (uint32_t)(code[row[i]] << 16) | (uint32_t)off;
                        val[slot] = val_bits[i];
                        if (is_wide)
                            wide[nwide * 64 + l] = col_idx[i];
                    } else {
                        pk[slot] = 0xFFFF0000u;
                        val[slot] = 0u;
                        if (is_wide)
                            wide[nwide * 64 + l] = 0;
                    }
                }
            }
            nwide += is_wide;
            ++ngrp;
        }
        if (chunk_grp) {
            chunk_grp[c + 1] = (int32_t)ngrp;
            chunk_blk[c] = (int32_t)(s % B);
        }
    }
    if (chunk_grp) {
        for (int64_t k = 0; k <= S; ++k) {
            slice_chunk[k] = (int32_t)slice_first_chunk[k];
            slice_item[k] = (int32_t)slice_first_item[k];
        }
        for (int64_t i = 0; i <= nitem; ++i)
            item_chunk[i] = (int32_t)item_first[i];
    }
    sizes[0] = nch;
    sizes[1] = ngrp;
    sizes[2] = nwide;
    sizes[3] = nitem;
    sizes[4] = nbal;
    free(lines); free(rate); free(load); free(cut); free(ch); free(item_first);
    free(slice_first_item); free(slice_first_chunk);
    free(row); free(by_col); free(order); free(cnt_col); free(seg_start);
    free(len); free(code); free(cand);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Blocked COO block height: RT = 32768, unless that layout (orc_coo_blocked */
/* with the given chunk size and hot-row rule) cuts some slice into         */
/* balanced work items; then RT = 38912.  Reading of [INTRO, memory-        */
/* efficiency check]: a taller block puts more of a segment's entries on    */
/* each x line; it is taken only where the chunks no longer fill the CUs in */
/* whole rounds anyway.  Returns -1 on a refused layout.                    */
/* ------------------------------------------------------------------------ */
int64_t orc_bc_block_rows(int64_t R, int64_t C, int64_t nnz, const int32_t *row_ptrs,
                          const int32_t *col_idx, int64_t S, int64_t E, int64_t H,
                          int64_t hot_min_len)
{
    int64_t sizes[5] = {0, 0, 0, 0, 0};
    int st = orc_coo_blocked(R, C, nnz, row_ptrs, col_idx, NULL, S, 32768, E, H, hot_min_len,
                             sizes, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL);
    if (st != ORC_OK)
        return -1;
    return sizes[4] > 0 ? 38912 : 32768;
}

/* ------------------------------------------------------------------------ */
/* Blocked COO chunk size (reading of [INTRO, split by nonzeros]: each      */
/* workgroup gets an equal share of the nonzeros, one share per CU): T =    */
/* ceil(11*nnz / 2560) rounded up to a multiple of 64, at least 8192; a     */
/* segment is cut into runs of T entries, the last one the remainder        */
/* (orc_coo_blocked's E).                                                   */
/* ------------------------------------------------------------------------ */
int64_t orc_bc_chunk_entries(int64_t nnz)
{
    int64_t t = (11 * nnz + 2559) / 2560;
    t = (t + 63) / 64 * 64;
    return t < 8192 ? 8192 : t;
}

/* ------------------------------------------------------------------------ */
/* The automatic build's choice (the library's SPMV_AUTO), written out: the */
/* selector of orc_select, then the build-time readings of x blocking       */
/* [INTRO, memory-efficiency check: gathers from an x that does not fit the */
/* cache; keep the x a block touches close]:                                */
/*   spread = floor(mean over non-empty rows r of |first column of r -      */
/*            floor(r*C/R)|); scattered = spread*8 > C; big_x = 4C > 4 MiB. */
/*   1. scattered, big_x and 32*nnz*min(R, RT) >= R*C (a row block holds an */
/*      entry per 128-byte line of x on average) -> blocked COO with S =    */
/*      the smallest power of two with 4C <= S * 4 MiB, at most 8.          */
/*   2. scattered and big_x otherwise -> x slices, each merge-based CSR:    */
/*      4C <= 16 MiB: K = the smallest of 2, 4, 8 with 4C <= K * 2 MiB,     */
/*      halved (not below 2) while 3*K*R > nnz; beyond: K = ceil(4C/4 MiB); */
/*      K capped at 64 and at C; the slices number ceil(C / ceil(C/K)).     */
/*   3. otherwise the selector's format, except that ELL becomes ELL with x */
/*      tiles when R >= 16384, W*R <= INT32_MAX, every 256-row block's tile */
/*      qualifies (orc_csr_to_ell_xtile's limits) and nnz >= 2 * (sum of    */
/*      the blocks' distinct column counts).                                */
/* out[0] format, out[1] HYB width, out[2] CSR-vector lanes, out[3] x       */
/* slices (1 when unsplit; S for blocked COO).                              */
/* ------------------------------------------------------------------------ */

#define ORC_FMT_ELL_XTILE 10
#define ORC_FMT_COO_BLOCKED 11

int orc_select_build(int64_t R, int64_t C, int64_t nnz, const int32_t *row_ptrs,
                     const int32_t *col_idx, int64_t RT, int64_t *out)
{
    int64_t W = 0, nonempty = 0, dist = 0;
    for (int64_t r = 0; r < R; ++r) {
        int64_t len = (int64_t)row_ptrs[r + 1] - row_ptrs[r];
        if (len > W)
            W = len;
        if (len > 0) {
            int64_t diag = r * C / R;
            int64_t d = (int64_t)col_idx[row_ptrs[r]] - diag;
            dist += d < 0 ? -d : d;
            ++nonempty;
        }
    }
    int64_t *hist = (int64_t *)calloc((size_t)(W + 1), sizeof(int64_t));
    if (!hist)
        return ORC_ERR_INVALID_ARG;
    for (int64_t r = 0; r < R; ++r)
        hist[row_ptrs[r + 1] - row_ptrs[r]]++;
    int64_t sel[3];
    orc_select(R, nnz, W, hist, 0, 0, sel);
    out[0] = sel[0];
    out[1] = sel[1];
    out[2] = sel[2];
    out[3] = 1;
    int64_t spread = nonempty > 0 ? dist / nonempty : 0;
    int scattered = spread * 8 > C;
    int big_x = 4 * C > (4 << 20);
    int64_t rows = R < RT ? R : RT;
    if (nnz > 0 && R > 0 && scattered && big_x && 32 * nnz * rows >= R * C) {
        int64_t S = 1;
        while (S < 8 && 4 * C > S * (4 << 20))
            S *= 2;
        free(hist);
        out[0] = ORC_FMT_COO_BLOCKED;
        out[1] = 0;
        out[2] = 0;
        out[3] = S;
        return ORC_OK;
    }
    free(hist);
    if (nnz > 0 && scattered && big_x) {
        int64_t K;
        if (4 * C <= 8 * (2 << 20)) {
            K = 2;
            while (K < 8 && 4 * C > K * (2 << 20))
                K *= 2;
            while (K > 2 && 3 * K * R > nnz)
                K /= 2;
        } else {
            K = (4 * C + (4 << 20) - 1) / (4 << 20);
        }
        if (K > 64)
            K = 64;
        if (K > C)
            K = C;
        if (K < 1)
            K = 1;
        if (K > 1) {
            int64_t slice = (C + K - 1) / K;
            out[0] = ORC_FMT_CSR_MERGE;
            out[1] = 0;
            out[2] = 0;
            out[3] = (C + slice - 1) / slice;
            return ORC_OK;
        }
    }
    if (out[0] == ORC_FMT_ELL && R >= 64 * 256 && W * R <= ORC_INT32_MAX) {
        int64_t runs = 0;
        if (orc_csr_to_ell_xtile(R, row_ptrs, col_idx, NULL, W, 256, NULL, NULL, NULL, NULL,
                                 NULL, &runs) == ORC_OK) {
            /* distinct columns of each 256-row block */
            int64_t tiles = 0, maxn = 0;
            for (int64_t b = 0; b * 256 < R; ++b) {
                int64_t r1 = (b + 1) * 256 < R ? (b + 1) * 256 : R;
                int64_t n = (int64_t)row_ptrs[r1] - row_ptrs[b * 256];
                if (n > maxn)
                    maxn = n;
            }
            int32_t *t = (int32_t *)malloc(sizeof(int32_t) * (size_t)(maxn > 0 ? maxn : 1));
            if (!t)
                return ORC_ERR_INVALID_ARG;
            for (int64_t b = 0; b * 256 < R; ++b) {
                int64_t r1 = (b + 1) * 256 < R ? (b + 1) * 256 : R;
                int64_t s0 = row_ptrs[b * 256], n = (int64_t)row_ptrs[r1] - s0;
                for (int64_t i = 0; i < n; ++i)
                    t[i] = col_idx[s0 + i];
                qsort(t, (size_t)n, sizeof(int32_t), orc_cmp_i32);
                for (int64_t i = 0; i < n; ++i)
                    tiles += (i == 0 || t[i] != t[i - 1]);
            }
            free(t);
            if (nnz >= 2 * tiles)
                out[0] = ORC_FMT_ELL_XTILE;
        }
    }
    return ORC_OK;
}
