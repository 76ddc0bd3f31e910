/*
 * OpenMP CSR SpMV, y <- A*x + y: the multi-core CPU baseline that the
 * benchmark times beside the single-threaded oracle.
 *
 * BENCHMARK INFRASTRUCTURE ONLY, like the oracle in this directory: only the
 * tests and the benchmark's CPU-baseline leg load it; the GPU library never
 * does.  Rows are split over the threads in chunks (dynamic schedule, so a
 * few very long rows do not stall one thread); each row is summed in fp64 in
 * row order, as in the oracle, and y is stored rounded to fp32.
 */
#include <omp.h>
#include <stdint.h>

int csr_omp_threads(void) { return omp_get_max_threads(); }

void csr_spmv_omp(int64_t R, const int32_t *row_ptrs, const int32_t *col_idx,
                  const float *values, const float *x, float *y)
{
#pragma omp parallel for schedule(dynamic, 2048)
    for (int64_t r = 0; r < R; ++r) {
        double s = (double)y[r];
        for (int64_t i = row_ptrs[r]; i < row_ptrs[r + 1]; ++i)
            s += (double)values[i] * (double)x[col_idx[i]];
        y[r] = (float)s;
    }
}
