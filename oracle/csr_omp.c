/*
 * OpenMP CSR SpMV, y <- A*x + y: the multi-core CPU baseline that the
 * benchmark times beside the single-threaded oracle.
 *
 * BENCHMARK INFRASTRUCTURE ONLY, like the oracle in this directory: only the
 * tests and the benchmark's CPU-baseline leg load it; the GPU library never
 * does.
 *
 * csr_omp_bench follows a plain multi-core CSR baseline: rows split over the
 * threads by a `parallel for` with schedule(static) (schedule_dynamic = 0) or
 * schedule(dynamic, 64) (1); each row summed in fp32 in row order, starting
 * from y; private copies of every array first touched by the threads that use
 * them (same schedule), so their pages sit with those threads' memory; reps
 * timed runs with a monotonic clock (y reset before each, untimed); returns
 * the median seconds and leaves the last run's y in y_out.  Thread placement
 * (OMP_PROC_BIND, OMP_PLACES) is the caller's environment.
 */
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

int csr_omp_threads(void) { return omp_get_max_threads(); }

static double now_s(void)
{
    struct timespec t;
    clock_gettime(CLOCK_MONOTONIC, &t);
    return (double)t.tv_sec + 1e-9 * (double)t.tv_nsec;
}

static int cmp_d(const void *a, const void *b)
{
    const double x = *(const double *)a, y = *(const double *)b;
    return (x > y) - (x < y);
}

#define ROWS_LOOP(body)                                                     \
    do {                                                                    \
        if (dyn) {                                                          \
            _Pragma("omp parallel for schedule(dynamic, 64)")               \
            for (int64_t r = 0; r < R; ++r) { body; }                       \
        } else {                                                            \
            _Pragma("omp parallel for schedule(static)")                    \
            for (int64_t r = 0; r < R; ++r) { body; }                       \
        }                                                                   \
    } while (0)

double csr_omp_bench(int64_t R, int64_t C, const int32_t *row_ptrs, const int32_t *col_idx,
                     const float *values, const float *x, const float *y0, float *y_out,
                     int schedule_dynamic, int reps)
{
    const int dyn = schedule_dynamic != 0;
    const int64_t nnz = R > 0 ? row_ptrs[R] : 0;
    int32_t *rp = (int32_t *)malloc(sizeof(int32_t) * (size_t)(R + 1));
    int32_t *ci = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nnz > 0 ? nnz : 1));
    float *va = (float *)malloc(sizeof(float) * (size_t)(nnz > 0 ? nnz : 1));
    float *xx = (float *)malloc(sizeof(float) * (size_t)(C > 0 ? C : 1));
    float *y = (float *)malloc(sizeof(float) * (size_t)(R > 0 ? R : 1));
    double *t = (double *)malloc(sizeof(double) * (size_t)(reps > 0 ? reps : 1));
    if (!rp || !ci || !va || !xx || !y || !t || reps < 1) {
        free(rp); free(ci); free(va); free(xx); free(y); free(t);
        return -1.0;
    }
    /* first touch: each row's pointers and entries by the thread that sums it */
    rp[0] = row_ptrs[0];
    ROWS_LOOP({
        rp[r + 1] = row_ptrs[r + 1];
        y[r] = y0[r];
        for (int64_t i = row_ptrs[r]; i < row_ptrs[r + 1]; ++i) {
            ci[i] = col_idx[i];
            va[i] = values[i];
        }
    });
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c)
        xx[c] = x[c];
    for (int k = 0; k < reps; ++k) {
        ROWS_LOOP(y[r] = y0[r]);
        const double a = now_s();
        ROWS_LOOP({
            float s = y[r];
            for (int64_t i = rp[r]; i < rp[r + 1]; ++i)
                s += va[i] * xx[ci[i]];
            y[r] = s;
        });
        t[k] = now_s() - a;
    }
    memcpy(y_out, y, sizeof(float) * (size_t)R);
    qsort(t, (size_t)reps, sizeof(double), cmp_d);
    const double med = t[reps / 2];
    free(rp); free(ci); free(va); free(xx); free(y); free(t);
    return med;
}
