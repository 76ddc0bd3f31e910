// Input checks and row-length statistics.
//
// Checks follow the CSR definition of the PMPP notes page "Sparse Matrices
// and Basic Formats (COO & CSR)" (rowPtrs[r] is where row r starts, so the
// pointers never decrease, rowPtrs[0] = 0 and rowPtrs[numRows] = nnz) and the
// input checks listed in section 5.3 of the SpGEMM/AIA article (row_ptr
// monotone, every column index below the column count).  Statistics are the
// ones the format-choice article uses to pick a format (section 4.1: row
// length histogram and variance; 4.3: mean and maximum row length).
#include "internal.h"

namespace spmv {
namespace {

constexpr int kThreads = 256;
constexpr int kHistLds = 4096;   // lengths below this are binned in LDS first
// Capped grids of the check kernels (one partial record or flags word per
// block, added or ORed on the host).
constexpr int kRowCheckMaxBlocks = 2048;
constexpr int kCooCheckMaxBlocks = 4096;
constexpr int kRowsInFlight = 4;   // rows a thread of k_row_checks loads at a time

__device__ inline int wave_max(int v) {
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
    return v;
}

__device__ inline unsigned long long wave_sum(unsigned long long v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// One lane per row: length, monotonicity, the two end conditions, and the
// reductions W = max len, sum len^2, number of empty rows.
//
// Also sums, over non-empty rows, the distance between the row's first column
// and its diagonal position r*C/R: small for banded matrices, about C/3 for
// uniformly scattered columns (used to decide on x slices).  The column is
// read only when the row's start lies inside [0, nnz).
//
// Grid-stride over rows with a capped grid; each block reduces its waves in
// LDS and writes one partial record (no atomics: same-address atomics from
// thousands of waves serialise in the L2).  The host adds the partials.
__global__ __launch_bounds__(kThreads) void k_row_checks(int32_t R, int32_t C, int32_t nnz,
                                                         const int32_t *__restrict__ rp,
                                                         const int32_t *__restrict__ col,
                                                         RowStatsDev *__restrict__ partial) {
    int bad = 0, wlen = 0;
    unsigned long long sq = 0, empty = 0, dist = 0;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    // kRowsInFlight rows at a time: their pointers, then their first columns,
    // are loaded together (every reduction here is order-free)
    for (int64_t r0 = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; r0 < R;
         r0 += kRowsInFlight * stride) {
        int a[kRowsInFlight], len[kRowsInFlight], c0[kRowsInFlight];
#pragma unroll
        for (int u = 0; u < kRowsInFlight; ++u) {
            const int64_t r = r0 + u * stride;
            a[u] = 0;
            len[u] = 0;
            if (r < R) {
                const int b = rp[r + 1];
                a[u] = rp[r];
                // compared directly (no subtraction that could wrap) and kept
                // within [0, nnz], so a wrapped pair such as INT32_MAX then
                // INT32_MIN is flagged like any decreasing pair
                const bool ok = b >= a[u] && a[u] >= 0 && b <= nnz;
                if (!ok) bad = 1;
                if (r == 0 && a[u] != 0) bad = 1;
                if (r == R - 1 && b != nnz) bad = 1;
                len[u] = ok ? b - a[u] : 0;
            }
        }
#pragma unroll
        for (int u = 0; u < kRowsInFlight; ++u)
            c0[u] = (len[u] > 0 && a[u] >= 0 && a[u] < nnz) ? col[a[u]] : 0;
#pragma unroll
        for (int u = 0; u < kRowsInFlight; ++u) {
            const int64_t r = r0 + u * stride;
            if (r >= R) continue;
            wlen = max(wlen, len[u]);
            sq += static_cast<unsigned long long>(len[u]) * static_cast<unsigned long long>(len[u]);
            empty += (len[u] == 0);
            if (len[u] > 0 && a[u] >= 0 && a[u] < nnz) {
                const int64_t diag = r * static_cast<int64_t>(C) / R;
                const int64_t d = static_cast<int64_t>(c0[u]) - diag;
                dist += static_cast<unsigned long long>(d < 0 ? -d : d);
            }
        }
    }
    if (R == 0 && blockIdx.x == 0 && threadIdx.x == 0) {  // rowPtrs = [0], nnz must be 0
        if (rp[0] != 0 || nnz != 0) bad = 1;
    }
    __shared__ RowStatsDev waves[kThreads / kWave];
    const unsigned long long any_bad = __ballot(bad != 0);
    const int wmax = wave_max(wlen);
    const unsigned long long wsq = wave_sum(sq);
    const unsigned long long wempty = wave_sum(empty);
    const unsigned long long wdist = wave_sum(dist);
    const int w = threadIdx.x / kWave;
    if (__lane_id() == 0) {
        waves[w].flags = any_bad ? kFlagBadRowPtrs : 0;
        waves[w].max_len = wmax;
        waves[w].sum_len_sq = wsq;
        waves[w].empty_rows = wempty;
        waves[w].sum_first_dist = wdist;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        RowStatsDev t = waves[0];
        for (int i = 1; i < kThreads / kWave; ++i) {
            t.flags |= waves[i].flags;
            t.max_len = max(t.max_len, waves[i].max_len);
            t.sum_len_sq += waves[i].sum_len_sq;
            t.empty_rows += waves[i].empty_rows;
            t.sum_first_dist += waves[i].sum_first_dist;
        }
        partial[blockIdx.x] = t;
    }
}

__global__ __launch_bounds__(kThreads) void k_col_checks(int32_t nnz, int32_t C,
                                                         const int32_t *__restrict__ col,
                                                         RowStatsDev *__restrict__ st) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    bool bad = false;
    if (i < nnz) {
        const int32_t c = ld_nt(col + i);
        bad = static_cast<uint32_t>(c) >= static_cast<uint32_t>(C);
    }
    if (__ballot(bad) != 0 && __lane_id() == 0) atomicOr(&st->flags, kFlagBadCol);
}

// COO input checks: row and column ranges, and whether the rows are already
// sorted.  Grid-stride over a capped grid; each block writes its flags to
// partial[blockIdx.x] (no same-address atomics: on an unsorted list every wave
// would set the flag) and the host ORs them.
__global__ __launch_bounds__(kThreads) void k_coo_checks(int32_t nnz, int32_t R, int32_t C,
                                                         const int32_t *__restrict__ row,
                                                         const int32_t *__restrict__ col,
                                                         int check_cols,
                                                         int *__restrict__ partial) {
    bool bad_row = false, bad_col = false, unsorted = false;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    constexpr int U = 4;   // entries of a thread loaded together
    for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i0 < nnz;
         i0 += U * stride) {
        int32_t r[U], rn[U], c[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = i0 + u * stride;
            r[u] = i < nnz ? ld_nt(row + i) : 0;
            rn[u] = i + 1 < nnz ? row[i + 1] : INT32_MAX;
            c[u] = (check_cols && i < nnz) ? ld_nt(col + i) : 0;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (i0 + u * stride >= nnz) continue;
            bad_row |= static_cast<uint32_t>(r[u]) >= static_cast<uint32_t>(R);
            if (check_cols) bad_col |= static_cast<uint32_t>(c[u]) >= static_cast<uint32_t>(C);
            unsorted |= rn[u] < r[u];
        }
    }
    const int f = (__ballot(bad_row) ? kFlagBadRow : 0) | (__ballot(bad_col) ? kFlagBadCol : 0) |
                  (__ballot(unsorted) ? kFlagUnsortedRows : 0);
    __shared__ int wf[kThreads / kWave];
    if (__lane_id() == 0) wf[threadIdx.x / kWave] = f;
    __syncthreads();
    if (threadIdx.x == 0) {
        int t = 0;
        for (int k = 0; k < kThreads / kWave; ++k) t |= wf[k];
        partial[blockIdx.x] = t;
    }
}

// hist[len] += 1 per row; short lengths are binned in LDS, long ones directly.
__global__ __launch_bounds__(kThreads) void k_len_hist(int32_t R, const int32_t *__restrict__ rp,
                                                       int32_t W, int32_t *__restrict__ hist) {
    __shared__ int sh[kHistLds];
    const int nb = W + 1 < kHistLds ? W + 1 : kHistLds;
    for (int i = threadIdx.x; i < nb; i += kThreads) sh[i] = 0;
    __syncthreads();
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; r < R;
         r += static_cast<int64_t>(gridDim.x) * kThreads) {
        const int len = rp[r + 1] - rp[r];
        if (len < kHistLds) atomicAdd(&sh[len], 1);
        else atomicAdd(&hist[len], 1);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nb; i += kThreads)
        if (sh[i]) atomicAdd(&hist[i], sh[i]);
}

}  // namespace

int row_check_blocks(int32_t R) {
    unsigned g = grid_for(R > 0 ? R : 1, kThreads);
    return static_cast<int>(g > kRowCheckMaxBlocks ? kRowCheckMaxBlocks : g);
}

hipError_t launch_row_checks(int32_t R, int32_t C, int32_t nnz, const int32_t *rp,
                             const int32_t *col, RowStatsDev *partial, hipStream_t s) {
    k_row_checks<<<row_check_blocks(R), kThreads, 0, s>>>(R, C, nnz, rp, col, partial);
    return hipGetLastError();
}

hipError_t launch_col_checks(int32_t nnz, int32_t C, const int32_t *col, RowStatsDev *st,
                             hipStream_t s) {
    if (nnz <= 0) return hipSuccess;
    k_col_checks<<<grid_for(nnz, kThreads), kThreads, 0, s>>>(nnz, C, col, st);
    return hipGetLastError();
}

int coo_check_blocks(int32_t nnz) {
    unsigned g = grid_for(nnz > 0 ? nnz : 1, kThreads);
    return static_cast<int>(g > kCooCheckMaxBlocks ? kCooCheckMaxBlocks : g);
}

hipError_t launch_coo_checks(int32_t nnz, int32_t R, int32_t C, const int32_t *row,
                             const int32_t *col, int check_cols, int *partial, hipStream_t s) {
    k_coo_checks<<<coo_check_blocks(nnz), kThreads, 0, s>>>(nnz, R, C, row, col, check_cols,
                                                            partial);
    return hipGetLastError();
}

hipError_t launch_len_hist(int32_t R, const int32_t *rp, int32_t W, int32_t *hist,
                           hipStream_t s) {
    if (R <= 0) return hipSuccess;
    unsigned g = grid_for(R, kThreads);
    if (g > 2048) g = 2048;
    k_len_hist<<<g, kThreads, 0, s>>>(R, rp, W, hist);
    return hipGetLastError();
}

}  // namespace spmv
