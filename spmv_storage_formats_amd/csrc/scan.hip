// Exclusive prefix sum of int32 counts: the step that turns per-row counts
// into CSR row pointers (PMPP notes, "Sparse Matrices and Basic Formats
// (COO & CSR)": rowPtrs[r] is the offset where row r starts, rowPtrs[numRows]
// the total), and radix-sort digit counts into scatter offsets.
//
// Reduce-then-scan over tiles of 2048 values (256 threads x 8): tile sums,
// a recursive scan of the sums, then a per-tile scan seeded with its offset.
#include "internal.h"

namespace spmv {
namespace {

constexpr int kThreads = 256;
constexpr int kItems = 8;
constexpr int kTile = kThreads * kItems;
constexpr int kWaves = kThreads / kWave;

__device__ inline int wave_inclusive(int v) {
    const int lane = __lane_id();
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int t = __shfl_up(v, o);
        if (lane >= o) v += t;
    }
    return v;
}

// Exclusive prefix of v over the block, plus the block total.
__device__ inline int block_exclusive(int v, int *total, int *lds) {
    const int w = threadIdx.x / kWave;
    const int incl = wave_inclusive(v);
    if (__lane_id() == kWave - 1) lds[w] = incl;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const int x = lds[i];
        before += (i < w) ? x : 0;
        tot += x;
    }
    __syncthreads();
    *total = tot;
    return before + incl - v;
}

__global__ __launch_bounds__(kThreads) void k_tile_sums(const int32_t *__restrict__ in,
                                                        int64_t n, int32_t *__restrict__ sums) {
    __shared__ int lds[kWaves];
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kTile;
    int s = 0;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        const int64_t i = base + j * kThreads + threadIdx.x;
        if (i < n) s += in[i];
    }
    int tot;
    block_exclusive(s, &tot, lds);
    if (threadIdx.x == 0) sums[blockIdx.x] = tot;
}

// Thread t scans the 8 consecutive values [base + 8t, base + 8t + 8).  in and
// out may alias: every thread reads its own values before writing them.
__global__ __launch_bounds__(kThreads) void k_scan_tiles(const int32_t *in, int32_t *out,
                                                         int64_t n,
                                                         const int32_t *__restrict__ tile_off,
                                                         int write_total) {
    __shared__ int lds[kWaves];
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kTile + threadIdx.x * kItems;
    int v[kItems];
    int s = 0;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        v[j] = (base + j < n) ? in[base + j] : 0;
        s += v[j];
    }
    int tot;
    const int excl = block_exclusive(s, &tot, lds);
    const int off0 = tile_off ? tile_off[blockIdx.x] : 0;
    int run = off0 + excl;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        if (base + j < n) out[base + j] = run;
        run += v[j];
    }
    if (write_total && blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) out[n] = off0 + tot;
}

}  // namespace

spmv_status exclusive_scan(const int32_t *in, int32_t *out, int64_t n, bool write_total,
                           hipStream_t s, Scratch &scratch) {
    if (n <= 0) {
        if (write_total) SPMV_HIP(hipMemsetAsync(out, 0, sizeof(int32_t), s));
        return SPMV_OK;
    }
    const int64_t tiles = (n + kTile - 1) / kTile;
    if (tiles == 1) {
        k_scan_tiles<<<1, kThreads, 0, s>>>(in, out, n, nullptr, write_total ? 1 : 0);
        SPMV_HIP(hipGetLastError());
        return SPMV_OK;
    }
    int32_t *sums = nullptr;
    SPMV_TRY(scratch.alloc(&sums, static_cast<size_t>(tiles)));
    k_tile_sums<<<static_cast<unsigned>(tiles), kThreads, 0, s>>>(in, n, sums);
    SPMV_HIP(hipGetLastError());
    SPMV_TRY(exclusive_scan(sums, sums, tiles, false, s, scratch));
    k_scan_tiles<<<static_cast<unsigned>(tiles), kThreads, 0, s>>>(in, out, n, sums,
                                                                   write_total ? 1 : 0);
    SPMV_HIP(hipGetLastError());
    return SPMV_OK;
}

}  // namespace spmv
