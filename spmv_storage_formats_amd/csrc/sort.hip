// Stable LSD radix sort of (uint32 key, int32 value) pairs, 8 bits per pass.
//
// Used where a builder must reorder entries without disturbing equal keys:
// COO -> CSR of an unsorted COO list (entries of one row keep their input
// order), and the JDS row sort by length (PMPP notes, "Regularized Formats",
// JDS section: sort rows by their nonzero count while recording each row's
// original index; equal lengths keep their original order).
//
// Per pass: (1) every block of 2048 keys builds a 256-bin digit histogram;
// (2) an exclusive scan over the digit-major [digit][block] counts gives each
// (digit, block) its output offset; (3) every block scatters its keys in
// input order.  Ranks inside a block come from wave ballots: the lanes that
// share a digit are found by AND-ing one ballot per digit bit, and a lane's
// rank is the number of such lanes below it.  Waves and rounds are ordered
// through LDS counters, so equal keys keep their input order.
#include "internal.h"

namespace spmv {
namespace {

constexpr int kThreads = 256;
constexpr int kRounds = 8;
constexpr int kTile = kThreads * kRounds;
constexpr int kRadix = 256;
constexpr int kWaves = kThreads / kWave;

__global__ __launch_bounds__(kThreads) void k_radix_count(const uint32_t *__restrict__ keys,
                                                          int64_t n, int shift,
                                                          int32_t *__restrict__ counts,
                                                          int32_t nblocks) {
    __shared__ int h[kRadix];
    h[threadIdx.x] = 0;
    __syncthreads();
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kTile;
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
        const int64_t i = base + j * kThreads + threadIdx.x;
        if (i < n) atomicAdd(&h[(keys[i] >> shift) & (kRadix - 1)], 1);
    }
    __syncthreads();
    counts[static_cast<int64_t>(threadIdx.x) * nblocks + blockIdx.x] = h[threadIdx.x];
}

__global__ __launch_bounds__(kThreads) void k_radix_scatter(
    const uint32_t *__restrict__ kin, const int32_t *__restrict__ vin,
    uint32_t *__restrict__ kout, int32_t *__restrict__ vout, int64_t n, int shift,
    const int32_t *__restrict__ offsets, int32_t nblocks) {
    __shared__ int running[kRadix];
    __shared__ int wcnt[kWaves][kRadix];
    const int tid = threadIdx.x;
    running[tid] = offsets[static_cast<int64_t>(tid) * nblocks + blockIdx.x];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) wcnt[w][tid] = 0;
    __syncthreads();

    const int lane = __lane_id();
    const int w = tid / kWave;
    const unsigned long long below = (1ull << lane) - 1ull;
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kTile;
    for (int j = 0; j < kRounds; ++j) {
        const int64_t i = base + j * kThreads + tid;
        const bool valid = i < n;
        const uint32_t k = valid ? kin[i] : 0u;
        const int32_t v = valid ? vin[i] : 0;
        const uint32_t d = (k >> shift) & (kRadix - 1);
        unsigned long long peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const bool bit = (d >> b) & 1u;
            const unsigned long long m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        const int rank = __popcll(peers & below);
        if (valid && rank == 0) wcnt[w][d] = __popcll(peers);
        __syncthreads();
        if (valid) {
            int pos = running[d] + rank;
            for (int ww = 0; ww < w; ++ww) pos += wcnt[ww][d];
            kout[pos] = k;
            vout[pos] = v;
        }
        __syncthreads();
        int add = 0;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            add += wcnt[ww][tid];
            wcnt[ww][tid] = 0;
        }
        running[tid] += add;
        __syncthreads();
    }
}

}  // namespace

spmv_status radix_sort_pairs(const uint32_t *keys_in, const int32_t *vals_in,
                             uint32_t *keys_out, int32_t *vals_out, int64_t n, int key_bits,
                             hipStream_t s, Scratch &scratch) {
    if (n <= 0) return SPMV_OK;
    if (n > INT32_MAX) return SPMV_ERR_TOO_LARGE;
    const int passes = key_bits <= 8 ? 1 : (key_bits + 7) / 8;
    const int32_t nblocks = static_cast<int32_t>((n + kTile - 1) / kTile);
    if (static_cast<int64_t>(nblocks) * kRadix > INT32_MAX) return SPMV_ERR_TOO_LARGE;
    int32_t *counts = nullptr;
    uint32_t *kt = nullptr;
    int32_t *vt = nullptr;
    SPMV_TRY(scratch.alloc(&counts, static_cast<size_t>(nblocks) * kRadix));
    if (passes > 1) {
        SPMV_TRY(scratch.alloc(&kt, static_cast<size_t>(n)));
        SPMV_TRY(scratch.alloc(&vt, static_cast<size_t>(n)));
    }
    // Ping-pong so that the last pass lands in keys_out / vals_out.
    const uint32_t *src_k = keys_in;
    const int32_t *src_v = vals_in;
    for (int p = 0; p < passes; ++p) {
        const bool to_out = ((passes - 1 - p) % 2) == 0;
        uint32_t *dst_k = to_out ? keys_out : kt;
        int32_t *dst_v = to_out ? vals_out : vt;
        const int shift = 8 * p;
        k_radix_count<<<nblocks, kThreads, 0, s>>>(src_k, n, shift, counts, nblocks);
        SPMV_HIP(hipGetLastError());
        SPMV_TRY(exclusive_scan(counts, counts, static_cast<int64_t>(nblocks) * kRadix, false, s,
                                scratch));
        k_radix_scatter<<<nblocks, kThreads, 0, s>>>(src_k, src_v, dst_k, dst_v, n, shift,
                                                     counts, nblocks);
        SPMV_HIP(hipGetLastError());
        src_k = dst_k;
        src_v = dst_v;
    }
    return SPMV_OK;
}

}  // namespace spmv
