// Stable LSD radix sort of uint32 keys, 8 bits per pass, with one to three
// 32-bit payload arrays that move along with the keys.
//
// Used where a builder must reorder entries without disturbing equal keys:
// COO -> CSR of an unsorted COO list (entries of one row keep their input
// order; the columns and values ride along as payload, so no permutation has
// to be gathered afterwards), the grouping of entries by x slice, and the JDS
// row sort by length (PMPP notes, "Regularized Formats", JDS section: sort
// rows by their nonzero count while recording each row's original index;
// equal lengths keep their original order).
//
// Per pass:
//   (1) every tile of kTile keys builds a 256-bin digit histogram;
//   (2) an exclusive scan over the digit-major [digit][tile] counts gives each
//       (digit, tile) its output offset;
//   (3) every tile orders its entries by digit in LDS, stably, and then
//       writes them out: the entries of one digit form one run of
//       consecutive output addresses, so the stores coalesce.
// Ranks inside a tile: each wave owns a contiguous quarter of the tile and
// walks it 64 entries at a time; the lanes that share a digit are found by
// AND-ing one ballot per digit bit, and a lane's rank is the number of such
// lanes below it plus the wave's running count for that digit.  Wave order,
// then step order, then lane order is input order, so equal keys keep it.
#include "internal.h"

namespace spmv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTile = 4096;
constexpr int kPerThread = kTile / kThreads;  // steps per wave
constexpr int kPerWave = kTile / kWaves;
constexpr int kRadix = 256;
constexpr int kMaxPayload = 3;

struct PayloadIn {
    const uint32_t *p[kMaxPayload];
};
struct PayloadOut {
    uint32_t *p[kMaxPayload];
};

__global__ __launch_bounds__(kThreads) void k_radix_count(const uint32_t *__restrict__ keys,
                                                          int64_t n, int shift,
                                                          int32_t *__restrict__ counts,
                                                          int32_t nblocks) {
    __shared__ int h[kRadix];
    h[threadIdx.x] = 0;
    __syncthreads();
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kTile;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
        const int64_t i = base + j * kThreads + threadIdx.x;
        if (i < n) atomicAdd(&h[(__builtin_nontemporal_load(keys + i) >> shift) & (kRadix - 1)], 1);
    }
    __syncthreads();
    counts[static_cast<int64_t>(threadIdx.x) * nblocks + blockIdx.x] = h[threadIdx.x];
}

template <int P>
__global__ __launch_bounds__(kThreads) void k_radix_scatter(
    const uint32_t *__restrict__ kin, PayloadIn pin, uint32_t *__restrict__ kout,
    PayloadOut pout, int64_t n, int shift, const int32_t *__restrict__ offsets,
    int32_t nblocks) {
    __shared__ uint32_t s_key[kTile];
    __shared__ uint32_t s_pay[P][kTile];
    __shared__ int s_wrun[kWaves][kRadix];
    __shared__ int s_start[kRadix];
    __shared__ int s_goff[kRadix];
    __shared__ int s_wsum[kWaves];

    const int tid = threadIdx.x;
    const int lane = __lane_id();
    const int w = tid / kWave;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) s_wrun[ww][tid] = 0;
    s_goff[tid] = offsets[static_cast<int64_t>(tid) * nblocks + blockIdx.x];
    __syncthreads();

    // every wave loads its quarter of the tile, 64 consecutive entries per step
    const int64_t tile0 = static_cast<int64_t>(blockIdx.x) * kTile;
    const int64_t base = tile0 + w * kPerWave + lane;
    uint32_t key[kPerThread];
    uint32_t pay[P][kPerThread];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
        const int64_t i = base + j * kWave;
        const bool valid = i < n;
        key[j] = valid ? __builtin_nontemporal_load(kin + i) : 0u;
#pragma unroll
        for (int q = 0; q < P; ++q) pay[q][j] = valid ? __builtin_nontemporal_load(pin.p[q] + i) : 0u;
    }

    // rank of every entry among the wave's earlier entries of its digit
    const unsigned long long below = (1ull << lane) - 1ull;
    int rank[kPerThread];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
        const bool valid = base + j * kWave < n;
        const uint32_t d = (key[j] >> shift) & (kRadix - 1);
        unsigned long long peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const bool bit = (d >> b) & 1u;
            const unsigned long long m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        const int r = __popcll(peers & below);
        // one LDS read per lane, then one write by the lowest lane of each
        // digit; a wave's LDS accesses complete in program order
        const int before = valid ? s_wrun[w][d] : 0;
        rank[j] = before + r;
        if (valid && r == 0) s_wrun[w][d] = before + __popcll(peers);
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();

    // thread tid = digit: per-wave exclusive prefix, the tile's count, and the
    // digit's start inside the tile (exclusive scan over the 256 digits)
    int total = 0;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
        const int c = s_wrun[ww][tid];
        s_wrun[ww][tid] = total;
        total += c;
    }
    int incl = total;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
    }
    if (lane == kWave - 1) s_wsum[w] = incl;
    __syncthreads();
    int pre = 0;
    for (int ww = 0; ww < w; ++ww) pre += s_wsum[ww];
    s_start[tid] = pre + incl - total;
    __syncthreads();

    // entries to their place in the digit-ordered tile
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
        if (base + j * kWave < n) {
            const uint32_t d = (key[j] >> shift) & (kRadix - 1);
            const int pos = s_start[d] + s_wrun[w][d] + rank[j];
            s_key[pos] = key[j];
#pragma unroll
            for (int q = 0; q < P; ++q) s_pay[q][pos] = pay[q][j];
        }
    }
    __syncthreads();

    // runs of one digit go to consecutive output addresses
    const int count = static_cast<int>(n - tile0 < kTile ? n - tile0 : kTile);
    for (int p = tid; p < count; p += kThreads) {
        const uint32_t k = s_key[p];
        const uint32_t d = (k >> shift) & (kRadix - 1);
        const int g = s_goff[d] + (p - s_start[d]);
        kout[g] = k;
#pragma unroll
        for (int q = 0; q < P; ++q) pout.p[q][g] = s_pay[q][p];
    }
}

}  // namespace

spmv_status radix_sort(const uint32_t *keys_in, uint32_t *keys_out, int num_payloads,
                       const uint32_t *const *pay_in, uint32_t *const *pay_out, int64_t n,
                       int key_bits, hipStream_t s, Scratch &scratch,
                       const uint32_t **keys_result) {
    if (num_payloads < 1 || num_payloads > kMaxPayload) return SPMV_ERR_INVALID_ARG;
    if (!keys_out && !keys_result) return SPMV_ERR_INVALID_ARG;
    if (n <= 0) return SPMV_OK;
    if (n > INT32_MAX) return SPMV_ERR_TOO_LARGE;
    const int passes = key_bits <= 8 ? 1 : (key_bits + 7) / 8;
    const int32_t nblocks = static_cast<int32_t>((n + kTile - 1) / kTile);
    if (static_cast<int64_t>(nblocks) * kRadix > INT32_MAX) return SPMV_ERR_TOO_LARGE;
    // one allocation (each free of a large buffer costs host time): the
    // [digit][tile] counts, the sorted keys when the caller leaves them to
    // scratch, then (more than one pass) the ping-pong keys and payloads;
    // every array 256-byte aligned
    const size_t n_counts = (static_cast<size_t>(nblocks) * kRadix + 63) & ~size_t{63};
    const size_t n_words = (static_cast<size_t>(n) + 63) & ~size_t{63};
    const size_t own_keys = keys_out ? 0 : n_words;
    const int tmp_arrays = passes > 1 ? 1 + num_payloads : 0;
    uint32_t *block = nullptr;
    SPMV_TRY(scratch.alloc(&block, n_counts + own_keys + n_words * tmp_arrays));
    int32_t *counts = reinterpret_cast<int32_t *>(block);
    if (!keys_out) keys_out = block + n_counts;
    if (keys_result) *keys_result = keys_out;
    block += own_keys;
    uint32_t *kt = nullptr;
    PayloadOut tmp{}, out{};
    PayloadIn src{};
    for (int q = 0; q < num_payloads; ++q) {
        out.p[q] = pay_out[q];
        src.p[q] = pay_in[q];
    }
    if (passes > 1) {
        kt = block + n_counts;
        for (int q = 0; q < num_payloads; ++q) tmp.p[q] = block + n_counts + n_words * (1 + q);
    }
    // Ping-pong so that the last pass lands in the outputs.
    const uint32_t *src_k = keys_in;
    for (int p = 0; p < passes; ++p) {
        const bool to_out = ((passes - 1 - p) % 2) == 0;
        uint32_t *dst_k = to_out ? keys_out : kt;
        const PayloadOut &dst = to_out ? out : tmp;
        const int shift = 8 * p;
        k_radix_count<<<nblocks, kThreads, 0, s>>>(src_k, n, shift, counts, nblocks);
        SPMV_HIP(hipGetLastError());
        SPMV_TRY(exclusive_scan(counts, counts, static_cast<int64_t>(nblocks) * kRadix, false, s,
                                scratch));
        switch (num_payloads) {
            case 1:
                k_radix_scatter<1><<<nblocks, kThreads, 0, s>>>(src_k, src, dst_k, dst, n, shift,
                                                                counts, nblocks);
                break;
            case 2:
                k_radix_scatter<2><<<nblocks, kThreads, 0, s>>>(src_k, src, dst_k, dst, n, shift,
                                                                counts, nblocks);
                break;
            default:
                k_radix_scatter<3><<<nblocks, kThreads, 0, s>>>(src_k, src, dst_k, dst, n, shift,
                                                                counts, nblocks);
                break;
        }
        SPMV_HIP(hipGetLastError());
        src_k = dst_k;
        for (int q = 0; q < num_payloads; ++q) src.p[q] = dst.p[q];
    }
    return SPMV_OK;
}

spmv_status radix_sort_pairs(const uint32_t *keys_in, const int32_t *vals_in,
                             uint32_t *keys_out, int32_t *vals_out, int64_t n, int key_bits,
                             hipStream_t s, Scratch &scratch) {
    const uint32_t *pin[1] = {reinterpret_cast<const uint32_t *>(vals_in)};
    uint32_t *pout[1] = {reinterpret_cast<uint32_t *>(vals_out)};
    return radix_sort(keys_in, keys_out, 1, pin, pout, n, key_bits, s, scratch);
}

}  // namespace spmv
