// Microbenchmarks of the two memory paths the SpMV kernels depend on, for the
// benchmark's report (not part of the SpMV library):
//   - x gathers: n 4-byte loads x[idx[i]] whose index pattern the caller
//     chooses (random, sorted with a given spacing, consecutive), 8 per lane
//     in flight, the way the kernels gather x;
//   - LDS updates: random-address float adds into a 16384-float LDS array by
//     the hardware float atomic, a compare-and-swap loop, or the integer
//     atomic (the blocked-COO kernel's partial sums use the CAS loop).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kThreads = 256;
constexpr int kPerLane = 8;

__global__ __launch_bounds__(kThreads) void k_gather(int64_t n, const int32_t *__restrict__ idx,
                                                     const float *__restrict__ x,
                                                     float *__restrict__ out) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    int32_t c[kPerLane];
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) {
        const int64_t i = t + k * stride;
        c[k] = i < n ? __builtin_nontemporal_load(idx + i) : -1;
    }
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) acc += c[k] >= 0 ? x[c[k]] : 0.f;
    out[t] = acc;
}

constexpr int kLdsWords = 16384;
constexpr int kLdsThreads = 1024;

template <int MODE>
__global__ __launch_bounds__(kLdsThreads) void k_lds_update(int32_t iters,
                                                            const uint32_t *__restrict__ addr,
                                                            float *__restrict__ out) {
    __shared__ float a[kLdsWords];
    for (int i = threadIdx.x; i < kLdsWords; i += kLdsThreads) a[i] = 0.f;
    __syncthreads();
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    for (int it = 0; it < iters; ++it) {
        const uint32_t i = addr[((it + wave) & 63) * 64 + lane] % kLdsWords;
        if (MODE == 0) {
            __hip_atomic_fetch_add(&a[i], 1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        } else if (MODE == 1) {
            uint32_t *p = reinterpret_cast<uint32_t *>(&a[i]);
            uint32_t old = *p;
            while (!__hip_atomic_compare_exchange_strong(
                p, &old, __float_as_uint(__uint_as_float(old) + 1.0f), __ATOMIC_RELAXED,
                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) {
            }
        } else {
            __hip_atomic_fetch_add(reinterpret_cast<uint32_t *>(&a[i]), 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    }
    __syncthreads();
    out[static_cast<int64_t>(blockIdx.x) * kLdsThreads + threadIdx.x] = a[threadIdx.x];
}

}  // namespace

extern "C" {

// out: float[grid * 256] with grid = ceil(n / (256 * 8)); idx values in [0, len(x)).
int mb_gather(int64_t n, const int32_t *idx, const float *x, float *out, void *stream) {
    if (n <= 0) return 0;
    const int64_t grid = (n + kThreads * kPerLane - 1) / (kThreads * kPerLane);
    k_gather<<<static_cast<unsigned>(grid), kThreads, 0, static_cast<hipStream_t>(stream)>>>(
        n, idx, x, out);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

int64_t mb_gather_out_len(int64_t n) {
    return ((n + kThreads * kPerLane - 1) / (kThreads * kPerLane)) * kThreads;
}

// mode 0: LDS float atomic add, 1: compare-and-swap float add, 2: integer
// atomic add.  addr: uint32[4096]; out: float[blocks * 1024].
int mb_lds_update(int mode, int32_t blocks, int32_t iters, const uint32_t *addr, float *out,
                  void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (blocks <= 0 || iters < 0 || mode < 0 || mode > 2) return 2;
    if (mode == 0) k_lds_update<0><<<blocks, kLdsThreads, 0, s>>>(iters, addr, out);
    if (mode == 1) k_lds_update<1><<<blocks, kLdsThreads, 0, s>>>(iters, addr, out);
    if (mode == 2) k_lds_update<2><<<blocks, kLdsThreads, 0, s>>>(iters, addr, out);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // extern "C"
