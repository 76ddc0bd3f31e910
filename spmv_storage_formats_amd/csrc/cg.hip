// Conjugate gradient for A x = b, A symmetric positive definite: the iterative
// method SpMV serves (PMPP notes, "Sparse Matrices and Basic Formats (COO &
// CSR)", background section: for positive-definite A conjugate gradient
// guesses X, evaluates A·X, and corrects X along the gradient; the SpMV is
// the most expensive step of each iteration).
//
// Per iteration: Ap = A p (the handle's spmv, into a zeroed Ap), pAp = p·Ap,
// alpha = rr / pAp, x += alpha p, r -= alpha Ap (fused with the partial sums
// of r·r), beta = rr_new / rr, p = r + beta p.  Dot products reduce in fp64
// (per-block partials, then one block); alpha and beta are computed on the
// device from device scalars, so an iteration never waits on the host.  The
// host reads r·r every kCheckEvery iterations to test convergence.
#include <cmath>
#include <vector>

#include "internal.h"

namespace spmv {
namespace {

constexpr int kThreads = 256;
constexpr int kDotBlocks = 1024;
constexpr int kCheckEvery = 8;

// device scalars
enum { kRR = 0, kPAP = 1, kRRNew = 2, kBB = 3, kNumScalars = 4 };

__device__ inline double block_sum(double v, double *lds) {
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int w = threadIdx.x / kWave;
    if (__lane_id() == 0) lds[w] = v;
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x == 0)
        for (int i = 0; i < kThreads / kWave; ++i) t += lds[i];
    return t;   // valid in thread 0
}

__global__ __launch_bounds__(kThreads) void k_fill(int32_t n, float v, float *__restrict__ a) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (i < n) a[i] = v;
}

// partial[b] = sum over the block's grid-stride share of a[i] * b[i]
__global__ __launch_bounds__(kThreads) void k_dot_partial(int32_t n, const float *__restrict__ a,
                                                          const float *__restrict__ b,
                                                          double *__restrict__ partial) {
    __shared__ double lds[kThreads / kWave];
    double s = 0.0;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * kThreads)
        s += static_cast<double>(a[i]) * static_cast<double>(b[i]);
    const double t = block_sum(s, lds);
    if (threadIdx.x == 0) partial[blockIdx.x] = t;
}

// scalars[slot] = sum of partial[0..np)
__global__ __launch_bounds__(kThreads) void k_dot_final(int32_t np, const double *__restrict__ partial,
                                                        double *__restrict__ scalars, int slot) {
    __shared__ double lds[kThreads / kWave];
    double s = 0.0;
    for (int i = threadIdx.x; i < np; i += kThreads) s += partial[i];
    const double t = block_sum(s, lds);
    if (threadIdx.x == 0) scalars[slot] = t;
}

// r = b - Ap (Ap holds A x), p = r
__global__ __launch_bounds__(kThreads) void k_cg_start(int32_t n, const float *__restrict__ b,
                                                       const float *__restrict__ ax,
                                                       float *__restrict__ r,
                                                       float *__restrict__ p) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (i < n) {
        const float v = b[i] - ax[i];
        r[i] = v;
        p[i] = v;
    }
}

// alpha = rr / pAp (0 when pAp == 0); x += alpha p; r -= alpha Ap;
// partial sums of the new r·r
__global__ __launch_bounds__(kThreads) void k_cg_update(int32_t n, const double *__restrict__ sc,
                                                        const float *__restrict__ p,
                                                        const float *__restrict__ ap,
                                                        float *__restrict__ x,
                                                        float *__restrict__ r,
                                                        double *__restrict__ partial) {
    __shared__ double lds[kThreads / kWave];
    const double pap = sc[kPAP];
    const float alpha = pap != 0.0 ? static_cast<float>(sc[kRR] / pap) : 0.f;
    double s = 0.0;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * kThreads) {
        x[i] += alpha * p[i];
        const float ri = r[i] - alpha * ap[i];
        r[i] = ri;
        s += static_cast<double>(ri) * static_cast<double>(ri);
    }
    const double t = block_sum(s, lds);
    if (threadIdx.x == 0) partial[blockIdx.x] = t;
}

// beta = rr_new / rr; p = r + beta p; Ap = 0 for the next SpMV; (rr <- rr_new
// is done by k_cg_roll after every block has read rr)
__global__ __launch_bounds__(kThreads) void k_cg_direction(int32_t n, const double *__restrict__ sc,
                                                           const float *__restrict__ r,
                                                           float *__restrict__ p,
                                                           float *__restrict__ ap) {
    const double rr = sc[kRR];
    const float beta = rr != 0.0 ? static_cast<float>(sc[kRRNew] / rr) : 0.f;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (i < n) {
        p[i] = r[i] + beta * p[i];
        ap[i] = 0.f;
    }
}

__global__ void k_cg_roll(double *__restrict__ sc) {
    if (threadIdx.x == 0) sc[kRR] = sc[kRRNew];
}

unsigned dot_blocks(int32_t n) {
    unsigned g = grid_for(n, kThreads);
    return g > kDotBlocks ? kDotBlocks : g;
}

hipError_t dot(int32_t n, const float *a, const float *b, double *partial, double *sc, int slot,
               hipStream_t s) {
    const unsigned g = dot_blocks(n);
    k_dot_partial<<<g, kThreads, 0, s>>>(n, a, b, partial);
    k_dot_final<<<1, kThreads, 0, s>>>(static_cast<int32_t>(g), partial, sc, slot);
    return hipGetLastError();
}

}  // namespace

spmv_status conjugate_gradient(const spmv_handle *A, const float *b, float *x, int32_t max_iter,
                               float rtol, int32_t *iters, float *rel_resid, hipStream_t s,
                               Scratch &scratch) {
    const int32_t n = static_cast<int32_t>(A->stats.num_rows);
    *iters = 0;
    *rel_resid = 0.f;
    if (n == 0) return SPMV_OK;
    float *r = nullptr, *p = nullptr, *ap = nullptr;
    double *partial = nullptr, *sc = nullptr;
    SPMV_TRY(scratch.alloc(&r, n));
    SPMV_TRY(scratch.alloc(&p, n));
    SPMV_TRY(scratch.alloc(&ap, n));
    SPMV_TRY(scratch.alloc(&partial, kDotBlocks));
    SPMV_TRY(scratch.alloc(&sc, kNumScalars));
    const unsigned gn = grid_for(n, kThreads);
    const unsigned gd = dot_blocks(n);
    // Ap = A x (into zeros), r = p = b - A x, rr = r.r, bb = b.b
    k_fill<<<gn, kThreads, 0, s>>>(n, 0.f, ap);
    SPMV_HIP(hipGetLastError());
    SPMV_TRY(launch_spmv(A, x, ap, s));
    k_cg_start<<<gn, kThreads, 0, s>>>(n, b, ap, r, p);
    SPMV_HIP(hipGetLastError());
    SPMV_HIP(dot(n, r, r, partial, sc, kRR, s));
    SPMV_HIP(dot(n, b, b, partial, sc, kBB, s));
    double host[kNumScalars] = {0, 0, 0, 0};
    SPMV_HIP(hipMemcpyAsync(host, sc, sizeof(host), hipMemcpyDeviceToHost, s));
    SPMV_HIP(hipStreamSynchronize(s));
    const double bnorm = std::sqrt(host[kBB]);
    const double target = static_cast<double>(rtol) * (bnorm > 0.0 ? bnorm : 1.0);
    double rnorm = std::sqrt(host[kRR]);
    int32_t it = 0;
    while (it < max_iter && rnorm > target) {
        const int32_t batch = std::min(kCheckEvery, max_iter - it);
        for (int32_t k = 0; k < batch; ++k) {
            k_fill<<<gn, kThreads, 0, s>>>(n, 0.f, ap);
            SPMV_HIP(hipGetLastError());
            SPMV_TRY(launch_spmv(A, p, ap, s));
            SPMV_HIP(dot(n, p, ap, partial, sc, kPAP, s));
            k_cg_update<<<gd, kThreads, 0, s>>>(n, sc, p, ap, x, r, partial);
            SPMV_HIP(hipGetLastError());
            k_dot_final<<<1, kThreads, 0, s>>>(static_cast<int32_t>(gd), partial, sc, kRRNew);
            SPMV_HIP(hipGetLastError());
            k_cg_direction<<<gn, kThreads, 0, s>>>(n, sc, r, p, ap);
            SPMV_HIP(hipGetLastError());
            k_cg_roll<<<1, 64, 0, s>>>(sc);
            SPMV_HIP(hipGetLastError());
        }
        it += batch;
        SPMV_HIP(hipMemcpyAsync(host, sc, sizeof(host), hipMemcpyDeviceToHost, s));
        SPMV_HIP(hipStreamSynchronize(s));
        rnorm = std::sqrt(host[kRR]);
        if (!std::isfinite(rnorm)) break;
    }
    *iters = it;
    *rel_resid = static_cast<float>(bnorm > 0.0 ? rnorm / bnorm : rnorm);
    return SPMV_OK;
}

}  // namespace spmv
