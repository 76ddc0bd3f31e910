// Conjugate gradient for A x = b, A symmetric positive definite: the iterative
// method SpMV serves (PMPP notes, "Sparse Matrices and Basic Formats (COO &
// CSR)", background section: for positive-definite A conjugate gradient
// guesses X, evaluates A·X, and corrects X along the gradient; the SpMV is
// the most expensive step of each iteration).
//
// Per iteration, three launches besides the handle's SpMV:
//   Ap = A p                         the handle's spmv, into an Ap already zero
//   k_dot:          partials of p·Ap
//   k_cg_update:    alpha = rr / pAp; x += alpha p; r -= alpha Ap; partials of r'·r'
//   k_cg_direction: beta = r'·r' / rr; p = r' + beta p; Ap = 0
// On a plain ELL handle of up to kDotBlocks * kThreads rows two launches do
// the same arithmetic: k_cg_ell_step (the previous iteration's new direction,
// Ap = A p and p·Ap) and k_cg_update.
// Dot products are fp64 per-block partials.  A kernel that needs a dot product
// adds the partials itself, every block in the same order, so all blocks agree
// bit for bit and the whole solve is deterministic when the SpMV is; no grid-
// wide synchronisation or atomics are needed (the launch boundary orders the
// partials' writes before their reads).  rr partials alternate between two
// buffers.  The host adds the rr partials every kCheckEvery iterations to test
// convergence.
#include <array>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "internal.h"

namespace spmv {
namespace {

constexpr int kThreads = 256;
constexpr int kDotBlocks = 1024;   // partials per dot product (grid of the dot kernels)
constexpr int kCheckEvery = 8;

// Sum over the block of one double per thread; the result is returned to
// every thread.
__device__ inline double block_sum_all(double v, double *lds) {
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int w = threadIdx.x / kWave;
    __syncthreads();   // lds may still be read from a previous call
    if (__lane_id() == 0) lds[w] = v;
    __syncthreads();
    double t = 0.0;
    for (int i = 0; i < kThreads / kWave; ++i) t += lds[i];
    return t;
}

// part[0..np) added in a fixed order: the same value in every block.
__device__ inline double sum_partials(const double *__restrict__ part, int np, double *lds) {
    double s = 0.0;
    for (int i = threadIdx.x; i < np; i += kThreads) s += part[i];
    return block_sum_all(s, lds);
}

__global__ __launch_bounds__(kThreads) void k_fill(int32_t n, float v, float *__restrict__ a) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (i < n) a[i] = v;
}

// part[block] = the block's grid-stride share of a·b
__global__ __launch_bounds__(kThreads) void k_dot(int32_t n, const float *__restrict__ a,
                                                  const float *__restrict__ b,
                                                  double *__restrict__ part) {
    __shared__ double lds[kThreads / kWave];
    double s = 0.0;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * kThreads)
        s += static_cast<double>(a[i]) * static_cast<double>(b[i]);
    const double t = block_sum_all(s, lds);
    if (threadIdx.x == 0) part[blockIdx.x] = t;
}

// r = b - Ap (Ap holds A x), p = r, Ap = 0; partials of r·r and b·b
__global__ __launch_bounds__(kThreads) void k_cg_start(int32_t n, const float *__restrict__ b,
                                                       float *__restrict__ ap,
                                                       float *__restrict__ r,
                                                       float *__restrict__ p,
                                                       double *__restrict__ part_rr,
                                                       double *__restrict__ part_bb) {
    __shared__ double lds[kThreads / kWave];
    double srr = 0.0, sbb = 0.0;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * kThreads) {
        const float bi = b[i];
        const float v = bi - ap[i];
        r[i] = v;
        p[i] = v;
        ap[i] = 0.f;
        srr += static_cast<double>(v) * static_cast<double>(v);
        sbb += static_cast<double>(bi) * static_cast<double>(bi);
    }
    const double trr = block_sum_all(srr, lds);
    const double tbb = block_sum_all(sbb, lds);
    if (threadIdx.x == 0) {
        part_rr[blockIdx.x] = trr;
        part_bb[blockIdx.x] = tbb;
    }
}

// alpha = rr / pAp (0 when pAp == 0); x += alpha p; r -= alpha Ap; partials of r·r
__global__ __launch_bounds__(kThreads) void k_cg_update(int32_t n, int np,
                                                        const double *__restrict__ part_rr,
                                                        const double *__restrict__ part_pap,
                                                        const float *__restrict__ p,
                                                        const float *__restrict__ ap,
                                                        float *__restrict__ x,
                                                        float *__restrict__ r,
                                                        double *__restrict__ part_rr_new) {
    __shared__ double lds[kThreads / kWave];
    // the thread's first element is loaded before the partials are added
    const int64_t i0 = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    float xv = 0.f, pv = 0.f, rv = 0.f, av = 0.f;
    if (i0 < n) {
        xv = x[i0];
        pv = p[i0];
        rv = r[i0];
        av = ap[i0];
    }
    const double rr = sum_partials(part_rr, np, lds);
    const double pap = sum_partials(part_pap, np, lds);
    const float alpha = pap != 0.0 ? static_cast<float>(rr / pap) : 0.f;
    double s = 0.0;
    for (int64_t i = i0; i < n; i += static_cast<int64_t>(gridDim.x) * kThreads) {
        if (i != i0) {
            xv = x[i];
            pv = p[i];
            rv = r[i];
            av = ap[i];
        }
        x[i] = xv + alpha * pv;
        const float ri = rv - alpha * av;
        r[i] = ri;
        s += static_cast<double>(ri) * static_cast<double>(ri);
    }
    const double t = block_sum_all(s, lds);
    if (threadIdx.x == 0) part_rr_new[blockIdx.x] = t;
}

// beta = rr_new / rr (0 when rr == 0); p = r + beta p; Ap = 0 for the next SpMV
__global__ __launch_bounds__(kThreads) void k_cg_direction(int32_t n, int np,
                                                           const double *__restrict__ part_rr,
                                                           const double *__restrict__ part_rr_new,
                                                           const float *__restrict__ r,
                                                           float *__restrict__ p,
                                                           float *__restrict__ ap) {
    __shared__ double lds[kThreads / kWave];
    const int64_t i0 = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    float rv = 0.f, pv = 0.f;
    if (i0 < n) {
        rv = r[i0];
        pv = p[i0];
    }
    const double rr = sum_partials(part_rr, np, lds);
    const double rr_new = sum_partials(part_rr_new, np, lds);
    const float beta = rr != 0.0 ? static_cast<float>(rr_new / rr) : 0.f;
    for (int64_t i = i0; i < n; i += static_cast<int64_t>(gridDim.x) * kThreads) {
        if (i != i0) {
            rv = r[i];
            pv = p[i];
        }
        p[i] = rv + beta * pv;
        ap[i] = 0.f;
    }
}

// ELL handles: one kernel for the new direction, the SpMV and p·Ap.
// beta = rr_new / rr_old (0 when rr_old == 0) from the partials, the same
// expression as k_cg_direction; every row of p_new is r + beta p_old, formed
// again wherever the SpMV gathers it (the same fp32 expression, so the same
// bits), and written once by its own lane into the other p buffer (the
// gathers read only p_old, so no block sees a half-updated p).  Row i is
// handled by block (i / kThreads) % gridDim.x, in the thread and order k_dot
// uses for element i, so the p·Ap partials equal k_dot's, and each row sums
// its slots in slot order like k_ell: the iterates are those of the
// four-launch iteration.
__global__ __launch_bounds__(kThreads) void k_cg_ell_step(
    int32_t n, int32_t W, const int32_t *__restrict__ col, const float *__restrict__ val,
    const int32_t *__restrict__ len, int np, const double *__restrict__ part_rr_old,
    const double *__restrict__ part_rr_new, const float *__restrict__ r,
    const float *__restrict__ p_old, float *__restrict__ p_new, float *__restrict__ ap,
    double *__restrict__ part_pap) {
    // one row per thread (the host launches this only when the grid covers
    // every row); the first kPre slots, their gathers and the row's own r and
    // p are loaded before the partials are added, hiding that latency
    constexpr int kPre = 8;
    __shared__ double lds[kThreads / kWave];
    const uint32_t nu = static_cast<uint32_t>(n), wu = static_cast<uint32_t>(W);
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const bool has = i < n;
    const uint32_t row = has ? static_cast<uint32_t>(i) : 0u;
    const int32_t m = has ? len[row] : 0;
    int32_t c[kPre];
    float v[kPre], rc[kPre], pc[kPre];
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
        const bool ok = has && static_cast<uint32_t>(u) < wu;
        const uint32_t slot = static_cast<uint32_t>(u) * nu + row;
        c[u] = ok ? ld_nt(col + slot) : 0;
        v[u] = ok ? ld_nt(val + slot) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
        const bool live = u < m;
        rc[u] = live ? r[c[u]] : 0.f;
        pc[u] = live ? p_old[c[u]] : 0.f;
    }
    const float r_own = has ? r[row] : 0.f, p_own = has ? p_old[row] : 0.f;
    const double rr = sum_partials(part_rr_old, np, lds);
    const double rr_new = sum_partials(part_rr_new, np, lds);
    const float beta = rr != 0.0 ? static_cast<float>(rr_new / rr) : 0.f;
    double s = 0.0;
    if (has) {
        float sum = 0.f;
#pragma unroll
        for (int u = 0; u < kPre; ++u) {
            const float pv = u < m ? rc[u] + beta * pc[u] : 0.f;
            if (static_cast<uint32_t>(u) < wu) sum += v[u] * pv;
        }
        for (uint32_t t = kPre; t < wu; ++t) {
            const uint32_t slot = t * nu + row;
            const int32_t ct = ld_nt(col + slot);
            const float vt = ld_nt(val + slot);
            const float pv = t < static_cast<uint32_t>(m) ? r[ct] + beta * p_old[ct] : 0.f;
            sum += vt * pv;
        }
        const float pi = r_own + beta * p_own;
        const float q = 0.f + sum;
        p_new[row] = pi;
        ap[row] = q;
        s += static_cast<double>(pi) * static_cast<double>(q);
    }
    const double t = block_sum_all(s, lds);
    if (threadIdx.x == 0) part_pap[blockIdx.x] = t;
}

// The fused step applies to a plain (unsliced) ELL handle whose rows one pass
// of the dot grid covers (a row per thread): past that its threads walk rows
// one after another and the kernel runs at well under half of k_ell's rate
// (2048^2 Laplacian: 97 against 41 us), so the four-launch iteration is
// faster.  SPMV_CG_FUSED=0 asks for the four launches everywhere.
bool fused_ell(const spmv_handle *A) {
    const char *v = std::getenv("SPMV_CG_FUSED");
    if (v && std::strcmp(v, "0") == 0) return false;
    return A->format == SPMV_ELL && A->parts.empty() && A->ell_width > 0 &&
           A->stats.num_rows <= static_cast<int64_t>(kDotBlocks) * kThreads;
}

// One CG iteration's launches on `st`: SpMV, p·Ap, update, new direction.
spmv_status enqueue_iteration(const spmv_handle *A, int32_t n, int np, float *x, float *r,
                              float *const pbuf[2], float *ap, double *part_pap,
                              double *const part_rr[2], int cur, bool fused, hipStream_t st) {
    if (fused) {
        // direction of the previous iteration, SpMV and p·Ap in one launch;
        // the new p goes to the other buffer
        float *p_old = pbuf[cur], *p = pbuf[cur ^ 1];
        k_cg_ell_step<<<np, kThreads, 0, st>>>(n, A->ell_width, A->a.ell_col, A->a.ell_val,
                                               A->a.ell_nnz, np, part_rr[cur ^ 1], part_rr[cur],
                                               r, p_old, p, ap, part_pap);
        k_cg_update<<<np, kThreads, 0, st>>>(n, np, part_rr[cur], part_pap, p, ap, x, r,
                                             part_rr[cur ^ 1]);
        SPMV_HIP(hipGetLastError());
        return SPMV_OK;
    }
    float *p = pbuf[0];
    SPMV_TRY(launch_spmv(A, p, ap, st));
    k_dot<<<np, kThreads, 0, st>>>(n, p, ap, part_pap);
    k_cg_update<<<np, kThreads, 0, st>>>(n, np, part_rr[cur], part_pap, p, ap, x, r,
                                         part_rr[cur ^ 1]);
    k_cg_direction<<<np, kThreads, 0, st>>>(n, np, part_rr[cur], part_rr[cur ^ 1], r, p, ap);
    SPMV_HIP(hipGetLastError());
    return SPMV_OK;
}

// A batch of kCheckEvery iterations captured once as a HIP graph and replayed
// for every full batch: one launch instead of 4 * kCheckEvery (plus the
// SpMV's own).  kCheckEvery is even, so every batch starts with the r·r
// partials in the same buffer and one graph serves them all.  Nothing in the
// batch allocates, synchronises or sets memory.
struct BatchGraph {
    hipStream_t launch = nullptr;   // where the replays run (drained before teardown)
    hipStream_t cs = nullptr;       // capture stream
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    explicit BatchGraph(hipStream_t s) : launch(s) {}
    ~BatchGraph() {
        if (exec) (void)hipStreamSynchronize(launch);
        if (exec) (void)hipGraphExecDestroy(exec);
        if (graph) (void)hipGraphDestroy(graph);
        if (cs) (void)hipStreamDestroy(cs);
    }
};

static_assert(kCheckEvery % 2 == 0,
              "a batch must return the r.r partials and the p buffers to their places");

spmv_status capture_batch(BatchGraph &g, const spmv_handle *A, int32_t n, int np, float *x,
                          float *r, float *const pbuf[2], float *ap, double *part_pap,
                          double *const part_rr[2], int cur, bool fused) {
    SPMV_HIP(hipStreamCreateWithFlags(&g.cs, hipStreamNonBlocking));
    SPMV_HIP(hipStreamBeginCapture(g.cs, hipStreamCaptureModeThreadLocal));
    spmv_status st = SPMV_OK;
    for (int k = 0; k < kCheckEvery && st == SPMV_OK; ++k)
        st = enqueue_iteration(A, n, np, x, r, pbuf, ap, part_pap, part_rr, cur ^ (k & 1), fused,
                               g.cs);
    const hipError_t e = hipStreamEndCapture(g.cs, &g.graph);
    if (st != SPMV_OK) return st;
    SPMV_HIP(e);
    SPMV_HIP(hipGraphInstantiate(&g.exec, g.graph, nullptr, nullptr, 0));
    return SPMV_OK;
}

// Graphs are used unless SPMV_CG_GRAPH=0 (eager launches, for comparison).
bool graphs_enabled() {
    const char *v = std::getenv("SPMV_CG_GRAPH");
    return !(v && std::strcmp(v, "0") == 0);
}

// Host sum of device partials, in block order.
spmv_status host_sum(const double *part, int np, std::array<double, kDotBlocks> &buf,
                     double *out, hipStream_t s) {
    SPMV_HIP(hipMemcpyAsync(buf.data(), part, sizeof(double) * np, hipMemcpyDeviceToHost, s));
    SPMV_HIP(hipStreamSynchronize(s));
    double t = 0.0;
    for (int i = 0; i < np; ++i) t += buf[i];
    *out = t;
    return SPMV_OK;
}

}  // namespace

// Floats of the CG workspace for n rows: r, two p buffers, Ap (each padded to
// 64 floats, 256 bytes), then the fp64 partials [pAp | rr slot 0 | rr slot 1 |
// bb], kDotBlocks each.
size_t cg_workspace_floats(int64_t n) {
    const size_t nv = (static_cast<size_t>(n) + 63) & ~size_t{63};
    return 4 * nv + 2 * 4 * kDotBlocks;
}

// The solve on a caller-provided workspace of cg_workspace_floats(R) floats;
// with allow_graph false every iteration is launched directly.
spmv_status cg_on_workspace(const spmv_handle *A, const float *b, float *x, int32_t max_iter,
                            float rtol, int32_t *iters, float *rel_resid, hipStream_t s,
                            float *vecs, bool allow_graph) {
    const int32_t n = static_cast<int32_t>(A->stats.num_rows);
    *iters = 0;
    *rel_resid = 0.f;
    if (n == 0) return SPMV_OK;
    const bool fused = fused_ell(A);
    const size_t nv = (static_cast<size_t>(n) + 63) & ~size_t{63};
    float *r = vecs, *ap = vecs + 3 * nv;
    float *const pbuf[2] = {vecs + nv, vecs + 2 * nv};
    double *part = reinterpret_cast<double *>(vecs + 4 * nv);
    double *part_pap = part, *part_bb = part + 3 * kDotBlocks;
    double *part_rr[2] = {part + kDotBlocks, part + 2 * kDotBlocks};
    const unsigned gn = grid_for(n, kThreads);
    const int np = static_cast<int>(gn < static_cast<unsigned>(kDotBlocks) ? gn : kDotBlocks);
    std::array<double, kDotBlocks> host{};

    // Ap = A x (into zeros); r = p = b - A x; Ap = 0; partials of r·r and b·b
    k_fill<<<gn, kThreads, 0, s>>>(n, 0.f, ap);
    SPMV_HIP(hipGetLastError());
    SPMV_TRY(launch_spmv(A, x, ap, s));
    k_cg_start<<<np, kThreads, 0, s>>>(n, b, ap, r, pbuf[0], part_rr[0], part_bb);
    SPMV_HIP(hipGetLastError());
    if (fused) {
        // the fused iteration forms p = r + beta p_old: p_old = 0 and the
        // previous r·r slot equal to the current one give p = r at the start
        // (beta = 1, or 0 when r·r = 0), with every iteration alike
        k_fill<<<gn, kThreads, 0, s>>>(n, 0.f, pbuf[0]);
        SPMV_HIP(hipGetLastError());
        SPMV_HIP(hipMemcpyAsync(part_rr[1], part_rr[0], sizeof(double) * kDotBlocks,
                                hipMemcpyDeviceToDevice, s));
    }
    double bb = 0.0, rr = 0.0;
    SPMV_TRY(host_sum(part_bb, np, host, &bb, s));
    SPMV_TRY(host_sum(part_rr[0], np, host, &rr, s));
    const double bnorm = std::sqrt(bb);
    const double target = static_cast<double>(rtol) * (bnorm > 0.0 ? bnorm : 1.0);
    double rnorm = std::sqrt(rr);
    int cur = 0;   // part_rr[cur] holds the current r·r partials
    int32_t it = 0;
    // a graph pays for its capture from the second full batch on
    const bool use_graph = allow_graph && graphs_enabled() && max_iter >= 2 * kCheckEvery;
    BatchGraph g(s);
    while (it < max_iter && rnorm > target) {
        const int32_t batch = std::min(kCheckEvery, max_iter - it);
        if (use_graph && batch == kCheckEvery) {
            if (!g.exec)
                SPMV_TRY(capture_batch(g, A, n, np, x, r, pbuf, ap, part_pap, part_rr, cur,
                                       fused));
            SPMV_HIP(hipGraphLaunch(g.exec, s));
        } else {
            for (int32_t k = 0; k < batch; ++k) {
                SPMV_TRY(enqueue_iteration(A, n, np, x, r, pbuf, ap, part_pap, part_rr, cur,
                                           fused, s));
                cur ^= 1;
            }
        }
        it += batch;
        SPMV_TRY(host_sum(part_rr[cur], np, host, &rr, s));
        rnorm = std::sqrt(rr);
        if (!std::isfinite(rnorm)) break;
    }
    *iters = it;
    *rel_resid = static_cast<float>(bnorm > 0.0 ? rnorm / bnorm : rnorm);
    return SPMV_OK;
}

spmv_status conjugate_gradient(const spmv_handle *A, const float *b, float *x, int32_t max_iter,
                               float rtol, int32_t *iters, float *rel_resid, hipStream_t s,
                               Scratch &scratch) {
    float *vecs = nullptr;
    if (A->stats.num_rows > 0)
        SPMV_TRY(scratch.alloc(&vecs, cg_workspace_floats(A->stats.num_rows)));
    return cg_on_workspace(A, b, x, max_iter, rtol, iters, rel_resid, s, vecs, true);
}

// ------------------------------------------------------------------------
// The allocation-free variant: the workspace is this file-scope device array,
// one per GPU the library runs on (reserved when the code object is loaded
// there and held until the process ends).  Its device address is looked up
// once per device with that device current; host code uses only that
// address, never the array's name (a host-side stand-in).
// ------------------------------------------------------------------------
constexpr int64_t kCgNoAllocFloats =
    4 * static_cast<int64_t>(SPMV_CG_NOALLOC_MAX_ROWS) + 2 * 4 * kDotBlocks;
static __device__ __align__(256) float scratch[kCgNoAllocFloats];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float *g_scratch_ptr[kMaxDevices] = {};

spmv_status device_scratch(int device, float **out) {
    if (device < 0 || device >= kMaxDevices) return SPMV_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[device]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return SPMV_ERR_HIP;
        }
        g_scratch_ptr[device] = static_cast<float *>(p);
    }
    *out = g_scratch_ptr[device];
    return SPMV_OK;
}
}  // namespace

spmv_status conjugate_gradient_noalloc(const spmv_handle *A, const float *b, float *x,
                                       int32_t max_iter, float rtol, int32_t *iters,
                                       float *rel_resid, hipStream_t s) {
    if (A->stats.num_rows > SPMV_CG_NOALLOC_MAX_ROWS) return SPMV_ERR_TOO_LARGE;
    static_assert(2 * 4 * kDotBlocks % 64 == 0, "partials keep 256-byte alignment");
    float *ws = nullptr;
    SPMV_TRY(device_scratch(A->device, &ws));
    return cg_on_workspace(A, b, x, max_iter, rtol, iters, rel_resid, s, ws, false);
}

}  // namespace spmv
