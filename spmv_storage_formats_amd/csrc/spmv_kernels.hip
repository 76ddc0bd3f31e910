// SpMV kernels for gfx950: y <- A*x + y.
//
// All kernels accumulate into y (PMPP notes, "Sparse Matrices and Basic
// Formats (COO & CSR)": SpMV computes A*X + Y; its CSR kernel adds the row sum
// into y[row]).  Streams of matrix data are read with non-temporal loads so the
// gathered x stays resident in the per-XCD L2.
//
// y updates: ELL reads y together with its matrix stream (coalesced, issued
// early) and writes y once.  Every other kernel adds its row sums with
// non-returning hardware fp32 atomics: a scattered or late read of y would
// stall the wave, a non-returning atomic does not, and a row that receives a
// single contribution still ends as exactly y + sum.  Rows split over several
// waves or blocks (COO runs, deep JDS tiles, merge-path boundary rows) get one
// atomic per piece.  Rows without nonzeros are never written.
#include <cmath>

#include "internal.h"

namespace spmv {
namespace {

constexpr int kThreads = 256;

__device__ inline void atomic_add_f32(float *p, float v) { unsafeAtomicAdd(p, v); }

// x[c], kept only where the lane's condition holds.  c must be a column on
// every lane (the kernels set it to 0 where a lane has no entry), so the load
// needs no per-lane branch: a branch around a gather makes the wave wait for
// it before the next one is issued, while unconditional gathers all go out
// before the first is used.  The condition goes through a lane mask (ballot,
// then inverse ballot), since a select on a plain comparison whose operand is
// a just-loaded value is turned back into a branch around the load.
__device__ inline float gather_kept(const float *__restrict__ x, int32_t c, bool keep) {
    const float g = x[c];
    return __builtin_amdgcn_inverse_ballot_w64(__builtin_amdgcn_ballot_w64(keep)) ? g : 0.f;
}

__device__ inline void lds_add_f32(float *p, float v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// ---------------------------------------------------------------------------
// COO, one atomic add per nonzero [COO/CSR page, COO kernel: each thread takes
// a nonzero; two threads may hit the same y[row], hence the atomic add].  The
// entries are row-sorted, so neighbouring entries usually share a row, and
// same-address atomics in one wave instruction serialise in the L2.  Each
// lane therefore takes RUN consecutive entries (16-byte loads) and the wave
// issues its atomics run position by run position: the lanes of one atomic
// instruction are RUN entries apart, in different rows whenever rows are
// shorter than RUN.  The launcher picks RUN from the row-length statistics.
// ---------------------------------------------------------------------------
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int RUN>
__global__ __launch_bounds__(kThreads) void k_coo_atomic(int32_t nnz,
                                                         const int32_t *__restrict__ row,
                                                         const int32_t *__restrict__ col,
                                                         const float *__restrict__ val,
                                                         const float *__restrict__ x,
                                                         float *__restrict__ y) {
    static_assert(RUN % 4 == 0, "16-byte loads");
    const int64_t base = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) * RUN;
    if (base >= nnz) return;
    int32_t r[RUN], c[RUN];
    float v[RUN];
    if (base + RUN <= nnz) {
#pragma unroll
        for (int k = 0; k < RUN; k += 4) {
            const i32x4 rr = ld_nt(reinterpret_cast<const i32x4 *>(row + base + k));
            const i32x4 cc = ld_nt(reinterpret_cast<const i32x4 *>(col + base + k));
            const f32x4 vv = ld_nt(reinterpret_cast<const f32x4 *>(val + base + k));
            r[k] = rr.x; r[k + 1] = rr.y; r[k + 2] = rr.z; r[k + 3] = rr.w;
            c[k] = cc.x; c[k + 1] = cc.y; c[k + 2] = cc.z; c[k + 3] = cc.w;
            v[k] = vv.x; v[k + 1] = vv.y; v[k + 2] = vv.z; v[k + 3] = vv.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < RUN; ++k) {
            const bool ok = base + k < nnz;
            r[k] = ok ? row[base + k] : 0;
            c[k] = ok ? col[base + k] : 0;
            v[k] = ok ? val[base + k] : 0.f;
        }
    }
    float xv[RUN];
#pragma unroll
    for (int k = 0; k < RUN; ++k) xv[k] = gather_kept(x, c[k], base + k < nnz);
#pragma unroll
    for (int k = 0; k < RUN; ++k)
        if (base + k < nnz) atomic_add_f32(&y[r[k]], v[k] * xv[k]);
}

// ---------------------------------------------------------------------------
// COO segmented: the COO entries are sorted by row.  One wave walks 64*8
// consecutive entries, 64 at a time (coalesced); a segmented inclusive scan
// over the wave (DPP row shifts and row broadcasts, no LDS permutes) sums each
// run of equal rows, the last lane of a run adds the
// run's total into y, and the wave's last run is carried into the next 64
// entries.  Used for COO input, the HYB tail and short-row x slices.
// ---------------------------------------------------------------------------

// one step of a segmented inclusive scan by DPP (GFX9 wave scan: row shifts
// 1/2/4/8, then row_bcast:15 and row_bcast:31); lanes without a source get a
// key no row has
template <int CTRL, int RMASK>
__device__ inline void seg_step(int32_t r, float &p) {
    const int32_t ru = __builtin_amdgcn_update_dpp(INT32_MIN, r, CTRL, RMASK, 0xF, false);
    const float pu = __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, p), CTRL, RMASK, 0xF, false));
    if (ru == r) p += pu;
}

constexpr int kSegIters = 8;

__global__ __launch_bounds__(kThreads) void k_coo_segmented(int32_t nnz,
                                                            const int32_t *__restrict__ row,
                                                            const int32_t *__restrict__ col,
                                                            const float *__restrict__ val,
                                                            const float *__restrict__ x,
                                                            float *__restrict__ y) {
    const int lane = __lane_id();
    const int64_t wave = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / kWave;
    const int64_t base = wave * (kWave * kSegIters);
    if (base >= nnz) return;
    // Every run total goes to y with a non-returning hardware atomic: unlike a
    // plain read-modify-write it never makes the wave wait on a scattered load
    // (measured faster on MI355X even for runs no other wave touches).
    auto flush = [&](int32_t r, float v) { atomic_add_f32(&y[r], v); };
    // all 8 batches' loads, then all 8 gathers, before the first scan
    int32_t rr[kSegIters], cc[kSegIters];
    float vv[kSegIters], pp[kSegIters];
#pragma unroll
    for (int it = 0; it < kSegIters; ++it) {
        const int64_t i = base + it * kWave + lane;
        const bool valid = i < nnz;
        rr[it] = valid ? ld_nt(row + i) : INT32_MAX;
        cc[it] = valid ? ld_nt(col + i) : 0;
        vv[it] = valid ? ld_nt(val + i) : 0.f;
    }
#pragma unroll
    for (int it = 0; it < kSegIters; ++it)   // vv = 0 where there is no entry
        pp[it] = vv[it] * gather_kept(x, cc[it], rr[it] != INT32_MAX);
    int carry_row = INT32_MAX;
    float carry = 0.f;
#pragma unroll
    for (int it = 0; it < kSegIters; ++it) {
        const int64_t i = base + it * kWave + lane;
        const bool valid = i < nnz;
        const int32_t r = rr[it];
        float p = pp[it];
        seg_step<0x111, 0xF>(r, p);
        seg_step<0x112, 0xF>(r, p);
        seg_step<0x114, 0xF>(r, p);
        seg_step<0x118, 0xF>(r, p);
        seg_step<0x142, 0xA>(r, p);
        seg_step<0x143, 0xC>(r, p);
        // The carried run either continues into this batch (same row as lane
        // 0) or ended exactly at the previous batch's last entry: flush it.
        const int32_t r_first = __builtin_amdgcn_readfirstlane(r);
        if (carry_row != INT32_MAX && carry_row != r_first && lane == 0) flush(carry_row, carry);
        if (r == carry_row) p += carry;
        const int32_t rn = __shfl_down(r, 1);
        if (valid && lane != kWave - 1 && rn != r) flush(r, p);
        carry_row = __builtin_amdgcn_readlane(r, kWave - 1);
        carry = __builtin_bit_cast(float,
                                   __builtin_amdgcn_readlane(__builtin_bit_cast(int, p), kWave - 1));
    }
    if (lane == 0 && carry_row != INT32_MAX) flush(carry_row, carry);
}

// ---------------------------------------------------------------------------
// CSR scalar: one lane per row [COO/CSR page, CSR kernel; format-choice
// article 2.1], with the block's 257 row pointers staged in LDS (article 4.2).
// ---------------------------------------------------------------------------
// CSR scalar with the rows' entries staged through LDS: a wave's 64 rows
// are one contiguous CSR segment; when it holds at most kCsrStage entries the
// wave copies its columns and values into LDS with coalesced loads (skewed one
// word per 32 against bank conflicts), then every lane walks its own row from
// LDS.  Longer segments read their rows directly.  The sum of each row is
// taken in the same order as k_csr_scalar, so the two give the same bits.
constexpr int kCsrStage = 2048;   // entries per wave staged in LDS
__device__ inline int csr_skew(int i) { return i + (i >> 5); }
constexpr int kCsrStageWords = kCsrStage + kCsrStage / 32;

__global__ __launch_bounds__(kThreads) void k_csr_scalar_lds(int32_t R, const int32_t *__restrict__ rp,
                                                         const int32_t *__restrict__ col,
                                                         const float *__restrict__ val,
                                                         const float *__restrict__ x,
                                                         float *__restrict__ y) {
    __shared__ int32_t s_col[kThreads / kWave][kCsrStageWords];
    __shared__ float s_val[kThreads / kWave][kCsrStageWords];
    const uint32_t b = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t r = static_cast<int64_t>(b) * kThreads + threadIdx.x;
    const int w = threadIdx.x / kWave;
    const int lane = __lane_id();
    const bool ok = r < R;
    const int32_t a = ok ? ld_nt(rp + r) : 0;
    const int32_t e = ok ? ld_nt(rp + r + 1) : 0;
    const unsigned long long live = __ballot(ok);
    if (!live) return;
    const int last = 63 - __clzll(static_cast<long long>(live));
    const int32_t s0 = __builtin_amdgcn_readfirstlane(a);
    const int32_t s1 = __shfl(e, last);
    const int64_t seg = static_cast<int64_t>(s1) - s0;
    const uint32_t len = static_cast<uint32_t>(e - a);
    float sum = 0.f;
    if (seg <= kCsrStage) {   // wave-uniform
        const int32_t n = static_cast<int32_t>(seg);
        int32_t i = lane;
        for (; i + 3 * kWave < n; i += 4 * kWave) {
            const int32_t c0 = ld_nt(col + s0 + i), c1 = ld_nt(col + s0 + i + kWave),
                          c2 = ld_nt(col + s0 + i + 2 * kWave), c3 = ld_nt(col + s0 + i + 3 * kWave);
            const float v0 = ld_nt(val + s0 + i), v1 = ld_nt(val + s0 + i + kWave),
                        v2 = ld_nt(val + s0 + i + 2 * kWave), v3 = ld_nt(val + s0 + i + 3 * kWave);
            s_col[w][csr_skew(i)] = c0; s_col[w][csr_skew(i + kWave)] = c1;
            s_col[w][csr_skew(i + 2 * kWave)] = c2; s_col[w][csr_skew(i + 3 * kWave)] = c3;
            s_val[w][csr_skew(i)] = v0; s_val[w][csr_skew(i + kWave)] = v1;
            s_val[w][csr_skew(i + 2 * kWave)] = v2; s_val[w][csr_skew(i + 3 * kWave)] = v3;
        }
        for (; i < n; i += kWave) {
            s_col[w][csr_skew(i)] = ld_nt(col + s0 + i);
            s_val[w][csr_skew(i)] = ld_nt(val + s0 + i);
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        if (!ok || len == 0) return;
        const int32_t off = a - s0;
        for (uint32_t t = 0; t < len; ++t) {
            const int k = csr_skew(off + static_cast<int32_t>(t));
            sum += s_val[w][k] * x[s_col[w][k]];
        }
    } else {
        if (!ok || len == 0) return;
        const int32_t *rc = col + a;
        const float *rv = val + a;
        uint32_t o = 0;
        for (; o + 4 <= len; o += 4) {
            const int32_t c0 = ld_nt(rc + o), c1 = ld_nt(rc + o + 1), c2 = ld_nt(rc + o + 2),
                          c3 = ld_nt(rc + o + 3);
            const float v0 = ld_nt(rv + o), v1 = ld_nt(rv + o + 1), v2 = ld_nt(rv + o + 2),
                        v3 = ld_nt(rv + o + 3);
            sum += v0 * x[c0];
            sum += v1 * x[c1];
            sum += v2 * x[c2];
            sum += v3 * x[c3];
        }
        for (; o < len; ++o) sum += ld_nt(rv + o) * x[ld_nt(rc + o)];
    }
    atomic_add_f32(&y[r], sum);
}

__global__ __launch_bounds__(kThreads) void k_csr_scalar(int32_t R, const int32_t *__restrict__ rp,
                                                         const int32_t *__restrict__ col,
                                                         const float *__restrict__ val,
                                                         const float *__restrict__ x,
                                                         float *__restrict__ y) {
    __shared__ int32_t srp[kThreads + 1];
    const uint32_t b = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t r0 = static_cast<int64_t>(b) * kThreads;
    const int64_t r = r0 + threadIdx.x;
    if (r <= R) srp[threadIdx.x] = ld_nt(rp + r);
    if (threadIdx.x == 0 && r0 + kThreads <= R) srp[kThreads] = ld_nt(rp + r0 + kThreads);
    __syncthreads();
    if (r >= R) return;
    const int32_t a = srp[threadIdx.x], e = srp[threadIdx.x + 1];
    if (a == e) return;
    // offsets inside the row, unsigned: a row may end at INT32_MAX, and
    // o + 4 <= len < 2^31 + 4 cannot wrap in 32 bits
    const int32_t *rc = col + a;
    const float *rv = val + a;
    const uint32_t len = static_cast<uint32_t>(e - a);
    float sum = 0.f;
    uint32_t o = 0;
    for (; o + 4 <= len; o += 4) {
        const int32_t c0 = ld_nt(rc + o), c1 = ld_nt(rc + o + 1), c2 = ld_nt(rc + o + 2),
                      c3 = ld_nt(rc + o + 3);
        const float v0 = ld_nt(rv + o), v1 = ld_nt(rv + o + 1), v2 = ld_nt(rv + o + 2),
                    v3 = ld_nt(rv + o + 3);
        sum += v0 * x[c0];
        sum += v1 * x[c1];
        sum += v2 * x[c2];
        sum += v3 * x[c3];
    }
    for (; o < len; ++o) sum += ld_nt(rv + o) * x[ld_nt(rc + o)];
    atomic_add_f32(&y[r], sum);
}

// ---------------------------------------------------------------------------
// CSR vector: a group of L lanes per row (format-choice article 2.2 gives one
// 32-lane warp per row; here L = 2..64 of a 64-lane wavefront).  Lanes stride
// the row by L; the group sum uses DPP / ds_swizzle (group_sum).
// ---------------------------------------------------------------------------
template <int L, int kRpg>
__global__ __launch_bounds__(kThreads) void k_csr_vector(int32_t R, const int32_t *__restrict__ rp,
                                                         const int32_t *__restrict__ col,
                                                         const float *__restrict__ val,
                                                         const float *__restrict__ x,
                                                         float *__restrict__ y) {
    // Each group of L lanes takes kRpg rows, interleaved so that at every step
    // the block's groups work on consecutive rows (contiguous nonzeros).  The
    // first 2 elements per lane of all kRpg rows are loaded before any gather,
    // so a wave keeps 2*kRpg loads per lane in flight; longer rows finish in a
    // remainder loop.  kRpg = 4 only when no row needs the remainder loop and
    // the grid stays large (run_vector); otherwise one row per group.
    constexpr int kGroups = kThreads / L;
    constexpr int kRows = kGroups * kRpg;
    __shared__ int32_t srp[kRows + 1];
    const uint32_t b = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t r0 = static_cast<int64_t>(b) * kRows;
    for (int i = threadIdx.x; i <= kRows; i += kThreads)
        if (r0 + i <= R) srp[i] = ld_nt(rp + r0 + i);
    __syncthreads();
    const int g = threadIdx.x / L, lg = threadIdx.x % L;
    // Offsets inside a row are unsigned and relative to the row start: a row
    // may end at INT32_MAX, and offset + 4L stays below 2^32.
    int32_t a[kRpg], c0[kRpg], c1[kRpg];
    uint32_t n[kRpg];
    float v0[kRpg], v1[kRpg], acc[kRpg];
#pragma unroll
    for (int m = 0; m < kRpg; ++m) {
        const int lr = m * kGroups + g;
        const bool ok = r0 + lr < R;
        a[m] = ok ? srp[lr] : 0;
        n[m] = ok ? static_cast<uint32_t>(srp[lr + 1] - a[m]) : 0u;
        const uint32_t j = lg;
        c0[m] = j < n[m] ? ld_nt(col + a[m] + j) : 0;
        v0[m] = j < n[m] ? ld_nt(val + a[m] + j) : 0.f;
        c1[m] = j + L < n[m] ? ld_nt(col + a[m] + (j + L)) : 0;
        v1[m] = j + L < n[m] ? ld_nt(val + a[m] + (j + L)) : 0.f;
    }
#pragma unroll
    for (int m = 0; m < kRpg; ++m) {
        const uint32_t j = lg;
        const float x0 = j < n[m] ? x[c0[m]] : 0.f;
        const float x1 = j + L < n[m] ? x[c1[m]] : 0.f;
        acc[m] = v0[m] * x0 + v1[m] * x1;
        // long rows: 4 elements per lane per step, loads before gathers
        const int32_t *rc = col + a[m];
        const float *rv = val + a[m];
        uint32_t jj = j + 2 * L;
        for (; jj + 3 * L < n[m]; jj += 4 * L) {
            int32_t cq[4];
            float vq[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                cq[q] = ld_nt(rc + (jj + q * L));
                vq[q] = ld_nt(rv + (jj + q * L));
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[m] += vq[q] * x[cq[q]];
        }
        for (; jj < n[m]; jj += L) acc[m] += ld_nt(rv + jj) * x[ld_nt(rc + jj)];
    }
#pragma unroll
    for (int m = 0; m < kRpg; ++m) {
        const float sum = group_sum<L>(acc[m]);
        const int64_t r = r0 + m * kGroups + g;
        if (lg == 0 && n[m] > 0) atomic_add_f32(&y[r], sum);
    }
}

// ---------------------------------------------------------------------------
// ELL: one lane per row, slot t of row r at t*R + r, so at every step the
// lanes of a wave read one contiguous 256-byte run of values and of columns
// [Regularized formats page, ELL section].  Slots past nnzPerRow[r] are
// padding and contribute nothing.  The slots are walked U at a time with the
// next U slots' loads issued before the current U gathers, so every wave keeps
// its HBM stream in flight while it waits on x.  The first U slots are loaded
// alongside nnzPerRow[r]; later slots only up to the row's length, so a lane
// past its row issues no loads (the page's kernel likewise stops at each row's
// own length): HYB's width-150 ELL part on the power-law matrix 1.52 -> 1.27 ms,
// no change on full rows.
// ---------------------------------------------------------------------------
template <int U>
__global__ __launch_bounds__(kThreads) void k_ell(int32_t R, int32_t W,
                                                  const int32_t *__restrict__ ell_col,
                                                  const float *__restrict__ ell_val,
                                                  const int32_t *__restrict__ ell_nnz,
                                                  const float *__restrict__ x,
                                                  float *__restrict__ y) {
    const uint32_t b = xcd_remap(blockIdx.x, gridDim.x);
    const uint32_t r = b * kThreads + threadIdx.x;
    if (r >= static_cast<uint32_t>(R)) return;
    const uint32_t ru = static_cast<uint32_t>(R);
    const int32_t n = ld_nt(ell_nnz + r);
    const float y0 = ld_nt(y + r);   // y is streamed too: non-temporal
    int32_t c[U];
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t slot = static_cast<uint32_t>(u) * ru + r;
        c[u] = u < W ? ld_nt(ell_col + slot) : 0;
        v[u] = u < W ? ld_nt(ell_val + slot) : 0.f;
    }
    float sum = 0.f;
    // slot counters unsigned: W may be INT32_MAX (one row), and t0 + 2U stays
    // below 2^32; a slot t*R + r is formed only for t < W, where it is < 2^31
    const uint32_t wu = static_cast<uint32_t>(W), nu = static_cast<uint32_t>(n);
    for (uint32_t t0 = 0; t0 < wu; t0 += U) {
        int32_t cn[U];
        float vn[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t t = t0 + U + u;
            const uint32_t slot = t * ru + r;
            cn[u] = t < nu ? ld_nt(ell_col + slot) : 0;
            vn[u] = t < nu ? ld_nt(ell_val + slot) : 0.f;
        }
        float xv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) xv[u] = (t0 + u < nu) ? x[c[u]] : 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u) sum += v[u] * xv[u];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            c[u] = cn[u];
            v[u] = vn[u];
        }
    }
    if (n > 0) __builtin_nontemporal_store(y0 + sum, y + r);
}

// ELL, 4 consecutive rows per lane: for narrow widths the wave's slot loads
// become 16-byte vectors (1 KB per wave per array) and every lane keeps 4x
// the gathers in flight; measured faster than one row per lane on the random
// 5-per-row matrix (1M rows), slower on the 27-wide stencil and on small
// grids.  Needs R % 4 == 0 and a 16-byte aligned y (checked by the launcher).
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(kThreads) void k_ell4(int32_t R, int32_t W,
                                                   const int32_t *__restrict__ ell_col,
                                                   const float *__restrict__ ell_val,
                                                   const int32_t *__restrict__ ell_nnz,
                                                   const float *__restrict__ x,
                                                   float *__restrict__ y) {
    const uint32_t q = xcd_remap(blockIdx.x, gridDim.x) * kThreads + threadIdx.x;
    const uint32_t r = q * 4;   // first of the lane's 4 rows
    if (r >= static_cast<uint32_t>(R)) return;
    const uint32_t ru = static_cast<uint32_t>(R), wu = static_cast<uint32_t>(W);
    const i32x4 n = ld_nt(reinterpret_cast<const i32x4 *>(ell_nnz + r));
    const f32x4 y0 = ld_nt(reinterpret_cast<const f32x4 *>(y + r));
    const uint32_t nmax = static_cast<uint32_t>(max(max(n.x, n.y), max(n.z, n.w)));
    i32x4 c[U];
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t slot = static_cast<uint32_t>(u) * ru + r;
        c[u] = u < W ? ld_nt(reinterpret_cast<const i32x4 *>(ell_col + slot)) : i32x4(0);
        v[u] = u < W ? ld_nt(reinterpret_cast<const f32x4 *>(ell_val + slot)) : f32x4(0.f);
    }
    f32x4 sum = f32x4(0.f);
    for (uint32_t t0 = 0; t0 < wu; t0 += U) {
        i32x4 cn[U];
        f32x4 vn[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t t = t0 + U + u;
            const uint32_t slot = t * ru + r;
            cn[u] = t < nmax ? ld_nt(reinterpret_cast<const i32x4 *>(ell_col + slot)) : i32x4(0);
            vn[u] = t < nmax ? ld_nt(reinterpret_cast<const f32x4 *>(ell_val + slot)) : f32x4(0.f);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t t = t0 + u;
            if (t < nmax) {
                f32x4 xv;
                xv.x = t < static_cast<uint32_t>(n.x) ? x[c[u].x] : 0.f;
                xv.y = t < static_cast<uint32_t>(n.y) ? x[c[u].y] : 0.f;
                xv.z = t < static_cast<uint32_t>(n.z) ? x[c[u].z] : 0.f;
                xv.w = t < static_cast<uint32_t>(n.w) ? x[c[u].w] : 0.f;
                sum += v[u] * xv;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            c[u] = cn[u];
            v[u] = vn[u];
        }
    }
    // rows without entries are written back unchanged (bit-identical y)
    f32x4 out = y0;
    if (n.x > 0) out.x = y0.x + sum.x;
    if (n.y > 0) out.y = y0.y + sum.y;
    if (n.z > 0) out.z = y0.z + sum.z;
    if (n.w > 0) out.w = y0.w + sum.w;
    __builtin_nontemporal_store(out, reinterpret_cast<f32x4 *>(y + r));
}

// ---------------------------------------------------------------------------
// ELL with x tiles: the block of 256 rows first copies its x tile into LDS,
// run by run (a wave per run, lanes over consecutive columns: coalesced), then
// each lane walks its row's ELL slots as k_ell does, reading 16-bit tile
// positions instead of 32-bit columns and gathering x from LDS instead of
// through the vector memory path (which bounds k_ell on banded matrices).
// ---------------------------------------------------------------------------
template <int U>
__global__ __launch_bounds__(kThreads) void k_ell_xtile(int32_t R, int32_t W,
                                                        const int32_t *__restrict__ run_ptr,
                                                        const int32_t *__restrict__ runs,
                                                        const int16_t *__restrict__ lidx,
                                                        const float *__restrict__ ell_val,
                                                        const int32_t *__restrict__ ell_nnz,
                                                        const float *__restrict__ x,
                                                        float *__restrict__ y) {
    extern __shared__ float tile[];
    const uint32_t b = xcd_remap(blockIdx.x, gridDim.x);
    const int k0 = run_ptr[b], k1 = run_ptr[b + 1];
    const int lane = __lane_id();
    // a wave per run; each lane keeps 8 loads in flight before its LDS stores
    constexpr int kCopy = 8;
    for (int k = k0 + static_cast<int>(threadIdx.x / kWave); k < k1; k += kThreads / kWave) {
        const int64_t q = 3 * static_cast<int64_t>(k);
        const int32_t start = runs[q], off = runs[q + 1], len = runs[q + 2];
        for (int i0 = 0; i0 < len; i0 += kCopy * kWave) {
            float v[kCopy];
#pragma unroll
            for (int u = 0; u < kCopy; ++u) {
                const int i = i0 + u * kWave + lane;
                v[u] = i < len ? x[start + i] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < kCopy; ++u) {
                const int i = i0 + u * kWave + lane;
                if (i < len) tile[off + i] = v[u];
            }
        }
    }
    __syncthreads();
    const uint32_t r = b * kThreads + threadIdx.x;
    if (r >= static_cast<uint32_t>(R)) return;
    const uint32_t ru = static_cast<uint32_t>(R), wu = static_cast<uint32_t>(W);
    const int32_t n = ld_nt(ell_nnz + r);
    const float y0 = ld_nt(y + r);
    int32_t c[U];
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t slot = static_cast<uint32_t>(u) * ru + r;
        c[u] = u < W ? ld_nt(lidx + slot) : 0;
        v[u] = u < W ? ld_nt(ell_val + slot) : 0.f;
    }
    float sum = 0.f;
    for (uint32_t t0 = 0; t0 < wu; t0 += U) {
        int32_t cn[U];
        float vn[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t t = t0 + U + u;
            const uint32_t slot = t * ru + r;
            cn[u] = t < static_cast<uint32_t>(n) ? ld_nt(lidx + slot) : 0;
            vn[u] = t < static_cast<uint32_t>(n) ? ld_nt(ell_val + slot) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (t0 + u < static_cast<uint32_t>(n)) sum += v[u] * tile[c[u]];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            c[u] = cn[u];
            v[u] = vn[u];
        }
    }
    if (n > 0) __builtin_nontemporal_store(y0 + sum, y + r);
}

// ---------------------------------------------------------------------------
// JDS: rows sorted by length (longest first) in jagged columns; entry t of
// sorted row s at iterPtr[t] + s [Regularized formats page, JDS section: one
// thread per row, iterPtr gives each iteration's start].  One wave takes a
// tile of 64 consecutive sorted rows x `depth` jagged columns, so a few very
// long rows are split over many waves instead of serialising one lane; the
// split rows are combined with atomics.  iterPtr[t] is wave-uniform (scalar
// load); lane s reads iterPtr[t] + s, contiguous across the wave.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_jds(int32_t R, int32_t ntiles, int32_t depth,
                                                  const int2 *__restrict__ tiles,
                                                  const int32_t *__restrict__ jds_len,
                                                  const int32_t *__restrict__ iter_ptr,
                                                  const int32_t *__restrict__ perm,
                                                  const int32_t *__restrict__ col,
                                                  const float *__restrict__ val,
                                                  const float *__restrict__ x,
                                                  float *__restrict__ y) {
    const int64_t tile = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / kWave;
    if (tile >= ntiles) return;
    const int lane = __lane_id();
    const int2 gc = tiles[tile];
    const int g = __builtin_amdgcn_readfirstlane(gc.x);
    const int chunk = __builtin_amdgcn_readfirstlane(gc.y);
    const int64_t s = static_cast<int64_t>(g) * kWave + lane;
    const int32_t len = s < R ? ld_nt(jds_len + s) : 0;
    const int32_t glen = __builtin_amdgcn_readfirstlane(jds_len[static_cast<int64_t>(g) * kWave]);
    // jagged-column counters in 64 bits: a row may hold INT32_MAX entries
    const int64_t t0 = static_cast<int64_t>(chunk) * depth;
    const int64_t t1 = min(t0 + depth, static_cast<int64_t>(glen));
    // jagged columns U at a time, the next U columns' loads issued before the
    // current U gathers (as in ELL)
    constexpr int U = 8;
    int32_t c[U];
    float v[U];
    auto load = [&](int64_t tb, int32_t *cc, float *vv) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t t = tb + u;
            const int32_t p = t < t1 ? iter_ptr[t] : 0;   // wave-uniform
            const bool ok = t < t1 && t < len;
            cc[u] = ok ? ld_nt(col + p + s) : 0;
            vv[u] = ok ? ld_nt(val + p + s) : 0.f;
        }
    };
    load(t0, c, v);
    float sum = 0.f;
    for (int64_t tb = t0; tb < t1; tb += U) {
        int32_t cn[U];
        float vn[U];
        load(tb + U, cn, vn);
        float xv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) xv[u] = gather_kept(x, c[u], tb + u < t1 && tb + u < len);
#pragma unroll
        for (int u = 0; u < U; ++u) sum += v[u] * xv[u];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            c[u] = cn[u];
            v[u] = vn[u];
        }
    }
    // y[perm[s]] is scattered: a non-returning atomic never stalls the wave on a
    // load (and with one contribution per row the result is still exact-order).
    if (len > t0) atomic_add_f32(&y[ld_nt(perm + s)], sum);
}

// ---------------------------------------------------------------------------
// Sectioned ELL, the JDS variant [Regularized formats page, JDS variant
// section]: section k = 64 consecutive sorted rows, an ELL padded to its own
// longest row, column-major inside the section: entry t of its row i at
// sect_ptr[k] + t*m_k + i.  One wave per (section, chunk of `depth` padded
// columns); a step reads one contiguous run of m_k words, with no per-column
// pointer load (unlike JDS); the next U columns are loaded before the current
// U gathers.  Padding lanes (t >= the row's length) load nothing.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_sell(int32_t R, int32_t ntiles, int32_t depth,
                                                   const int2 *__restrict__ tiles,
                                                   const int32_t *__restrict__ sell_len,
                                                   const int32_t *__restrict__ sect_ptr,
                                                   const int32_t *__restrict__ perm,
                                                   const int32_t *__restrict__ col,
                                                   const float *__restrict__ val,
                                                   const float *__restrict__ x,
                                                   float *__restrict__ y) {
    const int64_t tile = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / kWave;
    if (tile >= ntiles) return;
    const int lane = __lane_id();
    const int2 gc = tiles[tile];
    const int k = __builtin_amdgcn_readfirstlane(gc.x);
    const int chunk = __builtin_amdgcn_readfirstlane(gc.y);
    const int64_t first = static_cast<int64_t>(k) * kWave;
    const int32_t m = static_cast<int32_t>(min(static_cast<int64_t>(kWave), R - first));
    const int64_t s = first + lane;
    const int32_t len = lane < m ? ld_nt(sell_len + s) : 0;
    const int32_t width = __builtin_amdgcn_readfirstlane(sell_len[first]);
    const int64_t base = __builtin_amdgcn_readfirstlane(sect_ptr[k]);
    const int64_t t0 = static_cast<int64_t>(chunk) * depth;
    const int64_t t1 = min(t0 + depth, static_cast<int64_t>(width));
    constexpr int U = 8;
    int32_t c[U];
    float v[U];
    auto load = [&](int64_t tb, int32_t *cc, float *vv) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t t = tb + u;
            const bool ok = t < t1 && t < len;
            const int64_t slot = base + t * m + lane;
            cc[u] = ok ? ld_nt(col + slot) : 0;
            vv[u] = ok ? ld_nt(val + slot) : 0.f;
        }
    };
    load(t0, c, v);
    float sum = 0.f;
    for (int64_t tb = t0; tb < t1; tb += U) {
        int32_t cn[U];
        float vn[U];
        load(tb + U, cn, vn);
        float xv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) xv[u] = gather_kept(x, c[u], tb + u < t1 && tb + u < len);
#pragma unroll
        for (int u = 0; u < U; ++u) sum += v[u] * xv[u];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            c[u] = cn[u];
            v[u] = vn[u];
        }
    }
    if (len > t0) atomic_add_f32(&y[ld_nt(perm + s)], sum);
}

constexpr int kMaxMergeSlices = 8;

// ---------------------------------------------------------------------------
// Merge-path CSR [format-choice article 5.2: merge-based CSR for power-law
// graphs; "Introduction to sparse computing", parallel efficiency: split by
// nonzero count, split long rows].  The rows' end markers and the nonzeros
// form one sequence of R + nnz items; block b owns items
// [b*NB, (b+1)*NB) (NB = kMergeItemsPerBlock), starting at row row_start[b].
// The block stages its row ends and its products val*x[col] (coalesced loads)
// in LDS, each thread consumes kMergeItemsPerThread items of the merged
// sequence and adds its per-row partial sums
// into LDS accumulators, then the block adds each row's sum into y (a row cut
// by the block's ends receives one piece from each block it touches).
// ---------------------------------------------------------------------------
__device__ inline void merge_tile(int32_t tile, int32_t R, int32_t nnz,
                                                         const int32_t *__restrict__ row_start,
                                                         const int32_t *__restrict__ rp,
                                                         const int32_t *__restrict__ col,
                                                         const float *__restrict__ val,
                                                         const float *__restrict__ x,
                                                         float *__restrict__ y,
                                                         int32_t *s_end, float *s_prod,
                                                         float *s_acc) {
    constexpr int NB = kMergeItemsPerBlock;
    constexpr int IPT = kMergeItemsPerThread;
    const int tid = threadIdx.x;
    const int64_t total = static_cast<int64_t>(R) + nnz;
    const int64_t d0 = static_cast<int64_t>(tile) * NB;
    const int64_t d1 = min(d0 + NB, total);
    const int32_t r0 = row_start[tile];
    const int32_t r1 = row_start[tile + 1];
    const int32_t k0 = static_cast<int32_t>(d0 - r0);
    const int32_t k1 = static_cast<int32_t>(d1 - r1);
    const int32_t nr = r1 - r0;
    const int32_t nk = k1 - k0;

    for (int i = tid; i < nr; i += kMergeThreads) s_end[i] = ld_nt(rp + r0 + 1 + i) - k0;
    for (int j = tid; j < nk; j += kMergeThreads) {
        const int32_t kk = k0 + j;
        s_prod[j] = ld_nt(val + kk) * x[ld_nt(col + kk)];
    }
    for (int i = tid; i <= nr; i += kMergeThreads) s_acc[i] = 0.f;
    __syncthreads();

    // Start of this thread's IPT items on the merge path: the number i of row
    // ends before diagonal dt (row end i sits at local position s_end[i] + i).
    const int32_t items = nr + nk;
    const int32_t dt = min(tid * IPT, items);
    int32_t lo = max(0, dt - nk), hi = min(dt, nr);
    while (lo < hi) {
        const int32_t mid = (lo + hi) >> 1;
        if (s_end[mid] + mid < dt) lo = mid + 1; else hi = mid;
    }
    // A row whose end item lies in this thread's range has exactly one such
    // thread: it stores its part of the row with a plain LDS write.  What a
    // thread holds of the row still open at the end of its range (its tail)
    // belongs to a row ending in a later thread; the tails are combined below.
    // (LDS float atomics cost ~190 clocks per wave instruction on gfx950,
    // plain LDS writes a few clocks.)
    int32_t i = lo, k = dt - lo;
    const int32_t dend = min(dt + IPT, items);
    float sum = 0.f;
    bool any = false;
    for (int32_t d = dt; d < dend; ++d) {
        if (i < nr && k >= s_end[i]) {   // row i ends here
            if (any) s_acc[i] = sum;
            sum = 0.f;
            any = false;
            ++i;
        } else {
            sum += s_prod[k];
            ++k;
            any = true;
        }
    }
    __syncthreads();
    // Tails, in thread order, have non-decreasing rows: a segmented scan over
    // the wave sums each run of equal rows, and the run's last lane adds it to
    // the row's LDS accumulator.  A run that starts at lane 0 or reaches lane
    // 63 may share its row with a neighbouring wave's run: those two add
    // atomically; every other run is the only writer of its row after the
    // barrier above.
    {
        const int lane = __lane_id();
        const int32_t tr = any ? i : INT32_MAX;
        float p = any ? sum : 0.f;
        seg_step<0x111, 0xF>(tr, p);
        seg_step<0x112, 0xF>(tr, p);
        seg_step<0x114, 0xF>(tr, p);
        seg_step<0x118, 0xF>(tr, p);
        seg_step<0x142, 0xA>(tr, p);
        seg_step<0x143, 0xC>(tr, p);
        const int32_t tn = __shfl_down(tr, 1);
        const int32_t t_first = __builtin_amdgcn_readfirstlane(tr);
        if (tr != INT32_MAX && (lane == kWave - 1 || tn != tr)) {
            if (lane == kWave - 1 || tr == t_first) lds_add_f32(&s_acc[tr], p);
            else s_acc[tr] += p;
        }
    }
    __syncthreads();

    for (int li = tid; li <= nr; li += kMergeThreads) {
        const int32_t r = r0 + li;
        if (r >= R) continue;
        const int32_t start = li == 0 ? rp[r0] - k0 : s_end[li - 1];   // local offsets
        const int32_t end = li < nr ? s_end[li] : nk;
        const int32_t lo_k = max(start, 0), hi_k = min(end, nk);
        if (hi_k <= lo_k) continue;                 // no nonzero of row r in this block
        atomic_add_f32(&y[r], s_acc[li]);
    }
}

__global__ __launch_bounds__(kMergeThreads) void k_merge(int32_t R, int32_t nnz,
                                                         const int32_t *__restrict__ row_start,
                                                         const int32_t *__restrict__ rp,
                                                         const int32_t *__restrict__ col,
                                                         const float *__restrict__ val,
                                                         const float *__restrict__ x,
                                                         float *__restrict__ y) {
    __shared__ int32_t s_end[kMergeItemsPerBlock];
    __shared__ float s_prod[kMergeItemsPerBlock];
    __shared__ float s_acc[kMergeItemsPerBlock + 1];
    merge_tile(static_cast<int32_t>(blockIdx.x), R, nnz, row_start, rp, col, val, x, y, s_end,
               s_prod, s_acc);
}

// All x slices of a handle in one launch, each slice pinned to its own XCDs:
// blocks reach the 8 XCDs round-robin (block b on XCD b % 8), slice k takes
// XCDs [k * per, (k + 1) * per) with per = 8 / n, so every XCD's L2 holds
// one slice of x while the slices run side by side.  Every row's sum goes to
// y by an atomic add, so slices may overlap in time.  Blocks past their
// slice's tile count exit at once.
struct MergeSlices {
    int32_t n;
    int32_t nnz[kMaxMergeSlices];
    int32_t tiles[kMaxMergeSlices];
    const int32_t *row_start[kMaxMergeSlices];
    const int32_t *rp[kMaxMergeSlices];
    const int32_t *col[kMaxMergeSlices];
    const float *val[kMaxMergeSlices];
};

__global__ __launch_bounds__(kMergeThreads) void k_merge_slices(int32_t R, MergeSlices m,
                                                                const float *__restrict__ x,
                                                                float *__restrict__ y) {
    __shared__ int32_t s_end[kMergeItemsPerBlock];
    __shared__ float s_prod[kMergeItemsPerBlock];
    __shared__ float s_acc[kMergeItemsPerBlock + 1];
    const int per = 8 / m.n;
    const int xcd = static_cast<int>(blockIdx.x % 8);
    const int k = xcd / per;
    const int32_t tile = static_cast<int32_t>((blockIdx.x / 8) * per + xcd % per);
    if (tile >= m.tiles[k]) return;
    merge_tile(tile, R, m.nnz[k], m.row_start[k], m.rp[k], m.col[k], m.val[k], x, y, s_end,
               s_prod, s_acc);
}

unsigned blocks_of(int64_t n, int per_block) { return grid_for(n, per_block); }

template <int L>
hipError_t run_vector(const spmv_handle *h, const float *x, float *y, hipStream_t s) {
    const int32_t R = static_cast<int32_t>(h->stats.num_rows);
    constexpr int kRows4 = kThreads / L * 4;
    const bool four = h->stats.max_len <= 2 * L && blocks_of(R, kRows4) >= 2048;
    if (four)
        k_csr_vector<L, 4><<<blocks_of(R, kRows4), kThreads, 0, s>>>(
            R, h->a.row_ptrs, h->a.col_idx, h->a.values, x, y);
    else
        k_csr_vector<L, 1><<<blocks_of(R, kThreads / L), kThreads, 0, s>>>(
            R, h->a.row_ptrs, h->a.col_idx, h->a.values, x, y);
    return hipGetLastError();
}

hipError_t run_ell(int32_t R, int32_t W, bool scattered, const int32_t *col, const float *val,
                   const int32_t *nnz_per_row, const float *x, float *y, hipStream_t s) {
    if (R <= 0 || W <= 0) return hipSuccess;
    // 4 rows per lane only for scattered columns (with banded columns the
    // gathers of neighbouring one-row lanes coalesce, which 4 interleaved rows
    // per lane break) and while the grid still spreads over the chip (>= 2
    // blocks per CU); at any width (1M rows of 12-64 random columns: 5-10 %
    // faster than one row per lane)
    if (scattered && R % 4 == 0 && blocks_of(R / 4, kThreads) >= 512 &&
        reinterpret_cast<uintptr_t>(y) % 16 == 0) {
        k_ell4<4><<<blocks_of(R / 4, kThreads), kThreads, 0, s>>>(R, W, col, val, nnz_per_row, x,
                                                                 y);
        return hipGetLastError();
    }
    const unsigned g = blocks_of(R, kThreads);
    if (W <= 4) k_ell<4><<<g, kThreads, 0, s>>>(R, W, col, val, nnz_per_row, x, y);
    else k_ell<8><<<g, kThreads, 0, s>>>(R, W, col, val, nnz_per_row, x, y);
    return hipGetLastError();
}

// RUN = the smallest power of two above mean + one standard deviation of the
// row lengths, within 4..32 (1M x 5 random: 8; 27-point stencil, skewed and
// power-law rows: 32).  Measured against one entry per lane: 222 -> 55 us on
// the 1M x 5 matrix, 3062 -> 499 us on the stencil, 10.0 -> 6.0 ms on the
// power-law matrix.
hipError_t run_coo_atomic(const spmv_stats &st, int32_t nnz, const int32_t *row,
                          const int32_t *col, const float *val, const float *x, float *y,
                          hipStream_t s) {
    if (nnz <= 0) return hipSuccess;
    const double R = static_cast<double>(st.num_rows > 0 ? st.num_rows : 1);
    const double mean = static_cast<double>(st.nnz) / R;
    const double var = static_cast<double>(st.sum_len_sq) / R - mean * mean;
    const double spread = mean + (var > 0.0 ? std::sqrt(var) : 0.0);
    int run = 4;
    while (run < 32 && run <= spread) run *= 2;
    const int64_t n = nnz;
    switch (run) {
    case 4:
        k_coo_atomic<4><<<blocks_of((n + 3) / 4, kThreads), kThreads, 0, s>>>(nnz, row, col, val,
                                                                             x, y);
        break;
    case 8:
        k_coo_atomic<8><<<blocks_of((n + 7) / 8, kThreads), kThreads, 0, s>>>(nnz, row, col, val,
                                                                             x, y);
        break;
    case 16:
        k_coo_atomic<16><<<blocks_of((n + 15) / 16, kThreads), kThreads, 0, s>>>(nnz, row, col,
                                                                                val, x, y);
        break;
    default:
        k_coo_atomic<32><<<blocks_of((n + 31) / 32, kThreads), kThreads, 0, s>>>(nnz, row, col,
                                                                                val, x, y);
        break;
    }
    return hipGetLastError();
}

hipError_t run_coo_segmented(int32_t n, const int32_t *row, const int32_t *col,
                             const float *val, const float *x, float *y, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t waves = (static_cast<int64_t>(n) + kWave * kSegIters - 1) / (kWave * kSegIters);
    k_coo_segmented<<<blocks_of(waves * kWave, kThreads), kThreads, 0, s>>>(n, row, col, val, x,
                                                                            y);
    return hipGetLastError();
}

}  // namespace

spmv_status launch_spmv(const spmv_handle *h, const float *x, float *y, hipStream_t s) {
    const int32_t R = static_cast<int32_t>(h->stats.num_rows);
    const int32_t nnz = static_cast<int32_t>(h->stats.nnz);
    if (R == 0 || nnz == 0) return SPMV_OK;
    if (!h->parts.empty()) {
        // x slices that are all merge CSR, 2, 4 or 8 of them: one launch with
        // each slice on its own XCDs
        const int np = static_cast<int>(h->parts.size());
        bool together = np >= 2 && np <= kMaxMergeSlices && 8 % np == 0;
        for (const spmv_handle *p : h->parts)
            together = together && p->format == SPMV_CSR_MERGE && p->num_tiles > 0;
        if (together) {
            MergeSlices m{};
            m.n = np;
            int64_t most = 0;
            for (int k = 0; k < np; ++k) {
                const spmv_handle *p = h->parts[k];
                m.nnz[k] = static_cast<int32_t>(p->stats.nnz);
                m.tiles[k] = static_cast<int32_t>(p->num_tiles);
                m.row_start[k] = p->a.merge_row_start;
                m.rp[k] = p->a.row_ptrs;
                m.col[k] = p->a.col_idx;
                m.val[k] = p->a.values;
                most = std::max<int64_t>(most, p->num_tiles);
            }
            const int per = 8 / np;
            const int64_t grid = 8 * ((most + per - 1) / per);
            k_merge_slices<<<static_cast<unsigned>(grid), kMergeThreads, 0, s>>>(R, m, x, y);
            return hipGetLastError() == hipSuccess ? SPMV_OK : SPMV_ERR_HIP;
        }
        // otherwise one pass per slice over y, in stream order
        for (const spmv_handle *p : h->parts) {
            const spmv_status st = launch_spmv(p, x, y, s);
            if (st != SPMV_OK) return st;
        }
        return SPMV_OK;
    }
    const DevArrays &a = h->a;
    // scattered columns: rows' first columns lie more than C/8 from the
    // diagonal on average (the statistic the x-slice decision uses)
    const bool scattered = h->stats.col_spread * 8 > h->stats.num_cols;
    hipError_t e = hipSuccess;
    switch (h->format) {
    case SPMV_COO_ATOMIC:
        e = run_coo_atomic(h->stats, nnz, a.row_idx, a.col_idx, a.values, x, y, s);
        break;
    case SPMV_COO_SEGMENTED:
        e = run_coo_segmented(nnz, a.row_idx, a.col_idx, a.values, x, y, s);
        break;
    case SPMV_CSR_SCALAR:
        if (h->csr_staged)
            k_csr_scalar_lds<<<blocks_of(R, kThreads), kThreads, 0, s>>>(R, a.row_ptrs, a.col_idx,
                                                                        a.values, x, y);
        else
            k_csr_scalar<<<blocks_of(R, kThreads), kThreads, 0, s>>>(R, a.row_ptrs, a.col_idx,
                                                                    a.values, x, y);
        e = hipGetLastError();
        break;
    case SPMV_CSR_VECTOR:
        switch (h->lanes) {
        case 1:
            k_csr_scalar<<<blocks_of(R, kThreads), kThreads, 0, s>>>(R, a.row_ptrs, a.col_idx,
                                                                    a.values, x, y);
            e = hipGetLastError();
            break;
        case 2: e = run_vector<2>(h, x, y, s); break;
        case 4: e = run_vector<4>(h, x, y, s); break;
        case 8: e = run_vector<8>(h, x, y, s); break;
        case 16: e = run_vector<16>(h, x, y, s); break;
        case 32: e = run_vector<32>(h, x, y, s); break;
        case 64: e = run_vector<64>(h, x, y, s); break;
        default: return SPMV_ERR_INVALID_ARG;
        }
        break;
    case SPMV_ELL:
        e = run_ell(R, h->ell_width, scattered, a.ell_col, a.ell_val, a.ell_nnz, x, y, s);
        break;
    case SPMV_HYB:
        // ELL part first (plain y update per row), then the COO tail with
        // atomics, in stream order: the two never touch y concurrently.
        e = run_ell(R, h->ell_width, scattered, a.ell_col, a.ell_val, a.ell_nnz, x, y, s);
        if (e == hipSuccess)
            e = run_coo_segmented(static_cast<int32_t>(h->tail_nnz), a.tail_row, a.tail_col,
                                  a.tail_val, x, y, s);
        break;
    case SPMV_ELL_XTILE:
        if (h->ell_width > 0) {
            const unsigned g = blocks_of(R, kTileRows);
            const size_t lds = sizeof(float) * static_cast<size_t>(std::max(h->xt_max_tile, 1));
            if (h->ell_width <= 4)
                k_ell_xtile<4><<<g, kThreads, lds, s>>>(R, h->ell_width, a.xt_run_ptr, a.xt_runs,
                                                        a.xt_lidx, a.ell_val, a.ell_nnz, x, y);
            else
                k_ell_xtile<8><<<g, kThreads, lds, s>>>(R, h->ell_width, a.xt_run_ptr, a.xt_runs,
                                                        a.xt_lidx, a.ell_val, a.ell_nnz, x, y);
            e = hipGetLastError();
        }
        break;
    case SPMV_JDS:
        if (h->num_tiles > 0) {
            k_jds<<<blocks_of(h->num_tiles * kWave, kThreads), kThreads, 0, s>>>(
                R, static_cast<int32_t>(h->num_tiles), h->jds_depth, a.jds_tiles, a.jds_len,
                a.jds_iter_ptr, a.jds_perm, a.jds_col, a.jds_val, x, y);
            e = hipGetLastError();
        }
        break;
    case SPMV_SELL:
        if (h->num_tiles > 0) {
            k_sell<<<blocks_of(h->num_tiles * kWave, kThreads), kThreads, 0, s>>>(
                R, static_cast<int32_t>(h->num_tiles), h->jds_depth, a.jds_tiles, a.jds_len,
                a.sell_ptr, a.jds_perm, a.sell_col, a.sell_val, x, y);
            e = hipGetLastError();
        }
        break;
    case SPMV_COO_BLOCKED:
        e = launch_coo_blocked(h, x, y, s);
        break;
    case SPMV_CSR_MERGE:
        k_merge<<<static_cast<unsigned>(h->num_tiles), kMergeThreads, 0, s>>>(
            R, nnz, a.merge_row_start, a.row_ptrs, a.col_idx, a.values, x, y);
        e = hipGetLastError();
        break;
    default:
        return SPMV_ERR_INVALID_ARG;
    }
    return e == hipSuccess ? SPMV_OK : from_hip(e);
}

}  // namespace spmv
