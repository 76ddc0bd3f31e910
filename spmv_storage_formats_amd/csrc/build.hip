// Device format builders.  Every builder moves values as raw 32-bit words,
// so the built arrays hold exactly the input's bits.
//
//   COO -> CSR   PMPP notes, "Sparse Matrices and Basic Formats (COO & CSR)":
//                count entries per row, exclusive scan (scan.hip), then a
//                stable scatter (sort.hip) so each row keeps its input order.
//   CSR -> ELL   PMPP notes, "Regularized Formats", ELL section: pad every row
//                to the longest one (value 0, column 0) and store the padded
//                rows column-major, slot t of row r at t*R + r.
//   CSR -> HYB   same page, hybrid ELL-COO section: entries past position K of
//                each row go to a COO tail (rows in order, positions in
//                order); the rest is an ELL of width min(K, W).
//   CSR -> JDS   same page, JDS section: rows sorted by length, longest first
//                (original order among equals), perm records the original
//                row, iterPtr[t] = where jagged column t starts, entry t of
//                sorted row s at iterPtr[t] + s.
//   merge path   format-choice article 5.2 (merge-based CSR for power-law
//                rows): first row of each block's equal share of the
//                rows-plus-nonzeros sequence.
#include "internal.h"

namespace spmv {
namespace {

constexpr int kThreads = 256;

// Per-row counts with one atomic per run of equal row indices in a wave step:
// a row-sorted COO list costs one atomic per row segment, not per entry.  A
// wave takes kCountSteps consecutive steps of 64 entries, their loads issued
// together.
constexpr int kCountSteps = 4;

__global__ __launch_bounds__(kThreads) void k_count_rows(int32_t nnz,
                                                         const int32_t *__restrict__ row,
                                                         int32_t *__restrict__ counts) {
    const int64_t wave = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / kWave;
    const int lane = __lane_id();
    const int64_t base = wave * kWave * kCountSteps + lane;
    int32_t rv[kCountSteps];
#pragma unroll
    for (int k = 0; k < kCountSteps; ++k) {
        const int64_t i = base + k * kWave;
        rv[k] = i < nnz ? ld_nt(row + i) : -1;
    }
#pragma unroll
    for (int k = 0; k < kCountSteps; ++k) {
        const bool valid = base + k * kWave < nnz;
        const int32_t r = rv[k];
        const int32_t prev = __shfl_up(r, 1);
        const bool head = valid && (lane == 0 || prev != r);
        const unsigned long long heads = __ballot(head);
        const unsigned long long live = __ballot(valid);
        if (head) {
            const unsigned long long after = heads & ~((2ull << lane) - 1ull);
            const int end = after ? (__ffsll(static_cast<long long>(after)) - 1)
                                  : (64 - __clzll(static_cast<long long>(live)));
            atomicAdd(&counts[r], end - lane);
        }
    }
}

// One wave per 64 consecutive rows; all 64 lanes fill each row's range in turn.
__global__ __launch_bounds__(kThreads) void k_expand_rows(int32_t R,
                                                          const int32_t *__restrict__ rp,
                                                          int32_t *__restrict__ row_idx) {
    const int64_t wave = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / kWave;
    const int lane = __lane_id();
    const int64_t r0 = wave * kWave;
    if (r0 >= R) return;
    const int64_t my = r0 + lane;
    const int32_t a = my < R ? rp[my] : 0;
    const int32_t b = my < R ? rp[my + 1] : 0;
    for (int k = 0; k < kWave && r0 + k < R; ++k) {
        const int32_t ak = __shfl(a, k), bk = __shfl(b, k);
        // 64-bit position: a row may end at INT32_MAX
        for (int64_t i = static_cast<int64_t>(ak) + lane; i < bk; i += kWave)
            row_idx[i] = static_cast<int32_t>(r0 + k);
    }
}

// ---------------------------------------------------------------------------
// Row-to-column transposes (ELL, JDS, sectioned ELL).  One lane per row; for a
// fixed entry position t the lanes of a wave write neighbouring words, so the
// stores coalesce.  Reading row r's entries lane by lane would touch a
// different cache line in every lane, so when the wave's rows form one
// contiguous CSR segment of at most kStage entries the wave first copies the
// segment into LDS with coalesced loads and each lane then reads its row from
// LDS.  Word i of the segment is stored at i + i/32, so rows of a power-of-two
// length do not fall in one bank.  Columns and values are staged in two
// phases to halve the LDS footprint.  Other waves read global memory directly.
// ---------------------------------------------------------------------------
constexpr int kStage = 2048;
constexpr int kStageWords = kStage + kStage / 32;

__device__ inline int32_t skew(int32_t i) { return i + (i >> 5); }

// lds[skew(i)] = src[i] for i in [0, n), the wave's 64 lanes together.
template <typename T>
__device__ inline void stage_segment(const T *__restrict__ src, int32_t n, T *lds, int lane) {
    int32_t i = lane;
    for (; i + 3 * kWave < n; i += 4 * kWave) {
        const T v0 = src[i], v1 = src[i + kWave], v2 = src[i + 2 * kWave], v3 = src[i + 3 * kWave];
        lds[skew(i)] = v0;
        lds[skew(i + kWave)] = v1;
        lds[skew(i + 2 * kWave)] = v2;
        lds[skew(i + 3 * kWave)] = v3;
    }
    for (; i < n; i += kWave) lds[skew(i)] = src[i];
}

// CSR -> ELL [Regularized formats page, ELL section]: row r's entry t goes to
// slot t*R + r; slots past the row's length (or past `width`) are padding
// (column 0, +0.0f).
__global__ __launch_bounds__(kThreads) void k_build_ell(int32_t R, int32_t width,
                                                        const int32_t *__restrict__ rp,
                                                        const int32_t *__restrict__ col,
                                                        const uint32_t *__restrict__ val,
                                                        int32_t *__restrict__ ell_col,
                                                        uint32_t *__restrict__ ell_val,
                                                        int32_t *__restrict__ ell_nnz) {
    __shared__ uint32_t lds[kThreads / kWave][kStageWords];
    const int w = threadIdx.x / kWave;
    const int lane = __lane_id();
    const int64_t r = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const bool ok = r < R;
    const int32_t a = ok ? rp[r] : 0;
    const int32_t e = ok ? rp[r + 1] : 0;
    int32_t n = e - a;
    if (n > width) n = width;
    if (ok) ell_nnz[r] = n;
    // the wave's segment [s0, s1): lane 0's start to the last valid lane's end
    const unsigned long long live = __ballot(ok);
    const int last = live ? 63 - __clzll(static_cast<long long>(live)) : 0;
    const int32_t s0 = __builtin_amdgcn_readfirstlane(a);
    const int32_t s1 = __shfl(e, last);
    const int64_t seg = live ? static_cast<int64_t>(s1) - s0 : 0;
    const bool staged = seg <= kStage;   // wave-uniform
    const int32_t off = a - s0;
    for (int phase = 0; phase < 2; ++phase) {
        const uint32_t *src = phase == 0 ? reinterpret_cast<const uint32_t *>(col) : val;
        uint32_t *dst = phase == 0 ? reinterpret_cast<uint32_t *>(ell_col) : ell_val;
        if (staged) stage_segment(src + s0, static_cast<int32_t>(seg), lds[w], lane);
        __syncthreads();
        if (ok) {
            for (int32_t t = 0; t < width; ++t) {
                uint32_t v = 0u;   // padding: column 0 / +0.0f
                if (t < n) v = staged ? lds[w][skew(off + t)] : src[static_cast<int64_t>(a) + t];
                dst[static_cast<int64_t>(t) * R + r] = v;
            }
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(kThreads) void k_tail_lengths(int32_t R, int32_t K,
                                                           const int32_t *__restrict__ rp,
                                                           int32_t *__restrict__ tail_len) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (r < R) {
        const int32_t len = rp[r + 1] - rp[r];
        tail_len[r] = len > K ? len - K : 0;
    }
}

// One lane per tail entry e: its row is the last r with tail_off[r] <= e.
__global__ __launch_bounds__(kThreads) void k_fill_tail(
    int32_t R, int32_t K, int32_t ntail, const int32_t *__restrict__ rp,
    const int32_t *__restrict__ tail_off, const int32_t *__restrict__ col,
    const uint32_t *__restrict__ val, int32_t *__restrict__ tail_row,
    int32_t *__restrict__ tail_col, uint32_t *__restrict__ tail_val) {
    const int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (e >= ntail) return;
    const int64_t r = upper_index(tail_off, R, e);
    const int64_t src = static_cast<int64_t>(rp[r]) + K + (e - tail_off[r]);
    tail_row[e] = static_cast<int32_t>(r);
    tail_col[e] = col[src];
    tail_val[e] = val[src];
}

// ---------------------------------------------------------------------------
// ELL with x tiles [Regularized formats page, ELL section, for the slot layout;
// "Introduction to sparse computing", x blocking: keep the x a block gathers
// in fast memory; format-choice article 4.2: stage in shared memory].
// Block b = rows [256b, 256b + 256).  Its tile is the sorted set of distinct
// columns of its entries; a run is a maximal stretch of consecutive columns
// in the tile; a column's tile position is the number of tile columns below
// it.  The block marks its columns in an LDS bitmap over [lo, lo + span)
// (lo = least column, span = greatest - lo + 1), so tile positions are
// popcounts and runs are bit boundaries.
// ---------------------------------------------------------------------------
constexpr int kBmWords = kTileMaxSpan / 32;
static_assert(kTileRows == kThreads, "one row per thread in the x-tile kernels");

__device__ inline int block_min_max(int v, bool want_max, int *red) {
    for (int o = kWave / 2; o > 0; o >>= 1) {
        const int u = __shfl_xor(v, o);
        v = want_max ? max(v, u) : min(v, u);
    }
    __syncthreads();
    if (__lane_id() == 0) red[threadIdx.x / kWave] = v;
    __syncthreads();
    int t = red[0];
    for (int i = 1; i < kThreads / kWave; ++i) t = want_max ? max(t, red[i]) : min(t, red[i]);
    return t;
}

// Exclusive prefix over the block of one int per thread; *total = block sum.
__device__ inline int block_excl_scan(int v, int *total, int *red) {
    const int lane = __lane_id();
    int incl = v;
    for (int o = 1; o < kWave; o <<= 1) {
        const int u = __shfl_up(incl, o);
        if (lane >= o) incl += u;
    }
    __syncthreads();
    if (lane == kWave - 1) red[threadIdx.x / kWave] = incl;
    __syncthreads();
    int before = 0, tot = 0;
    for (int i = 0; i < kThreads / kWave; ++i) {
        const int x = red[i];
        before += i < static_cast<int>(threadIdx.x / kWave) ? x : 0;
        tot += x;
    }
    *total = tot;
    return before + incl - v;
}

struct XtBlock {
    int32_t r0, r1;     // rows of the block
    int64_t s0, s1;     // its entries [s0, s1)
    int32_t lo, span;   // column window
};

// Marks the block's columns in bm.  Returns false (the same in every thread)
// when the window exceeds the bitmap.  Every thread passes every barrier.
__device__ bool xt_mark(int32_t R, const int32_t *__restrict__ rp,
                        const int32_t *__restrict__ col, uint32_t *bm, int *red, XtBlock &xb) {
    xb.r0 = static_cast<int32_t>(blockIdx.x) * kTileRows;
    xb.r1 = min(R, xb.r0 + kTileRows);
    xb.s0 = rp[xb.r0];
    xb.s1 = rp[xb.r1];
    int lo = INT32_MAX, hi = -1;
    for (int64_t i = xb.s0 + threadIdx.x; i < xb.s1; i += kThreads) {
        const int c = col[i];
        lo = min(lo, c);
        hi = max(hi, c);
    }
    lo = block_min_max(lo, false, red);
    hi = block_min_max(hi, true, red);
    xb.lo = lo;
    xb.span = hi < lo ? 0 : (static_cast<int64_t>(hi) - lo + 1 > kTileMaxSpan ? -1 : hi - lo + 1);
    if (xb.span < 0) return false;
    const int words = (xb.span + 31) / 32;
    for (int w = threadIdx.x; w < words; w += kThreads) bm[w] = 0u;
    __syncthreads();
    for (int64_t i = xb.s0 + threadIdx.x; i < xb.s1; i += kThreads) {
        const int c = col[i] - lo;
        atomicOr(&bm[c >> 5], 1u << (c & 31));
    }
    __syncthreads();
    return true;
}

// bits of word w that start / end a run (a set bit whose lower / upper
// neighbour is clear)
__device__ inline uint32_t run_starts(const uint32_t *bm, int w) {
    const uint32_t m = bm[w];
    const uint32_t below = w > 0 ? bm[w - 1] >> 31 : 0u;
    return m & ~((m << 1) | below);
}
__device__ inline uint32_t run_ends(const uint32_t *bm, int w, int words) {
    const uint32_t m = bm[w];
    const uint32_t above = w + 1 < words ? (bm[w + 1] & 1u) << 31 : 0u;
    return m & ~((m >> 1) | above);
}

// counts[3b] = distinct columns, counts[3b+1] = runs, counts[3b+2] = 1 if the
// window fits the bitmap (else 0 and the other two are 0)
__global__ __launch_bounds__(kThreads) void k_xt_count(int32_t R, const int32_t *__restrict__ rp,
                                                       const int32_t *__restrict__ col,
                                                       int32_t *__restrict__ counts) {
    __shared__ uint32_t bm[kBmWords];
    __shared__ int red[kThreads / kWave];
    XtBlock xb;
    const bool ok = xt_mark(R, rp, col, bm, red, xb);
    int distinct = 0, runs = 0;
    if (ok) {
        const int words = (xb.span + 31) / 32;
        int d = 0, n = 0;
        for (int w = threadIdx.x; w < words; w += kThreads) {
            d += __popc(bm[w]);
            n += __popc(run_starts(bm, w));
        }
        block_excl_scan(d, &distinct, red);
        block_excl_scan(n, &runs, red);
    }
    if (threadIdx.x == 0) {
        counts[3 * blockIdx.x] = distinct;
        counts[3 * blockIdx.x + 1] = runs;
        counts[3 * blockIdx.x + 2] = ok ? 1 : 0;
    }
}

// Writes the block's runs (first column, tile offset, length) at
// runs[3 * (run_ptr[b] + k)] and, for every row, its ELL slots: tile position
// (int16) and value, padding (0, +0.0f) past the row's length.  The host has
// checked that every block fits (window, kTileMaxCols, kTileMaxRuns).
__global__ __launch_bounds__(kThreads) void k_xt_fill(int32_t R, int32_t W,
                                                      const int32_t *__restrict__ rp,
                                                      const int32_t *__restrict__ col,
                                                      const uint32_t *__restrict__ val,
                                                      const int32_t *__restrict__ run_ptr,
                                                      int32_t *__restrict__ runs,
                                                      int16_t *__restrict__ lidx,
                                                      uint32_t *__restrict__ ell_val,
                                                      int32_t *__restrict__ ell_nnz) {
    __shared__ uint32_t bm[kBmWords];
    __shared__ int32_t rank[kBmWords];      // tile position of each word's first bit
    __shared__ int32_t rstart[kTileMaxRuns], rend[kTileMaxRuns];   // relative columns
    __shared__ int red[kThreads / kWave];
    XtBlock xb;
    if (!xt_mark(R, rp, col, bm, red, xb)) return;   // (excluded by the host)
    const int words = (xb.span + 31) / 32;
    // each thread owns a contiguous chunk of words
    const int cw = (words + kThreads - 1) / kThreads;
    const int w0 = min(words, static_cast<int>(threadIdx.x) * cw), w1 = min(words, w0 + cw);
    int d = 0, ns = 0, ne = 0;
    for (int w = w0; w < w1; ++w) {
        d += __popc(bm[w]);
        ns += __popc(run_starts(bm, w));
        ne += __popc(run_ends(bm, w, words));
    }
    int tot;
    int rk = block_excl_scan(d, &tot, red);
    int sk = block_excl_scan(ns, &tot, red);
    int ek = block_excl_scan(ne, &tot, red);
    for (int w = w0; w < w1; ++w) {
        rank[w] = rk;
        rk += __popc(bm[w]);
        for (uint32_t m = run_starts(bm, w); m; m &= m - 1) rstart[sk++] = 32 * w + __ffs(m) - 1;
        for (uint32_t m = run_ends(bm, w, words); m; m &= m - 1) rend[ek++] = 32 * w + __ffs(m) - 1;
    }
    __syncthreads();
    auto position = [&](int c) {   // tile position of relative column c (a tile column)
        const int w = c >> 5, bit = c & 31;
        return rank[w] + __popc(bm[w] & ((1u << bit) - 1u));
    };
    const int base = run_ptr[blockIdx.x];
    const int nruns = run_ptr[blockIdx.x + 1] - base;
    for (int k = threadIdx.x; k < nruns; k += kThreads) {
        const int st = rstart[k];
        runs[3 * (static_cast<int64_t>(base) + k)] = xb.lo + st;
        runs[3 * (static_cast<int64_t>(base) + k) + 1] = position(st);
        runs[3 * (static_cast<int64_t>(base) + k) + 2] = rend[k] - st + 1;
    }
    const int32_t r = xb.r0 + static_cast<int32_t>(threadIdx.x);
    if (r >= xb.r1) return;
    const int32_t a = rp[r];
    const int32_t n = rp[r + 1] - a;
    ell_nnz[r] = n;
    for (int32_t t = 0; t < W; ++t) {
        const int64_t slot = static_cast<int64_t>(t) * R + r;
        int16_t p = 0;
        uint32_t v = 0u;   // padding: position 0, +0.0f
        if (t < n) {
            p = static_cast<int16_t>(position(col[static_cast<int64_t>(a) + t] - xb.lo));
            v = val[static_cast<int64_t>(a) + t];
        }
        lidx[slot] = p;
        ell_val[slot] = v;
    }
}

// JDS sort key: W - len, so an ascending stable sort puts longer rows first and
// keeps the original order among equal lengths.
__global__ __launch_bounds__(kThreads) void k_jds_keys(int32_t R, int32_t W,
                                                       const int32_t *__restrict__ rp,
                                                       uint32_t *__restrict__ keys,
                                                       int32_t *__restrict__ rows) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (r < R) {
        keys[r] = static_cast<uint32_t>(W - (rp[r + 1] - rp[r]));
        rows[r] = static_cast<int32_t>(r);
    }
}

__global__ __launch_bounds__(kThreads) void k_jds_lengths(int32_t R, int32_t W,
                                                          const uint32_t *__restrict__ keys,
                                                          int32_t *__restrict__ jds_len) {
    const int64_t s = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (s < R) jds_len[s] = W - static_cast<int32_t>(keys[s]);
}

// counts[t] = number of sorted rows longer than t = first s with len[s] <= t.
__global__ __launch_bounds__(kThreads) void k_jds_counts(int32_t R, int32_t W,
                                                         const int32_t *__restrict__ jds_len,
                                                         int32_t *__restrict__ counts) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (t >= W) return;
    int64_t lo = 0, hi = R;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (jds_len[mid] > t) lo = mid + 1; else hi = mid;
    }
    counts[t] = static_cast<int32_t>(lo);
}

// One wave per JDS tile (64 consecutive sorted rows x `depth` jagged columns,
// the tiles the SpMV kernel walks): lane i takes sorted row s = 64g + i and
// copies its entries t in the tile's column range from original row perm[s]
// to iter_ptr[t] + s.  A first-chunk tile whose rows are consecutive original
// rows (the common case: equal lengths keep their order) stages its CSR
// segment in LDS as the ELL builder does.
__global__ __launch_bounds__(kThreads) void k_jds_fill(int32_t R, int32_t ntiles, int32_t depth,
                                                       const int2 *__restrict__ tiles,
                                                       const int32_t *__restrict__ iter_ptr,
                                                       const int32_t *__restrict__ perm,
                                                       const int32_t *__restrict__ jds_len,
                                                       const int32_t *__restrict__ rp,
                                                       const int32_t *__restrict__ col,
                                                       const uint32_t *__restrict__ val,
                                                       int32_t *__restrict__ jds_col,
                                                       uint32_t *__restrict__ jds_val) {
    __shared__ uint32_t lds[kThreads / kWave][kStageWords];
    const int w = threadIdx.x / kWave;
    const int lane = __lane_id();
    const int64_t tile = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / kWave;
    const bool tile_ok = tile < ntiles;
    const int2 gc = tile_ok ? tiles[tile] : make_int2(0, 0);
    const int64_t s = static_cast<int64_t>(gc.x) * kWave + lane;
    const bool ok = tile_ok && s < R;
    const int64_t t0 = static_cast<int64_t>(gc.y) * depth;
    const int64_t t1 = ok ? min(t0 + depth, static_cast<int64_t>(jds_len[s])) : 0;
    const int32_t p = ok ? perm[s] : 0;
    const int32_t a = ok ? rp[p] : 0;
    // staged when the tile is its group's first chunk and the rows are
    // consecutive original rows forming one segment of <= kStage entries
    const unsigned long long live = __ballot(ok);
    const int last = live ? 63 - __clzll(static_cast<long long>(live)) : 0;
    const int32_t p0 = __builtin_amdgcn_readfirstlane(p);
    const bool consecutive = __ballot(ok && p != p0 + lane) == 0;
    const int32_t s0 = __builtin_amdgcn_readfirstlane(a);
    const int32_t s1 = live ? rp[__shfl(p, last) + 1] : s0;
    const int64_t seg = static_cast<int64_t>(s1) - s0;
    const bool staged = live && gc.y == 0 && consecutive && seg <= kStage;   // wave-uniform
    const int32_t off = a - s0;
    for (int phase = 0; phase < 2; ++phase) {
        const uint32_t *src = phase == 0 ? reinterpret_cast<const uint32_t *>(col) : val;
        uint32_t *dst = phase == 0 ? reinterpret_cast<uint32_t *>(jds_col) : jds_val;
        if (staged) stage_segment(src + s0, static_cast<int32_t>(seg), lds[w], lane);
        __syncthreads();
        for (int64_t t = t0; t < t1; ++t) {
            const uint32_t v = staged ? lds[w][skew(off + static_cast<int32_t>(t))]
                                      : src[static_cast<int64_t>(a) + t];
            dst[static_cast<int64_t>(iter_ptr[t]) + s] = v;
        }
        __syncthreads();
    }
}

// Sectioned ELL (JDS variant): section k = sorted rows [64k, 64k + m_k),
// padded to its first (longest) row; slot (t, i) at sect_ptr[k] + t*m_k + i.
__global__ __launch_bounds__(kThreads) void k_sell_sizes(int32_t R,
                                                         const int32_t *__restrict__ jds_len,
                                                         int32_t *__restrict__ sizes) {
    const int64_t k = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const int64_t nsect = (static_cast<int64_t>(R) + kWave - 1) / kWave;
    if (k < nsect) {
        const int64_t m = min(static_cast<int64_t>(kWave), R - k * kWave);
        sizes[k] = static_cast<int32_t>(m * jds_len[k * kWave]);   // total checked on the host
    }
}

// One wave per tile (section k, chunk of `depth` padded columns), the tiles
// the SpMV kernel walks: lane i writes slots sect_ptr[k] + t*m + i of the
// chunk, its row's entry t or padding (column 0, +0.0f) past its length.
// Staged in LDS like the JDS fill when the section's rows are consecutive.
__global__ __launch_bounds__(kThreads) void k_sell_fill(
    int32_t R, int32_t ntiles, int32_t depth, const int2 *__restrict__ tiles,
    const int32_t *__restrict__ sect_ptr, const int32_t *__restrict__ jds_len,
    const int32_t *__restrict__ perm, const int32_t *__restrict__ rp,
    const int32_t *__restrict__ col, const uint32_t *__restrict__ val,
    int32_t *__restrict__ sell_col, uint32_t *__restrict__ sell_val) {
    __shared__ uint32_t lds[kThreads / kWave][kStageWords];
    const int w = threadIdx.x / kWave;
    const int lane = __lane_id();
    const int64_t tile = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / kWave;
    const bool tile_ok = tile < ntiles;
    const int2 gc = tile_ok ? tiles[tile] : make_int2(0, 0);
    const int64_t first = static_cast<int64_t>(gc.x) * kWave;
    const int64_t m = tile_ok ? min(static_cast<int64_t>(kWave), R - first) : 0;
    const bool ok = lane < m;
    const int64_t s = first + lane;
    const int64_t width = tile_ok ? jds_len[first] : 0;
    const int64_t t0 = static_cast<int64_t>(gc.y) * depth;
    const int64_t t1 = min(t0 + depth, width);
    const int64_t len = ok ? jds_len[s] : 0;
    const int32_t p = ok ? perm[s] : 0;
    const int32_t a = ok ? rp[p] : 0;
    const int64_t base = tile_ok ? static_cast<int64_t>(sect_ptr[gc.x]) + lane : 0;
    const unsigned long long live = __ballot(ok);
    const int last = live ? 63 - __clzll(static_cast<long long>(live)) : 0;
    const int32_t p0 = __builtin_amdgcn_readfirstlane(p);
    const bool consecutive = __ballot(ok && p != p0 + lane) == 0;
    const int32_t s0 = __builtin_amdgcn_readfirstlane(a);
    const int32_t s1 = live ? rp[__shfl(p, last) + 1] : s0;
    const int64_t seg = static_cast<int64_t>(s1) - s0;
    const bool staged = live && gc.y == 0 && consecutive && seg <= kStage;   // wave-uniform
    const int32_t off = a - s0;
    for (int phase = 0; phase < 2; ++phase) {
        const uint32_t *src = phase == 0 ? reinterpret_cast<const uint32_t *>(col) : val;
        uint32_t *dst = phase == 0 ? reinterpret_cast<uint32_t *>(sell_col) : sell_val;
        if (staged) stage_segment(src + s0, static_cast<int32_t>(seg), lds[w], lane);
        __syncthreads();
        if (ok) {
            for (int64_t t = t0; t < t1; ++t) {
                uint32_t v = 0u;   // padding: column 0 / +0.0f
                if (t < len)
                    v = staged ? lds[w][skew(off + static_cast<int32_t>(t))]
                               : src[static_cast<int64_t>(a) + t];
                dst[base + t * m] = v;
            }
        }
        __syncthreads();
    }
}

// Tiles of the JDS kernel: 64 consecutive sorted rows x `depth` jagged columns.
// Group g needs ceil(len[64 g] / depth) tiles (its first row is its longest).
__global__ __launch_bounds__(kThreads) void k_jds_chunks(int32_t R, int32_t depth,
                                                         const int32_t *__restrict__ jds_len,
                                                         int32_t *__restrict__ chunks) {
    const int64_t g = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const int64_t groups = (static_cast<int64_t>(R) + kWave - 1) / kWave;
    if (g < groups) {
        const int64_t len = jds_len[g * kWave];
        chunks[g] = static_cast<int32_t>((len + depth - 1) / depth);
    }
}

__global__ __launch_bounds__(kThreads) void k_jds_tiles(int32_t groups, int32_t ntiles,
                                                        const int32_t *__restrict__ tile_off,
                                                        int2 *__restrict__ tiles) {
    const int64_t tile = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (tile >= ntiles) return;
    const int64_t g = upper_index(tile_off, groups, tile);
    tiles[tile] = make_int2(static_cast<int>(g), static_cast<int>(tile - tile_off[g]));
}

// Column slices: entry i belongs to slice col[i] / slice_cols.  A stable sort
// by slice (sort.hip) groups each slice's entries in their original, row-major
// order; bounds[b] = first sorted position of slice b (binary search).
__global__ __launch_bounds__(kThreads) void k_slice_keys(int32_t nnz,
                                                         const int32_t *__restrict__ col,
                                                         int32_t slice_cols,
                                                         uint32_t *__restrict__ keys) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (i < nnz) keys[i] = static_cast<uint32_t>(col[i] / slice_cols);
}

__global__ __launch_bounds__(kThreads) void k_slice_bounds(int32_t nnz, int32_t K,
                                                           const uint32_t *__restrict__ keys,
                                                           int32_t *__restrict__ bounds) {
    const int b = blockIdx.x * kThreads + threadIdx.x;
    if (b > K) return;
    int64_t lo = 0, hi = nnz;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (keys[mid] < static_cast<uint32_t>(b)) lo = mid + 1; else hi = mid;
    }
    bounds[b] = static_cast<int32_t>(lo);
}

// Merge path over rows (their end markers) and nonzeros: row r's end marker
// sits at position rowPtrs[r+1] + r.  row_start[b] = number of rows whose end
// marker lies before diagonal b * items_per_block.
__global__ __launch_bounds__(kThreads) void k_merge_partition(int32_t R, int32_t nnz,
                                                              const int32_t *__restrict__ rp,
                                                              int32_t nblocks,
                                                              int32_t *__restrict__ row_start) {
    const int64_t b = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (b > nblocks) return;
    const int64_t total = static_cast<int64_t>(R) + nnz;
    int64_t d = b * kMergeItemsPerBlock;
    if (d > total) d = total;
    int64_t lo = 0, hi = R;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (static_cast<int64_t>(rp[mid + 1]) + mid < d) lo = mid + 1; else hi = mid;
    }
    row_start[b] = static_cast<int32_t>(lo);
}

}  // namespace

hipError_t launch_count_rows(int32_t nnz, const int32_t *row, int32_t *counts, hipStream_t s) {
    if (nnz <= 0) return hipSuccess;
    const int64_t waves = (static_cast<int64_t>(nnz) + kWave * kCountSteps - 1) /
                          (kWave * kCountSteps);
    k_count_rows<<<grid_for(waves * kWave, kThreads), kThreads, 0, s>>>(nnz, row, counts);
    return hipGetLastError();
}

hipError_t launch_expand_rows(int32_t R, int32_t nnz, const int32_t *rp, int32_t *row_idx,
                              hipStream_t s) {
    if (R <= 0 || nnz <= 0) return hipSuccess;
    const int64_t waves = (static_cast<int64_t>(R) + kWave - 1) / kWave;
    k_expand_rows<<<grid_for(waves * kWave, kThreads), kThreads, 0, s>>>(R, rp, row_idx);
    return hipGetLastError();
}

hipError_t launch_build_ell(int32_t R, int32_t width, const int32_t *rp, const int32_t *col,
                            const float *val, int32_t *ell_col, float *ell_val,
                            int32_t *ell_nnz, hipStream_t s) {
    if (R <= 0) return hipSuccess;
    k_build_ell<<<grid_for(R, kThreads), kThreads, 0, s>>>(
        R, width, rp, col, reinterpret_cast<const uint32_t *>(val), ell_col,
        reinterpret_cast<uint32_t *>(ell_val), ell_nnz);
    return hipGetLastError();
}

hipError_t launch_xt_count(int32_t R, const int32_t *rp, const int32_t *col, int32_t *counts,
                           hipStream_t s) {
    if (R <= 0) return hipSuccess;
    k_xt_count<<<grid_for(R, kTileRows), kThreads, 0, s>>>(R, rp, col, counts);
    return hipGetLastError();
}

hipError_t launch_xt_fill(int32_t R, int32_t W, const int32_t *rp, const int32_t *col,
                          const float *val, const int32_t *run_ptr, int32_t *runs,
                          int16_t *lidx, float *ell_val, int32_t *ell_nnz, hipStream_t s) {
    if (R <= 0) return hipSuccess;
    k_xt_fill<<<grid_for(R, kTileRows), kThreads, 0, s>>>(
        R, W, rp, col, reinterpret_cast<const uint32_t *>(val), run_ptr, runs, lidx,
        reinterpret_cast<uint32_t *>(ell_val), ell_nnz);
    return hipGetLastError();
}

hipError_t launch_tail_lengths(int32_t R, int32_t K, const int32_t *rp, int32_t *tail_len,
                               hipStream_t s) {
    if (R <= 0) return hipSuccess;
    k_tail_lengths<<<grid_for(R, kThreads), kThreads, 0, s>>>(R, K, rp, tail_len);
    return hipGetLastError();
}

hipError_t launch_fill_tail(int32_t R, int32_t K, int32_t ntail, const int32_t *rp,
                            const int32_t *tail_off, const int32_t *col, const float *val,
                            int32_t *tail_row, int32_t *tail_col, float *tail_val,
                            hipStream_t s) {
    if (ntail <= 0) return hipSuccess;
    k_fill_tail<<<grid_for(ntail, kThreads), kThreads, 0, s>>>(
        R, K, ntail, rp, tail_off, col, reinterpret_cast<const uint32_t *>(val), tail_row,
        tail_col, reinterpret_cast<uint32_t *>(tail_val));
    return hipGetLastError();
}

hipError_t launch_jds_keys(int32_t R, int32_t W, const int32_t *rp, uint32_t *keys,
                           int32_t *rows, hipStream_t s) {
    if (R <= 0) return hipSuccess;
    k_jds_keys<<<grid_for(R, kThreads), kThreads, 0, s>>>(R, W, rp, keys, rows);
    return hipGetLastError();
}

hipError_t launch_jds_lengths(int32_t R, int32_t W, const uint32_t *sorted_keys,
                              int32_t *jds_len, hipStream_t s) {
    if (R <= 0) return hipSuccess;
    k_jds_lengths<<<grid_for(R, kThreads), kThreads, 0, s>>>(R, W, sorted_keys, jds_len);
    return hipGetLastError();
}

hipError_t launch_jds_counts(int32_t R, int32_t W, const int32_t *jds_len, int32_t *counts,
                             hipStream_t s) {
    if (W <= 0) return hipSuccess;
    k_jds_counts<<<grid_for(W, kThreads), kThreads, 0, s>>>(R, W, jds_len, counts);
    return hipGetLastError();
}

hipError_t launch_jds_fill(int32_t R, int32_t ntiles, int32_t depth, const int2 *tiles,
                           const int32_t *iter_ptr, const int32_t *perm, const int32_t *jds_len,
                           const int32_t *rp, const int32_t *col, const float *val,
                           int32_t *jds_col, float *jds_val, hipStream_t s) {
    if (ntiles <= 0) return hipSuccess;
    k_jds_fill<<<grid_for(static_cast<int64_t>(ntiles) * kWave, kThreads), kThreads, 0, s>>>(
        R, ntiles, depth, tiles, iter_ptr, perm, jds_len, rp, col,
        reinterpret_cast<const uint32_t *>(val), jds_col, reinterpret_cast<uint32_t *>(jds_val));
    return hipGetLastError();
}

hipError_t launch_sell_sizes(int32_t R, const int32_t *jds_len, int32_t *sizes, hipStream_t s) {
    if (R <= 0) return hipSuccess;
    const int64_t nsect = (static_cast<int64_t>(R) + kWave - 1) / kWave;
    k_sell_sizes<<<grid_for(nsect, kThreads), kThreads, 0, s>>>(R, jds_len, sizes);
    return hipGetLastError();
}

hipError_t launch_sell_fill(int32_t R, int32_t ntiles, int32_t depth, const int2 *tiles,
                            const int32_t *sect_ptr, const int32_t *jds_len, const int32_t *perm,
                            const int32_t *rp, const int32_t *col, const float *val,
                            int32_t *sell_col, float *sell_val, hipStream_t s) {
    if (ntiles <= 0) return hipSuccess;
    k_sell_fill<<<grid_for(static_cast<int64_t>(ntiles) * kWave, kThreads), kThreads, 0, s>>>(
        R, ntiles, depth, tiles, sect_ptr, jds_len, perm, rp, col,
        reinterpret_cast<const uint32_t *>(val), sell_col, reinterpret_cast<uint32_t *>(sell_val));
    return hipGetLastError();
}

hipError_t launch_jds_chunks(int32_t R, int32_t depth, const int32_t *jds_len,
                             int32_t *chunks, hipStream_t s) {
    if (R <= 0) return hipSuccess;
    const int64_t groups = (static_cast<int64_t>(R) + kWave - 1) / kWave;
    k_jds_chunks<<<grid_for(groups, kThreads), kThreads, 0, s>>>(R, depth, jds_len, chunks);
    return hipGetLastError();
}

hipError_t launch_jds_tiles(int32_t groups, int32_t ntiles, const int32_t *tile_off,
                            int2 *tiles, hipStream_t s) {
    if (ntiles <= 0) return hipSuccess;
    k_jds_tiles<<<grid_for(ntiles, kThreads), kThreads, 0, s>>>(groups, ntiles, tile_off, tiles);
    return hipGetLastError();
}

hipError_t launch_slice_keys(int32_t nnz, const int32_t *col, int32_t slice_cols,
                             uint32_t *keys, hipStream_t s) {
    if (nnz <= 0) return hipSuccess;
    k_slice_keys<<<grid_for(nnz, kThreads), kThreads, 0, s>>>(nnz, col, slice_cols, keys);
    return hipGetLastError();
}

hipError_t launch_slice_bounds(int32_t nnz, int32_t K, const uint32_t *keys, int32_t *bounds,
                               hipStream_t s) {
    k_slice_bounds<<<grid_for(static_cast<int64_t>(K) + 1, kThreads), kThreads, 0, s>>>(
        nnz, K, keys, bounds);
    return hipGetLastError();
}

hipError_t launch_merge_partition(int32_t R, int32_t nnz, const int32_t *rp, int32_t nblocks,
                                  int32_t *row_start, hipStream_t s) {
    k_merge_partition<<<grid_for(static_cast<int64_t>(nblocks) + 1, kThreads), kThreads, 0, s>>>(
        R, nnz, rp, nblocks, row_start);
    return hipGetLastError();
}

}  // namespace spmv
