// C ABI of the SpMV engine (include/spmv.h): argument checks, the analysis and
// build flow, the format selector, run dispatch, export and teardown.
#include <algorithm>
#include <cstring>
#include <memory>

#include "internal.h"

namespace spmv {

spmv_status from_hip(hipError_t e) {
    return e == hipErrorOutOfMemory ? SPMV_ERR_OOM : SPMV_ERR_HIP;
}

Scratch::~Scratch() {
    if (ptrs_.empty()) return;
    (void)hipStreamSynchronize(stream_);
    for (void *p : ptrs_) (void)hipFree(p);
}

spmv_status Scratch::alloc_bytes(void **p, size_t bytes) {
    *p = nullptr;
    hipError_t e = hipMalloc(p, bytes < 4 ? 4 : bytes);
    if (e != hipSuccess) {
        *p = nullptr;
        (void)hipGetLastError();
        return from_hip(e);
    }
    ptrs_.push_back(*p);
    return SPMV_OK;
}

namespace {

constexpr int64_t kInt32Max = 2147483647LL;

struct HandleDeleter {
    void operator()(spmv_handle *h) const {
        if (!h) return;
        for (spmv_handle *p : h->parts) (*this)(p);
        for (void *p : h->owned) (void)hipFree(p);
        delete h;
    }
};
using HandlePtr = std::unique_ptr<spmv_handle, HandleDeleter>;

template <typename T>
spmv_status halloc(spmv_handle *h, T **p, int64_t count) {
    *p = nullptr;
    const size_t bytes = static_cast<size_t>(count) * sizeof(T);
    void *q = nullptr;
    hipError_t e = hipMalloc(&q, bytes < 4 ? 4 : bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return from_hip(e);
    }
    h->owned.push_back(q);
    h->device_bytes += static_cast<int64_t>(bytes);
    *p = static_cast<T *>(q);
    return SPMV_OK;
}

spmv_opts resolve_opts(const spmv_opts *o) {
    spmv_opts r;
    spmv_opts_default(&r);
    if (o) r = *o;
    return r;
}

bool valid_lanes(int32_t l) { return l == 0 || (l >= 1 && l <= 64 && (l & (l - 1)) == 0); }

bool valid_opts(const spmv_opts &o) {
    return valid_lanes(o.lanes_per_row) && o.jds_depth >= 0 && o.max_bytes >= 0 &&
           o.col_blocks >= 0 && o.col_blocks <= kMaxColBlocks && o.reserved == 0;
}

bool valid_format(int32_t f) { return f >= SPMV_AUTO && f <= SPMV_COO_BLOCKED; }

// ---------------------------------------------------------------- analysis
struct Analysis {
    spmv_stats st{};
    std::vector<int64_t> hist;
};

spmv_status analyze_csr(int32_t R, int32_t C, int32_t nnz, const int32_t *rp,
                        const int32_t *col, bool validate, bool want_hist, Analysis &out,
                        hipStream_t s, Scratch &scratch) {
    // record 0: column-check flags; records 1..G: per-block row statistics
    const int G = row_check_blocks(R);
    RowStatsDev *d = nullptr;
    SPMV_TRY(scratch.alloc(&d, static_cast<size_t>(G) + 1));
    SPMV_HIP(hipMemsetAsync(d, 0, sizeof(RowStatsDev), s));
    SPMV_HIP(launch_row_checks(R, C, nnz, rp, col, d + 1, s));
    if (validate) SPMV_HIP(launch_col_checks(nnz, C, col, d, s));
    std::vector<RowStatsDev> parts(static_cast<size_t>(G) + 1);
    SPMV_HIP(hipMemcpyAsync(parts.data(), d, sizeof(RowStatsDev) * parts.size(),
                            hipMemcpyDeviceToHost, s));
    SPMV_HIP(hipStreamSynchronize(s));
    RowStatsDev h = parts[0];
    for (int i = 1; i <= G; ++i) {
        h.flags |= parts[i].flags;
        h.max_len = std::max(h.max_len, parts[i].max_len);
        h.sum_len_sq += parts[i].sum_len_sq;
        h.empty_rows += parts[i].empty_rows;
        h.sum_first_dist += parts[i].sum_first_dist;
    }
    if (h.flags & kFlagBadRowPtrs) return SPMV_ERR_BAD_ROWPTRS;
    if (h.flags & kFlagBadCol) return SPMV_ERR_BAD_COLIDX;
    out.st.num_rows = R;
    out.st.num_cols = C;
    out.st.nnz = nnz;
    out.st.max_len = h.max_len;
    out.st.sum_len_sq = static_cast<int64_t>(h.sum_len_sq);
    out.st.empty_rows = static_cast<int64_t>(h.empty_rows);
    const int64_t nonempty = static_cast<int64_t>(R) - out.st.empty_rows;
    out.st.col_spread =
        nonempty > 0 ? static_cast<int64_t>(h.sum_first_dist / static_cast<uint64_t>(nonempty)) : 0;
    if (want_hist) {
        const int64_t bins = out.st.max_len + 1;
        out.hist.assign(static_cast<size_t>(bins), 0);
        if (R > 0) {
            int32_t *dh = nullptr;
            SPMV_TRY(scratch.alloc(&dh, static_cast<size_t>(bins)));
            SPMV_HIP(hipMemsetAsync(dh, 0, sizeof(int32_t) * bins, s));
            SPMV_HIP(launch_len_hist(R, rp, static_cast<int32_t>(out.st.max_len), dh, s));
            std::vector<int32_t> tmp(static_cast<size_t>(bins));
            SPMV_HIP(hipMemcpyAsync(tmp.data(), dh, sizeof(int32_t) * bins,
                                    hipMemcpyDeviceToHost, s));
            SPMV_HIP(hipStreamSynchronize(s));
            for (int64_t i = 0; i < bins; ++i) out.hist[i] = tmp[i];
        }
    }
    return SPMV_OK;
}

// ---------------------------------------------------------------- selector
// Smallest k such that at least 99% of the rows have length <= k.
int64_t hyb_percentile_width(int64_t R, const int64_t *hist, int64_t bins) {
    int64_t below = 0;
    for (int64_t k = 0; k < bins; ++k) {
        below += hist[k];
        if (below * 100 >= R * 99) return k;
    }
    return bins - 1;
}

int32_t lanes_from_mean(int64_t R, int64_t nnz) {
    const int64_t mean_up = R > 0 ? (nnz + R - 1) / R : 0;
    int32_t L = 2;
    while (L < 64 && L < mean_up) L <<= 1;
    return L;
}

void select_format(const spmv_stats &st, const int64_t *hist, const spmv_opts &o,
                   int32_t *fmt, int32_t *K, int32_t *L) {
    const int64_t R = st.num_rows, nnz = st.nnz, W = st.max_len;
    *K = 0;
    *L = 0;
    const int64_t padded = W * R;             // slots of a full-width ELL
    // a padded format is taken only while its slots fit int32 indices
    if (padded <= 2 * nnz && padded <= kInt32Max) {   // max <= 2 * mean
        *fmt = SPMV_ELL;
    } else if (nnz < 10 * R) {                // mean < 10
        *fmt = SPMV_COO_SEGMENTED;
    } else if (padded > 5 * nnz) {            // max > 5 * mean
        const int64_t k = o.hyb_width > 0 ? o.hyb_width : hyb_percentile_width(R, hist, W + 1);
        if (2 * R * k <= 3 * nnz && R * k <= kInt32Max) {   // ELL part <= 1.5 * nnz slots
            *fmt = SPMV_HYB;
            *K = static_cast<int32_t>(k);
        } else {
            *fmt = SPMV_CSR_MERGE;
        }
    } else {
        *fmt = SPMV_CSR_VECTOR;
        *L = o.lanes_per_row > 0 ? o.lanes_per_row : lanes_from_mean(R, nnz);
    }
}

// ------------------------------------------------------------------ builds
spmv_status check_budget(const spmv_opts &o, int64_t bytes) {
    if (o.max_bytes > 0 && bytes > o.max_bytes) return SPMV_ERR_TOO_LARGE;
    return SPMV_OK;
}

spmv_status copy_csr(spmv_handle *h, int32_t R, int32_t nnz, const int32_t *rp,
                     const int32_t *col, const float *val, hipStream_t s) {
    SPMV_TRY(halloc(h, &h->a.row_ptrs, static_cast<int64_t>(R) + 1));
    SPMV_TRY(halloc(h, &h->a.col_idx, nnz));
    SPMV_TRY(halloc(h, &h->a.values, nnz));
    SPMV_HIP(hipMemcpyAsync(h->a.row_ptrs, rp, sizeof(int32_t) * (static_cast<size_t>(R) + 1),
                            hipMemcpyDeviceToDevice, s));
    if (nnz > 0) {
        SPMV_HIP(hipMemcpyAsync(h->a.col_idx, col, sizeof(int32_t) * nnz,
                                hipMemcpyDeviceToDevice, s));
        SPMV_HIP(hipMemcpyAsync(h->a.values, val, sizeof(float) * nnz, hipMemcpyDeviceToDevice,
                                s));
    }
    return SPMV_OK;
}

spmv_status build_ell_part(spmv_handle *h, int32_t R, int32_t width, const int32_t *rp,
                           const int32_t *col, const float *val, hipStream_t s) {
    const int64_t slots = static_cast<int64_t>(R) * width;
    if (slots > kInt32Max) return SPMV_ERR_TOO_LARGE;
    h->ell_width = width;
    SPMV_TRY(halloc(h, &h->a.ell_col, slots));
    SPMV_TRY(halloc(h, &h->a.ell_val, slots));
    SPMV_TRY(halloc(h, &h->a.ell_nnz, R));
    SPMV_HIP(launch_build_ell(R, width, rp, col, val, h->a.ell_col, h->a.ell_val, h->a.ell_nnz,
                              s));
    return SPMV_OK;
}

spmv_status build_hyb_tail(spmv_handle *h, int32_t R, int32_t K, const int32_t *rp,
                           const int32_t *col, const float *val, hipStream_t s,
                           Scratch &scratch) {
    int32_t *off = nullptr;
    SPMV_TRY(scratch.alloc(&off, static_cast<size_t>(R) + 1));
    SPMV_HIP(launch_tail_lengths(R, K, rp, off, s));
    SPMV_TRY(exclusive_scan(off, off, R, true, s, scratch));
    int32_t ntail = 0;
    SPMV_HIP(hipMemcpyAsync(&ntail, off + R, sizeof(int32_t), hipMemcpyDeviceToHost, s));
    SPMV_HIP(hipStreamSynchronize(s));
    h->tail_nnz = ntail;
    SPMV_TRY(halloc(h, &h->a.tail_row, ntail));
    SPMV_TRY(halloc(h, &h->a.tail_col, ntail));
    SPMV_TRY(halloc(h, &h->a.tail_val, ntail));
    SPMV_HIP(launch_fill_tail(R, K, ntail, rp, off, col, val, h->a.tail_row, h->a.tail_col,
                              h->a.tail_val, s));
    return SPMV_OK;
}

// JDS sort [REG, JDS: sort rows by nonzero count, longest first, recording
// the original index]: stable radix sort of (W - len, row) -> perm, lengths.
spmv_status jds_sort(spmv_handle *h, int32_t R, const int32_t *rp, hipStream_t s,
                     Scratch &scratch) {
    const int32_t W = static_cast<int32_t>(h->stats.max_len);
    uint32_t *keys = nullptr, *sorted = nullptr;
    int32_t *rows = nullptr;
    SPMV_TRY(scratch.alloc(&keys, R));
    SPMV_TRY(scratch.alloc(&sorted, R));
    SPMV_TRY(scratch.alloc(&rows, R));
    SPMV_TRY(halloc(h, &h->a.jds_perm, R));
    SPMV_TRY(halloc(h, &h->a.jds_len, R));
    SPMV_HIP(launch_jds_keys(R, W, rp, keys, rows, s));
    SPMV_TRY(radix_sort_pairs(keys, rows, sorted, h->a.jds_perm, R, bits_for(W), s, scratch));
    SPMV_HIP(launch_jds_lengths(R, W, sorted, h->a.jds_len, s));
    return SPMV_OK;
}

// Wave tiles over groups of 64 sorted rows: (group, chunk of `depth` columns).
spmv_status jds_tiles(spmv_handle *h, int32_t R, hipStream_t s, Scratch &scratch) {
    const int32_t groups = static_cast<int32_t>((static_cast<int64_t>(R) + kWave - 1) / kWave);
    int32_t *off = nullptr;
    SPMV_TRY(scratch.alloc(&off, static_cast<size_t>(groups) + 1));
    SPMV_HIP(launch_jds_chunks(R, h->jds_depth, h->a.jds_len, off, s));
    SPMV_TRY(exclusive_scan(off, off, groups, true, s, scratch));
    int32_t ntiles = 0;
    SPMV_HIP(hipMemcpyAsync(&ntiles, off + groups, sizeof(int32_t), hipMemcpyDeviceToHost, s));
    SPMV_HIP(hipStreamSynchronize(s));
    h->num_tiles = ntiles;
    SPMV_TRY(halloc(h, &h->a.jds_tiles, ntiles));
    SPMV_HIP(launch_jds_tiles(groups, ntiles, off, h->a.jds_tiles, s));
    return SPMV_OK;
}

spmv_status build_jds(spmv_handle *h, int32_t R, int32_t nnz, const int32_t *rp,
                      const int32_t *col, const float *val, hipStream_t s, Scratch &scratch) {
    const int32_t W = static_cast<int32_t>(h->stats.max_len);
    SPMV_TRY(jds_sort(h, R, rp, s, scratch));
    SPMV_TRY(halloc(h, &h->a.jds_iter_ptr, static_cast<int64_t>(W) + 1));
    SPMV_TRY(halloc(h, &h->a.jds_col, nnz));
    SPMV_TRY(halloc(h, &h->a.jds_val, nnz));
    SPMV_HIP(launch_jds_counts(R, W, h->a.jds_len, h->a.jds_iter_ptr, s));
    SPMV_TRY(exclusive_scan(h->a.jds_iter_ptr, h->a.jds_iter_ptr, W, true, s, scratch));
    SPMV_TRY(jds_tiles(h, R, s, scratch));
    SPMV_HIP(launch_jds_fill(R, h->num_tiles, h->jds_depth, h->a.jds_tiles, h->a.jds_iter_ptr,
                             h->a.jds_perm, h->a.jds_len, rp, col, val, h->a.jds_col,
                             h->a.jds_val, s));
    return SPMV_OK;
}

// Padded slots of the sectioned ELL, exactly, from the length histogram: the
// sorted lengths run from W down; section k starts at sorted position 64k and
// is as wide as the length found there.
int64_t sell_slots_from_hist(int64_t R, const std::vector<int64_t> &hist) {
    int64_t total = 0, pos = 0;
    for (int64_t l = static_cast<int64_t>(hist.size()) - 1; l >= 0; --l) {
        const int64_t c = hist[l];
        if (c == 0) continue;
        for (int64_t st = (pos + kWave - 1) / kWave * kWave; st < pos + c; st += kWave)
            total += std::min<int64_t>(kWave, R - st) * l;
        pos += c;
    }
    return total;
}

spmv_status build_sell(spmv_handle *h, int32_t R, const int32_t *rp, const int32_t *col,
                       const float *val, hipStream_t s, Scratch &scratch) {
    const int64_t slots = sell_slots_from_hist(R, h->hist);
    if (slots > kInt32Max) return SPMV_ERR_TOO_LARGE;
    h->sell_slots = slots;
    const int32_t nsect = static_cast<int32_t>((static_cast<int64_t>(R) + kWave - 1) / kWave);
    SPMV_TRY(jds_sort(h, R, rp, s, scratch));
    SPMV_TRY(halloc(h, &h->a.sell_ptr, static_cast<int64_t>(nsect) + 1));
    SPMV_TRY(halloc(h, &h->a.sell_col, slots));
    SPMV_TRY(halloc(h, &h->a.sell_val, slots));
    SPMV_HIP(launch_sell_sizes(R, h->a.jds_len, h->a.sell_ptr, s));
    SPMV_TRY(exclusive_scan(h->a.sell_ptr, h->a.sell_ptr, nsect, true, s, scratch));
    SPMV_TRY(jds_tiles(h, R, s, scratch));
    SPMV_HIP(launch_sell_fill(R, h->num_tiles, h->jds_depth, h->a.jds_tiles, h->a.sell_ptr,
                              h->a.jds_len, h->a.jds_perm, rp, col, val, h->a.sell_col,
                              h->a.sell_val, s));
    return SPMV_OK;
}

// Device bytes a format needs (checked against opts.max_bytes before building).
int64_t format_bytes(int32_t fmt, int64_t R, int64_t nnz, int64_t W, int64_t K,
                     const std::vector<int64_t> &hist) {
    switch (fmt) {
    case SPMV_COO_ATOMIC:
    case SPMV_COO_SEGMENTED: return 12 * nnz;
    case SPMV_CSR_SCALAR:
    case SPMV_CSR_VECTOR: return 8 * nnz + 4 * (R + 1);
    case SPMV_CSR_MERGE:
        return 8 * nnz + 4 * (R + 1) + 4 * ((R + nnz) / kMergeItemsPerBlock + 2);
    case SPMV_ELL: return 8 * R * W + 4 * R;
    case SPMV_HYB: {
        const int64_t w = std::min(K, W);
        int64_t tail = 0;
        for (int64_t l = w + 1; l < static_cast<int64_t>(hist.size()); ++l) tail += (l - w) * hist[l];
        return 8 * R * w + 4 * R + 12 * tail;
    }
    case SPMV_JDS: return 8 * nnz + 8 * R + 4 * (W + 1) + 8 * (R / kWave + 1 + nnz / kWave);
    case SPMV_SELL: {
        const int64_t slots = sell_slots_from_hist(R, hist);
        return 8 * slots + 8 * R + 4 * (R / kWave + 2) + 8 * (R / kWave + 1 + slots / kWave);
    }
    case SPMV_COO_BLOCKED: {
        // upper bound: every segment, chunk and work-item cut may end in a
        // partial group, and the group arrays carry kBcUnroll - 1 groups of
        // tail padding; chunks and work items are at most one per group
        const int64_t nblk = (R + kBcRows - 1) / kBcRows;
        const int64_t groups = nnz / kWave + nnz / bc_chunk_entries(nnz) + kNumXcd * nblk +
                               kBcCus + kBcUnroll;
        return 8 * kWave * groups + 4 * groups + 4 * nblk * kBcHot + 12 * (groups + 1) +
               8 * (kNumXcd + 1);
    }
    default: return 0;
    }
}

// ELL with x tiles: per-block counts from the device, checked and summed on
// the host.
struct XtPlan {
    bool ok = false;
    int64_t blocks = 0, tile_total = 0, runs = 0;
    int32_t max_tile = 0;
    std::vector<int32_t> run_ptr;   // [blocks + 1]
};

spmv_status plan_xtiles(int32_t R, const int32_t *rp, const int32_t *col, XtPlan &p,
                        hipStream_t s, Scratch &scratch) {
    p = XtPlan{};
    p.blocks = (static_cast<int64_t>(R) + kTileRows - 1) / kTileRows;
    p.run_ptr.assign(static_cast<size_t>(p.blocks) + 1, 0);
    if (p.blocks == 0) {
        p.ok = true;
        return SPMV_OK;
    }
    int32_t *counts = nullptr;
    SPMV_TRY(scratch.alloc(&counts, static_cast<size_t>(3 * p.blocks)));
    SPMV_HIP(launch_xt_count(R, rp, col, counts, s));
    std::vector<int32_t> hc(static_cast<size_t>(3 * p.blocks));
    SPMV_HIP(hipMemcpyAsync(hc.data(), counts, sizeof(int32_t) * hc.size(), hipMemcpyDeviceToHost,
                            s));
    SPMV_HIP(hipStreamSynchronize(s));
    p.ok = true;
    for (int64_t b = 0; b < p.blocks; ++b) {
        const int32_t d = hc[3 * b], n = hc[3 * b + 1], fits = hc[3 * b + 2];
        if (!fits || d > kTileMaxCols || n > kTileMaxRuns) p.ok = false;
        p.tile_total += d;
        p.max_tile = std::max(p.max_tile, d);
        p.run_ptr[b + 1] = static_cast<int32_t>(p.run_ptr[b] + n);
    }
    p.runs = p.run_ptr[p.blocks];
    return SPMV_OK;
}

int64_t xtile_bytes(int64_t R, int64_t W, const XtPlan &p) {
    return 6 * R * W + 4 * R + 12 * p.runs + 4 * (p.blocks + 1);
}

spmv_status build_ell_xtile(spmv_handle *h, int32_t R, int32_t W, const int32_t *rp,
                            const int32_t *col, const float *val, const XtPlan &p,
                            hipStream_t s) {
    h->ell_width = W;
    h->xt_runs = p.runs;
    h->xt_max_tile = p.max_tile;
    const int64_t slots = static_cast<int64_t>(R) * W;
    SPMV_TRY(halloc(h, &h->a.xt_run_ptr, p.blocks + 1));
    SPMV_TRY(halloc(h, &h->a.xt_runs, 3 * p.runs));
    SPMV_TRY(halloc(h, &h->a.xt_lidx, slots));
    SPMV_TRY(halloc(h, &h->a.ell_val, slots));
    SPMV_TRY(halloc(h, &h->a.ell_nnz, R));
    SPMV_HIP(hipMemcpyAsync(h->a.xt_run_ptr, p.run_ptr.data(), sizeof(int32_t) * p.run_ptr.size(),
                            hipMemcpyHostToDevice, s));
    SPMV_HIP(launch_xt_fill(R, W, rp, col, val, h->a.xt_run_ptr, h->a.xt_runs, h->a.xt_lidx,
                            h->a.ell_val, h->a.ell_nnz, s));
    return SPMV_OK;
}

// Number of x slices.  Automatic only for SPMV_AUTO: when x is larger than
// one XCD's L2 and the rows' columns are scattered (their first column lies
// more than C/8 from the diagonal on average), gathers from the whole x miss
// the L2 and go to the Infinity Cache; slices keep the gathers L2-resident at
// the price of one more visit to every row per slice.  Up to 16 MiB of x: 2,
// 4 or 8 slices of at most kXSliceXcdBytes (fewer while slices x rows would
// exceed a third of the nonzeros), run side by side on their own XCDs;
// beyond that, kXSliceBytes slices run one after another.
int32_t choose_col_blocks(const spmv_stats &st, spmv_format fmt, const spmv_opts &o) {
    const int64_t C = st.num_cols;
    int64_t K = 1;
    if (o.col_blocks > 0) {
        K = o.col_blocks;
    } else if (fmt == SPMV_AUTO && 4 * C > kL2Bytes && st.col_spread * 8 > C && st.nnz > 0 &&
               !bc_auto_rule(st)) {
        const int64_t xbytes = 4 * C;
        if (xbytes <= kNumXcd * kXSliceXcdBytes) {
            K = 2;
            while (K < kNumXcd && xbytes > K * kXSliceXcdBytes) K *= 2;
            // every slice visits every row: keep that work (K * R merge items)
            // within a third of the nonzeros (power law 4M: 8 slices 445 us,
            // 4 slices 440 us)
            while (K > 2 && 3 * K * st.num_rows > st.nnz) K /= 2;
        } else {
            K = (xbytes + kXSliceBytes - 1) / kXSliceBytes;
        }
    }
    K = std::min<int64_t>(K, kMaxColBlocks);
    K = std::min<int64_t>(K, std::max<int64_t>(C, 1));
    return static_cast<int32_t>(std::max<int64_t>(K, 1));
}

spmv_status build_csr_impl(spmv_handle **out, spmv_format fmt, int32_t R, int32_t C,
                           int32_t nnz, const int32_t *rp, const int32_t *col,
                           const float *val, const spmv_opts &o, hipStream_t s,
                           Scratch &scratch);

// A handle made of column slices: slice k holds the entries with column in
// [k*slice, (k+1)*slice) in their original order (global column indices) and
// is built as a matrix of its own.  Running the handle runs the slices in
// stream order.
spmv_status build_sliced(spmv_handle **out, spmv_format fmt, int32_t R, int32_t C, int32_t nnz,
                         const int32_t *rp, const int32_t *col, const float *val,
                         const spmv_opts &o, int32_t K, const Analysis &an, hipStream_t s,
                         Scratch &scratch) {
    HandlePtr h(new spmv_handle());
    SPMV_HIP(hipGetDevice(&h->device));
    h->stats = an.st;
    h->hist = an.hist;
    const int64_t slice = (static_cast<int64_t>(C) + K - 1) / K;
    h->slice_cols = static_cast<int32_t>(slice);
    h->col_blocks = static_cast<int32_t>((C + slice - 1) / slice);
    spmv_opts po = o;
    po.col_blocks = 1;
    po.validate = 0;
    // A slice of scattered columns is a thin matrix whose row lengths follow
    // the whole matrix's spread: an automatic build runs every slice as
    // merge-path CSR (balanced for any length distribution; measured fastest
    // per slice on the skewed and power-law workloads).  An explicit format is
    // kept as asked.
    if (fmt == SPMV_AUTO) fmt = SPMV_CSR_MERGE;
    // Group the entries by slice: row index per entry, then a stable sort on
    // the slice number (entries of a slice keep their row-major order) that
    // carries each entry's row, column and value along.  Slice b is the
    // sorted range [bounds[b], bounds[b+1]); its row pointers come from
    // counting its row indices and scanning, as in COO -> CSR.
    const int32_t nb = h->col_blocks;
    int32_t *row_idx = nullptr, *bounds = nullptr;
    uint32_t *keys = nullptr;
    const uint32_t *keys_sorted = nullptr;
    int32_t *rows_s = nullptr, *col_s = nullptr;
    float *val_s = nullptr;
    // one allocation for the five entry arrays (row index and slice key in,
    // rows, columns and values out), each 256-byte aligned
    const size_t nw = (static_cast<size_t>(nnz) + 63) & ~size_t{63};
    uint32_t *arrays = nullptr;
    SPMV_TRY(scratch.alloc(&arrays, 5 * nw));
    row_idx = reinterpret_cast<int32_t *>(arrays);
    keys = arrays + nw;
    rows_s = reinterpret_cast<int32_t *>(arrays + 2 * nw);
    col_s = reinterpret_cast<int32_t *>(arrays + 3 * nw);
    val_s = reinterpret_cast<float *>(arrays + 4 * nw);
    SPMV_TRY(scratch.alloc(&bounds, static_cast<size_t>(nb) + 1));
    SPMV_HIP(launch_expand_rows(R, nnz, rp, row_idx, s));
    SPMV_HIP(launch_slice_keys(nnz, col, static_cast<int32_t>(slice), keys, s));
    const uint32_t *pin[3] = {reinterpret_cast<const uint32_t *>(row_idx),
                              reinterpret_cast<const uint32_t *>(col),
                              reinterpret_cast<const uint32_t *>(val)};
    uint32_t *pout[3] = {reinterpret_cast<uint32_t *>(rows_s), reinterpret_cast<uint32_t *>(col_s),
                         reinterpret_cast<uint32_t *>(val_s)};
    SPMV_TRY(radix_sort(keys, nullptr, 3, pin, pout, nnz, bits_for(static_cast<uint64_t>(nb - 1)),
                        s, scratch, &keys_sorted));
    SPMV_HIP(launch_slice_bounds(nnz, nb, keys_sorted, bounds, s));
    std::vector<int32_t> hb(static_cast<size_t>(nb) + 1);
    SPMV_HIP(hipMemcpyAsync(hb.data(), bounds, sizeof(int32_t) * hb.size(), hipMemcpyDeviceToHost,
                            s));
    SPMV_HIP(hipStreamSynchronize(s));
    int64_t best_nnz = -1;
    // one row-pointer buffer serves every slice: each sub-build copies or
    // consumes it on this stream before the next slice overwrites it
    int32_t *prp = nullptr;
    SPMV_TRY(scratch.alloc(&prp, static_cast<size_t>(R) + 1));
    for (int32_t b = 0; b < nb; ++b) {
        const int32_t p0 = hb[b], pn = hb[b + 1] - hb[b];
        if (pn == 0) continue;
        SPMV_HIP(hipMemsetAsync(prp, 0, sizeof(int32_t) * (static_cast<size_t>(R) + 1), s));
        SPMV_HIP(launch_count_rows(pn, rows_s + p0, prp, s));
        SPMV_TRY(exclusive_scan(prp, prp, R, true, s, scratch));
        spmv_handle *part = nullptr;
        SPMV_TRY(build_csr_impl(&part, fmt, R, C, pn, prp, col_s + p0, val_s + p0, po, s,
                                scratch));
        h->parts.push_back(part);
        h->device_bytes += part->device_bytes;
        if (pn > best_nnz) {
            best_nnz = pn;
            h->format = part->format;
        }
    }
    if (h->parts.empty()) h->format = SPMV_ELL;
    SPMV_HIP(hipStreamSynchronize(s));
    if (o.max_bytes > 0 && h->device_bytes > o.max_bytes) return SPMV_ERR_TOO_LARGE;
    *out = h.release();
    return SPMV_OK;
}

spmv_status build_csr_impl(spmv_handle **out, spmv_format fmt, int32_t R, int32_t C,
                           int32_t nnz, const int32_t *rp, const int32_t *col,
                           const float *val, const spmv_opts &o, hipStream_t s,
                           Scratch &scratch) {
    Analysis an;
    SPMV_TRY(analyze_csr(R, C, nnz, rp, col, o.validate != 0, true, an, s, scratch));
    // Blocked COO: asked for, or taken by SPMV_AUTO (without an explicit slice
    // count) for scattered columns over an x larger than one L2, when a row
    // block holds at least one entry per 128-byte line of x on average.
    int32_t bc_slices = 0;
    if (fmt == SPMV_COO_BLOCKED) {
        bc_slices = o.col_blocks > 0 ? o.col_blocks : bc_auto_slices(C);
        if (bc_slices != 1 && bc_slices != 2 && bc_slices != 4 && bc_slices != 8)
            return SPMV_ERR_INVALID_ARG;
    } else if (fmt == SPMV_AUTO && o.col_blocks == 0 && bc_auto_rule(an.st)) {
        bc_slices = bc_auto_slices(C);
    } else {
        const int32_t K_slices = choose_col_blocks(an.st, fmt, o);
        if (K_slices > 1)
            return build_sliced(out, fmt, R, C, nnz, rp, col, val, o, K_slices, an, s, scratch);
    }
    int32_t f = bc_slices > 0 ? static_cast<int32_t>(SPMV_COO_BLOCKED) : fmt, K = 0, L = 0;
    if (f == SPMV_AUTO) {
        select_format(an.st, an.hist.data(), o, &f, &K, &L);
    } else if (f == SPMV_HYB) {
        K = o.hyb_width > 0 ? o.hyb_width
                            : static_cast<int32_t>(hyb_percentile_width(
                                  R, an.hist.data(), static_cast<int64_t>(an.hist.size())));
    } else if (f == SPMV_CSR_VECTOR) {
        L = o.lanes_per_row > 0 ? o.lanes_per_row : lanes_from_mean(R, nnz);
    }
    const int64_t W = an.st.max_len;
    // x tiles: asked for explicitly, or taken by SPMV_AUTO in place of ELL when
    // the matrix has at least kXtileAutoRows rows, every 256-row block
    // qualifies and each staged x word serves two gathers or more on average
    // (nnz >= 2 * total tile size)
    XtPlan xt;
    const bool ell_fits = static_cast<int64_t>(R) * W <= kInt32Max;
    if (f == SPMV_ELL_XTILE ||
        (fmt == SPMV_AUTO && f == SPMV_ELL && ell_fits && R >= kXtileAutoRows)) {
        SPMV_TRY(plan_xtiles(R, rp, col, xt, s, scratch));
        if (f == SPMV_ELL_XTILE && !xt.ok) return SPMV_ERR_TOO_LARGE;
        if (f == SPMV_ELL && xt.ok && static_cast<int64_t>(nnz) >= 2 * xt.tile_total)
            f = SPMV_ELL_XTILE;
    }
    if ((f == SPMV_ELL || f == SPMV_ELL_XTILE) && !ell_fits) return SPMV_ERR_TOO_LARGE;
    if (f == SPMV_HYB && static_cast<int64_t>(R) * std::min<int64_t>(K, W) > kInt32Max)
        return SPMV_ERR_TOO_LARGE;
    SPMV_TRY(check_budget(o, f == SPMV_ELL_XTILE ? xtile_bytes(R, W, xt)
                                                : format_bytes(f, R, nnz, W, K, an.hist)));

    HandlePtr h(new spmv_handle());
    SPMV_HIP(hipGetDevice(&h->device));
    h->format = f;
    h->stats = an.st;
    h->hist = an.hist;
    h->jds_depth = o.jds_depth > 0 ? o.jds_depth : kJdsDepthDefault;
    h->slice_cols = C;
    switch (f) {
    case SPMV_COO_ATOMIC:
    case SPMV_COO_SEGMENTED:
        SPMV_TRY(halloc(h.get(), &h->a.row_idx, nnz));
        SPMV_TRY(halloc(h.get(), &h->a.col_idx, nnz));
        SPMV_TRY(halloc(h.get(), &h->a.values, nnz));
        SPMV_HIP(launch_expand_rows(R, nnz, rp, h->a.row_idx, s));
        if (nnz > 0) {
            SPMV_HIP(hipMemcpyAsync(h->a.col_idx, col, sizeof(int32_t) * nnz,
                                    hipMemcpyDeviceToDevice, s));
            SPMV_HIP(hipMemcpyAsync(h->a.values, val, sizeof(float) * nnz,
                                    hipMemcpyDeviceToDevice, s));
        }
        break;
    case SPMV_CSR_SCALAR: {
        SPMV_TRY(copy_csr(h.get(), R, nnz, rp, col, val, s));
        // LDS staging pays for rows longer than 8 on average when almost no
        // wave holds a row longer than 32 (whose wave would fall back to
        // direct loads at the staging kernel's lower occupancy)
        int64_t over32 = 0;
        for (size_t k = 33; k < an.hist.size(); ++k) over32 += an.hist[k];
        h->csr_staged = (nnz > 8 * static_cast<int64_t>(R) && 100 * over32 < R) ? 1 : 0;
        break;
    }
    case SPMV_CSR_VECTOR:
        h->lanes = L;
        SPMV_TRY(copy_csr(h.get(), R, nnz, rp, col, val, s));
        break;
    case SPMV_CSR_MERGE: {
        SPMV_TRY(copy_csr(h.get(), R, nnz, rp, col, val, s));
        const int64_t blocks =
            (static_cast<int64_t>(R) + nnz + kMergeItemsPerBlock - 1) / kMergeItemsPerBlock;
        h->num_tiles = blocks;
        SPMV_TRY(halloc(h.get(), &h->a.merge_row_start, blocks + 1));
        SPMV_HIP(launch_merge_partition(R, nnz, h->a.row_ptrs, static_cast<int32_t>(blocks),
                                        h->a.merge_row_start, s));
        break;
    }
    case SPMV_ELL:
        SPMV_TRY(build_ell_part(h.get(), R, static_cast<int32_t>(W), rp, col, val, s));
        break;
    case SPMV_HYB: {
        h->hyb_width = K;
        const int32_t w = static_cast<int32_t>(std::min<int64_t>(K, W));
        SPMV_TRY(build_ell_part(h.get(), R, w, rp, col, val, s));
        SPMV_TRY(build_hyb_tail(h.get(), R, w, rp, col, val, s, scratch));
        break;
    }
    case SPMV_JDS:
        SPMV_TRY(build_jds(h.get(), R, nnz, rp, col, val, s, scratch));
        break;
    case SPMV_SELL:
        SPMV_TRY(build_sell(h.get(), R, rp, col, val, s, scratch));
        break;
    case SPMV_ELL_XTILE:
        SPMV_TRY(build_ell_xtile(h.get(), R, static_cast<int32_t>(W), rp, col, val, xt, s));
        break;
    case SPMV_COO_BLOCKED:
        SPMV_TRY(build_coo_blocked(h.get(), R, C, nnz, rp, col, val, bc_slices, s, scratch));
        break;
    default:
        return SPMV_ERR_INVALID_ARG;
    }
    SPMV_HIP(hipStreamSynchronize(s));
    // the estimate checked before building can fall short (blocked COO's wide
    // groups, JDS tiles at a small depth): the budget bounds what the handle
    // actually keeps, so a larger result is freed and refused
    if (o.max_bytes > 0 && h->device_bytes > o.max_bytes) return SPMV_ERR_TOO_LARGE;
    *out = h.release();
    return SPMV_OK;
}

spmv_status coo_to_csr_impl(int32_t R, int32_t C, int32_t nnz, const int32_t *ri,
                            const int32_t *ci, const float *v, int32_t *rp_out, int32_t *c_out,
                            float *v_out, bool validate, hipStream_t s, Scratch &scratch) {
    int flags = 0;
    if (nnz > 0) {
        const int nb = coo_check_blocks(nnz);
        int *part = nullptr;
        SPMV_TRY(scratch.alloc(&part, static_cast<size_t>(nb)));
        SPMV_HIP(launch_coo_checks(nnz, R, C, ri, ci, validate ? 1 : 0, part, s));
        std::vector<int> hp(static_cast<size_t>(nb));
        SPMV_HIP(hipMemcpyAsync(hp.data(), part, sizeof(int) * nb, hipMemcpyDeviceToHost, s));
        SPMV_HIP(hipStreamSynchronize(s));
        for (int f : hp) flags |= f;
    }
    if (flags & kFlagBadRow) return SPMV_ERR_BAD_ROWIDX;
    if (flags & kFlagBadCol) return SPMV_ERR_BAD_COLIDX;
    if (nnz == 0) {
        SPMV_HIP(hipMemsetAsync(rp_out, 0, sizeof(int32_t) * (static_cast<size_t>(R) + 1), s));
        return SPMV_OK;
    }
    if (!(flags & kFlagUnsortedRows)) {
        // already grouped by row: (i) entries per row (one atomic per run),
        // (ii) exclusive scan -> rowPtrs, (iii) the entries stay where they are
        SPMV_HIP(hipMemsetAsync(rp_out, 0, sizeof(int32_t) * (static_cast<size_t>(R) + 1), s));
        SPMV_HIP(launch_count_rows(nnz, ri, rp_out, s));
        SPMV_TRY(exclusive_scan(rp_out, rp_out, R, true, s, scratch));
        SPMV_HIP(hipMemcpyAsync(c_out, ci, sizeof(int32_t) * nnz, hipMemcpyDeviceToDevice, s));
        SPMV_HIP(hipMemcpyAsync(v_out, v, sizeof(float) * nnz, hipMemcpyDeviceToDevice, s));
        return SPMV_OK;
    }
    // stable sort of the entries by row (entries of a row keep their input
    // order), columns and values moving with their rows straight into the
    // outputs; the row counts are then taken on the sorted rows (one atomic
    // per run of equal rows per wave instead of one per entry) and scanned
    // into rowPtrs
    const uint32_t *keys_sorted = nullptr;
    const uint32_t *pin[2] = {reinterpret_cast<const uint32_t *>(ci),
                              reinterpret_cast<const uint32_t *>(v)};
    uint32_t *pout[2] = {reinterpret_cast<uint32_t *>(c_out), reinterpret_cast<uint32_t *>(v_out)};
    SPMV_TRY(radix_sort(reinterpret_cast<const uint32_t *>(ri), nullptr, 2, pin, pout, nnz,
                        bits_for(R > 0 ? static_cast<uint64_t>(R - 1) : 0), s, scratch,
                        &keys_sorted));
    SPMV_HIP(hipMemsetAsync(rp_out, 0, sizeof(int32_t) * (static_cast<size_t>(R) + 1), s));
    SPMV_HIP(launch_count_rows(nnz, reinterpret_cast<const int32_t *>(keys_sorted), rp_out, s));
    SPMV_TRY(exclusive_scan(rp_out, rp_out, R, true, s, scratch));
    return SPMV_OK;
}

bool bad_sizes(int32_t R, int32_t C, int32_t nnz) { return R < 0 || C < 0 || nnz < 0; }

spmv_status check_device(const spmv_handle *h) {
    int dev = -1;
    SPMV_HIP(hipGetDevice(&dev));
    return dev == h->device ? SPMV_OK : SPMV_ERR_DEVICE;
}

}  // namespace
}  // namespace spmv

using namespace spmv;

extern "C" {

void spmv_opts_default(spmv_opts *o) {
    if (!o) return;
    std::memset(o, 0, sizeof(*o));
    o->validate = 1;
}

spmv_status spmv_analyze(int32_t R, int32_t C, int32_t nnz, const int32_t *rp,
                         const int32_t *col, int32_t validate, spmv_stats *st, int64_t *hist,
                         int64_t hist_cap, void *stream) {
    if (bad_sizes(R, C, nnz) || !rp || !st || (nnz > 0 && !col) ||
        (hist && hist_cap < 0))
        return SPMV_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Scratch scratch(s);
    Analysis an;
    SPMV_TRY(analyze_csr(R, C, nnz, rp, col, validate != 0, hist != nullptr, an, s, scratch));
    *st = an.st;
    if (hist) {
        const int64_t n = std::min<int64_t>(hist_cap, static_cast<int64_t>(an.hist.size()));
        for (int64_t i = 0; i < n; ++i) hist[i] = an.hist[i];
    }
    return SPMV_OK;
}

spmv_status spmv_select(const spmv_stats *st, const int64_t *hist, const spmv_opts *opts,
                        int32_t *fmt, int32_t *K, int32_t *L) {
    if (!st || !hist || !fmt || !K || !L) return SPMV_ERR_INVALID_ARG;
    const spmv_opts o = resolve_opts(opts);
    if (!valid_lanes(o.lanes_per_row) || st->num_rows < 0 || st->nnz < 0 || st->max_len < 0)
        return SPMV_ERR_INVALID_ARG;
    select_format(*st, hist, o, fmt, K, L);
    return SPMV_OK;
}

spmv_status spmv_build(spmv_handle **out, spmv_format fmt, int32_t R, int32_t C, int32_t nnz,
                       const int32_t *rp, const int32_t *col, const float *val,
                       const spmv_opts *opts, void *stream) {
    if (!out) return SPMV_ERR_INVALID_ARG;
    *out = nullptr;
    const spmv_opts o = resolve_opts(opts);
    if (bad_sizes(R, C, nnz) || !rp || (nnz > 0 && (!col || !val)) || !valid_format(fmt) ||
        !valid_opts(o))
        return SPMV_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Scratch scratch(s);
    return build_csr_impl(out, fmt, R, C, nnz, rp, col, val, o, s, scratch);
}

spmv_status spmv_build_tuned(spmv_handle **out, int32_t R, int32_t C, int32_t nnz,
                             const int32_t *rp, const int32_t *col, const float *val,
                             const spmv_opts *opts, uint32_t format_mask, int32_t runs,
                             spmv_tune_report *report, void *stream) {
    if (!out) return SPMV_ERR_INVALID_ARG;
    *out = nullptr;
    const spmv_opts o = resolve_opts(opts);
    if (bad_sizes(R, C, nnz) || !rp || (nnz > 0 && (!col || !val)) || !valid_opts(o) ||
        runs < 0 || runs > 1000 || (format_mask & ~0xFFEu) != 0)
        return SPMV_ERR_INVALID_ARG;
    if (format_mask == 0) format_mask = 0xFFEu;   // formats 1..11
    if (runs == 0) runs = 5;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Scratch scratch(s);
    // checks and statistics once; candidates then build without the column pass
    Analysis an;
    SPMV_TRY(analyze_csr(R, C, nnz, rp, col, o.validate != 0, true, an, s, scratch));
    const int32_t auto_slices = choose_col_blocks(an.st, SPMV_AUTO, spmv_opts{});
    float *x = nullptr, *y = nullptr;
    SPMV_TRY(scratch.alloc(&x, static_cast<size_t>(std::max(C, 1))));
    SPMV_TRY(scratch.alloc(&y, static_cast<size_t>(std::max(R, 1))));
    SPMV_HIP(hipMemsetAsync(x, 0, sizeof(float) * std::max(C, 1), s));
    SPMV_HIP(hipMemsetAsync(y, 0, sizeof(float) * std::max(R, 1), s));
    hipEvent_t e0 = nullptr, e1 = nullptr;
    SPMV_HIP(hipEventCreate(&e0));
    hipError_t ee = hipEventCreate(&e1);
    if (ee != hipSuccess) {
        (void)hipEventDestroy(e0);
        return from_hip(ee);
    }
    spmv_tune_report rep{};
    rep.chosen = -1;
    HandlePtr best;
    float best_us = 0.f;
    spmv_status first_err = SPMV_OK;
    spmv_status fatal = SPMV_OK;
    for (int f = SPMV_COO_ATOMIC; f <= SPMV_COO_BLOCKED && fatal == SPMV_OK; ++f) {
        if (!(format_mask & (1u << f))) continue;
        for (int variant = 0; variant < 2 && fatal == SPMV_OK; ++variant) {
            // blocked COO slices x itself: one candidate, its automatic count
            const bool blocked = f == SPMV_COO_BLOCKED;
            const int32_t K = blocked ? 0 : variant == 0 ? 1 : auto_slices;
            if (variant == 1 && (blocked || auto_slices <= 1)) continue;
            if (rep.count >= SPMV_TUNE_MAX) break;
            spmv_tune_entry &ent = rep.entry[rep.count++];
            ent.format = f;
            ent.col_blocks = blocked ? bc_auto_slices(C) : K;
            spmv_opts oc = o;
            oc.validate = 0;
            oc.col_blocks = K;
            if (oc.max_bytes == 0) {   // not worth timing: more than 8x the CSR arrays
                const int64_t csr = 8 * static_cast<int64_t>(nnz) + 4 * (static_cast<int64_t>(R) + 1);
                oc.max_bytes = std::max<int64_t>(int64_t(64) << 20, 8 * csr);
            }
            spmv_handle *raw = nullptr;
            spmv_status st;
            {
                Scratch cand(s);   // the candidate's build scratch, freed before the next
                st = build_csr_impl(&raw, static_cast<spmv_format>(f), R, C, nnz, rp, col, val,
                                    oc, s, cand);
            }
            HandlePtr h(raw);
            ent.status = st;
            if (st != SPMV_OK) {
                if (first_err == SPMV_OK) first_err = st;
                if (st == SPMV_ERR_HIP) fatal = st;   // the device is in trouble: stop
                continue;
            }
            // one warm-up run, then `runs` individually timed runs
            std::vector<float> t;
            st = launch_spmv(h.get(), x, y, s);
            for (int i = 0; i < runs && st == SPMV_OK; ++i) {
                hipError_t he = hipEventRecord(e0, s);
                if (he == hipSuccess) st = launch_spmv(h.get(), x, y, s);
                if (he == hipSuccess && st == SPMV_OK) he = hipEventRecord(e1, s);
                if (he == hipSuccess && st == SPMV_OK) he = hipEventSynchronize(e1);
                float ms = 0.f;
                if (he == hipSuccess && st == SPMV_OK) he = hipEventElapsedTime(&ms, e0, e1);
                if (he != hipSuccess) st = from_hip(he);
                t.push_back(ms);
            }
            if (st != SPMV_OK) {
                ent.status = st;
                fatal = st;
                continue;
            }
            std::sort(t.begin(), t.end());
            ent.us = 1000.f * t[t.size() / 2];
            if (!best || ent.us < best_us) {
                best = std::move(h);
                best_us = ent.us;
                rep.chosen = rep.count - 1;
            }
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (report) *report = rep;
    if (fatal != SPMV_OK) return fatal;
    if (!best) return first_err != SPMV_OK ? first_err : SPMV_ERR_INVALID_ARG;
    SPMV_HIP(hipStreamSynchronize(s));
    *out = best.release();
    return SPMV_OK;
}

spmv_status spmv_coo_to_csr(int32_t R, int32_t C, int32_t nnz, const int32_t *ri,
                            const int32_t *ci, const float *v, int32_t *rp_out, int32_t *c_out,
                            float *v_out, int32_t validate, void *stream) {
    if (bad_sizes(R, C, nnz) || !rp_out || (nnz > 0 && (!ri || !ci || !v || !c_out || !v_out)))
        return SPMV_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Scratch scratch(s);
    SPMV_TRY(coo_to_csr_impl(R, C, nnz, ri, ci, v, rp_out, c_out, v_out, validate != 0, s,
                             scratch));
    SPMV_HIP(hipStreamSynchronize(s));
    return SPMV_OK;
}

spmv_status spmv_build_coo(spmv_handle **out, spmv_format fmt, int32_t R, int32_t C,
                           int32_t nnz, const int32_t *ri, const int32_t *ci, const float *v,
                           const spmv_opts *opts, void *stream) {
    if (!out) return SPMV_ERR_INVALID_ARG;
    *out = nullptr;
    const spmv_opts o = resolve_opts(opts);
    if (bad_sizes(R, C, nnz) || (nnz > 0 && (!ri || !ci || !v)) || !valid_format(fmt) ||
        !valid_opts(o))
        return SPMV_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Scratch scratch(s);
    int32_t *rp = nullptr, *c = nullptr;
    float *val = nullptr;
    SPMV_TRY(scratch.alloc(&rp, static_cast<size_t>(R) + 1));
    SPMV_TRY(scratch.alloc(&c, static_cast<size_t>(nnz)));
    SPMV_TRY(scratch.alloc(&val, static_cast<size_t>(nnz)));
    SPMV_TRY(coo_to_csr_impl(R, C, nnz, ri, ci, v, rp, c, val, o.validate != 0, s, scratch));
    spmv_opts o2 = o;
    o2.validate = 0;  // columns were checked on the COO input
    return build_csr_impl(out, fmt, R, C, nnz, rp, c, val, o2, s, scratch);
}

spmv_status spmv_run(const spmv_handle *h, const float *x, float *y, void *stream) {
    if (!h) return SPMV_ERR_INVALID_ARG;
    if (h->stats.num_rows == 0 || h->stats.nnz == 0) return SPMV_OK;
    if (!x || !y) return SPMV_ERR_INVALID_ARG;
    SPMV_TRY(check_device(h));
    return launch_spmv(h, x, y, static_cast<hipStream_t>(stream));
}

spmv_status spmv_cg(const spmv_handle *h, const float *b, float *x, int32_t max_iter, float rtol,
                    int32_t *iters, float *rel_resid, void *stream) {
    if (!h || !iters || !rel_resid || max_iter < 0 || !(rtol >= 0.f) ||
        h->stats.num_rows != h->stats.num_cols)
        return SPMV_ERR_INVALID_ARG;
    if (h->stats.num_rows > 0 && (!b || !x)) return SPMV_ERR_INVALID_ARG;
    SPMV_TRY(check_device(h));
    hipStream_t s = static_cast<hipStream_t>(stream);
    Scratch scratch(s);
    return conjugate_gradient(h, b, x, max_iter, rtol, iters, rel_resid, s, scratch);
}

spmv_status spmv_cg_noalloc(const spmv_handle *h, const float *b, float *x, int32_t max_iter,
                            float rtol, int32_t *iters, float *rel_resid, void *stream) {
    if (!h || !iters || !rel_resid || max_iter < 0 || !(rtol >= 0.f) ||
        h->stats.num_rows != h->stats.num_cols)
        return SPMV_ERR_INVALID_ARG;
    if (h->stats.num_rows > 0 && (!b || !x)) return SPMV_ERR_INVALID_ARG;
    SPMV_TRY(check_device(h));
    return conjugate_gradient_noalloc(h, b, x, max_iter, rtol, iters, rel_resid,
                                      static_cast<hipStream_t>(stream));
}

spmv_status spmv_get_info(const spmv_handle *h, spmv_info *info) {
    if (!h || !info) return SPMV_ERR_INVALID_ARG;
    std::memset(info, 0, sizeof(*info));
    info->format = h->format;
    info->hyb_width = h->hyb_width;
    info->lanes_per_row = h->lanes;
    info->ell_width = h->ell_width;
    info->col_blocks = h->col_blocks;
    info->slice_cols = h->slice_cols;
    info->stats = h->stats;
    info->tail_nnz = h->tail_nnz;
    info->num_tiles = h->num_tiles;
    info->device_bytes = h->device_bytes;
    if (h->format == SPMV_COO_BLOCKED) {
        info->groups = h->bc_groups;
        info->wide_groups = h->bc_wide_groups;
        info->block_rows = h->bc_rows;
        info->chunk_entries = static_cast<int32_t>(h->bc_chunk);
        info->hot_slots = kBcHot;
        info->hot_min_len = h->bc_hot_min_len;
        info->work_items = static_cast<int32_t>(h->bc_items);
    }
    return SPMV_OK;
}

}  // extern "C"

// Internal helper (C++ linkage): where an exportable array lives.
namespace {
struct ArrayRef {
    const void *dev = nullptr;
    const void *host = nullptr;
    size_t bytes = 0;
};

ArrayRef array_ref(const spmv_handle *h, spmv_array which) {
    const int64_t R = h->stats.num_rows, nnz = h->stats.nnz, W = h->stats.max_len;
    const int64_t slots = R * h->ell_width;
    const DevArrays &a = h->a;
    ArrayRef r;
    auto set = [&](const void *p, int64_t n, size_t elem) {
        if (p) {
            r.dev = p;
            r.bytes = static_cast<size_t>(n) * elem;
        }
    };
    switch (which) {
    case SPMV_A_ROW_PTRS: set(a.row_ptrs, R + 1, 4); break;
    case SPMV_A_COL_IDX: set(a.col_idx, nnz, 4); break;
    case SPMV_A_VALUES: set(a.values, nnz, 4); break;
    case SPMV_A_ROW_IDX: set(a.row_idx, nnz, 4); break;
    case SPMV_A_ELL_COL: set(a.ell_col, slots, 4); break;
    case SPMV_A_ELL_VAL: set(a.ell_val, slots, 4); break;
    case SPMV_A_ELL_NNZ: set(a.ell_nnz, R, 4); break;
    case SPMV_A_TAIL_ROW: set(a.tail_row, h->tail_nnz, 4); break;
    case SPMV_A_TAIL_COL: set(a.tail_col, h->tail_nnz, 4); break;
    case SPMV_A_TAIL_VAL: set(a.tail_val, h->tail_nnz, 4); break;
    case SPMV_A_JDS_PERM: set(a.jds_perm, R, 4); break;
    case SPMV_A_JDS_LEN: set(a.jds_len, R, 4); break;
    case SPMV_A_JDS_ITER_PTR: set(a.jds_iter_ptr, W + 1, 4); break;
    case SPMV_A_JDS_COL: set(a.jds_col, nnz, 4); break;
    case SPMV_A_JDS_VAL: set(a.jds_val, nnz, 4); break;
    case SPMV_A_SELL_SECT_PTR: set(a.sell_ptr, (R + kWave - 1) / kWave + 1, 4); break;
    case SPMV_A_SELL_COL: set(a.sell_col, h->sell_slots, 4); break;
    case SPMV_A_SELL_VAL: set(a.sell_val, h->sell_slots, 4); break;
    case SPMV_A_XT_RUN_PTR:
        set(a.xt_run_ptr, (R + kTileRows - 1) / kTileRows + 1, 4);
        break;
    case SPMV_A_XT_RUNS: set(a.xt_runs, 3 * h->xt_runs, 4); break;
    case SPMV_A_XT_LIDX: set(a.xt_lidx, slots, 2); break;
    case SPMV_A_BC_CHUNK_GRP: set(a.bc_chunk_grp, h->num_tiles + 1, 4); break;
    case SPMV_A_BC_CHUNK_BLK: set(a.bc_chunk_blk, h->num_tiles, 4); break;
    case SPMV_A_BC_SLICE_CHUNK: set(a.bc_slice_chunk, h->col_blocks + 1, 4); break;
    case SPMV_A_BC_HOT: set(a.bc_hot, h->bc_blocks * kBcHot, 4); break;
    case SPMV_A_BC_BASE: set(a.bc_base, h->bc_groups, 4); break;
    case SPMV_A_BC_PK: set(a.bc_pk, h->bc_groups * kWave, 4); break;
    case SPMV_A_BC_VAL: set(a.bc_val, h->bc_groups * kWave, 4); break;
    case SPMV_A_BC_WIDE: set(a.bc_wide, h->bc_wide_groups * kWave, 4); break;
    case SPMV_A_BC_SLICE_ITEM: set(a.bc_slice_item, h->col_blocks + 1, 4); break;
    case SPMV_A_BC_ITEM_CHUNK: set(a.bc_item_chunk, h->bc_items + 1, 4); break;
    case SPMV_A_LEN_HIST:
        r.host = h->hist.data();
        r.bytes = h->hist.size() * sizeof(int64_t);
        break;
    default: break;
    }
    return r;
}
}  // namespace

extern "C" {

spmv_status spmv_array_bytes(const spmv_handle *h, spmv_array which, size_t *bytes) {
    if (!h || !bytes) return SPMV_ERR_INVALID_ARG;
    *bytes = array_ref(h, which).bytes;
    return SPMV_OK;
}

spmv_status spmv_export(const spmv_handle *h, spmv_array which, void *dst, size_t bytes) {
    if (!h) return SPMV_ERR_INVALID_ARG;
    const ArrayRef r = array_ref(h, which);
    if (bytes != r.bytes || (bytes > 0 && !dst)) return SPMV_ERR_INVALID_ARG;
    if (bytes == 0) return SPMV_OK;
    if (r.host) {
        std::memcpy(dst, r.host, bytes);
        return SPMV_OK;
    }
    SPMV_TRY(check_device(h));
    SPMV_HIP(hipMemcpy(dst, r.dev, bytes, hipMemcpyDeviceToHost));
    return SPMV_OK;
}

spmv_status spmv_destroy(spmv_handle *h) {
    if (!h) return SPMV_OK;
    int prev = -1;
    (void)hipGetDevice(&prev);
    if (prev != h->device) (void)hipSetDevice(h->device);
    (void)hipDeviceSynchronize();
    HandleDeleter()(h);
    if (prev >= 0 && prev != h->device) (void)hipSetDevice(prev);
    return SPMV_OK;
}

const char *spmv_status_string(spmv_status st) {
    switch (st) {
    case SPMV_OK: return "ok";
    case SPMV_ERR_INVALID_ARG: return "invalid argument";
    case SPMV_ERR_BAD_ROWPTRS: return "bad row pointers (rowPtrs[0] != 0, decreasing, or rowPtrs[R] != nnz)";
    case SPMV_ERR_BAD_COLIDX: return "column index out of range";
    case SPMV_ERR_BAD_ROWIDX: return "row index out of range";
    case SPMV_ERR_TOO_LARGE: return "format too large (int32 slots or max_bytes)";
    case SPMV_ERR_OOM: return "device out of memory";
    case SPMV_ERR_HIP: return "HIP runtime error";
    case SPMV_ERR_DEVICE: return "handle used on a different device";
    default: return "unknown status";
    }
}

const char *spmv_format_name(spmv_format f) {
    switch (f) {
    case SPMV_AUTO: return "auto";
    case SPMV_COO_ATOMIC: return "coo_atomic";
    case SPMV_COO_SEGMENTED: return "coo_segmented";
    case SPMV_CSR_SCALAR: return "csr_scalar";
    case SPMV_CSR_VECTOR: return "csr_vector";
    case SPMV_ELL: return "ell";
    case SPMV_HYB: return "hyb";
    case SPMV_JDS: return "jds";
    case SPMV_CSR_MERGE: return "csr_merge";
    case SPMV_SELL: return "sell";
    case SPMV_ELL_XTILE: return "ell_xtile";
    case SPMV_COO_BLOCKED: return "coo_blocked";
    default: return "unknown";
    }
}

}  // extern "C"
