// Internal declarations of the gfx950 SpMV library: handle layout, device
// helpers shared by the kernels, and the host-side launchers each .hip file
// provides.  Nothing here is part of the public C ABI (include/spmv.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <vector>

#include "spmv.h"

namespace spmv {

constexpr int kWave = 64;       // CDNA wavefront width
constexpr int kNumXcd = 8;      // MI355X: 8 accelerator complex dies, 32 CUs each
constexpr int kJdsDepthDefault = 128;
// x slices for column splitting.  Up to 8 * kXSliceXcdBytes of x, the
// slices (2, 4 or 8, each at most kXSliceXcdBytes) run side by side in one
// launch, each on its own XCDs, so a slice leaves room in the 4 MiB L2 for
// the stream (skewed 2M rows: 4 slices 196 us, 2 slices 210 us).  Larger x
// is cut into kXSliceBytes slices run one pass after another (one XCD's L2
// each; 4 MiB beat 2 MiB once each slice pays its own pass over the rows).
constexpr int64_t kXSliceXcdBytes = 2 << 20;
constexpr int64_t kXSliceBytes = 4 << 20;
constexpr int64_t kL2Bytes = 4 << 20;
constexpr int kMaxColBlocks = 64;

// Merge-path CSR: 512 threads x 5 merge items (row ends + nonzeros) per block.
// (Swept on MI355X over 2-16 items and 128-1024 threads: short per-thread
// chains in large blocks win; the power-law matrix in 4 x slices 512 -> 478
// us, the skewed one in 2 slices 235 -> 222 us against 256 x 8.)
constexpr int kMergeThreads = 512;
constexpr int kMergeItemsPerThread = 5;
constexpr int kMergeItemsPerBlock = kMergeThreads * kMergeItemsPerThread;

// ELL with x tiles: rows in blocks of kTileRows; a block qualifies when its
// columns span fewer than kTileMaxSpan and it has at most kTileMaxCols
// distinct columns in at most kTileMaxRuns runs of consecutive columns.
constexpr int kTileRows = 256;
constexpr int kTileMaxSpan = 1 << 18;
constexpr int kTileMaxCols = 8192;
constexpr int kTileMaxRuns = 1024;
// SPMV_AUTO considers x tiles only from this many rows on (8 blocks per XCD)
constexpr int kXtileAutoRows = 64 * kTileRows;

// Blocked COO (x-scattered matrices): rows per block (the LDS partials of one
// workgroup), hot-row slots per block and the length above which a row is hot
// (kBcHotPerSlice * slices), one workgroup's threads and groups in flight per
// wave, the largest x slice of the automatic slice count (4 MiB: one XCD's
// L2), and the chunk rule (bc_chunk_entries): a chunk holds about 1.1 * nnz /
// kBcCus entries, so that the chunks fill the CUs about once, and at least
// kBcChunkMin.  A slice whose chunks would leave the most loaded of its CUs
// with more than kBcSkewNum / kBcSkewDen of an even share is cut instead into
// one work item per CU of equal cost, an entry costing 1 and each x line its
// segment touches kBcLineCost more.
// Measured on the power-law 4M-row matrix and the 2M-row skewed one, with
// every group's loads and gathers in flight together: 16384-row blocks in
// chunks of 65536 with 6 groups per wave (two workgroups per CU) 274 and 107
// us; 32768-row blocks in chunks of 131072 (one workgroup per CU, twice the
// entries per x line) with 6, 8, 10 groups per wave 267, 272, 274 and 97 us
// (with 4 and 5 groups: 264 us); all before the chunk-relative addressing.
constexpr int kBcRows = SPMV_BC_BLOCK_ROWS;
constexpr int kBcRowsTall = SPMV_BC_BLOCK_ROWS_TALL;
constexpr int kBcHot = 32;
constexpr int kBcHotPerSlice = 64;
constexpr int kBcThreads = 1024;
constexpr int kBcUnroll = 6;
constexpr int64_t kBcSliceBytes = 4 << 20;
constexpr int64_t kBcCus = 256;
constexpr int64_t kBcChunkMin = kBcRows / 4;
constexpr int64_t kBcLineCost = 3;
constexpr int64_t kBcSkewNum = 9, kBcSkewDen = 8;

// Validation flags written by the analysis kernels.
enum : int { kFlagBadRowPtrs = 1, kFlagBadCol = 2, kFlagBadRow = 4, kFlagUnsortedRows = 8 };

// ---------------------------------------------------------------------------
// Handle: every device array the built format needs.  Unused ones are null.
// ---------------------------------------------------------------------------
struct DevArrays {
    // CSR (CSR scalar / vector / merge)
    int32_t *row_ptrs = nullptr;
    int32_t *col_idx = nullptr;
    float *values = nullptr;
    // COO (COO atomic / segmented): col_idx, values above plus row_idx
    int32_t *row_idx = nullptr;
    // ELL or the ELL part of HYB
    int32_t *ell_col = nullptr;
    float *ell_val = nullptr;
    int32_t *ell_nnz = nullptr;
    // HYB COO tail
    int32_t *tail_row = nullptr;
    int32_t *tail_col = nullptr;
    float *tail_val = nullptr;
    // JDS
    int32_t *jds_perm = nullptr;
    int32_t *jds_len = nullptr;
    int32_t *jds_iter_ptr = nullptr;
    int32_t *jds_col = nullptr;
    float *jds_val = nullptr;
    int2 *jds_tiles = nullptr;      // (group of 64 sorted rows, depth chunk); SELL too
    // sectioned ELL (uses jds_perm, jds_len, jds_tiles as well)
    int32_t *sell_ptr = nullptr;    // [sections + 1]
    int32_t *sell_col = nullptr;
    float *sell_val = nullptr;
    // CSR merge: first row of each block's merge-path segment, [blocks + 1]
    int32_t *merge_row_start = nullptr;
    // ELL with x tiles (values and row lengths in ell_val / ell_nnz)
    int32_t *xt_run_ptr = nullptr;  // [blocks + 1]
    int32_t *xt_runs = nullptr;     // [3 * runs]: first column, offset in the tile, length
    int16_t *xt_lidx = nullptr;     // [R * W]: slot t of row r at t*R + r, tile position
    // blocked COO (layout in coo_blocked.hip)
    int32_t *bc_chunk_grp = nullptr;   // [chunks + 1] first group of each chunk
    int32_t *bc_chunk_blk = nullptr;   // [chunks] row block of each chunk
    int32_t *bc_slice_chunk = nullptr; // [slices + 1] first chunk of each x slice
    int32_t *bc_slice_item = nullptr;  // [slices + 1] first work item of each x slice
    int32_t *bc_item_chunk = nullptr;  // [items + 1] first chunk of each work item
    int32_t *bc_hot = nullptr;         // [blocks * kBcHot] hot rows, -1 unused
    int32_t *bc_base = nullptr;        // [groups] smallest column, or -(w+1): wide group w
    uint32_t *bc_pk = nullptr;         // [groups * 64] code << 16 | column offset
    float *bc_val = nullptr;           // [groups * 64]
    int32_t *bc_wide = nullptr;        // [wide groups * 64] columns of wide groups
};

}  // namespace spmv

struct spmv_handle {
    int device = 0;
    int32_t format = 0;
    int32_t hyb_width = 0;
    int32_t lanes = 0;
    int32_t ell_width = 0;
    int32_t csr_staged = 0;         // CSR scalar: waves stage their rows' entries in LDS
    int32_t jds_depth = spmv::kJdsDepthDefault;
    spmv_stats stats{};
    std::vector<int64_t> hist;      // host copy of the row-length histogram
    int64_t tail_nnz = 0;
    int64_t sell_slots = 0;
    int64_t xt_runs = 0;            // ELL x tiles: runs over all blocks
    int32_t xt_max_tile = 0;        // ELL x tiles: largest tile (floats of LDS)
    int64_t num_tiles = 0;
    int64_t device_bytes = 0;
    spmv::DevArrays a;
    std::vector<void *> owned;      // every device allocation of this handle
    // x slices: when non-empty the handle runs parts[k] (the columns of slice k)
    // in order and holds no arrays of its own.
    std::vector<spmv_handle *> parts;
    int32_t col_blocks = 1;
    int32_t slice_cols = 0;
    // blocked COO
    int32_t bc_rows = 0;            // rows per row block (kBcRows or kBcRowsTall)
    int64_t bc_blocks = 0;          // row blocks
    int64_t bc_groups = 0;          // groups of 64 slots
    int64_t bc_chunk = 0;           // entries per chunk (a segment's last may hold fewer)
    int64_t bc_wide_groups = 0;
    int64_t bc_grid = 0;            // workgroups of one launch
    int64_t bc_items = 0;           // work items, one workgroup each
    int32_t bc_hot_min_len = 0;     // rows of at least this length may be hot
};

namespace spmv {

// ---------------------------------------------------------------------------
// Host helpers
// ---------------------------------------------------------------------------
spmv_status from_hip(hipError_t e);

#define SPMV_HIP(expr)                                      \
    do {                                                    \
        hipError_t _e = (expr);                             \
        if (_e != hipSuccess) return ::spmv::from_hip(_e);  \
    } while (0)

#define SPMV_TRY(expr)                                      \
    do {                                                    \
        spmv_status _s = (expr);                            \
        if (_s != SPMV_OK) return _s;                       \
    } while (0)

// Temporary device buffers of one host call; freed (after the stream drains)
// when the object goes out of scope.  Freeing a large buffer costs ~0.1-0.25
// ms of host time (small ones next to nothing), so callers that need several
// large temporaries at once take them as one allocation.
class Scratch {
  public:
    explicit Scratch(hipStream_t s) : stream_(s) {}
    ~Scratch();
    Scratch(const Scratch &) = delete;
    Scratch &operator=(const Scratch &) = delete;
    template <typename T>
    spmv_status alloc(T **p, size_t count) {
        return alloc_bytes(reinterpret_cast<void **>(p), count * sizeof(T));
    }
    spmv_status alloc_bytes(void **p, size_t bytes);

  private:
    hipStream_t stream_;
    std::vector<void *> ptrs_;
};

inline unsigned grid_for(int64_t n, int per_block) {
    int64_t g = (n + per_block - 1) / per_block;
    return static_cast<unsigned>(g < 1 ? 1 : g);
}

inline int bits_for(uint64_t max_value) {
    int b = 0;
    while (b < 64 && (max_value >> b) != 0) ++b;
    return b;
}

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

// Workgroups are dispatched to the 8 XCDs round-robin (block b -> XCD b % 8).
// Re-number blocks so each XCD works on one contiguous range of logical
// blocks: neighbouring rows (and the x entries they share) then meet in the
// same 4 MB L2.
__device__ inline uint32_t xcd_remap(uint32_t b, uint32_t nblocks) {
    uint32_t per = nblocks / kNumXcd, rem = nblocks % kNumXcd;
    uint32_t xcd = b % kNumXcd, idx = b / kNumXcd;
    return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

template <typename T>
__device__ inline T ld_nt(const T *p) {
    return __builtin_nontemporal_load(p);
}

// DPP controls (gfx9 encoding)
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

#define SPMV_DPP_F32(v, ctrl)                                                              \
    __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, (v)), \
                                                          (ctrl), 0xF, 0xF, false))

// Sum over aligned groups of L lanes (L = 1..64, power of two).  Every lane of
// the wave must execute this with EXEC full; the result is valid in every lane
// of the group for L <= 32 and wave-uniform for L = 64.
template <int L>
__device__ inline float group_sum(float v) {
    if constexpr (L >= 2) v += SPMV_DPP_F32(v, kDppQuadXor1);
    if constexpr (L >= 4) v += SPMV_DPP_F32(v, kDppQuadXor2);
    if constexpr (L >= 8) v += SPMV_DPP_F32(v, kDppRowHalfMirror);
    if constexpr (L >= 16) v += SPMV_DPP_F32(v, kDppRowMirror);
    if constexpr (L >= 32) {
        // ds_swizzle bit mode within 32 lanes: and 0x1f, or 0, xor 0x10
        v += __builtin_bit_cast(float,
                                __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
    }
    if constexpr (L >= 64) {
        int bits = __builtin_bit_cast(int, v);
        v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(bits, 0)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(bits, 32));
    }
    return v;
}

// Largest i in [0, n) with a[i] <= key, for non-decreasing a with a[0] <= key.
__device__ inline int64_t upper_index(const int32_t *a, int64_t n, int64_t key) {
    int64_t lo = 0, hi = n - 1;
    while (lo < hi) {
        int64_t mid = (lo + hi + 1) >> 1;
        if (a[mid] <= key) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// Launchers provided by the .hip files (all enqueue on `s`)
// ---------------------------------------------------------------------------

// analyze.hip
struct RowStatsDev {                 // device-side accumulators
    int flags;
    int max_len;
    unsigned long long sum_len_sq;
    unsigned long long empty_rows;
    unsigned long long sum_first_dist;   // sum over non-empty rows of |col[rp[r]] - r*C/R|
};
// Row checks write one RowStatsDev per block (row_check_blocks(R) records);
// the caller adds them up.
int row_check_blocks(int32_t R);
hipError_t launch_row_checks(int32_t R, int32_t C, int32_t nnz, const int32_t *rp,
                             const int32_t *col, RowStatsDev *partial, hipStream_t s);
hipError_t launch_col_checks(int32_t nnz, int32_t C, const int32_t *col, RowStatsDev *st,
                             hipStream_t s);
// COO checks write one flags word per block (coo_check_blocks(nnz) words);
// the caller ORs them.
int coo_check_blocks(int32_t nnz);
hipError_t launch_coo_checks(int32_t nnz, int32_t R, int32_t C, const int32_t *row,
                             const int32_t *col, int check_cols, int *partial, hipStream_t s);
hipError_t launch_len_hist(int32_t R, const int32_t *rp, int32_t W, int32_t *hist, hipStream_t s);

// scan.hip: exclusive scan of n int32 values; out[n] receives the total when
// write_total.  in and out may alias.
spmv_status exclusive_scan(const int32_t *in, int32_t *out, int64_t n, bool write_total,
                           hipStream_t s, Scratch &scratch);

// sort.hip: stable LSD radix sort by the low key_bits of the keys; the
// num_payloads (1..3) arrays pay_in[q] move with them into pay_out[q].
// Outputs must not alias inputs.  keys_out may be null: the sorted keys then
// live in scratch and *keys_result points to them.
spmv_status radix_sort(const uint32_t *keys_in, uint32_t *keys_out, int num_payloads,
                       const uint32_t *const *pay_in, uint32_t *const *pay_out, int64_t n,
                       int key_bits, hipStream_t s, Scratch &scratch,
                       const uint32_t **keys_result = nullptr);
// The same with one int32 payload.
spmv_status radix_sort_pairs(const uint32_t *keys_in, const int32_t *vals_in,
                             uint32_t *keys_out, int32_t *vals_out, int64_t n, int key_bits,
                             hipStream_t s, Scratch &scratch);

// build.hip
hipError_t launch_count_rows(int32_t nnz, const int32_t *row, int32_t *counts, hipStream_t s);
hipError_t launch_expand_rows(int32_t R, int32_t nnz, const int32_t *rp, int32_t *row_idx,
                              hipStream_t s);
// ELL x tiles.  counts[3*b + {0,1,2}] = distinct columns, runs, span ok (1/0)
// of block b (kTileRows rows); xt_fill writes run_ptr must already hold the
// exclusive scan of the run counts.
hipError_t launch_xt_count(int32_t R, const int32_t *rp, const int32_t *col, int32_t *counts,
                           hipStream_t s);
hipError_t launch_xt_fill(int32_t R, int32_t W, const int32_t *rp, const int32_t *col,
                          const float *val, const int32_t *run_ptr, int32_t *runs,
                          int16_t *lidx, float *ell_val, int32_t *ell_nnz, hipStream_t s);
hipError_t launch_build_ell(int32_t R, int32_t width, const int32_t *rp, const int32_t *col,
                            const float *val, int32_t *ell_col, float *ell_val,
                            int32_t *ell_nnz, hipStream_t s);
hipError_t launch_tail_lengths(int32_t R, int32_t K, const int32_t *rp, int32_t *tail_len,
                               hipStream_t s);
hipError_t launch_fill_tail(int32_t R, int32_t K, int32_t ntail, const int32_t *rp,
                            const int32_t *tail_off, const int32_t *col, const float *val,
                            int32_t *tail_row, int32_t *tail_col, float *tail_val,
                            hipStream_t s);
hipError_t launch_jds_keys(int32_t R, int32_t W, const int32_t *rp, uint32_t *keys,
                           int32_t *rows, hipStream_t s);
hipError_t launch_jds_lengths(int32_t R, int32_t W, const uint32_t *sorted_keys,
                              int32_t *jds_len, hipStream_t s);
hipError_t launch_jds_counts(int32_t R, int32_t W, const int32_t *jds_len, int32_t *counts,
                             hipStream_t s);
hipError_t launch_jds_fill(int32_t R, int32_t ntiles, int32_t depth, const int2 *tiles,
                           const int32_t *iter_ptr, const int32_t *perm, const int32_t *jds_len,
                           const int32_t *rp, const int32_t *col, const float *val,
                           int32_t *jds_col, float *jds_val, hipStream_t s);
// Sectioned ELL: slots of each section of 64 sorted rows, and the fill.
hipError_t launch_sell_sizes(int32_t R, const int32_t *jds_len, int32_t *sizes, hipStream_t s);
hipError_t launch_sell_fill(int32_t R, int32_t ntiles, int32_t depth, const int2 *tiles,
                            const int32_t *sect_ptr, const int32_t *jds_len, const int32_t *perm,
                            const int32_t *rp, const int32_t *col, const float *val,
                            int32_t *sell_col, float *sell_val, hipStream_t s);
hipError_t launch_jds_chunks(int32_t R, int32_t depth, const int32_t *jds_len,
                             int32_t *chunks, hipStream_t s);
hipError_t launch_jds_tiles(int32_t groups, int32_t ntiles, const int32_t *tile_off,
                            int2 *tiles, hipStream_t s);
// x slices: keys[i] = col[i] / slice_cols; bounds[b] = first sorted entry
// of slice b (bounds[K] = nnz).
hipError_t launch_slice_keys(int32_t nnz, const int32_t *col, int32_t slice_cols,
                             uint32_t *keys, hipStream_t s);
hipError_t launch_slice_bounds(int32_t nnz, int32_t K, const uint32_t *keys, int32_t *bounds,
                               hipStream_t s);
hipError_t launch_merge_partition(int32_t R, int32_t nnz, const int32_t *rp, int32_t nblocks,
                                  int32_t *row_start, hipStream_t s);

// spmv_kernels.hip: y <- A x + y for the handle's format
spmv_status launch_spmv(const spmv_handle *h, const float *x, float *y, hipStream_t s);

// coo_blocked.hip: the automatic rule (scattered columns, x beyond one L2,
// at least one entry of a row block per 128-byte x line on average), the
// automatic slice count, the builder and the launcher.
bool bc_auto_rule(const spmv_stats &st);
int32_t bc_auto_slices(int64_t num_cols);
int64_t bc_chunk_entries(int64_t nnz);
spmv_status build_coo_blocked(spmv_handle *h, int32_t R, int32_t C, int32_t nnz,
                              const int32_t *rp, const int32_t *col, const float *val, int32_t S,
                              hipStream_t s, Scratch &scratch);
hipError_t launch_coo_blocked(const spmv_handle *h, const float *x, float *y, hipStream_t s);

// cg.hip: conjugate gradient on a square handle (host-synchronous); the
// allocation-free variant uses a static per-device workspace and direct
// launches (the caller must be on the handle's device)
spmv_status conjugate_gradient(const spmv_handle *A, const float *b, float *x, int32_t max_iter,
                               float rtol, int32_t *iters, float *rel_resid, hipStream_t s,
                               Scratch &scratch);
spmv_status conjugate_gradient_noalloc(const spmv_handle *A, const float *b, float *x,
                                       int32_t max_iter, float rtol, int32_t *iters,
                                       float *rel_resid, hipStream_t s);

}  // namespace spmv
