/*
 * spmv.h -- C ABI of the MI355X (gfx950) sparse matrix-vector
 * multiply-accumulate engine.
 *
 * Operation: y <- A*x + y, with A sparse (fp32 values, int32 indices) and x, y
 * dense fp32 vectors.  This is the SpMV defined on the PMPP notes page
 * "Sparse Matrices and Basic Formats (COO & CSR)", background section:
 * sparse matrix-vector multiplication AND accumulation, the core of iterative
 * solvers such as conjugate gradient, with a standard library interface.
 *
 * Pages cited below:
 *   [COO/CSR]   PMPP notes ch.14, "Sparse Matrices and Basic Formats (COO & CSR)"
 *   [REG]       PMPP notes ch.14, "Regularized Formats (ELL, Hybrid ELL-COO, JDS)"
 *   [CHOICE]    "SpMV storage-format choice and performance comparison"
 *               (CUDA tuning article), numbered sections
 *   [INTRO]     "Introduction to sparse computing and locating performance
 *               bottlenecks", section on the three checks (density, memory
 *               efficiency, parallel efficiency)
 *   [SPGEMM]    SpGEMM/AIA article, section 5.3 (input checks for CSR)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Device pointers.  Every array argument named *_dev is a device pointer
 *    on the current HIP device (e.g. torch.Tensor.data_ptr() of a cuda
 *    tensor).  Host pointers are named *_host.
 *  - Streams.  `stream` is a hipStream_t passed as void* (NULL = the null
 *    stream).  Work is ordered on that stream.
 *  - Index types.  int32, signed.  nnz, rows and columns are below 2^31; an
 *    ELL slot index t*R + r must also stay below 2^31 (else
 *    SPMV_ERR_TOO_LARGE).
 *  - Ownership.  The caller owns every input array, x and y.  A handle owns
 *    device copies of every format array it needs; inputs may be freed or
 *    reused as soon as spmv_build / spmv_build_coo return.  spmv_destroy
 *    frees the handle's memory.
 *  - Synchronisation.  spmv_analyze, spmv_build, spmv_build_coo and
 *    spmv_coo_to_csr are host-synchronous (they read row statistics back and
 *    wait for their own stream before returning).  spmv_run is asynchronous on
 *    `stream`: it allocates nothing, never synchronises and only enqueues
 *    kernels.
 *  - Errors.  Every call returns a spmv_status; nothing throws across the ABI.
 *    On error no handle is returned (*out is set to NULL) and no memory is
 *    leaked.  A HIP runtime or launch failure maps to SPMV_ERR_HIP.
 *  - Concurrency.  A handle is read-only after build; it may be run from
 *    several streams at once provided each run writes a distinct y.  x and y
 *    must not overlap.
 */
#ifndef SPMV_MI355X_H
#define SPMV_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum spmv_status {
    SPMV_OK = 0,
    SPMV_ERR_INVALID_ARG = 1,  /* null pointer, negative size, bad option      */
    SPMV_ERR_BAD_ROWPTRS = 2,  /* rowPtrs[0] != 0, decreasing, or != nnz at end */
    SPMV_ERR_BAD_COLIDX = 3,   /* a column index outside [0, num_cols)          */
    SPMV_ERR_BAD_ROWIDX = 4,   /* a COO row index outside [0, num_rows)         */
    SPMV_ERR_TOO_LARGE = 5,    /* format exceeds int32 slots or opts.max_bytes  */
    SPMV_ERR_OOM = 6,          /* device allocation failed                      */
    SPMV_ERR_HIP = 7,          /* HIP runtime or kernel launch error            */
    SPMV_ERR_DEVICE = 8        /* handle used on another device than its own    */
} spmv_status;

/* Blocked COO layout constant (SPMV_COO_BLOCKED): rows per row block, whose
 * partials one workgroup keeps in LDS.  A chunk is a run of one segment's
 * entries (one x slice, one row block) whose partials are flushed to y
 * together; a work item, one workgroup's work, is one or more consecutive
 * chunks.  Each x slice takes one of two rules:
 *   - by chunk: segments cut into chunks of T = max(8192, ceil(ceil(11 * nnz /
 *     2560) / 64) * 64) entries (about 1.1 * nnz / 256, in whole groups of 64:
 *     the chunks cover the 256 CUs about once), the last one the remainder,
 *     joined to the chunk before it when shorter than T/2; one chunk per item;
 *     spmv_info.chunk_entries reports T;
 *   - balanced: P = 256 / S items of about equal cost.  An entry of segment s
 *     costs r_s = floor((n_s + 3 * lines_s) * 1024 / n_s), n_s being the
 *     segment's entries and lines_s the 128-byte lines of x they touch (an
 *     entry costs 1024, each line 3 * 1024 more, spread evenly over the
 *     segment); item w < P - 1 ends at the first position of the slice whose
 *     preceding entries cost at least floor(total * (w + 1) / P), and each
 *     item's range is cut at segment boundaries into chunks.
 * A slice takes the balanced rule when it holds at least P * 8192 entries and
 * its by-chunk chunks, dealt in order each to the least loaded of P
 * workgroups (a chunk costing its entries times r_s), would leave the most
 * loaded with more than 9/8 of total / P (8 * most * P > 9 * total). */
#define SPMV_BC_BLOCK_ROWS 32768
/* A blocked-COO build whose SPMV_BC_BLOCK_ROWS-row layout cuts some x slice
 * into balanced work items is redone with blocks of SPMV_BC_BLOCK_ROWS_TALL
 * rows (the most whose partials fit the LDS); spmv_info.block_rows tells
 * which. */
#define SPMV_BC_BLOCK_ROWS_TALL 38912

/* Storage formats / kernels.  SPMV_AUTO lets the selector choose. */
typedef enum spmv_format {
    SPMV_AUTO = 0,
    SPMV_COO_ATOMIC = 1,    /* one lane per nonzero, atomic add [COO/CSR, COO kernel]       */
    SPMV_COO_SEGMENTED = 2, /* wave-wide segmented sum of row runs, one atomic per run     */
    SPMV_CSR_SCALAR = 3,    /* one lane per row, row pointers staged in LDS [COO/CSR, CSR
                               kernel; CHOICE 2.1 and 4.2]                                  */
    SPMV_CSR_VECTOR = 4,    /* a group of 2..64 lanes per row [CHOICE 2.2]                 */
    SPMV_ELL = 5,           /* padded, column-major, one lane per row [REG, ELL]           */
    SPMV_HYB = 6,           /* ELL of width K + COO tail [REG, hybrid; CHOICE 3.2, 4.1]    */
    SPMV_JDS = 7,           /* rows sorted by length, jagged column-major [REG, JDS]       */
    SPMV_CSR_MERGE = 8,     /* merge-path: equal shares of rows+nonzeros per block
                               [CHOICE 5.2; INTRO, parallel efficiency]                    */
    SPMV_SELL = 9,          /* sectioned ELL, the JDS variant: rows sorted by length, cut
                               into sections of 64 sorted rows, each an ELL padded to its
                               own longest row [REG, JDS variant].  Never picked by
                               SPMV_AUTO (the selector rule has no branch for it).         */
    SPMV_ELL_XTILE = 10,    /* ELL whose x gathers come from LDS [REG, ELL slot layout;
                               INTRO x blocking; CHOICE 4.2 staging]: rows in blocks of
                               256; a block's tile is the sorted set of the distinct
                               columns of its entries, kept as runs of consecutive
                               columns; the column array holds int16 tile positions.
                               Refused (SPMV_ERR_TOO_LARGE) unless every block spans
                               < 2^18 columns, has <= 8192 distinct ones in <= 1024 runs,
                               and R*W <= INT32_MAX.  SPMV_AUTO takes it in place of ELL
                               for R >= 16384 when every block qualifies and nnz >= 2 *
                               (sum over blocks of the tile sizes): each x word staged
                               serves two gathers or more, as on banded 3-D stencils.    */
    SPMV_COO_BLOCKED = 11   /* blocked COO [INTRO x blocking and split by nonzeros; CHOICE
                               3.2 segmented COO]: rows in blocks of SPMV_BC_BLOCK_ROWS, columns in S
                               x slices (S = opts.col_blocks in {1,2,4,8}; 0: the smallest
                               power of two that keeps a slice of x within 4 MiB, at most
                               8); the entries of each (slice, block) are ordered by
                               column, cut into chunks and work items (see
                               SPMV_BC_BLOCK_ROWS above) and groups of 64, and each
                               group is reordered by row so that runs of one row are
                               neighbouring lanes.  Neighbouring lanes therefore gather
                               neighbouring x words, and row partials are summed in LDS.
                               SPMV_AUTO takes it (with the automatic S) when the columns
                               are scattered (col_spread * 8 > C), x exceeds 4 MiB and a
                               block holds at least one entry per 128-byte line of x on
                               average (32 * nnz * min(R, SPMV_BC_BLOCK_ROWS) >= R * C). */
} spmv_format;

typedef struct spmv_opts {
    int32_t hyb_width;      /* HYB: ELL width K.  <= 0: smallest width that holds 99% of
                               rows entirely (the 99th percentile of row length).          */
    int32_t lanes_per_row;  /* CSR vector: 1,2,4,...,64.  0: smallest power of two >=
                               ceil(mean row length), clamped to [2, 64].                  */
    int32_t validate;       /* nonzero: also check every column index (one pass over
                               colIdx).  Row pointers are always checked.                  */
    int32_t jds_depth;      /* JDS: depth of one tile (jagged columns per wave).  0: 128.  */
    int32_t col_blocks;     /* x slices (column blocks), each a pass over y.
                               SPMV_COO_BLOCKED: its slice count S (0, 1, 2, 4 or 8; other
                               values are SPMV_ERR_INVALID_ARG), see above.  Otherwise:
                               0: automatic for SPMV_AUTO builds when x exceeds the 4 MiB
                               L2 of one XCD, the rows' columns are scattered and the
                               matrix is too sparse for SPMV_COO_BLOCKED's rule
                               (otherwise 1): up to 16 MiB of x, 2, 4 or 8 slices of at
                               most 2 MiB, fewer while slices x rows exceeds nnz / 3;
                               beyond 16 MiB, slices of 4 MiB.  An automatic sliced
                               build runs every slice as merge-path CSR.  When every
                               slice is merge CSR and their number divides 8, spmv_run
                               runs them in one launch, each slice on its own XCDs;
                               otherwise one launch per slice in order.  1: never
                               split.  K > 1: exactly K slices, each in the requested
                               format.                                                    */
    int32_t reserved;       /* must be 0                                                   */
    int64_t max_bytes;      /* > 0: refuse (SPMV_ERR_TOO_LARGE) a format whose device
                               arrays would exceed this many bytes.                        */
} spmv_opts;

/* Fills the defaults: every field 0 except validate = 1. */
void spmv_opts_default(spmv_opts *opts);

/* Row-length statistics [CHOICE 4.1 histogram/variance, 4.3 mean and max;
 * INTRO: max/mean of work per worker]. */
typedef struct spmv_stats {
    int64_t num_rows;
    int64_t num_cols;
    int64_t nnz;
    int64_t max_len;     /* W = longest row                         */
    int64_t sum_len_sq;  /* sum over rows of len^2 (variance = E[len^2] - mean^2) */
    int64_t empty_rows;
    int64_t col_spread;  /* mean over non-empty rows of |first column - r*C/R|: how far a
                            row's columns sit from its diagonal (small for banded matrices) */
} spmv_stats;

/* What a handle holds (spmv_get_info). */
typedef struct spmv_info {
    int32_t format;        /* built format (never SPMV_AUTO)              */
    int32_t hyb_width;     /* K used by HYB, else 0                       */
    int32_t lanes_per_row; /* lanes used by CSR vector, else 0            */
    int32_t ell_width;     /* width of the ELL arrays (ELL: W; HYB: min(K, W)) */
    int32_t col_blocks;    /* x slices the handle runs (1 = unsplit)      */
    int32_t slice_cols;    /* columns per x slice (num_cols if unsplit)   */
    spmv_stats stats;
    int64_t tail_nnz;      /* HYB: entries in the COO tail                */
    int64_t num_tiles;     /* JDS: wave tiles; CSR merge: blocks; blocked COO: chunks */
    int64_t device_bytes;  /* device memory owned by the handle           */
    int64_t groups;        /* blocked COO: groups of 64 slots             */
    int64_t wide_groups;   /* blocked COO: groups whose columns span > 65535 */
    int32_t block_rows;    /* blocked COO: SPMV_BC_BLOCK_ROWS or SPMV_BC_BLOCK_ROWS_TALL */
    int32_t chunk_entries; /* blocked COO: T, entries per chunk           */
    int32_t hot_slots;     /* blocked COO: hot rows per block (32)        */
    int32_t hot_min_len;   /* blocked COO: rows this long or longer may be hot (64*S+1) */
    int32_t work_items;    /* blocked COO: work items, one workgroup each */
} spmv_info;

/* Arrays a handle can export (spmv_export) for bit-exact comparison. */
typedef enum spmv_array {
    SPMV_A_ROW_PTRS = 0,   /* int32 [R+1]   CSR formats                       */
    SPMV_A_COL_IDX = 1,    /* int32 [nnz]   CSR and COO formats               */
    SPMV_A_VALUES = 2,     /* fp32  [nnz]   CSR and COO formats               */
    SPMV_A_ROW_IDX = 3,    /* int32 [nnz]   COO formats (sorted by row)       */
    SPMV_A_ELL_COL = 4,    /* int32 [R*w]   ELL/HYB, slot t of row r at t*R+r */
    SPMV_A_ELL_VAL = 5,    /* fp32  [R*w]                                     */
    SPMV_A_ELL_NNZ = 6,    /* int32 [R]     entries of row r in the ELL part  */
    SPMV_A_TAIL_ROW = 7,   /* int32 [tail]  HYB COO tail                      */
    SPMV_A_TAIL_COL = 8,   /* int32 [tail]                                    */
    SPMV_A_TAIL_VAL = 9,   /* fp32  [tail]                                    */
    SPMV_A_JDS_PERM = 10,  /* int32 [R]     original row of sorted row s      */
    SPMV_A_JDS_LEN = 11,   /* int32 [R]     length of sorted row s            */
    SPMV_A_JDS_ITER_PTR = 12, /* int32 [W+1] start of jagged column t         */
    SPMV_A_JDS_COL = 13,   /* int32 [nnz]   entry t of sorted row s at iterPtr[t]+s */
    SPMV_A_JDS_VAL = 14,   /* fp32  [nnz]                                     */
    SPMV_A_LEN_HIST = 15,  /* int64 [W+1]   rows of each length (every handle) */
    SPMV_A_SELL_SECT_PTR = 16, /* int32 [S+1] start of section k (S = ceil(R/64))  */
    SPMV_A_SELL_COL = 17,  /* int32 [slots] entry t of the section's row i at
                              sect_ptr[k] + t*m_k + i, m_k = rows in section k;
                              padding (0, +0.0f).  Sorted-row order and lengths
                              are SPMV_A_JDS_PERM / SPMV_A_JDS_LEN.          */
    SPMV_A_SELL_VAL = 18,  /* fp32  [slots]                                    */
    SPMV_A_XT_RUN_PTR = 19, /* int32 [B+1]  ELL x tiles: runs of block b (rows 256b ..
                              256b+255) are [run_ptr[b], run_ptr[b+1]), B = ceil(R/256) */
    SPMV_A_XT_RUNS = 20,   /* int32 [3*runs] run k: first column, offset in its block's
                              tile, length                                          */
    SPMV_A_XT_LIDX = 21,   /* int16 [R*W]   slot t of row r at t*R+r: tile position of
                              the entry's column, padding 0.  Values and row lengths:
                              SPMV_A_ELL_VAL, SPMV_A_ELL_NNZ.                       */
    /* blocked COO: segment k*B + b holds the entries of x slice k and row block b
       (B = ceil(R/SPMV_BC_BLOCK_ROWS) blocks) ordered by column, ties in CSR order;
       chunks are consecutive runs of a segment's entries and work items runs of
       chunks, by the rules at SPMV_BC_BLOCK_ROWS; groups a chunk's runs of 64.     */
    SPMV_A_BC_CHUNK_GRP = 22,  /* int32 [chunks+1] first group of chunk c          */
    SPMV_A_BC_CHUNK_BLK = 23,  /* int32 [chunks]   row block of chunk c             */
    SPMV_A_BC_SLICE_CHUNK = 24,/* int32 [S+1]      first chunk of x slice k         */
    SPMV_A_BC_HOT = 25,        /* int32 [B*32]     hot rows of block b: rows with at
                                  least hot_min_len entries, longest first, ties by
                                  row, at most 32; -1 fills                          */
    SPMV_A_BC_BASE = 26,       /* int32 [groups]   smallest column of group g, or
                                  -(w+1) if its columns span more than 65535 (wide
                                  group w)                                           */
    SPMV_A_BC_PK = 27,         /* uint32 [groups*64] slot g*64+i: code << 16 | column
                                  - base (0 in wide groups); code = row - RB*b, or
                                  RB + h for hot row h (RB = SPMV_BC_BLOCK_ROWS); the
                                  group's entries
                                  reordered by code, ties in column order; padding
                                  0xFFFF0000                                         */
    SPMV_A_BC_VAL = 28,        /* fp32 [groups*64]  values, padding +0.0f            */
    SPMV_A_BC_WIDE = 29,       /* int32 [wide*64]   columns of wide group w's slots,
                                  padding 0                                          */
    SPMV_A_BC_SLICE_ITEM = 30, /* int32 [S+1]      first work item of x slice k      */
    SPMV_A_BC_ITEM_CHUNK = 31  /* int32 [items+1]  first chunk of work item i        */
} spmv_array;

typedef struct spmv_handle spmv_handle;

/* One candidate timed by spmv_build_tuned. */
typedef struct spmv_tune_entry {
    int32_t format;      /* spmv_format tried                                          */
    int32_t col_blocks;  /* x slices of this candidate (1 = unsplit)                   */
    int32_t status;      /* SPMV_OK, or why it could not be built (e.g. TOO_LARGE)     */
    float us;            /* median time of one spmv_run, microseconds (0 if not built) */
} spmv_tune_entry;

#define SPMV_TUNE_MAX 32
typedef struct spmv_tune_report {
    int32_t count;                        /* entries filled                         */
    int32_t chosen;                       /* index of the fastest entry (-1: none)  */
    spmv_tune_entry entry[SPMV_TUNE_MAX];
} spmv_tune_report;

/*
 * spmv_analyze -- input checks and row-length statistics of a CSR matrix.
 *   Checks [COO/CSR, CSR section: rowPtrs[numRows] = nnz; SPGEMM 5.3: row_ptr
 *   monotone, column index below the column count, value count = nnz]:
 *   rowPtrs[0] = 0, rowPtrs non-decreasing, rowPtrs[R] = nnz
 *   (-> SPMV_ERR_BAD_ROWPTRS), and, if `validate`, 0 <= colIdx < C
 *   (-> SPMV_ERR_BAD_COLIDX).  Row pointers are checked first.
 *   row_ptrs_dev: int32[R+1]; col_idx_dev: int32[nnz] (may be NULL only if nnz = 0;
 *   the first column of each row is read even when `validate` is 0).
 *   stats_host: filled on success.  hist_host (nullable): int64 buffer of
 *   hist_cap entries; on success entries 0..min(hist_cap, W+1)-1 receive the
 *   number of rows of each length.
 */
spmv_status spmv_analyze(int32_t num_rows, int32_t num_cols, int32_t nnz,
                         const int32_t *row_ptrs_dev, const int32_t *col_idx_dev,
                         int32_t validate, spmv_stats *stats_host, int64_t *hist_host,
                         int64_t hist_cap, void *stream);

/*
 * spmv_select -- the format selector, a pure host function of the statistics
 * [CHOICE 4.3 rule on mean and max row length, operators restored as
 * W*R <= 2*nnz -> ELL; nnz < 10*R -> COO (segmented); W*R > 5*nnz -> HYB;
 * else CSR (vector); CHOICE 4.1 for the HYB width; CHOICE 5.2: power-law rows
 * -> merge-based CSR, taken when HYB's ELL part would exceed 1.5*nnz slots].
 *   ELL is not chosen when W*R exceeds INT32_MAX (the later rules decide), nor
 *   HYB when R*K does (merge-based CSR instead), so an automatic build never
 *   fails on the int32 slot limit.
 *   hist_host: int64[max_len+1] from spmv_analyze.  opts (nullable):
 *   hyb_width / lanes_per_row override the width and lane rules.
 *   Outputs: *format, *hyb_width (0 unless HYB), *lanes (0 unless CSR vector).
 */
spmv_status spmv_select(const spmv_stats *stats_host, const int64_t *hist_host,
                        const spmv_opts *opts, int32_t *format, int32_t *hyb_width,
                        int32_t *lanes);

/*
 * spmv_build -- build a handle in `format` from a CSR matrix on the device
 * [COO/CSR, CSR section: value/colIdx grouped by row, rowPtrs[r] = start of
 * row r, rowPtrs[numRows] = nnz; column order inside a row is free].
 *   Validates (as spmv_analyze), computes the statistics, resolves SPMV_AUTO
 *   with spmv_select, then runs the device builders:
 *     ELL  [REG, ELL: pad to the longest row with value 0 / column 0,
 *           transpose to column-major]
 *     HYB  [REG, hybrid: entries past position K of each row move to a COO
 *           list in row order; ELL of width min(K, W) for the rest]
 *     JDS  [REG, JDS: stable sort of rows by length, longest first; perm;
 *           iterPtr from the length counts; jagged column-major arrays]
 *     SELL [REG, JDS variant: the JDS sort, then sections of 64 sorted rows,
 *           each an ELL padded to its own longest row; section pointers]
 *     COO  row index expanded from rowPtrs [COO/CSR, COO section]
 *     CSR merge: per-block starting rows of the merge path
 *   Fails with SPMV_ERR_TOO_LARGE when an ELL (or HYB ELL part, or the padded
 *   SELL sections) would need more than 2^31-1 slots or when opts->max_bytes
 *   is exceeded.
 *   values_dev: fp32[nnz], moved bit for bit.  opts nullable (defaults).
 */
spmv_status spmv_build(spmv_handle **out, spmv_format format, int32_t num_rows,
                       int32_t num_cols, int32_t nnz, const int32_t *row_ptrs_dev,
                       const int32_t *col_idx_dev, const float *values_dev,
                       const spmv_opts *opts, void *stream);

/*
 * spmv_coo_to_csr -- COO -> CSR on the device [COO/CSR: COO stores one
 * (row, col, value) per nonzero; CSR groups them by row with rowPtrs].
 *   Count entries per row, exclusive scan of the counts -> rowPtrs, then a
 *   stable scatter: entries of one row keep their order in the COO input.
 *   Duplicates are kept (they add up in SpMV).  Checks row indices
 *   (SPMV_ERR_BAD_ROWIDX) and, if validate, column indices.
 *   Outputs (caller-allocated device arrays): row_ptrs_out int32[R+1],
 *   col_idx_out int32[nnz], values_out fp32[nnz].  Outputs must not alias
 *   inputs.
 */
spmv_status spmv_coo_to_csr(int32_t num_rows, int32_t num_cols, int32_t nnz,
                            const int32_t *row_idx_dev, const int32_t *col_idx_dev,
                            const float *values_dev, int32_t *row_ptrs_out_dev,
                            int32_t *col_idx_out_dev, float *values_out_dev,
                            int32_t validate, void *stream);

/*
 * spmv_build_tuned -- the empirical selector [CHOICE 4.3: a tool that times
 * the formats on the matrix itself and keeps the fastest].
 *   Tries every concrete format whose bit is set in `format_mask` (bit f for
 *   spmv_format f, 1..11; 0 = all eleven), each unsplit and -- when the matrix
 *   is one that SPMV_AUTO would cut into x slices -- also sliced (blocked COO
 *   once, with its automatic slice count).  Each
 *   candidate that builds is run once to warm up and then `runs` times
 *   (0: 5) back to back on device scratch vectors (x = 0, y = 0: the kernels
 *   do the same work for any values), each run timed with HIP events on
 *   `stream`; its median is its time.  The fastest candidate is returned in
 *   *out; all others are freed as soon as they lose.  `report` (nullable)
 *   receives one entry per candidate, including the ones that could not be
 *   built (status).  A candidate whose device arrays would exceed
 *   opts->max_bytes (0: 8x the CSR arrays, at least 64 MiB) is reported as
 *   SPMV_ERR_TOO_LARGE and not built.  Host-synchronous.  Input checks as
 *   spmv_build (once).
 *   Fails with the first candidate's error only when no candidate builds.
 */
spmv_status spmv_build_tuned(spmv_handle **out, int32_t num_rows, int32_t num_cols,
                             int32_t nnz, const int32_t *row_ptrs_dev,
                             const int32_t *col_idx_dev, const float *values_dev,
                             const spmv_opts *opts, uint32_t format_mask, int32_t runs,
                             spmv_tune_report *report, void *stream);

/* spmv_build_coo -- spmv_coo_to_csr into temporaries, then spmv_build. */
spmv_status spmv_build_coo(spmv_handle **out, spmv_format format, int32_t num_rows,
                           int32_t num_cols, int32_t nnz, const int32_t *row_idx_dev,
                           const int32_t *col_idx_dev, const float *values_dev,
                           const spmv_opts *opts, void *stream);

/*
 * spmv_run -- y <- A*x + y [COO/CSR background: SpMV computes A*X + Y].
 *   x_dev: fp32[num_cols]; y_dev: fp32[num_rows], read and written.
 *   Enqueues 1-2 kernels on `stream` (HYB: ELL part, then COO tail, in stream
 *   order).  No allocation, no synchronisation.  Rows with no nonzeros are
 *   left untouched.  Summation order is the kernel's own: results agree with
 *   the exact sum within |err| <= 1e-5 * (|y| + sum |a*x|) per row; the
 *   atomic formats (COO, HYB tail, JDS long rows, CSR merge) are not bit-
 *   reproducible from run to run.
 *   Must be called on the device the handle was built on (SPMV_ERR_DEVICE).
 */
spmv_status spmv_run(const spmv_handle *h, const float *x_dev, float *y_dev, void *stream);

/*
 * spmv_cg -- conjugate gradient for A x = b, A symmetric positive definite
 * (square), built in any format [COO/CSR, background: the iterative methods
 * SpMV serves; for positive-definite A, conjugate gradient evaluates A·X each
 * iteration and corrects X along the search direction].
 *   b_dev: fp32[R]; x_dev: fp32[R], the initial guess in, the solution out.
 *   Stops when ||b - A x|| <= rtol * ||b|| (the recurrence residual, fp64
 *   dot products, tested every 8 iterations, so up to 7 iterations may run
 *   past the first that meets it) or after max_iter iterations, never more.
 *   *iters and *rel_resid report the iterations run and ||r|| / ||b||.
 *   From max_iter >= 16 on, each batch of 8 iterations is captured once as a
 *   HIP graph and replayed (one launch per batch); setting the environment
 *   variable SPMV_CG_GRAPH=0 launches every kernel directly instead (same
 *   arithmetic, same results).  On a plain ELL handle of at most 262,144
 *   rows an iteration is two kernels (the new direction, A·p and p·Ap fused;
 *   then the update) instead of the SpMV and three vector kernels, with the
 *   same results bit for bit; SPMV_CG_FUSED=0 selects the four launches.
 *   Allocates its four work vectors (r, two p buffers, A·p) and the dot
 *   partials, runs every step on `stream`, host-synchronous.
 *   Symmetry and definiteness are the caller's promise (not checked).
 */
spmv_status spmv_cg(const spmv_handle *h, const float *b_dev, float *x_dev, int32_t max_iter,
                    float rtol, int32_t *iters, float *rel_resid, void *stream);

/*
 * spmv_cg_noalloc -- spmv_cg for callers that cannot allocate device memory
 * (code that must not call hipMalloc: work inside tight serving loops,
 * harnesses that forbid allocation).
 *   Same arguments, checks, arithmetic and results as spmv_cg, except:
 *   - the four work vectors and the dot partials live in one library-owned
 *     static device array per GPU, sized for SPMV_CG_NOALLOC_MAX_ROWS rows
 *     (about 16 MiB; reserved when the library's code is loaded on that GPU
 *     and held until the process ends).  A system with more rows is refused
 *     with SPMV_ERR_TOO_LARGE before any work;
 *   - no HIP graphs: every iteration is launched directly (SPMV_CG_GRAPH is
 *     ignored), so the results equal spmv_cg's with SPMV_CG_GRAPH=0, which
 *     are spmv_cg's own bit for bit;
 *   - it calls no hipMalloc, hipFree or other allocating routine.
 *   Every call on one GPU uses that GPU's array, which keeps the previous
 *   call's contents (each call initialises what it reads).  Calls that
 *   overlap in time on the same GPU -- from several host threads or streams
 *   -- race on the array and must be serialised by the caller.
 *   Must be called on the handle's device (SPMV_ERR_DEVICE).  Host-synchronous.
 */
#define SPMV_CG_NOALLOC_MAX_ROWS 1048576
spmv_status spmv_cg_noalloc(const spmv_handle *h, const float *b_dev, float *x_dev,
                            int32_t max_iter, float rtol, int32_t *iters, float *rel_resid,
                            void *stream);

spmv_status spmv_get_info(const spmv_handle *h, spmv_info *info_host);

/* Size in bytes of an exportable array (0 if the handle's format has none;
 * a handle split into x slices exports only SPMV_A_LEN_HIST). */
spmv_status spmv_array_bytes(const spmv_handle *h, spmv_array which, size_t *bytes);

/* Copy an array of the handle to host memory (synchronous).  `bytes` must
 * equal spmv_array_bytes(); else SPMV_ERR_INVALID_ARG. */
spmv_status spmv_export(const spmv_handle *h, spmv_array which, void *host_dst, size_t bytes);

/* Free the handle and its device memory (synchronises its device first).
 * NULL is accepted. */
spmv_status spmv_destroy(spmv_handle *h);

const char *spmv_status_string(spmv_status status);
const char *spmv_format_name(spmv_format format);

#ifdef __cplusplus
}
#endif

#endif /* SPMV_MI355X_H */
