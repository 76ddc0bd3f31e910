// Blocked COO for matrices whose columns are scattered over an x larger than
// one XCD's L2: the device builder and the SpMV kernel.
//
// Why: a random 4-byte x gather costs the memory pipeline one cache line per
// lane; when the 64 lanes of a wave instruction gather from nearby columns
// they share lines and the instruction costs far less (measured on MI355X,
// 64M gathers from a 2 MB x: random 206 G/s, two lanes per 128-byte line
// 338 G/s, eight per line 744 G/s).  Row-major formats give each lane its own
// row and hence an unrelated column.  This format orders a block of rows'
// entries by column instead, so neighbouring lanes gather neighbouring x, and
// sums the products into per-row partials held in LDS -- x blocking and
// splitting the work by nonzeros ("Introduction to sparse computing", the
// memory-efficiency and parallel-efficiency checks), with row runs summed by
// a segmented scan as in COO's segmented reduction (format-choice article,
// 3.2).
//
// Layout (every array owned by the handle; R rows, C columns):
//   - rows in blocks of RB = kBcRows, or kBcRowsTall when the kBcRows layout
//     cuts some slice into balanced work items (build_coo_blocked); columns in
//     S slices of sc = ceil(C/S); the
//     entries of (slice k, block b) form segment k*nblk + b, ordered by column
//     (ties keep CSR order); segments are cut into chunks of T entries (T =
//     bc_chunk_entries(nnz); the last of a segment the remainder, joined to
//     the chunk before it when shorter than T/2), one chunk per work item --
//     unless those chunks would leave a short last round on the slice's CUs:
//     then the slice is cut into one work item per CU of equal cost (an entry
//     1, each x line its segment touches kBcLineCost more) and each item's
//     range into chunks at segment ends; chunks into groups of 64 consecutive
//     entries;
//   - inside a group the entries are reordered by row code (stable), so equal
//     rows are neighbouring lanes; the code of an entry is its row's index
//     within the block, or RB + h for the block's hot row h (the
//     kBcHot longest rows with more than kBcHotPerSlice * S entries, longest
//     first, ties by row): hot rows get per-wave partials, so waves never
//     contend for them;
//   - bc_pk[g*64 + lane] = code << 16 | (col - base[g]); pads 0xFFFF0000;
//     bc_val the values (pads +0.0f); bc_base[g] the group's smallest column,
//     or -(w+1) when its columns span more than 65535, in which case the
//     columns are bc_wide[w*64 + lane] (pads 0);
//   - bc_chunk_grp[c] first group of chunk c, bc_chunk_blk[c] its row block,
//     bc_slice_chunk[k] the first chunk of slice k, bc_slice_item[k] its first
//     work item, bc_item_chunk[i] the first chunk of item i,
//     bc_hot[b*kBcHot + h] the hot rows of block b (-1 unused).
//
// Kernel: one workgroup per work item (slice k's items on the XCDs k*8/S ..
// (k+1)*8/S - 1, so each XCD's L2 holds one slice of x), walking the item's
// chunks one after another; a chunk's block's row partials live in LDS; each
// wave takes six consecutive groups at a time,
// gathers x, sums runs of equal codes with a DPP segmented scan (one ballot
// of neighbouring equal codes picks the steps the group's runs need, none
// when every row holds a single lane) and adds each run's total to its partial:
// hot rows by a plain add into the wave's own slot, other rows by a
// compare-and-swap loop (an LDS float atomic add costs ~190 clocks per wave
// instruction on gfx950, a CAS ~28, a plain read-modify-write ~16); finally
// every touched partial is added to y with a global atomic (chunks of the
// same rows run concurrently) and, when another chunk of the item follows,
// reset.
#include <algorithm>
#include <vector>

#include "internal.h"

namespace spmv {
namespace {

constexpr int kThreads = 256;
constexpr int kBcWaves = kBcThreads / kWave;
constexpr uint32_t kBcPadCode = 0xFFFFu;

// ------------------------------------------------------------------ builder

// Rows longer than min_len (hot candidates): appended in any order; the host
// sorts them.  At most nnz / (min_len + 1) rows qualify, the list's capacity.
__global__ __launch_bounds__(kThreads) void k_bc_hot_candidates(int32_t R,
                                                                const int32_t *__restrict__ rp,
                                                                int32_t min_len, int32_t cap,
                                                                int32_t *__restrict__ count,
                                                                int32_t *__restrict__ rows,
                                                                int32_t *__restrict__ lens) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (r >= R) return;
    const int32_t len = rp[r + 1] - rp[r];
    if (len <= min_len) return;
    const int32_t i = atomicAdd(count, 1);
    if (i < cap) {
        rows[i] = static_cast<int32_t>(r);
        lens[i] = len;
    }
}

// code[r] = r mod RB, then RB + h for hot row h of each block.
__global__ __launch_bounds__(kThreads) void k_bc_codes(int32_t R, int32_t RB,
                                                       int32_t *__restrict__ code) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (r < R) code[r] = static_cast<int32_t>(r % RB);
}

__global__ __launch_bounds__(kThreads) void k_bc_hot_codes(int64_t slots, int32_t RB,
                                                           const int32_t *__restrict__ hot,
                                                           int32_t *__restrict__ code) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (i >= slots) return;
    const int32_t r = hot[i];
    if (r >= 0) code[r] = RB + static_cast<int32_t>(i % kBcHot);
}

// Segment of each (column-sorted) entry: slice * nblk + block.
__global__ __launch_bounds__(kThreads) void k_bc_seg_keys(int32_t nnz, const int32_t *__restrict__ row,
                                                          const uint32_t *__restrict__ col,
                                                          int32_t slice_cols, int32_t nblk,
                                                          int32_t RB, uint32_t *__restrict__ key) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (i >= nnz) return;
    const uint32_t k = col[i] / static_cast<uint32_t>(slice_cols);
    key[i] = k * static_cast<uint32_t>(nblk) + static_cast<uint32_t>(row[i] / RB);
}

// 1 where an entry, in (segment, column) order, is its segment's first or
// lies in another 128-byte line of x than the entry before it: summed over a
// segment, the x lines the segment touches.
__global__ __launch_bounds__(kThreads) void k_bc_new_line(int32_t nnz,
                                                          const uint32_t *__restrict__ seg,
                                                          const int32_t *__restrict__ col,
                                                          int32_t *__restrict__ flag) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (i >= nnz) return;
    flag[i] = (i == 0 || seg[i] != seg[i - 1] || (col[i] >> 5) != (col[i - 1] >> 5)) ? 1 : 0;
}

// out[i] = src[at[i]]
__global__ __launch_bounds__(kThreads) void k_bc_take(int64_t n, const int32_t *__restrict__ at,
                                                      const int32_t *__restrict__ src,
                                                      int32_t *__restrict__ out) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (i < n) out[i] = src[at[i]];
}

// Entry range of group g: its chunk by binary search over chunk_grp.
__device__ inline void bc_group_range(int64_t g, int32_t nch, const int32_t *chunk_grp,
                                      const int32_t *chunk_e0, const int32_t *chunk_e1,
                                      int64_t &e0, int64_t &e1) {
    const int64_t c = upper_index(chunk_grp, nch, g);   // chunk_grp[c] <= g < chunk_grp[c+1]
    e0 = chunk_e0[c] + (g - chunk_grp[c]) * kWave;
    e1 = min(e0 + kWave, static_cast<int64_t>(chunk_e1[c]));
}

// wide[g] = 1 when group g's columns span more than 65535 (its first entry
// holds the smallest column, its last the largest).
__global__ __launch_bounds__(kThreads) void k_bc_wide(int64_t G, int32_t nch,
                                                      const int32_t *__restrict__ chunk_grp,
                                                      const int32_t *__restrict__ chunk_e0,
                                                      const int32_t *__restrict__ chunk_e1,
                                                      const int32_t *__restrict__ col,
                                                      int32_t *__restrict__ wide) {
    const int64_t g = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (g >= G) return;
    int64_t e0, e1;
    bc_group_range(g, nch, chunk_grp, chunk_e0, chunk_e1, e0, e1);
    wide[g] = (col[e1 - 1] - col[e0] > 65535) ? 1 : 0;
}

// One wave per group: codes, a 64-lane bitonic sort on (code, lane) -- the
// lane is the entry's position in column order, so equal codes keep column
// order -- then the packed words, values, base and wide columns.
__global__ __launch_bounds__(kThreads) void k_bc_fill(int64_t G, int32_t nch,
                                                      const int32_t *__restrict__ chunk_grp,
                                                      const int32_t *__restrict__ chunk_e0,
                                                      const int32_t *__restrict__ chunk_e1,
                                                      const int32_t *__restrict__ row,
                                                      const int32_t *__restrict__ col,
                                                      const uint32_t *__restrict__ val,
                                                      const int32_t *__restrict__ code_of_row,
                                                      const int32_t *__restrict__ wide_idx,
                                                      int32_t *__restrict__ base,
                                                      uint32_t *__restrict__ pk,
                                                      uint32_t *__restrict__ pval,
                                                      int32_t *__restrict__ wide_col) {
    const int64_t g = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / kWave;
    if (g >= G) return;   // wave-uniform
    const int lane = __lane_id();
    int64_t e0, e1;
    bc_group_range(g, nch, chunk_grp, chunk_e0, chunk_e1, e0, e1);
    const bool ok = e0 + lane < e1;
    const int32_t c = ok ? col[e0 + lane] : 0;
    const uint32_t v = ok ? val[e0 + lane] : 0u;
    const uint32_t code = ok ? static_cast<uint32_t>(code_of_row[row[e0 + lane]]) : kBcPadCode;
    uint32_t key = (code << 6) | static_cast<uint32_t>(lane);
    for (int k = 2; k <= kWave; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            const uint32_t other = static_cast<uint32_t>(__shfl_xor(static_cast<int>(key), j));
            const bool ascending = (lane & k) == 0;
            const bool lower = (lane & j) == 0;
            key = (lower == ascending) ? min(key, other) : max(key, other);
        }
    }
    const int src = static_cast<int>(key & 63u);
    const uint32_t code_s = key >> 6;
    const int32_t col_s = __shfl(c, src);
    const uint32_t val_s = static_cast<uint32_t>(__shfl(static_cast<int>(v), src));
    const int32_t first = __shfl(c, 0);
    const int32_t w0 = wide_idx[g], w1 = wide_idx[g + 1];
    const int64_t slot = g * kWave + lane;
    if (w1 > w0) {   // wide group w0: full columns on the side
        pk[slot] = code_s << 16;
        wide_col[static_cast<int64_t>(w0) * kWave + lane] = code_s == kBcPadCode ? 0 : col_s;
        if (lane == 0) base[g] = -(w0 + 1);
    } else {
        pk[slot] = (code_s << 16) | (code_s == kBcPadCode ? 0u : static_cast<uint32_t>(col_s - first));
        if (lane == 0) base[g] = first;
    }
    pval[slot] = code_s == kBcPadCode ? 0u : val_s;
}

// -------------------------------------------------------------------- SpMV

// One step of a segmented inclusive scan by row code: lane l adds the partial
// of the lane CTRL reads from when that lane holds the same row.  Keys are the
// codes plus one, so a lane outside the DPP pattern (reading 0) never matches.
template <int CTRL, int RMASK>
__device__ inline void bc_seg_step(uint32_t k, float &p) {
    const uint32_t ku = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(k), CTRL, RMASK, 0xF, true));
    const float pu = __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, p), CTRL, RMASK, 0xF, true));
    if (ku == k) p += pu;
}

__device__ inline void lds_cas_add(float *a, float v) {
    uint32_t *p = reinterpret_cast<uint32_t *>(a);
    uint32_t old = *p;
    while (!__hip_atomic_compare_exchange_strong(p, &old, __float_as_uint(__uint_as_float(old) + v),
                                                 __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_WORKGROUP)) {
    }
}

// One step of a wave: the U consecutive groups lw .. lw + U - 1 of its
// chunk (n groups).  Every load is unconditional, so the U groups' stream
// loads, then their U gathers, are all in flight at once (a gather under a
// divergent branch would be waited for before the next is issued).  In the
// chunk's last step (kTail) groups past its end, at most U - 1 of them and
// kept in bounds by the arrays' tail padding, become padding that gathers
// the slice's first column; a padding slot inside a group has offset 0 and
// gathers its group's base column.
template <int U, bool kFarX, bool kTail, int RB>
__device__ __forceinline__ void bc_wave_step(int lw, int n, int lane, const uint32_t *pkc,
                                             const float *valc, const int32_t *basec,
                                             const int32_t *wide_col, int32_t col0,
                                             const float *xs, float *part, float *mine) {
    const uint32_t off = static_cast<uint32_t>(lw * kWave + lane);
    uint32_t w[U];
    float v[U];
    int32_t bs[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        bs[u] = basec[lw + u];
        w[u] = ld_nt(pkc + off + u * kWave);
        v[u] = ld_nt(valc + off + u * kWave);
    }
    int32_t cx[U];
    bool wide = false;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (kTail && lw + u >= n) {   // past the chunk: wave-uniform
            w[u] = kBcPadCode << 16;
            bs[u] = col0;
        }
        cx[u] = (bs[u] - col0) + static_cast<int32_t>(w[u] & 0xFFFFu);
        wide |= bs[u] < 0;
    }
    if (wide) {   // wave-uniform and rare: groups spanning more than 2^16 columns
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (bs[u] < 0)   // a padding slot's column 0 becomes the slice's first
                cx[u] = max(ld_nt(wide_col + static_cast<int64_t>(-bs[u] - 1) * kWave + lane) - col0, 0);
    }
    float xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if constexpr (kFarX) {
            xv[u] = xs[cx[u]];
        } else {   // a slice of at most 2^30 columns: a 32-bit byte offset
            xv[u] = *reinterpret_cast<const float *>(reinterpret_cast<const char *>(xs) +
                                                     (static_cast<uint32_t>(cx[u]) << 2));
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float q = v[u] * xv[u];   // padding lanes' products are never read
        const uint32_t k = (w[u] >> 16) + 1;   // code + 1: a lane that DPP fills with 0 never matches
        // lane l + 1's key (wave_shl:1; lane 63 reads 0)
        const uint32_t kn = static_cast<uint32_t>(
            __builtin_amdgcn_update_dpp(0, static_cast<int>(k), 0x130, 0xF, 0xF, true));
        const bool real = k != kBcPadCode + 1;
        // bit l: lanes l and l + 1 hold the same row.  The scan runs only the
        // steps some run needs: shift s when a run spans more than s lanes
        // (m & m >> 1, ... find spans of 3, 5, 9), the broadcasts when a run
        // crosses a 16-lane DPP row
        // (padding lanes pair with each other only, and only a tail step has
        // whole groups of them: elsewhere their pairs cost nothing)
        const uint64_t m = kTail ? __builtin_amdgcn_ballot_w64(real && kn == k)
                                 : __builtin_amdgcn_ballot_w64(kn == k);
        if (m != 0) {
            bc_seg_step<0x111, 0xF>(k, q);   // row_shr:1
            const uint64_t m2 = m & (m >> 1);
            if (m2 != 0) {
                bc_seg_step<0x112, 0xF>(k, q);   // row_shr:2
                const uint64_t m4 = m2 & (m2 >> 2);
                if (m4 != 0) {
                    bc_seg_step<0x114, 0xF>(k, q);   // row_shr:4
                    if ((m4 & (m4 >> 4)) != 0) bc_seg_step<0x118, 0xF>(k, q);   // row_shr:8
                }
            }
            if ((m & 0x0000800000008000ull) != 0) bc_seg_step<0x142, 0xA>(k, q);   // row_bcast:15
            if ((m & 0x0000000080000000ull) != 0) bc_seg_step<0x143, 0xC>(k, q);   // row_bcast:31
        }
        // the last lane of each run adds the run's total to its row
        if (real && kn != k) {
            const uint32_t r = k - 1;
            if (r >= RB) mine[r - RB] += q;   // this wave's own slot
            else lds_cas_add(&part[r], q);
        }
    }
}

template <int U, bool kFarX, int RB>
__global__ __launch_bounds__(kBcThreads) void k_coo_blocked(
    int32_t R, int32_t per, int32_t slice_cols, const int32_t *__restrict__ slice_item,
    const int32_t *__restrict__ item_chunk, const int32_t *__restrict__ chunk_grp,
    const int32_t *__restrict__ chunk_blk, const int32_t *__restrict__ hot,
    const int32_t *__restrict__ base, const uint32_t *__restrict__ pk,
    const float *__restrict__ val, const int32_t *__restrict__ wide_col,
    const float *__restrict__ x, float *__restrict__ y) {
    __shared__ float part[RB];
    __shared__ float priv[kBcWaves * kBcHot];
    // slice k's work items on XCDs [k*per, (k+1)*per): block b runs on XCD b % 8
    const int xcd = static_cast<int>(blockIdx.x % kNumXcd);
    const int k = xcd / per;
    const int it = slice_item[k] + static_cast<int>(blockIdx.x / kNumXcd) * per + xcd % per;
    if (it >= slice_item[k + 1]) return;   // whole workgroup
    const int c0 = item_chunk[it], c1 = item_chunk[it + 1];
    if (c0 >= c1) return;                  // whole workgroup
    const int32_t col0 = k * slice_cols;   // a slice with a chunk starts below C
    const float *xs = x + col0;
    // -0.0 is the additive identity bit for bit: an untouched partial is
    // recognised and never added, so rows without entries keep their y bits
    for (int i = threadIdx.x; i < RB; i += kBcThreads) part[i] = -0.0f;
    for (int i = threadIdx.x; i < kBcWaves * kBcHot; i += kBcThreads) priv[i] = -0.0f;
    __syncthreads();
    const int lane = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    float *mine = priv + wave * kBcHot;
    // The item's chunks one after another, each with its block's partials
    // flushed to y before the next
    for (int c = c0; c < c1; ++c) {
        const int b = chunk_blk[c];
        const int32_t g0 = chunk_grp[c];
        const int32_t n = chunk_grp[c + 1] - g0;   // groups of this chunk
        const int64_t r0 = static_cast<int64_t>(b) * RB;
        const int nrows = static_cast<int>(min(static_cast<int64_t>(RB), R - r0));
        // the chunk's arrays through wave-uniform pointers, so every load
        // below takes a 32-bit offset (slots past 2^31 included)
        const uint32_t *pkc = pk + static_cast<int64_t>(g0) * kWave;
        const float *valc = val + static_cast<int64_t>(g0) * kWave;
        const int32_t *basec = base + g0;
        // The workgroup walks the chunk U * 16 groups at a time, wave w taking
        // the U consecutive groups lw .. lw + U - 1
        int lw = wave * U;
        for (; lw + U <= n; lw += kBcWaves * U)
            bc_wave_step<U, kFarX, false, RB>(lw, n, lane, pkc, valc, basec, wide_col, col0, xs, part,
                                          mine);
        if (lw < n)
            bc_wave_step<U, kFarX, true, RB>(lw, n, lane, pkc, valc, basec, wide_col, col0, xs, part,
                                         mine);
        __syncthreads();
        // every partial that was touched goes to y (a full block's partials
        // read 8 at a time, so one LDS wait covers 8 of them); when another
        // chunk follows, each thread resets the partials it has just read
        const bool more = c + 1 < c1;
        if (nrows == RB) {
            constexpr int P = RB / kBcThreads;   // partials per thread
#pragma unroll
            for (int j0 = 0; j0 < P; j0 += 8) {
                float s[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    s[j] = j0 + j < P ? part[threadIdx.x + (j0 + j) * kBcThreads] : -0.0f;
                if (more) {
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if (j0 + j < P) part[threadIdx.x + (j0 + j) * kBcThreads] = -0.0f;
                }
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (__float_as_uint(s[j]) != 0x80000000u)
                        unsafeAtomicAdd(&y[r0 + threadIdx.x + (j0 + j) * kBcThreads], s[j]);
            }
        } else {
            for (int i = threadIdx.x; i < nrows; i += kBcThreads) {
                const float s = part[i];
                if (more) part[i] = -0.0f;
                if (__float_as_uint(s) != 0x80000000u) unsafeAtomicAdd(&y[r0 + i], s);
            }
        }
        if (threadIdx.x < kBcHot) {
            const int32_t hr = hot[static_cast<int64_t>(b) * kBcHot + threadIdx.x];
            float w[kBcWaves];
#pragma unroll
            for (int wv = 0; wv < kBcWaves; ++wv) w[wv] = priv[wv * kBcHot + threadIdx.x];
            if (more) {
#pragma unroll
                for (int wv = 0; wv < kBcWaves; ++wv) priv[wv * kBcHot + threadIdx.x] = -0.0f;
            }
            if (hr >= 0) {
                float s = -0.0f;   // summed in wave order
#pragma unroll
                for (int wv = 0; wv < kBcWaves; ++wv) s += w[wv];
                if (__float_as_uint(s) != 0x80000000u) unsafeAtomicAdd(&y[hr], s);
            }
        }
        if (!more) break;
        __syncthreads();   // the resets land before the next chunk's updates
    }
}

template <typename T>
spmv_status owned(spmv_handle *h, T **p, int64_t count) {
    *p = nullptr;
    const size_t bytes = static_cast<size_t>(std::max<int64_t>(count, 1)) * sizeof(T);
    void *q = nullptr;
    hipError_t e = hipMalloc(&q, bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return from_hip(e);
    }
    h->owned.push_back(q);
    h->device_bytes += static_cast<int64_t>(bytes);
    *p = static_cast<T *>(q);
    return SPMV_OK;
}

}  // namespace

int32_t bc_auto_slices(int64_t num_cols) {
    // Fewer slices mean fewer chunks, and each chunk flushes its block's
    // partials to y; a slice of x up to one L2 (4 MiB) keeps the gathers
    // cheap (power-law 4M x 4M, one chunk per segment: 4 slices 221 us, 8
    // slices 251 us, 2 slices of 8 MB 267 us).
    int32_t S = 1;
    while (S < kNumXcd && 4 * num_cols > S * kBcSliceBytes) S *= 2;
    return S;
}

int64_t bc_chunk_entries(int64_t nnz) {
    // about 1.1 * nnz / 256 entries, in whole groups: the chunks, one
    // workgroup per CU, cover the 256 CUs about once, and each flushes its
    // block's partials for a full share of the work (power law 4M: 221 us
    // against 251 us in chunks of at most 131,072; two rounds' worth on the
    // skewed 2M matrix: 108 against 90 us)
    const int64_t t = (11 * nnz + 10 * kBcCus - 1) / (10 * kBcCus);
    return std::max<int64_t>((t + kWave - 1) / kWave * kWave, kBcChunkMin);
}

bool bc_auto_rule(const spmv_stats &st) {
    const int64_t R = st.num_rows, C = st.num_cols, nnz = st.nnz;
    if (nnz <= 0 || R <= 0) return false;
    const bool scattered = st.col_spread * 8 > C;
    const int64_t rows = std::min<int64_t>(R, kBcRows);
    // 32 * nnz * rows / (R * C) = expected entries of a block per 128-byte x line
    return scattered && 4 * C > kL2Bytes && 32 * nnz * rows >= R * C;
}

namespace {

// One build at block height RB; *balanced tells whether some slice took
// balanced work items.
spmv_status build_coo_blocked_at(spmv_handle *h, int32_t R, int32_t C, int32_t nnz,
                                 const int32_t *rp, const int32_t *col, const float *val,
                                 int32_t S, int32_t RB, bool *balanced_any, hipStream_t s,
                                 Scratch &scratch) {
    *balanced_any = false;
    const int64_t sc = std::max<int64_t>((static_cast<int64_t>(C) + S - 1) / S, 1);
    const int64_t nblk = (static_cast<int64_t>(R) + RB - 1) / RB;
    const int64_t nseg = S * nblk;
    h->col_blocks = S;
    h->slice_cols = static_cast<int32_t>(sc);
    h->bc_rows = RB;
    h->bc_blocks = nblk;
    h->bc_hot_min_len = kBcHotPerSlice * S + 1;
    h->bc_chunk = bc_chunk_entries(nnz);
    if (nnz == 0 || R == 0) return SPMV_OK;
    if (nseg > 2147483647LL) return SPMV_ERR_TOO_LARGE;

    // 1. hot rows of each block: rows longer than kBcHotPerSlice * S, longest
    //    first (ties by row), at most kBcHot per block
    const int32_t min_len = kBcHotPerSlice * S;
    const int32_t cap = nnz / (min_len + 1) + 1;
    int32_t *cand = nullptr;
    SPMV_TRY(scratch.alloc(&cand, 2 * static_cast<size_t>(cap) + 1));
    SPMV_HIP(hipMemsetAsync(cand, 0, sizeof(int32_t), s));
    SPMV_HIP(hipGetLastError());
    k_bc_hot_candidates<<<grid_for(R, kThreads), kThreads, 0, s>>>(R, rp, min_len, cap, cand,
                                                                   cand + 1, cand + 1 + cap);
    SPMV_HIP(hipGetLastError());
    int32_t ncand = 0;
    SPMV_HIP(hipMemcpyAsync(&ncand, cand, sizeof(int32_t), hipMemcpyDeviceToHost, s));
    SPMV_HIP(hipStreamSynchronize(s));
    ncand = std::min(ncand, cap);
    std::vector<int32_t> crow(static_cast<size_t>(ncand)), clen(static_cast<size_t>(ncand));
    if (ncand > 0) {
        SPMV_HIP(hipMemcpyAsync(crow.data(), cand + 1, sizeof(int32_t) * ncand,
                                hipMemcpyDeviceToHost, s));
        SPMV_HIP(hipMemcpyAsync(clen.data(), cand + 1 + cap, sizeof(int32_t) * ncand,
                                hipMemcpyDeviceToHost, s));
        SPMV_HIP(hipStreamSynchronize(s));
    }
    std::vector<int32_t> order(static_cast<size_t>(ncand));
    for (int32_t i = 0; i < ncand; ++i) order[i] = i;
    std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
        const int32_t ba = crow[a] / RB, bb = crow[b] / RB;
        if (ba != bb) return ba < bb;
        if (clen[a] != clen[b]) return clen[a] > clen[b];
        return crow[a] < crow[b];
    });
    std::vector<int32_t> hot(static_cast<size_t>(nblk * kBcHot), -1);
    for (int32_t i = 0, prev = -1, h_in = 0; i < ncand; ++i) {
        const int32_t r = crow[order[i]], b = r / RB;
        h_in = (b == prev) ? h_in + 1 : 0;
        prev = b;
        if (h_in < kBcHot) hot[static_cast<size_t>(b) * kBcHot + h_in] = r;
    }
    SPMV_TRY(owned(h, &h->a.bc_hot, nblk * kBcHot));
    SPMV_HIP(hipMemcpyAsync(h->a.bc_hot, hot.data(), sizeof(int32_t) * hot.size(),
                            hipMemcpyHostToDevice, s));
    int32_t *code = nullptr;
    SPMV_TRY(scratch.alloc(&code, static_cast<size_t>(R)));
    k_bc_codes<<<grid_for(R, kThreads), kThreads, 0, s>>>(R, RB, code);
    SPMV_HIP(hipGetLastError());
    k_bc_hot_codes<<<grid_for(nblk * kBcHot, kThreads), kThreads, 0, s>>>(nblk * kBcHot, RB,
                                                                         h->a.bc_hot, code);
    SPMV_HIP(hipGetLastError());

    // 2. entries ordered by (segment, column), ties in CSR order: a stable
    //    sort by column, then a stable sort by segment
    const size_t nw = (static_cast<size_t>(nnz) + 63) & ~size_t{63};
    uint32_t *arr = nullptr;
    SPMV_TRY(scratch.alloc(&arr, 8 * nw));
    int32_t *row0 = reinterpret_cast<int32_t *>(arr);
    uint32_t *col1 = arr + nw;
    int32_t *row1 = reinterpret_cast<int32_t *>(arr + 2 * nw);
    uint32_t *val1 = arr + 3 * nw;
    uint32_t *seg = arr + 4 * nw;
    int32_t *row2 = reinterpret_cast<int32_t *>(arr + 5 * nw);
    int32_t *col2 = reinterpret_cast<int32_t *>(arr + 6 * nw);
    uint32_t *val2 = arr + 7 * nw;
    SPMV_HIP(launch_expand_rows(R, nnz, rp, row0, s));
    {
        const uint32_t *pin[2] = {reinterpret_cast<const uint32_t *>(row0),
                                  reinterpret_cast<const uint32_t *>(val)};
        uint32_t *pout[2] = {reinterpret_cast<uint32_t *>(row1), val1};
        SPMV_TRY(radix_sort(reinterpret_cast<const uint32_t *>(col), col1, 2, pin, pout, nnz,
                            bits_for(static_cast<uint64_t>(C > 0 ? C - 1 : 0)), s, scratch));
    }
    k_bc_seg_keys<<<grid_for(nnz, kThreads), kThreads, 0, s>>>(
        nnz, row1, col1, static_cast<int32_t>(sc), static_cast<int32_t>(nblk), RB, seg);
    SPMV_HIP(hipGetLastError());
    const uint32_t *seg_sorted = nullptr;
    {
        const uint32_t *pin[3] = {reinterpret_cast<const uint32_t *>(row1), val1, col1};
        uint32_t *pout[3] = {reinterpret_cast<uint32_t *>(row2), val2,
                             reinterpret_cast<uint32_t *>(col2)};
        SPMV_TRY(radix_sort(seg, nullptr, 3, pin, pout, nnz,
                            bits_for(static_cast<uint64_t>(nseg - 1)), s, scratch, &seg_sorted));
    }
    int32_t *bounds = nullptr;
    SPMV_TRY(scratch.alloc(&bounds, static_cast<size_t>(nseg) + 1));
    SPMV_HIP(launch_slice_bounds(nnz, static_cast<int32_t>(nseg), seg_sorted, bounds, s));
    std::vector<int32_t> hb(static_cast<size_t>(nseg) + 1);
    SPMV_HIP(hipMemcpyAsync(hb.data(), bounds, sizeof(int32_t) * hb.size(), hipMemcpyDeviceToHost,
                            s));
    SPMV_HIP(hipStreamSynchronize(s));

    // x lines touched per segment: new-line flags, their exclusive sum, read
    // at the segment bounds
    std::vector<int32_t> hl(static_cast<size_t>(nseg) + 1);
    {
        int32_t *flag = nullptr, *at = nullptr;
        SPMV_TRY(scratch.alloc(&flag, static_cast<size_t>(nnz) + 1));
        SPMV_TRY(scratch.alloc(&at, static_cast<size_t>(nseg) + 1));
        k_bc_new_line<<<grid_for(nnz, kThreads), kThreads, 0, s>>>(nnz, seg_sorted, col2, flag);
        SPMV_HIP(hipGetLastError());
        SPMV_TRY(exclusive_scan(flag, flag, nnz, true, s, scratch));
        k_bc_take<<<grid_for(nseg + 1, kThreads), kThreads, 0, s>>>(nseg + 1, bounds, flag, at);
        SPMV_HIP(hipGetLastError());
        SPMV_HIP(hipMemcpyAsync(hl.data(), at, sizeof(int32_t) * hl.size(),
                                hipMemcpyDeviceToHost, s));
        SPMV_HIP(hipStreamSynchronize(s));
    }

    // 3. chunks and work items, slice by slice.  By chunk: chunks of T
    //    entries per segment, the last one the remainder, which joins the
    //    chunk before it when shorter than T/2 (a sliver chunk would flush a
    //    whole block's partials for a sliver of work: on 3.6M x 2M, 15 per
    //    row, 2 slices, 444 chunks 232 us against 222 chunks 146 us), one
    //    chunk per work item.  When those chunks, dealt in order each to the
    //    least loaded of the slice's P CUs, would load one CU with more than
    //    9/8 of an even share (a last round of a few chunks: 2 x 65 blocks of
    //    32,768 rows, 15 per row, 149 us against 93 for 2 x 64), the slice is
    //    cut instead into P work items of equal cost, each an entry plus
    //    kBcLineCost per x line of its segment (2 x 65 blocks: 100 us; a
    //    partial last block, whose few rows share fewer x lines, costs more
    //    per entry: 118 against 135 us with items of equal entries); groups
    //    of 64 per chunk
    const int64_t T = h->bc_chunk;
    const int32_t per = kNumXcd / S;
    const int64_t P = kBcCus / S;
    std::vector<int32_t> cgrp{0}, cblk, ce0, ce1, schunk(static_cast<size_t>(S) + 1, 0),
        sitem(static_cast<size_t>(S) + 1, 0), ichunk;
    std::vector<int64_t> dyn, load, cut(static_cast<size_t>(P) + 1);
    int64_t groups = 0;
    auto add_chunk = [&](int64_t sg, int64_t e, int64_t e1) {
        groups += (e1 - e + kWave - 1) / kWave;
        cgrp.push_back(static_cast<int32_t>(groups));
        cblk.push_back(static_cast<int32_t>(sg % nblk));
        ce0.push_back(static_cast<int32_t>(e));
        ce1.push_back(static_cast<int32_t>(e1));
    };
    // cost of one entry of segment sg, in 1/1024
    auto rate = [&](int64_t sg) -> int64_t {
        const int64_t n = hb[sg + 1] - hb[sg];
        return n > 0 ? (n + kBcLineCost * (hl[sg + 1] - hl[sg])) * 1024 / n : 0;
    };
    for (int32_t k = 0; k < S; ++k) {
        const int64_t sg0 = static_cast<int64_t>(k) * nblk, sg1 = sg0 + nblk;
        const int64_t s0 = hb[sg0], s1 = hb[sg1];
        schunk[k] = static_cast<int32_t>(cblk.size());
        sitem[k] = static_cast<int32_t>(ichunk.size());
        dyn.clear();
        int64_t total = 0;
        for (int64_t sg = sg0; sg < sg1; ++sg) {
            total += (hb[sg + 1] - hb[sg]) * rate(sg);
            for (int64_t e = hb[sg], e1 = 0; e < hb[sg + 1]; e = e1) {
                e1 = std::min<int64_t>(e + T, hb[sg + 1]);
                if (hb[sg + 1] - e1 < T / 2) e1 = hb[sg + 1];   // a short last piece joins this chunk
                dyn.insert(dyn.end(), {sg, e, e1});
            }
        }
        bool balanced = false;
        if (s1 - s0 >= P * std::max<int64_t>(RB / 4, kWave)) {
            load.assign(static_cast<size_t>(P), 0);
            int64_t most = 0;
            for (size_t i = 0; i < dyn.size(); i += 3) {
                auto least = std::min_element(load.begin(), load.end());
                *least += (dyn[i + 2] - dyn[i + 1]) * rate(dyn[i]);
                most = std::max(most, *least);
            }
            balanced = kBcSkewDen * most * P > kBcSkewNum * total;
        }
        *balanced_any = *balanced_any || balanced;
        if (!balanced) {
            for (size_t i = 0; i < dyn.size(); i += 3) {
                ichunk.push_back(static_cast<int32_t>(cblk.size()));
                add_chunk(dyn[i], dyn[i + 1], dyn[i + 2]);
            }
        } else {
            // item w ends at the first position whose preceding entries of
            // the slice cost at least total * (w + 1) / P
            cut[0] = s0;
            cut[static_cast<size_t>(P)] = s1;
            for (int64_t w = 1, sg = sg0, acc = 0; w < P; ++w) {
                const int64_t t = total * w / P;
                while (acc + (hb[sg + 1] - hb[sg]) * rate(sg) < t) {
                    acc += (hb[sg + 1] - hb[sg]) * rate(sg);
                    ++sg;
                }
                const int64_t r = rate(sg);
                cut[static_cast<size_t>(w)] = hb[sg] + (r > 0 ? (t - acc + r - 1) / r : 0);
            }
            for (int64_t w = 0, sg = sg0; w < P; ++w) {
                ichunk.push_back(static_cast<int32_t>(cblk.size()));
                for (int64_t e = cut[static_cast<size_t>(w)]; e < cut[static_cast<size_t>(w) + 1];) {
                    while (hb[sg + 1] <= e) ++sg;
                    const int64_t e1 = std::min<int64_t>(cut[static_cast<size_t>(w) + 1], hb[sg + 1]);
                    add_chunk(sg, e, e1);
                    e = e1;
                }
            }
        }
        if (groups * kWave > (int64_t{1} << 40)) return SPMV_ERR_TOO_LARGE;
    }
    schunk[static_cast<size_t>(S)] = static_cast<int32_t>(cblk.size());
    sitem[static_cast<size_t>(S)] = static_cast<int32_t>(ichunk.size());
    ichunk.push_back(static_cast<int32_t>(cblk.size()));
    const int32_t nch = static_cast<int32_t>(cblk.size());
    int32_t most_items = 0;
    for (int32_t k = 0; k < S; ++k) most_items = std::max(most_items, sitem[k + 1] - sitem[k]);
    h->bc_grid = static_cast<int64_t>(kNumXcd) * ((most_items + per - 1) / per);
    h->bc_items = sitem[static_cast<size_t>(S)];
    h->num_tiles = nch;
    h->bc_groups = groups;
    SPMV_TRY(owned(h, &h->a.bc_chunk_grp, nch + 1));
    SPMV_TRY(owned(h, &h->a.bc_chunk_blk, nch));
    SPMV_TRY(owned(h, &h->a.bc_slice_chunk, S + 1));
    SPMV_HIP(hipMemcpyAsync(h->a.bc_chunk_grp, cgrp.data(), sizeof(int32_t) * cgrp.size(),
                            hipMemcpyHostToDevice, s));
    SPMV_HIP(hipMemcpyAsync(h->a.bc_chunk_blk, cblk.data(), sizeof(int32_t) * cblk.size(),
                            hipMemcpyHostToDevice, s));
    SPMV_HIP(hipMemcpyAsync(h->a.bc_slice_chunk, schunk.data(), sizeof(int32_t) * schunk.size(),
                            hipMemcpyHostToDevice, s));
    SPMV_TRY(owned(h, &h->a.bc_slice_item, S + 1));
    SPMV_TRY(owned(h, &h->a.bc_item_chunk, static_cast<int64_t>(ichunk.size())));
    SPMV_HIP(hipMemcpyAsync(h->a.bc_slice_item, sitem.data(), sizeof(int32_t) * sitem.size(),
                            hipMemcpyHostToDevice, s));
    SPMV_HIP(hipMemcpyAsync(h->a.bc_item_chunk, ichunk.data(), sizeof(int32_t) * ichunk.size(),
                            hipMemcpyHostToDevice, s));
    int32_t *e01 = nullptr;
    SPMV_TRY(scratch.alloc(&e01, 2 * static_cast<size_t>(nch)));
    SPMV_HIP(hipMemcpyAsync(e01, ce0.data(), sizeof(int32_t) * nch, hipMemcpyHostToDevice, s));
    SPMV_HIP(hipMemcpyAsync(e01 + nch, ce1.data(), sizeof(int32_t) * nch, hipMemcpyHostToDevice,
                            s));

    // 4. wide groups (columns spanning more than 16 bits) and their numbering
    int32_t *widx = nullptr;
    SPMV_TRY(scratch.alloc(&widx, static_cast<size_t>(groups) + 1));
    k_bc_wide<<<grid_for(groups, kThreads), kThreads, 0, s>>>(groups, nch, h->a.bc_chunk_grp, e01,
                                                              e01 + nch, col2, widx);
    SPMV_HIP(hipGetLastError());
    SPMV_TRY(exclusive_scan(widx, widx, groups, true, s, scratch));
    int32_t nwide = 0;
    SPMV_HIP(hipMemcpyAsync(&nwide, widx + groups, sizeof(int32_t), hipMemcpyDeviceToHost, s));
    SPMV_HIP(hipStreamSynchronize(s));
    h->bc_wide_groups = nwide;

    // 5. the groups themselves
    // kBcUnroll - 1 groups of tail padding: a wave's last step may read that
    // far past the final chunk (the kernel marks those groups as padding)
    const int64_t padded = groups + kBcUnroll - 1;
    SPMV_TRY(owned(h, &h->a.bc_base, padded));
    SPMV_TRY(owned(h, &h->a.bc_pk, padded * kWave));
    SPMV_TRY(owned(h, &h->a.bc_val, padded * kWave));
    SPMV_HIP(hipMemsetAsync(h->a.bc_base + groups, 0, sizeof(int32_t) * (kBcUnroll - 1), s));
    SPMV_HIP(hipMemsetAsync(h->a.bc_pk + groups * kWave, 0,
                            sizeof(uint32_t) * kWave * (kBcUnroll - 1), s));
    SPMV_HIP(hipMemsetAsync(h->a.bc_val + groups * kWave, 0,
                            sizeof(float) * kWave * (kBcUnroll - 1), s));
    SPMV_TRY(owned(h, &h->a.bc_wide, static_cast<int64_t>(nwide) * kWave));
    k_bc_fill<<<grid_for(groups * kWave, kThreads), kThreads, 0, s>>>(
        groups, nch, h->a.bc_chunk_grp, e01, e01 + nch, row2, col2, val2, code, widx,
        h->a.bc_base, h->a.bc_pk, reinterpret_cast<uint32_t *>(h->a.bc_val), h->a.bc_wide);
    SPMV_HIP(hipGetLastError());
    SPMV_HIP(hipStreamSynchronize(s));
    return SPMV_OK;
}

}  // namespace

spmv_status build_coo_blocked(spmv_handle *h, int32_t R, int32_t C, int32_t nnz,
                              const int32_t *rp, const int32_t *col, const float *val, int32_t S,
                              hipStream_t s, Scratch &scratch) {
    // Blocks of kBcRows rows; when that cuts some slice into balanced work
    // items (the chunks would not fill the CUs in whole rounds), the chunk
    // rounds no longer matter and the build is redone with kBcRowsTall-row
    // blocks, the tallest whose partials still fit the LDS: more of a
    // segment's entries then share each x line
    const size_t mark = h->owned.size();
    const int64_t bytes = h->device_bytes;
    const DevArrays arrays = h->a;
    bool balanced = false;
    SPMV_TRY(build_coo_blocked_at(h, R, C, nnz, rp, col, val, S, kBcRows, &balanced, s, scratch));
    if (!balanced) return SPMV_OK;
    SPMV_HIP(hipStreamSynchronize(s));
    for (size_t i = mark; i < h->owned.size(); ++i) SPMV_HIP(hipFree(h->owned[i]));
    h->owned.resize(mark);
    h->device_bytes = bytes;
    h->a = arrays;
    return build_coo_blocked_at(h, R, C, nnz, rp, col, val, S, kBcRowsTall, &balanced, s, scratch);
}

hipError_t launch_coo_blocked(const spmv_handle *h, const float *x, float *y, hipStream_t s) {
    if (h->bc_grid <= 0) return hipSuccess;
    const int32_t R = static_cast<int32_t>(h->stats.num_rows);
    const int32_t per = kNumXcd / h->col_blocks;
    const DevArrays &a = h->a;
    const dim3 grid(static_cast<unsigned>(h->bc_grid));
    const bool far = h->slice_cols > (1 << 30);
    const bool tall = h->bc_rows == kBcRowsTall;
#define SPMV_BC_LAUNCH(FAR, RB)                                                                   \
    k_coo_blocked<kBcUnroll, FAR, RB><<<grid, kBcThreads, 0, s>>>(                                \
        R, per, h->slice_cols, a.bc_slice_item, a.bc_item_chunk, a.bc_chunk_grp, a.bc_chunk_blk,  \
        a.bc_hot, a.bc_base, a.bc_pk, a.bc_val, a.bc_wide, x, y)
    if (far && tall)
        SPMV_BC_LAUNCH(true, kBcRowsTall);
    else if (far)
        SPMV_BC_LAUNCH(true, kBcRows);
    else if (tall)
        SPMV_BC_LAUNCH(false, kBcRowsTall);
    else
        SPMV_BC_LAUNCH(false, kBcRows);
#undef SPMV_BC_LAUNCH
    return hipGetLastError();
}

}  // namespace spmv
