// CSR transpose on the device: the CSR of A^T (k x m) from the CSR of A
// (m x k), which the backward pass of a sparse layer needs for the input
// gradient dB = A^T dC ("Sparse GPU Kernels for Deep Learning", summary card,
// "Summary": the kernels serve training, and its gradients take the
// transposed operand).
//
// Method.  A^T in CSR is A's entries ordered by (column, row).  A's arrays
// already list them by (row, column), so a stable sort of the entry indices
// by column gives the order: a least-significant-digit radix sort of the
// column indices, 8 bits per pass, ceil(log2(k) / 8) passes, carrying each
// entry's index.  Every pass has three launches:
//   upsweep   -- each 4096-entry tile counts its digits (LDS counters);
//   scan      -- one workgroup per digit turns its per-tile counts into
//                exclusive offsets within the digit and the digit's total;
//   downsweep -- each tile ranks its entries within the tile, stably, with
//                wave ballots (the lanes that share a digit, and how many of
//                them come before), and scatters them to
//                digit base + tile offset + rank.
// No atomic operation decides any position, so the result is the same on
// every run.  Then the row offsets of A^T come from the sorted columns (the
// first position of each column), and a last pass writes each transposed
// entry's row (the source entry's row, from an expanded row-id array), value
// and source index.
//
// Counting method, for k <= kCountMaxK and nnz <= kCountMaxNnz (four
// launches instead of three per radix pass plus three; FFN-sized problems).  The rows are cut into
// ranges of S consecutive rows, and:
//   rank    -- one wave per range walks its rows in order.  A row's entries
//              have distinct columns, so each lane reads its column's running
//              count (LDS) as the entry's rank among the range's entries of
//              that column and advances it; the entry's row is recorded too.
//              The range's per-column counts go to tbl[c * R + r].
//   columns -- one wave per column: tbl[c * R + r] becomes the column's count
//              over the ranges before r, and tot[c] its total.
//   offsets -- one workgroup: t_row_offsets is the exclusive scan of tot.
//   scatter -- entry p of column c in range r goes to position
//              t_row_offsets[c] + tbl[c * R + r] + rank[p].
// Within a column, ranges come in order and rows in order within a range, so
// the positions are exactly the stable order of the radix method; no count
// depends on the order of concurrent updates (LDS counters of one wave,
// updated by distinct lanes for distinct columns).
#include <algorithm>

#include "sp_device.h"
#include "sp_launch.h"
#include "sp_scan.h"

namespace spk {

namespace {

constexpr int kSortThreads = 256;
constexpr int kSortWaves = kSortThreads / kWave;
constexpr int kItems = 16;                              // entries per thread
constexpr int kTile = kSortThreads * kItems;            // entries per tile
constexpr int kDigits = 256;                            // 8-bit digits
constexpr int kDigitScanThreads = 1024;
static_assert(kSortThreads == kDigits, "one thread per digit in the bases");

// Entry `j` of thread (wave w, lane l) in tile b is entry
// b * kTile + w * (kItems * kWave) + j * kWave + l: a wave's entries in
// (j, lane) order, waves in order, tiles in order -- the original order.
__device__ __forceinline__ long long item_index(int tile, int wave, int j, int lane)
{
    return (long long)tile * kTile + wave * (kItems * kWave) + j * kWave + lane;
}

// rowid[p] = the row of entry p (one wave per row).
__global__ __launch_bounds__(kWave) void expand_rows_kernel(const int *__restrict__ row_offsets,
                                                            int *__restrict__ rowid)
{
    const int row = blockIdx.x;
    const int p1 = row_offsets[row + 1];
    for (int p = row_offsets[row] + (int)threadIdx.x; p < p1; p += kWave) rowid[p] = row;
}

// key[p] = (row << row_shift) | col_indices[p] for the entries p of each row
// (one wave per row): the row rides in the key's bits above the sorted ones.
__global__ __launch_bounds__(kWave) void pack_keys_kernel(const int *__restrict__ row_offsets,
                                                          const int *__restrict__ col_indices,
                                                          int row_shift, int *__restrict__ key)
{
    const int row = blockIdx.x;
    const int p1 = row_offsets[row + 1];
    const int hi = row << row_shift;
    for (int p = row_offsets[row] + (int)threadIdx.x; p < p1; p += kWave)
        key[p] = hi | col_indices[p];
}

// hist[d * (tiles + 1) + b + 1] = number of entries of tile b whose digit is d.
__global__ __launch_bounds__(kSortThreads) void radix_upsweep_kernel(
    int nnz, int shift, const int *__restrict__ keys, int *__restrict__ hist, int tiles)
{
    __shared__ int s_count[kDigits];
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int b = blockIdx.x;
    s_count[tid] = 0;
    __syncthreads();
    int key[kItems];
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        const long long idx = item_index(b, wave, j, lane);
        key[j] = idx < nnz ? keys[idx] : -1;
    }
#pragma unroll
    for (int j = 0; j < kItems; ++j)
        if (key[j] >= 0) atomicAdd(&s_count[(key[j] >> shift) & (kDigits - 1)], 1);
    __syncthreads();
    hist[(size_t)tid * (tiles + 1) + b + 1] = s_count[tid];
}

// Per digit d: hist[d][b] = sum of tile counts of digit d before tile b, and
// hist[d][tiles] = the digit's total (in place; counts sit at b + 1).
__global__ __launch_bounds__(kDigitScanThreads) void digit_scan_kernel(int tiles, int *hist)
{
    int *row = hist + (size_t)blockIdx.x * (tiles + 1);
    exclusive_scan_block<kDigitScanThreads>(tiles, row + 1, row);
}

// Scatter tile b's entries to their sorted positions.  vals_in == NULL means
// the identity (entry index) as the carried value.
__global__ __launch_bounds__(kSortThreads) void radix_downsweep_kernel(
    int nnz, int shift, const int *__restrict__ keys_in, const int *__restrict__ vals_in,
    int *__restrict__ keys_out, int *__restrict__ vals_out, const int *__restrict__ hist,
    int tiles)
{
    __shared__ int s_wave_count[kSortWaves][kDigits];
    __shared__ int s_base[kDigits];
    __shared__ int s_wave_sum[kSortWaves];
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int b = blockIdx.x;

#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) s_wave_count[w][tid] = 0;
    // Digit bases: exclusive scan of the digit totals (thread d holds digit
    // d), plus this tile's offset within the digit.
    const int total = hist[(size_t)tid * (tiles + 1) + tiles];
    const int incl = wave_inclusive_sum(total);
    if (lane == kWave - 1) s_wave_sum[wave] = incl;

    int key[kItems], val[kItems], rank[kItems];
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        const long long idx = item_index(b, wave, j, lane);
        const bool ok = idx < nnz;
        key[j] = ok ? keys_in[idx] : -1;
        val[j] = vals_in ? (ok ? vals_in[idx] : 0) : (int)idx;
    }
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) before += w < wave ? s_wave_sum[w] : 0;
    s_base[tid] = before + incl - total + hist[(size_t)tid * (tiles + 1) + b];

    // Rank within the wave, round by round in (j, lane) order.  In a round,
    // the lanes sharing a digit read the wave's running count for it, take
    // their place among themselves, and the lowest of them advances the
    // count.  A wave's LDS operations complete in program order, so every
    // read of a round precedes that round's update.
    const uint64_t below = lanes_below(lane);
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        const bool ok = key[j] >= 0;
        const int d = ok ? (key[j] >> shift) & (kDigits - 1) : 0;
        uint64_t peers = __ballot(ok);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const uint64_t ones = __ballot((d >> bit) & 1);
            peers &= ((d >> bit) & 1) ? ones : ~ones;
        }
        const int ahead = __popcll(peers & below);
        const int old = s_wave_count[wave][d];
        if (ok && ahead == 0) s_wave_count[wave][d] = old + __popcll(peers);
        rank[j] = old + ahead;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        if (key[j] < 0) continue;
        const int d = (key[j] >> shift) & (kDigits - 1);
        int pos = s_base[d] + rank[j];
#pragma unroll
        for (int w = 0; w < kSortWaves; ++w) pos += w < wave ? s_wave_count[w][d] : 0;
        keys_out[pos] = key[j];
        vals_out[pos] = val[j];
    }
}

// t_row_offsets[c] = first position of column c in the sorted columns (nnz
// past the last): position q writes every column in (keys[q-1], keys[q]].
__global__ __launch_bounds__(256) void offsets_from_sorted_kernel(int nnz, int k,
                                                                  const int *__restrict__ keys,
                                                                  int *__restrict__ t_row_offsets)
{
    const long long q = (long long)blockIdx.x * 256 + threadIdx.x;
    if (q > nnz) return;
    const long long prev = q > 0 ? keys[q - 1] : -1;
    const long long cur = q < nnz ? min(keys[q], k) : k;  // (min: as in the packed form)
    for (long long c = prev + 1; c <= cur; ++c) t_row_offsets[c] = (int)q;
}

// Entry q of A^T: source entry p = perm[q] (q itself when perm == NULL).
__global__ __launch_bounds__(256) void transpose_finish_kernel(
    int nnz, const int *__restrict__ perm, const int *__restrict__ rowid,
    const float *__restrict__ values, int *__restrict__ t_col_indices,
    float *__restrict__ t_values, int *__restrict__ t_perm)
{
    const long long q = (long long)blockIdx.x * 256 + threadIdx.x;
    if (q >= nnz) return;
    const int p = perm ? perm[q] : (int)q;
    t_col_indices[q] = rowid[p];
    if (t_values) t_values[q] = values[p];
    if (t_perm) t_perm[q] = p;
}

// Entry q of A^T from packed keys sorted by column (column in the bits below
// row_shift, row above): its row of A and, through perm, its value and source
// entry; position q also writes t_row_offsets[c] for every column c in
// (column of q - 1, column of q] (through k at q = nnz), as
// offsets_from_sorted_kernel does.
__global__ __launch_bounds__(256) void transpose_finish_packed_kernel(
    int nnz, int k, int row_shift, const int *__restrict__ keys, const int *__restrict__ perm,
    const float *__restrict__ values, int *__restrict__ t_row_offsets,
    int *__restrict__ t_col_indices, float *__restrict__ t_values, int *__restrict__ t_perm)
{
    const long long q = (long long)blockIdx.x * 256 + threadIdx.x;
    if (q > nnz) return;
    const int mask = (1 << row_shift) - 1;
    // (min: a column index outside [0, k), which valid input never holds,
    // still writes no offset past t_row_offsets[k])
    const long long prev = q > 0 ? (keys[q - 1] & mask) : -1;
    const long long cur = q < nnz ? min(keys[q] & mask, k) : k;
    for (long long c = prev + 1; c <= cur; ++c) t_row_offsets[c] = (int)q;
    if (q == nnz) return;
    const int p = perm[q];
    t_col_indices[q] = keys[q] >> row_shift;
    if (t_values) t_values[q] = values[p];
    if (t_perm) t_perm[q] = p;
}

__global__ __launch_bounds__(256) void gather_values_kernel(int nnz, const int *__restrict__ perm,
                                                            const float *__restrict__ in,
                                                            float *__restrict__ out)
{
    const long long q = (long long)blockIdx.x * 256 + threadIdx.x;
    if (q < nnz) out[q] = in[perm[q]];
}

// ---- counting method
constexpr int kCountMaxK = 16384;     // LDS counters of the rank kernel: 64 KiB
constexpr int kCountMaxNnz = 1 << 18;
constexpr long long kCountMaxTable = 1 << 18;  // R * k: the table is written column-major
                                               // by range-major producers (scattered)
constexpr int kRangeEntries = 1024;   // aim: entries per range
constexpr int kRowsCap = 1024;        // rows per range at most (offsets staged in LDS)
constexpr int kPiece = 2048;          // column indices staged in LDS at a time

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(kWave) void count_rank_kernel(
    int m, int k, int rows_per_range, int ranges, const int *__restrict__ row_offsets,
    const int *__restrict__ col_indices, int *__restrict__ rank, int *__restrict__ rowid,
    int *__restrict__ tbl)
{
    extern __shared__ int s_cnt[];  // k counters
    __shared__ int s_ro[kRowsCap + 1];
    __shared__ int s_col[kPiece];
    const int r = blockIdx.x;
    const int lane = threadIdx.x;
    const int r0 = r * rows_per_range;
    const int nrows = min(m - r0, rows_per_range);
    for (int c = lane; c < k; c += kWave) s_cnt[c] = 0;
    for (int t = lane; t <= nrows; t += kWave) s_ro[t] = row_offsets[r0 + t];
    wave_lds_sync();
    const int e0 = __builtin_amdgcn_readfirstlane(s_ro[0]);
    const int e1 = __builtin_amdgcn_readfirstlane(s_ro[nrows]);
    int t = 0;  // the first row not finished
    for (int e = e0; e < e1; e += kPiece) {
        const int e_end = min(e1, e + kPiece);
        for (int i = lane; i < e_end - e; i += kWave) s_col[i] = col_indices[e + i];
        wave_lds_sync();
        while (t < nrows) {
            const int rs = __builtin_amdgcn_readfirstlane(s_ro[t]);
            const int re = __builtin_amdgcn_readfirstlane(s_ro[t + 1]);
            if (re <= e) {  // ended before this piece (or empty)
                ++t;
                continue;
            }
            if (rs >= e_end) break;
            const int hi = min(re, e_end);
            for (int base = max(rs, e); base < hi; base += kWave) {
                const int q = base + lane;
                if (q < hi) {
                    const int c = s_col[q - e];
                    const int old = s_cnt[c];
                    s_cnt[c] = old + 1;
                    rank[q] = old;
                    rowid[q] = r0 + t;
                }
                // The next chunk's reads follow these updates (one wave's LDS
                // operations complete in program order).
                wave_lds_sync();
            }
            if (re > e_end) break;  // the row goes on in the next piece
            ++t;
        }
        wave_lds_sync();  // before the next piece overwrites s_col
    }
    for (int c = lane; c < k; c += kWave) tbl[(size_t)c * ranges + r] = s_cnt[c];
}

// One wave per column: exclusive prefix over the ranges in place, and the total.
__global__ __launch_bounds__(256) void count_columns_kernel(int k, int ranges,
                                                           int *__restrict__ tbl,
                                                           int *__restrict__ tot)
{
    const int c = (int)blockIdx.x * 4 + (int)threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (c >= k) return;
    int *col = tbl + (size_t)c * ranges;
    int carry = 0;
    for (int base = 0; base < ranges; base += kWave) {
        const int i = base + lane;
        const int v = i < ranges ? col[i] : 0;
        const int incl = wave_inclusive_sum(v);
        if (i < ranges) col[i] = carry + incl - v;
        carry += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    if (lane == 0) tot[c] = carry;
}

__global__ __launch_bounds__(kDigitScanThreads) void count_offsets_kernel(int k,
                                                                         const int *__restrict__ tot,
                                                                         int *__restrict__ t_row_offsets)
{
    exclusive_scan_block<kDigitScanThreads>(k, tot, t_row_offsets);
}

__global__ __launch_bounds__(256) void count_scatter_kernel(
    int nnz, int ranges, int rows_per_range, const int *__restrict__ col_indices,
    const float *__restrict__ values, const int *__restrict__ rank,
    const int *__restrict__ rowid, const int *__restrict__ tbl,
    const int *__restrict__ t_row_offsets, int *__restrict__ t_col_indices,
    float *__restrict__ t_values, int *__restrict__ t_perm)
{
    const long long p = (long long)blockIdx.x * 256 + threadIdx.x;
    if (p >= nnz) return;
    const int c = col_indices[p];
    const int row = rowid[p];
    const int r = row / rows_per_range;
    const int q = t_row_offsets[c] + tbl[(size_t)c * ranges + r] + rank[p];
    t_col_indices[q] = row;
    if (t_values) t_values[q] = values[p];
    if (t_perm) t_perm[q] = (int)p;
}

struct Workspace {
    int *keys[2], *vals[2], *rowid, *hist;
    size_t bytes;
};

}  // namespace

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

namespace {

Workspace carve(int nnz, void *base)
{
    const size_t arr = align256((size_t)std::max(nnz, 1) * sizeof(int));
    const size_t hist = radix_hist_bytes(nnz);
    Workspace w;
    char *p = static_cast<char *>(base);
    w.keys[0] = reinterpret_cast<int *>(p);
    w.keys[1] = reinterpret_cast<int *>(p + arr);
    w.vals[0] = reinterpret_cast<int *>(p + 2 * arr);
    w.vals[1] = reinterpret_cast<int *>(p + 3 * arr);
    w.rowid = reinterpret_cast<int *>(p + 4 * arr);
    w.hist = reinterpret_cast<int *>(p + 5 * arr);
    w.bytes = 5 * arr + hist;
    return w;
}

unsigned blocks_for(long long count) { return (unsigned)((count + 255) / 256); }

// The counting method's ranges: about kRangeEntries entries each, at most
// kRowsCap rows, and a table of R * k + k ints within kCountMaxTable and the
// workspace's three nnz-sized arrays after the rank array.  0: use the radix
// method (larger problems, where its passes stream better than the rank
// kernel's row-by-row walk).
int count_rows_per_range(int m, int k, int nnz)
{
    if (k > kCountMaxK || nnz > kCountMaxNnz || m == 0) return 0;
    const long long cap = std::min<long long>(
        kCountMaxTable, 3 * (long long)(align256((size_t)nnz * sizeof(int)) / sizeof(int)));
    long long s = std::max(1LL, std::min<long long>(kRowsCap, (long long)kRangeEntries * m / nnz));
    for (;;) {
        const long long ranges = (m + s - 1) / s;
        if (ranges * k + k <= cap) return (int)s;
        if (s >= kRowsCap) return 0;
        s = std::min<long long>(kRowsCap, 2 * s);
    }
}

hipError_t launch_count_transpose(int m, int k, int nnz, int rows_per_range,
                                  const int *row_offsets, const int *col_indices,
                                  const float *values, int *t_row_offsets, int *t_col_indices,
                                  float *t_values, int *t_perm, const Workspace &w,
                                  hipStream_t stream)
{
    hipError_t e;
    const int ranges = (m + rows_per_range - 1) / rows_per_range;
    int *rank = w.keys[0];
    int *tbl = w.keys[1];  // keys[1], vals[0], vals[1] are contiguous
    int *tot = tbl + (size_t)ranges * k;
    const size_t lds = (size_t)k * sizeof(int);
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void *>(&count_rank_kernel),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) !=
        hipSuccess)
        return e;
    hipLaunchKernelGGL(count_rank_kernel, dim3((unsigned)ranges), dim3(kWave), lds, stream, m, k,
                       rows_per_range, ranges, row_offsets, col_indices, rank, w.rowid, tbl);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(count_columns_kernel, dim3((unsigned)((k + 3) / 4)), dim3(256), 0, stream,
                       k, ranges, tbl, tot);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(count_offsets_kernel, dim3(1), dim3(kDigitScanThreads), 0, stream, k, tot,
                       t_row_offsets);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(count_scatter_kernel, dim3(blocks_for(nnz)), dim3(256), 0, stream, nnz,
                       ranges, rows_per_range, col_indices, values, rank, w.rowid, tbl,
                       t_row_offsets, t_col_indices, t_values, t_perm);
    return hipGetLastError();
}

}  // namespace

size_t transpose_workspace_bytes(int nnz) { return carve(nnz, nullptr).bytes; }

size_t radix_hist_bytes(int n)
{
    const int tiles = (n + kTile - 1) / kTile;
    return align256((size_t)kDigits * (size_t)(tiles + 1) * sizeof(int));
}

int radix_passes(long long bound)
{
    int bits = 0;
    while (bits < 31 && (1LL << bits) < bound) ++bits;  // keys lie in [0, 2^bits)
    return (bits + 7) / 8;
}

hipError_t launch_radix_sort(int n, int passes, const int *keys_in, const int *vals_in,
                             int *const keys_buf[2], int *const vals_buf[2], int *vals_last,
                             int *hist, hipStream_t stream, const int **keys_sorted,
                             const int **vals_sorted)
{
    hipError_t e;
    const int tiles = (n + kTile - 1) / kTile;
    const int *keys = keys_in;
    const int *vals = vals_in;
    for (int pass = 0; pass < passes; ++pass) {
        const int shift = 8 * pass;
        int *keys_out = keys_buf[pass & 1];
        int *vals_out = (pass == passes - 1 && vals_last) ? vals_last : vals_buf[pass & 1];
        hipLaunchKernelGGL(radix_upsweep_kernel, dim3((unsigned)tiles), dim3(kSortThreads), 0,
                           stream, n, shift, keys, hist, tiles);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(digit_scan_kernel, dim3(kDigits), dim3(kDigitScanThreads), 0, stream,
                           tiles, hist);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(radix_downsweep_kernel, dim3((unsigned)tiles), dim3(kSortThreads), 0,
                           stream, n, shift, keys, vals, keys_out, vals_out, hist, tiles);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        keys = keys_out;
        vals = vals_out;
    }
    if (keys_sorted) *keys_sorted = keys;
    if (vals_sorted) *vals_sorted = vals;
    return hipSuccess;
}

hipError_t launch_csr_transpose(int m, int k, int nnz, const int *row_offsets,
                                const int *col_indices, const float *values,
                                int *t_row_offsets, int *t_col_indices, float *t_values,
                                int *t_perm, void *workspace, hipStream_t stream)
{
    hipError_t e;
    if (nnz == 0) return launch_fill_zero(reinterpret_cast<float *>(t_row_offsets), k + 1, stream);
    const Workspace w = carve(nnz, workspace);
    if (const int s = count_rows_per_range(m, k, nnz))
        return launch_count_transpose(m, k, nnz, s, row_offsets, col_indices, values,
                                      t_row_offsets, t_col_indices, t_values, t_perm, w, stream);

    // Columns lie in [0, k): the sort looks at the low 8 * passes bits.  When
    // the row fits above them in a non-negative int, it rides in the key, so
    // the sorted keys give A^T's column indices (rows of A) with no gather.
    // With no pass (k == 1) every column is 0: the entries are already in
    // order.
    const int passes = radix_passes(k);
    const int row_shift = 8 * passes;
    int row_bits = 0;
    while (row_bits < 31 && (1LL << row_bits) < (long long)m) ++row_bits;
    if (passes > 0 && row_shift + row_bits <= 31) {
        hipLaunchKernelGGL(pack_keys_kernel, dim3((unsigned)m), dim3(kWave), 0, stream,
                           row_offsets, col_indices, row_shift, w.rowid);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int *pkeys = nullptr;
        const int *perm = nullptr;
        if ((e = launch_radix_sort(nnz, passes, w.rowid, nullptr, w.keys, w.vals, nullptr,
                                   w.hist, stream, &pkeys, &perm)) != hipSuccess)
            return e;
        hipLaunchKernelGGL(transpose_finish_packed_kernel, dim3(blocks_for((long long)nnz + 1)),
                           dim3(256), 0, stream, nnz, k, row_shift, pkeys, perm, values,
                           t_row_offsets, t_col_indices, t_values, t_perm);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(expand_rows_kernel, dim3((unsigned)m), dim3(kWave), 0, stream,
                       row_offsets, w.rowid);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int *keys = col_indices;
    const int *vals = nullptr;
    if ((e = launch_radix_sort(nnz, passes, col_indices, nullptr, w.keys, w.vals,
                               nullptr, w.hist, stream, &keys, &vals)) != hipSuccess)
        return e;
    hipLaunchKernelGGL(offsets_from_sorted_kernel, dim3(blocks_for((long long)nnz + 1)),
                       dim3(256), 0, stream, nnz, k, keys, t_row_offsets);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(transpose_finish_kernel, dim3(blocks_for(nnz)), dim3(256), 0, stream, nnz,
                       vals, w.rowid, values, t_col_indices, t_values, t_perm);
    return hipGetLastError();
}

hipError_t launch_gather_values(int nnz, const int *perm, const float *in, float *out,
                                hipStream_t stream)
{
    if (nnz == 0) return hipSuccess;
    hipLaunchKernelGGL(gather_values_kernel, dim3(blocks_for(nnz)), dim3(256), 0, stream, nnz,
                       perm, in, out);
    return hipGetLastError();
}

}  // namespace spk
