// Row swizzle: the order in which rows are handed to workers, by nonzero
// count ("Sparse GPU Kernels for Deep Learning", summary card, "Interesting
// ideas" I4: load balancing by reordering rows, independent of how the
// kernels split their work).
//
// Order: longest row first; rows of equal length by ascending row index.  Each
// row gets the unique 64-bit key (length << 32) | (2^32 - 1 - row), so the
// wanted order is descending key order and a row's slot is its rank
//   rank(i) = #{j : key_j > key_i},
// a bijection onto 0..m-1 that needs no workspace and no atomics: the order is
// deterministic and identical to any stable descending sort by length.  Cost
// is m^2 64-bit comparisons, served from LDS as broadcast reads; the pass runs
// once per sparsity structure and its order is reused by every SpMM and SDDMM
// on that structure.
//
// Many rows (above kRankMaxRows) with a caller workspace: the same order by a
// stable radix sort of the keys k - length (in [0, k] for a structure whose
// rows hold at most k distinct columns), carrying the row index; ascending
// keys are descending lengths and the sort's stability keeps rows of equal
// length in ascending index order.  ceil(log2(k + 1) / 8) passes of three
// launches each, linear in m.
#include <algorithm>
#include <mutex>

#include "sp_device.h"
#include "sp_launch.h"
#include "sp_scan.h"

namespace spk {

namespace {

constexpr int kSwizzleThreads = 256;
// Lanes sharing one row's comparisons: 32 up to kFewRows rows (twice the
// workgroups, half the comparisons per lane: the order of a few thousand rows
// comes sooner), 16 above (fewer workgroups each staging all the keys).
constexpr int kFewRows = 4096;
template <int kLanes> constexpr int rows_per_block() { return kSwizzleThreads / kLanes; }
constexpr int kSwizzleTile = 2048;  // keys staged in LDS per pass (16 KB)
// Above this many rows the workspace form takes the radix sort.
constexpr int kRankMaxRows = 16384;

__device__ __forceinline__ unsigned long long row_key(int length, int row)
{
    return ((unsigned long long)(unsigned)length << 32) | (unsigned)(0xFFFFFFFFu - (unsigned)row);
}

// Row lengths from CSR row offsets, or given directly.
struct FromOffsets {
    const int *row_offsets;
    __device__ int operator()(int r) const { return row_offsets[r + 1] - row_offsets[r]; }
};
struct FromLengths {
    const int *lengths;
    __device__ int operator()(int r) const { return lengths[r]; }
};

// Each row's rank is counted by kLanesPerRow lanes, each taking every
// kLanesPerRow-th pair of staged keys; the partial counts are summed across
// the lanes (integer sums, so the order does not matter).  Lanes of a wave
// that read the same pair read the same LDS address (a broadcast), and the
// kLanesPerRow pairs a wave reads at once are contiguous.  Padding slots hold
// key 0, which is below every real key.
template <int kLanesPerRow, class Len>
__device__ void rank_rows(int m, Len len, int *__restrict__ row_indices, int block)
{
    constexpr int kRowsPerBlock = rows_per_block<kLanesPerRow>();
    __shared__ __align__(16) unsigned long long s_key[kSwizzleTile];
    const int t = threadIdx.x;
    const int sub = t % kLanesPerRow;
    const int i = block * kRowsPerBlock + t / kLanesPerRow;
    const bool mine = i < m;
    const unsigned long long key_i = mine ? row_key(len(i), i) : ~0ull;
    int rank = 0;
    for (int t0 = 0; t0 < m; t0 += kSwizzleTile) {
        const int cnt = min(kSwizzleTile, m - t0);
        // All of a thread's length loads are issued before any is used.
        constexpr int kPer = kSwizzleTile / kSwizzleThreads;
        int l[kPer];
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int j = t + q * kSwizzleThreads;
            l[q] = j < cnt ? len(t0 + j) : 0;
        }
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int j = t + q * kSwizzleThreads;
            s_key[j] = j < cnt ? row_key(l[q], t0 + j) : 0ull;
        }
        __syncthreads();
        // Eight independent LDS reads in flight per lane.  The tile's padding
        // keys are 0, so reading whole groups of eight past cnt is harmless.
        constexpr int kStep = kLanesPerRow * 8;
        const int pairs = min(kSwizzleTile / 2, ((cnt + 1) / 2 + kStep - 1) / kStep * kStep);
        const ulonglong2 *keys2 = reinterpret_cast<const ulonglong2 *>(s_key);
        for (int g0 = sub; g0 < pairs; g0 += kStep) {
            ulonglong2 k2[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) k2[u] = keys2[g0 + u * kLanesPerRow];
#pragma unroll
            for (int u = 0; u < 8; ++u) rank += (k2[u].x > key_i) + (k2[u].y > key_i);
        }
        __syncthreads();
    }
    rank = group_reduce<kLanesPerRow>(rank, OpAdd{});
    if (mine && sub == 0) row_indices[rank] = i;
}

template <int kLanes>
__global__ __launch_bounds__(kSwizzleThreads) void row_swizzle_kernel(
    int m, const int *__restrict__ row_offsets, int *__restrict__ row_indices)
{
    rank_rows<kLanes>(m, FromOffsets{row_offsets}, row_indices, blockIdx.x);
}

// CSR offsets and the swizzled order from row lengths in one launch: the
// order needs only the lengths, so the last workgroup scans them into the
// offsets while the others rank the rows.
template <int kLanes>
__global__ __launch_bounds__(kSwizzleThreads) void build_and_swizzle_kernel(
    int m, const int *__restrict__ lengths, int *__restrict__ row_offsets,
    int *__restrict__ row_indices)
{
    if (blockIdx.x == gridDim.x - 1) {
        exclusive_scan_block<kSwizzleThreads>(m, lengths, row_offsets);
        return;
    }
    rank_rows<kLanes>(m, FromLengths{lengths}, row_indices, blockIdx.x);
}

template <int kLanes>
hipError_t launch_build_t(int m, const int *lengths, int *row_offsets, int *row_indices,
                          hipStream_t stream)
{
    const int blocks = (m + rows_per_block<kLanes>() - 1) / rows_per_block<kLanes>() + 1;
    hipLaunchKernelGGL((build_and_swizzle_kernel<kLanes>), dim3(blocks), dim3(kSwizzleThreads),
                       0, stream, m, lengths, row_offsets, row_indices);
    return hipGetLastError();
}

template <int kLanes>
hipError_t launch_swizzle_t(int m, const int *row_offsets, int *row_indices, hipStream_t stream)
{
    const int blocks = (m + rows_per_block<kLanes>() - 1) / rows_per_block<kLanes>();
    hipLaunchKernelGGL((row_swizzle_kernel<kLanes>), dim3(blocks), dim3(kSwizzleThreads), 0,
                       stream, m, row_offsets, row_indices);
    return hipGetLastError();
}

// keys[i] = k - length of row i, clamped to [0, k]: a row longer than k (not a
// valid structure) sorts with the rows of length k.  The length is the 32-bit
// difference of the offsets, as the rank sort takes it.
__global__ __launch_bounds__(256) void swizzle_keys_kernel(int m, int k,
                                                           const int *__restrict__ row_offsets,
                                                           int *__restrict__ keys)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= m) return;
    const int len = (int)((unsigned)row_offsets[i + 1] - (unsigned)row_offsets[i]);
    const long long key = (long long)k - len;
    keys[i] = (int)(key < 0 ? 0 : key > k ? k : key);
}

struct SwizzleWorkspace {
    int *keys[2], *vals[2], *hist;
    size_t bytes;
};

SwizzleWorkspace carve_swizzle(int m, void *base)
{
    const size_t arr = align256((size_t)m * sizeof(int));
    char *p = static_cast<char *>(base);
    SwizzleWorkspace w;
    w.keys[0] = reinterpret_cast<int *>(p);
    w.keys[1] = reinterpret_cast<int *>(p + arr);
    w.vals[0] = reinterpret_cast<int *>(p + 2 * arr);
    w.vals[1] = reinterpret_cast<int *>(p + 3 * arr);
    w.hist = reinterpret_cast<int *>(p + 4 * arr);
    w.bytes = 4 * arr + radix_hist_bytes(m);
    return w;
}

}  // namespace

size_t row_swizzle_workspace_bytes(int m)
{
    return m <= kRankMaxRows ? 0 : carve_swizzle(m, nullptr).bytes;
}

// ---- the allocation-free form
// The radix sort's workspace for up to kNoAllocMaxRows rows, as a device
// global: every GPU the library runs on holds its own copy, from when the code
// object is loaded there until the process ends.  Nothing in it needs
// clearing between calls (every word the sort reads was written earlier in the
// same call), and calls that overlap on one GPU share it and race.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// The current device's address of `scratch`, looked up once per device with
// that device current.  In host code the name `scratch` denotes a host-side
// stand-in, so only this address may be handed to kernels.
hipError_t scratch_address(void **out)
{
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return e;
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[device] == nullptr) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (ptr == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[device] = ptr;
    }
    *out = g_scratch_ptr[device];
    return hipSuccess;
}

}  // namespace

bool row_swizzle_noalloc_fits(int m)
{
    return m >= 0 && row_swizzle_workspace_bytes(m) <= kScratchBytes;
}

hipError_t launch_row_swizzle_noalloc(int m, int k, const int *row_offsets, int *row_indices,
                                      hipStream_t stream)
{
    if (m <= kRankMaxRows) return launch_row_swizzle(m, row_offsets, row_indices, stream);
    if (!row_swizzle_noalloc_fits(m)) return hipErrorInvalidValue;
    void *ws = nullptr;
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return e;
    return launch_row_swizzle_ws(m, k, row_offsets, row_indices, ws, stream);
}

hipError_t launch_row_swizzle_ws(int m, int k, const int *row_offsets, int *row_indices,
                                 void *workspace, hipStream_t stream)
{
    if (m <= kRankMaxRows) return launch_row_swizzle(m, row_offsets, row_indices, stream);
    const SwizzleWorkspace w = carve_swizzle(m, workspace);
    // The initial keys go to keys[1]; the first pass writes keys[0] (see
    // launch_radix_sort), the second keys[1] again.
    hipLaunchKernelGGL(swizzle_keys_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0,
                       stream, m, k, row_offsets, w.keys[1]);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // keys in [0, k]; at least one pass, so the values always reach row_indices
    const int passes = std::max(1, radix_passes((long long)k + 1));
    return launch_radix_sort(m, passes, w.keys[1], nullptr, w.keys, w.vals, row_indices,
                             w.hist, stream, nullptr, nullptr);
}

hipError_t launch_build_and_swizzle(int m, const int *lengths, int *row_offsets,
                                   int *row_indices, hipStream_t stream)
{
    return m <= kFewRows ? launch_build_t<32>(m, lengths, row_offsets, row_indices, stream)
                         : launch_build_t<16>(m, lengths, row_offsets, row_indices, stream);
}

hipError_t launch_row_swizzle(int m, const int *row_offsets, int *row_indices,
                              hipStream_t stream)
{
    if (m == 0) return hipSuccess;
    return m <= kFewRows ? launch_swizzle_t<32>(m, row_offsets, row_indices, stream)
                         : launch_swizzle_t<16>(m, row_offsets, row_indices, stream);
}

}  // namespace spk
