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

}  // namespace

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
