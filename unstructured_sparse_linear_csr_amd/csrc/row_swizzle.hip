// Row swizzle: the order in which rows are handed to workers, by nonzero
// count ("Sparse GPU Kernels for Deep Learning", summary card, "Interesting
// ideas" I4: load balancing by reordering rows, independent of how the
// kernels split their work).
//
// Order: longest row first; rows of equal length by ascending row index.  The
// kernel is a stable rank sort: row i goes to slot
//   rank(i) = #{j : len_j > len_i} + #{j < i : len_j == len_i},
// which is a bijection onto 0..m-1 and needs no workspace and no atomics, so
// the order is deterministic and identical to any stable descending sort.
// Cost is m^2 comparisons, served from LDS as broadcast reads four lengths at
// a time; it runs once per sparsity structure and is reused by every SpMM and
// SDDMM on that structure.
#include "sp_device.h"
#include "sp_launch.h"

namespace spk {

namespace {

constexpr int kSwizzleThreads = 256;
constexpr int kSwizzleTile = 4096;  // lengths staged in LDS per pass (16 KB)

__global__ __launch_bounds__(kSwizzleThreads) void row_swizzle_kernel(
    int m, const int *__restrict__ row_offsets, int *__restrict__ row_indices)
{
    __shared__ int4 s_len4[kSwizzleTile / 4];
    const int i = blockIdx.x * kSwizzleThreads + threadIdx.x;
    const bool mine = i < m;
    const int len_i = mine ? row_offsets[i + 1] - row_offsets[i] : 0;
    int rank = 0;
    for (int t0 = 0; t0 < m; t0 += kSwizzleTile) {
        const int cnt = min(kSwizzleTile, m - t0);
        for (int j = threadIdx.x; j < kSwizzleTile; j += kSwizzleThreads) {
            // Padding slots get length -1: never greater than, never equal to,
            // any real length, so they never count.
            const int r = t0 + j;
            reinterpret_cast<int *>(s_len4)[j] =
                (j < cnt) ? row_offsets[r + 1] - row_offsets[r] : -1;
        }
        __syncthreads();
        if (mine) {
            const int groups = (cnt + 3) / 4;
            for (int g = 0; g < groups; ++g) {
                const int4 l4 = s_len4[g];
                const int j = t0 + 4 * g;
                rank += (l4.x > len_i) | ((l4.x == len_i) & (j + 0 < i));
                rank += (l4.y > len_i) | ((l4.y == len_i) & (j + 1 < i));
                rank += (l4.z > len_i) | ((l4.z == len_i) & (j + 2 < i));
                rank += (l4.w > len_i) | ((l4.w == len_i) & (j + 3 < i));
            }
        }
        __syncthreads();
    }
    if (mine) row_indices[rank] = i;
}

}  // namespace

hipError_t launch_row_swizzle(int m, const int *row_offsets, int *row_indices,
                              hipStream_t stream)
{
    if (m == 0) return hipSuccess;
    const int blocks = (m + kSwizzleThreads - 1) / kSwizzleThreads;
    hipLaunchKernelGGL(row_swizzle_kernel, dim3(blocks), dim3(kSwizzleThreads),
                       0, stream, m, row_offsets, row_indices);
    return hipGetLastError();
}

}  // namespace spk
