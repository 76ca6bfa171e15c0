// CSR build on the device: row offsets from row lengths (an exclusive prefix
// sum) and CSR from a dense byte mask (count, prefix sum, ordered compaction).
//
// The card ("Sparse GPU Kernels for Deep Learning", summary card: "Summary",
// "Interesting ideas" I5) has the kernels work on plain, standard CSR; these
// kernels produce exactly that format: rows ascending, columns ascending
// within a row, int32 offsets and indices.  Integer work only, so the result
// is bit-identical to any correct CSR construction.
#include "sp_device.h"
#include "sp_launch.h"
#include "sp_scan.h"

namespace spk {

namespace {

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void exclusive_scan_kernel(
    int m, const int *in, int *out)
{
    exclusive_scan_block<kScanThreads>(m, in, out);
}

// counts[row] = number of nonzero bytes in mask row `row` (one wave per row).
__global__ __launch_bounds__(kWave) void count_mask_rows_kernel(
    int m, int k, const unsigned char *__restrict__ mask, int *__restrict__ counts)
{
    const int row = blockIdx.x;
    const int lane = threadIdx.x;
    const unsigned char *r = mask + (size_t)row * (size_t)k;
    int total = 0;
    for (int c0 = 0; c0 < k; c0 += kWave) {
        const int c = c0 + lane;
        const bool set = c < k && r[c] != 0;
        total += __popcll(__ballot(set));
    }
    if (lane == 0) counts[row] = total;
}

// Ordered compaction of mask row `row` into its CSR slice (one wave per row):
// each 64-column window's set positions are written in column order at the
// row's running offset, via ballot and a lane-below popcount.
__global__ __launch_bounds__(kWave) void fill_mask_rows_kernel(
    int m, int k, const unsigned char *__restrict__ mask,
    const float *__restrict__ dense_values, const int *__restrict__ row_offsets,
    int *__restrict__ col_indices, float *__restrict__ values)
{
    const int row = blockIdx.x;
    const int lane = threadIdx.x;
    const size_t row_base = (size_t)row * (size_t)k;
    int p = row_offsets[row];
    const uint64_t below = lanes_below(lane);
    for (int c0 = 0; c0 < k; c0 += kWave) {
        const int c = c0 + lane;
        const bool set = c < k && mask[row_base + c] != 0;
        const uint64_t bits = __ballot(set);
        if (set) {
            const int at = p + __popcll(bits & below);
            col_indices[at] = c;
            if (dense_values != nullptr) values[at] = dense_values[row_base + c];
        }
        p += __popcll(bits);
    }
}

}  // namespace

hipError_t launch_offsets_from_lengths(int m, const int *lengths,
                                       int *row_offsets, hipStream_t stream)
{
    hipLaunchKernelGGL(exclusive_scan_kernel, dim3(1), dim3(kScanThreads), 0,
                       stream, m, lengths, row_offsets);
    return hipGetLastError();
}

hipError_t launch_count_dense(int m, int k, const unsigned char *mask,
                              int *row_offsets, hipStream_t stream)
{
    if (m > 0) {
        hipLaunchKernelGGL(count_mask_rows_kernel, dim3(m), dim3(kWave), 0,
                           stream, m, k, mask, row_offsets + 1);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // In place: row_offsets[1..m] holds the counts, the scan turns them into
    // offsets and writes row_offsets[0] = 0.
    hipLaunchKernelGGL(exclusive_scan_kernel, dim3(1), dim3(kScanThreads), 0,
                       stream, m, row_offsets + 1, row_offsets);
    return hipGetLastError();
}

hipError_t launch_fill_dense(int m, int k, const unsigned char *mask,
                             const float *dense_values, const int *row_offsets,
                             int *col_indices, float *values, hipStream_t stream)
{
    if (m == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_mask_rows_kernel, dim3(m), dim3(kWave), 0, stream,
                       m, k, mask, dense_values, row_offsets, col_indices,
                       values);
    return hipGetLastError();
}

}  // namespace spk
