// Host-side launchers of the device kernels, called by the C ABI layer after
// it has validated the arguments.  Each returns the launch's hipError_t.
#pragma once

#include <hip/hip_runtime.h>

#include "sp_types.h"

namespace spk {

struct SpmmArgs {
    int m, k, n, nnz;
    const int *row_indices;  // NULL = identity order
    const int *row_offsets;
    const int *col_indices;
    const void *values;  // element type `dtype`
    const void *b;       // element type `dtype`
    float *c;
    int batch;
    long long stride_values, stride_b, stride_c;  // elements
    Dtype dtype = Dtype::f32;
    bool balanced = false;  // wide B: waves share each group's entries evenly
    // wide B, one batch entry, a row order given: the balanced kernel (its
    // groups of rows of similar length run as the wide kernel does)
    bool auto_balance = true;
};

struct SddmmArgs {
    int m, k, d, nnz;
    const int *row_indices;  // NULL = identity order
    const int *row_offsets;
    const int *col_indices;
    const float *mask_values;  // NULL = no scaling by the mask's values
    const void *x;             // element type `dtype`
    const void *y;             // element type `dtype`
    int y_layout;  // 0: Y is k x d; 1: Y is d x k
    float alpha, beta;  // beta == 0: out is not read
    float *out;
    int batch;
    long long stride_values, stride_x, stride_y, stride_out;  // elements
    Dtype dtype = Dtype::f32;
    bool softmax = false;  // row softmax of alpha * scores (k x d layout, no v, beta 0)
    int parts = 1;         // > 1: waves sharing each row's 64-entry windows (not with softmax)
    void *workspace = nullptr;  // Y stored d x k: room for its k x d transpose, or NULL
};

struct AttnArgs {
    int m, k_rows, d, batch;
    const int *row_indices;  // NULL = identity order
    const int *row_offsets;
    const int *col_indices;
    const void *q, *k, *v;   // element type `dtype`
    float alpha;
    float *out;
    long long stride_q, stride_k, stride_v, stride_out;  // elements
    Dtype dtype = Dtype::f32;
};

hipError_t launch_offsets_from_lengths(int m, const int *lengths,
                                       int *row_offsets, hipStream_t stream);
hipError_t launch_count_dense(int m, int k, const unsigned char *mask,
                              int *row_offsets, hipStream_t stream);
hipError_t launch_fill_dense(int m, int k, const unsigned char *mask,
                             const float *dense_values, const int *row_offsets,
                             int *col_indices, float *values, hipStream_t stream);
hipError_t launch_build_and_swizzle(int m, const int *lengths, int *row_offsets,
                                   int *row_indices, hipStream_t stream);
hipError_t launch_row_swizzle(int m, const int *row_offsets, int *row_indices,
                              hipStream_t stream);
// The workspace form: the rank sort up to its row limit (no workspace), a
// radix sort above it in row_swizzle_workspace_bytes(m) bytes of workspace.
size_t row_swizzle_workspace_bytes(int m);
hipError_t launch_row_swizzle_ws(int m, int k, const int *row_offsets, int *row_indices,
                                 void *workspace, hipStream_t stream);
// The workspace form on the library's own per-device scratch array (for
// callers that cannot allocate); row_swizzle_noalloc_fits(m) says whether m
// rows fit it.
bool row_swizzle_noalloc_fits(int m);
hipError_t launch_row_swizzle_noalloc(int m, int k, const int *row_offsets, int *row_indices,
                                      hipStream_t stream);
hipError_t launch_spmm(const SpmmArgs &a, hipStream_t stream);
// Name of the kernel launch_spmm would run for `a` (host-only).
const char *spmm_kernel_name(const SpmmArgs &a);
const char *sddmm_kernel_name(const SddmmArgs &a);
hipError_t launch_sddmm(const SddmmArgs &a, hipStream_t stream);
hipError_t launch_spmm_sddmm(const SpmmArgs &x, const SddmmArgs &y, hipStream_t stream);
hipError_t launch_attention(const AttnArgs &a, hipStream_t stream);
hipError_t launch_row_softmax(int m, const int *row_indices, const int *row_offsets,
                              const float *in, float *out, int batch, long long stride_in,
                              long long stride_out, hipStream_t stream);
hipError_t launch_fill_zero(float *dst, long long count, hipStream_t stream);
size_t align256(size_t b);
// Stable least-significant-digit radix sort of n (key, value) int pairs, 8-bit
// digits, `passes` passes (keys in [0, 2^(8 * passes))), each pass three
// launches (tile digit counts, per-digit scan over tiles, stable scatter).
// keys_in / vals_in are read only (vals_in NULL: the identity 0..n-1); passes
// alternate between keys_buf[0/1] and vals_buf[0/1] (n ints each); the last
// pass writes its values to vals_last when that is not NULL.  hist needs
// radix_hist_bytes(n).  The sorted arrays' addresses are returned through
// keys_sorted / vals_sorted (the inputs themselves when passes == 0).
size_t radix_hist_bytes(int n);
int radix_passes(long long bound);  // passes for keys in [0, bound)
hipError_t launch_radix_sort(int n, int passes, const int *keys_in, const int *vals_in,
                             int *const keys_buf[2], int *const vals_buf[2], int *vals_last,
                             int *hist, hipStream_t stream, const int **keys_sorted,
                             const int **vals_sorted);
size_t transpose_workspace_bytes(int nnz);
hipError_t launch_csr_transpose(int m, int k, int nnz, const int *row_offsets,
                                const int *col_indices, const float *values,
                                int *t_row_offsets, int *t_col_indices, float *t_values,
                                int *t_perm, void *workspace, hipStream_t stream);
hipError_t launch_gather_values(int nnz, const int *perm, const float *in, float *out,
                                hipStream_t stream);

}  // namespace spk
