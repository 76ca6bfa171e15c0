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
hipError_t launch_spmm(const SpmmArgs &a, hipStream_t stream);
hipError_t launch_sddmm(const SddmmArgs &a, hipStream_t stream);
hipError_t launch_spmm_sddmm(const SpmmArgs &x, const SddmmArgs &y, hipStream_t stream);
hipError_t launch_attention(const AttnArgs &a, hipStream_t stream);
hipError_t launch_row_softmax(int m, const int *row_indices, const int *row_offsets,
                              const float *in, float *out, int batch, long long stride_in,
                              long long stride_out, hipStream_t stream);
hipError_t launch_fill_zero(float *dst, long long count, hipStream_t stream);
size_t transpose_workspace_bytes(int nnz);
hipError_t launch_csr_transpose(int m, int k, int nnz, const int *row_offsets,
                                const int *col_indices, const float *values,
                                int *t_row_offsets, int *t_col_indices, float *t_values,
                                int *t_perm, void *workspace, hipStream_t stream);
hipError_t launch_gather_values(int nnz, const int *perm, const float *in, float *out,
                                hipStream_t stream);

}  // namespace spk
