// The C ABI of include/sp_csr.h: argument checks on the host, then kernel
// launches on the caller's stream.  No allocation, no synchronisation, no
// global mutable state.
#include <climits>

#include "sp_csr.h"
#include "sp_launch.h"

namespace {

constexpr int kVersion = 10000;  // 1.0.0

sp_status_t from_hip(hipError_t e)
{
    if (e == hipSuccess) return SP_SUCCESS;
    if (e == hipErrorInvalidConfiguration) return SP_ERROR_NOT_SUPPORTED;
    return SP_ERROR_LAUNCH_FAILED;
}

hipStream_t as_stream(sp_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

// A pointer must be non-NULL when the buffer it describes is non-empty.
bool need(const void *ptr, long long elements) { return elements <= 0 || ptr != nullptr; }

bool dtype_of(int code, spk::Dtype *out)
{
    switch (code) {
    case SP_DTYPE_F32: *out = spk::Dtype::f32; return true;
    case SP_DTYPE_F16: *out = spk::Dtype::f16; return true;
    case SP_DTYPE_BF16: *out = spk::Dtype::bf16; return true;
    default: return false;
    }
}

// Bytes for the k x d transpose of Y (one per batch entry, or one shared).
size_t sddmm_workspace_bytes(int k, int d, int batch, long long stride_y, spk::Dtype dtype)
{
    const size_t copies = stride_y == 0 ? 1 : (size_t)(batch > 0 ? batch : 0);
    const size_t eb = dtype == spk::Dtype::f32 ? 4 : 2;
    return copies * (size_t)(k > 0 ? k : 0) * (size_t)(d > 0 ? d : 0) * eb;
}

// Checks an SDDMM's arguments and fills `a`; *work is false when there is
// nothing to launch.
sp_status_t sddmm_prepare(int m, int k, int d, int nnz, const int *row_indices,
                          const int *row_offsets, const int *col_indices,
                          const float *mask_values, spk::Dtype dtype, const void *x,
                          const void *y, int y_layout, float alpha, float beta, float *out,
                          int batch, long long stride_values, long long stride_x,
                          long long stride_y, long long stride_out, spk::SddmmArgs *args,
                          bool *work, void *workspace = nullptr, size_t workspace_bytes = 0)
{
    *work = false;
    if (m < 0 || k < 0 || d < 0 || nnz < 0 || batch < 0 || stride_values < 0 ||
        stride_x < 0 || stride_y < 0 || stride_out < 0)
        return SP_ERROR_INVALID_VALUE;
    if (y_layout != SP_Y_KD && y_layout != SP_Y_DK) return SP_ERROR_INVALID_VALUE;
    if (m == 0 || nnz == 0 || batch == 0) return SP_SUCCESS;
    if (!need(row_offsets, m) || !need(col_indices, nnz) || out == nullptr ||
        !need(x, (long long)m * d) || !need(y, (long long)k * d))
        return SP_ERROR_INVALID_VALUE;
    if (batch > 1 && stride_out < nnz) return SP_ERROR_INVALID_VALUE;
    spk::SddmmArgs &a = *args;
    a.m = m;
    a.k = k;
    a.d = d;
    a.nnz = nnz;
    a.row_indices = row_indices;
    a.row_offsets = row_offsets;
    a.col_indices = col_indices;
    a.mask_values = mask_values;
    a.x = x;
    a.y = y;
    a.y_layout = y_layout;
    a.alpha = alpha;
    a.beta = beta;
    a.out = out;
    a.batch = batch;
    a.stride_values = stride_values;
    a.stride_x = stride_x;
    a.stride_y = stride_y;
    a.stride_out = stride_out;
    a.dtype = dtype;
    if (y_layout == SP_Y_DK && workspace != nullptr) {
        if (workspace_bytes < sddmm_workspace_bytes(k, d, batch, stride_y, dtype) ||
            reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
            return SP_ERROR_INVALID_VALUE;
        a.workspace = workspace;
    }
    *work = true;
    return SP_SUCCESS;
}

sp_status_t sddmm_any(int m, int k, int d, int nnz, const int *row_indices,
                      const int *row_offsets, const int *col_indices,
                      const float *mask_values, spk::Dtype dtype, const void *x, const void *y,
                      int y_layout, float alpha, float beta, float *out, int batch,
                      long long stride_values, long long stride_x, long long stride_y,
                      long long stride_out, sp_stream_t stream, void *workspace = nullptr,
                      size_t workspace_bytes = 0)
{
    spk::SddmmArgs a;
    bool work = false;
    const sp_status_t st = sddmm_prepare(m, k, d, nnz, row_indices, row_offsets, col_indices,
                                         mask_values, dtype, x, y, y_layout, alpha, beta, out,
                                         batch, stride_values, stride_x, stride_y, stride_out,
                                         &a, &work, workspace, workspace_bytes);
    if (st != SP_SUCCESS || !work) return st;
    return from_hip(spk::launch_sddmm(a, as_stream(stream)));
}

// Checks an SpMM's arguments and fills `a`; *work is false when there is
// nothing to launch.
sp_status_t spmm_prepare(int m, int k, int n, int nnz, const int *row_indices,
                         spk::Dtype dt, const void *values, const int *row_offsets,
                         const int *col_indices, const void *b, float *c, int batch,
                         long long stride_values, long long stride_b, long long stride_c,
                         spk::SpmmArgs *args, bool *work)
{
    *work = false;
    if (m < 0 || k < 0 || n < 0 || nnz < 0 || batch < 0 || stride_values < 0 ||
        stride_b < 0 || stride_c < 0)
        return SP_ERROR_INVALID_VALUE;
    if (m == 0 || n == 0 || batch == 0) return SP_SUCCESS;
    if (!need(row_offsets, m) || !need(col_indices, nnz) || !need(values, nnz) ||
        !need(b, nnz > 0 ? (long long)k * n : 0) || c == nullptr)
        return SP_ERROR_INVALID_VALUE;
    if (batch > 1 && stride_c < (long long)m * n) return SP_ERROR_INVALID_VALUE;
    spk::SpmmArgs &a = *args;
    a.m = m;
    a.k = k;
    a.n = n;
    a.nnz = nnz;
    a.row_indices = row_indices;
    a.row_offsets = row_offsets;
    a.col_indices = col_indices;
    a.values = values;
    a.b = b;
    a.c = c;
    a.batch = batch;
    a.stride_values = stride_values;
    a.stride_b = stride_b;
    a.stride_c = stride_c;
    a.dtype = dt;
    *work = true;
    return SP_SUCCESS;
}

}  // namespace

extern "C" {

const char *sp_status_string(sp_status_t status)
{
    switch (status) {
    case SP_SUCCESS: return "success";
    case SP_ERROR_INVALID_VALUE: return "invalid argument";
    case SP_ERROR_NOT_SUPPORTED: return "problem shape or size not supported by these kernels";
    case SP_ERROR_LAUNCH_FAILED: return "kernel launch failed";
    }
    return "unknown status";
}

int sp_version(void) { return kVersion; }

sp_status_t sp_csr_offsets_from_lengths(int m, const int *lengths, int *row_offsets,
                                        sp_stream_t stream)
{
    if (m < 0 || !need(lengths, m) || row_offsets == nullptr)
        return SP_ERROR_INVALID_VALUE;
    return from_hip(spk::launch_offsets_from_lengths(m, lengths, row_offsets,
                                                     as_stream(stream)));
}

sp_status_t sp_csr_count_dense(int m, int k, const unsigned char *mask,
                               int *row_offsets, sp_stream_t stream)
{
    if (m < 0 || k < 0 || !need(mask, (long long)m * k) || row_offsets == nullptr)
        return SP_ERROR_INVALID_VALUE;
    return from_hip(spk::launch_count_dense(m, k, mask, row_offsets, as_stream(stream)));
}

sp_status_t sp_csr_fill_dense(int m, int k, const unsigned char *mask,
                              const float *dense_values, const int *row_offsets,
                              int *col_indices, float *values, sp_stream_t stream)
{
    // col_indices (and values, when dense_values is given) are written only at
    // the mask's set positions, so they may be NULL for a mask with none; the
    // host cannot know nnz without reading the device, so that is left to the
    // caller (documented precondition).
    if (m < 0 || k < 0 || !need(mask, (long long)m * k) || !need(row_offsets, m))
        return SP_ERROR_INVALID_VALUE;
    return from_hip(spk::launch_fill_dense(m, k, mask, dense_values, row_offsets,
                                           col_indices, values, as_stream(stream)));
}

sp_status_t sp_row_swizzle(int m, const int *row_offsets, int *row_indices,
                           sp_stream_t stream)
{
    if (m < 0 || !need(row_offsets, m) || !need(row_indices, m))
        return SP_ERROR_INVALID_VALUE;
    return from_hip(spk::launch_row_swizzle(m, row_offsets, row_indices,
                                            as_stream(stream)));
}

sp_status_t sp_row_swizzle_workspace(int m, size_t *bytes)
{
    if (m < 0 || bytes == nullptr) return SP_ERROR_INVALID_VALUE;
    *bytes = spk::row_swizzle_workspace_bytes(m);
    return SP_SUCCESS;
}

sp_status_t sp_row_swizzle_ws(int m, int k, const int *row_offsets, int *row_indices,
                              void *workspace, size_t workspace_bytes, sp_stream_t stream)
{
    if (m < 0 || k < 0 || !need(row_offsets, m) || !need(row_indices, m))
        return SP_ERROR_INVALID_VALUE;
    if (m == 0) return SP_SUCCESS;
    const size_t want = spk::row_swizzle_workspace_bytes(m);
    if (want > 0 && (workspace == nullptr || workspace_bytes < want ||
                     reinterpret_cast<uintptr_t>(workspace) % 256 != 0))
        return SP_ERROR_INVALID_VALUE;
    return from_hip(spk::launch_row_swizzle_ws(m, k, row_offsets, row_indices, workspace,
                                               as_stream(stream)));
}

sp_status_t sp_row_swizzle_noalloc(int m, int k, const int *row_offsets, int *row_indices,
                                   sp_stream_t stream)
{
    if (m < 0 || k < 0 || !need(row_offsets, m) || !need(row_indices, m))
        return SP_ERROR_INVALID_VALUE;
    if (m > SP_ROW_SWIZZLE_NOALLOC_MAX_ROWS || !spk::row_swizzle_noalloc_fits(m))
        return SP_ERROR_INVALID_VALUE;
    if (m == 0) return SP_SUCCESS;
    return from_hip(spk::launch_row_swizzle_noalloc(m, k, row_offsets, row_indices,
                                                    as_stream(stream)));
}

sp_status_t sp_csr_build_from_lengths(int m, const int *lengths, int *row_offsets,
                                      int *row_indices, sp_stream_t stream)
{
    if (m < 0 || !need(lengths, m) || row_offsets == nullptr || !need(row_indices, m))
        return SP_ERROR_INVALID_VALUE;
    return from_hip(spk::launch_build_and_swizzle(m, lengths, row_offsets, row_indices,
                                                  as_stream(stream)));
}

sp_status_t sp_spmm_ex(int m, int k, int n, int nnz, const int *row_indices, int dtype,
                       const void *values, const int *row_offsets, const int *col_indices,
                       const void *b, float *c, int batch, long long stride_values,
                       long long stride_b, long long stride_c, sp_stream_t stream)
{
    spk::Dtype dt;
    if (!dtype_of(dtype, &dt)) return SP_ERROR_INVALID_VALUE;
    spk::SpmmArgs a;
    bool work = false;
    const sp_status_t st = spmm_prepare(m, k, n, nnz, row_indices, dt, values, row_offsets,
                                        col_indices, b, c, batch, stride_values, stride_b,
                                        stride_c, &a, &work);
    if (st != SP_SUCCESS || !work) return st;
    return from_hip(spk::launch_spmm(a, as_stream(stream)));
}

sp_status_t sp_spmm_kernel_name(int m, int k, int n, int nnz, const int *row_indices, int dtype,
                                const void *values, const int *col_indices, const void *b,
                                const float *c, int batch, long long stride_values,
                                long long stride_b, long long stride_c, const char **name)
{
    if (name == nullptr) return SP_ERROR_INVALID_VALUE;
    spk::Dtype dt;
    if (!dtype_of(dtype, &dt)) return SP_ERROR_INVALID_VALUE;
    // The choice depends on sizes, element type and pointer alignment only, so
    // stand-ins take the place of the arrays the plan does not look at.
    static const int kStandIn[2] = {0, 0};
    spk::SpmmArgs a;
    bool work = false;
    const sp_status_t st = spmm_prepare(m, k, n, nnz, row_indices, dt, values, kStandIn, col_indices,
                                        b, const_cast<float *>(c), batch, stride_values,
                                        stride_b, stride_c, &a, &work);
    if (st != SP_SUCCESS) return st;
    *name = work ? spk::spmm_kernel_name(a) : "none";
    return SP_SUCCESS;
}

sp_status_t sp_sddmm_kernel_name(int m, int k, int d, int nnz, int dtype,
                                 const float *mask_values, const void *x, const void *y,
                                 int y_layout, float beta, int batch, long long stride_values,
                                 long long stride_x, long long stride_y, long long stride_out,
                                 void *workspace, size_t workspace_bytes, const char **name)
{
    if (name == nullptr) return SP_ERROR_INVALID_VALUE;
    spk::Dtype dt;
    if (!dtype_of(dtype, &dt)) return SP_ERROR_INVALID_VALUE;
    // As for SpMM: the arrays the plan does not look at get stand-ins.
    static const int kStandIn[2] = {0, 0};
    static float kOutStandIn[1] = {0.f};
    spk::SddmmArgs a;
    bool work = false;
    const sp_status_t st = sddmm_prepare(m, k, d, nnz, nullptr, kStandIn, kStandIn, mask_values,
                                         dt, x, y, y_layout, 1.f, beta, kOutStandIn, batch,
                                         stride_values, stride_x, stride_y, stride_out, &a,
                                         &work, workspace, workspace_bytes);
    if (st != SP_SUCCESS) return st;
    *name = work ? spk::sddmm_kernel_name(a) : "none";
    return SP_SUCCESS;
}

sp_status_t sp_spmm_sddmm(int m, int k, int n, int nnz, const int *row_indices,
                          const float *values, const int *row_offsets, const int *col_indices,
                          const float *b, float *c, int s_m, int s_k, int d, int s_nnz,
                          const int *s_row_indices, const int *s_row_offsets,
                          const int *s_col_indices, const float *x, const float *y,
                          float alpha, float *out, sp_stream_t stream)
{
    spk::SpmmArgs a;
    spk::SddmmArgs q;
    bool work_a = false, work_q = false;
    sp_status_t st = spmm_prepare(m, k, n, nnz, row_indices, spk::Dtype::f32, values,
                                  row_offsets, col_indices, b, c, 1, 0, 0, 0, &a, &work_a);
    if (st != SP_SUCCESS) return st;
    st = sddmm_prepare(s_m, s_k, d, s_nnz, s_row_indices, s_row_offsets, s_col_indices, nullptr,
                       spk::Dtype::f32, x, y, SP_Y_KD, alpha, 0.f, out, 1, 0, 0, 0, 0, &q,
                       &work_q);
    if (st != SP_SUCCESS) return st;
    const hipStream_t s = as_stream(stream);
    if (work_a && work_q) return from_hip(spk::launch_spmm_sddmm(a, q, s));
    if (work_a) return from_hip(spk::launch_spmm(a, s));
    if (work_q) return from_hip(spk::launch_sddmm(q, s));
    return SP_SUCCESS;
}

sp_status_t sp_spmm_balanced(int m, int k, int n, int nnz, const int *row_indices,
                             const float *values, const int *row_offsets,
                             const int *col_indices, const float *b, float *c,
                             sp_stream_t stream)
{
    spk::SpmmArgs a;
    bool work = false;
    const sp_status_t st = spmm_prepare(m, k, n, nnz, row_indices, spk::Dtype::f32, values,
                                        row_offsets, col_indices, b, c, 1, 0, 0, 0, &a, &work);
    if (st != SP_SUCCESS || !work) return st;
    a.balanced = true;
    return from_hip(spk::launch_spmm(a, as_stream(stream)));
}

sp_status_t sp_spmm_batched(int m, int k, int n, int nnz, const int *row_indices,
                            const float *values, const int *row_offsets,
                            const int *col_indices, const float *b, float *c,
                            int batch, long long stride_values, long long stride_b,
                            long long stride_c, sp_stream_t stream)
{
    return sp_spmm_ex(m, k, n, nnz, row_indices, SP_DTYPE_F32, values, row_offsets,
                      col_indices, b, c, batch, stride_values, stride_b, stride_c, stream);
}

sp_status_t sp_spmm(int m, int k, int n, int nnz, const int *row_indices,
                    const float *values, const int *row_offsets,
                    const int *col_indices, const float *b, float *c,
                    sp_stream_t stream)
{
    return sp_spmm_batched(m, k, n, nnz, row_indices, values, row_offsets,
                           col_indices, b, c, 1, 0, 0, 0, stream);
}

sp_status_t sp_sddmm_general_workspace(int k, int d, int batch, long long stride_y,
                                       size_t *bytes)
{
    if (k < 0 || d < 0 || batch < 0 || stride_y < 0 || bytes == nullptr)
        return SP_ERROR_INVALID_VALUE;
    *bytes = sddmm_workspace_bytes(k, d, batch, stride_y, spk::Dtype::f32);
    return SP_SUCCESS;
}

sp_status_t sp_sddmm_general(int m, int k, int d, int nnz, const int *row_indices,
                             const int *row_offsets, const int *col_indices,
                             const float *mask_values, const float *x, const float *y,
                             int y_layout, float alpha, float beta, float *out, int batch,
                             long long stride_values, long long stride_x,
                             long long stride_y, long long stride_out, void *workspace,
                             size_t workspace_bytes, sp_stream_t stream)
{
    return sddmm_any(m, k, d, nnz, row_indices, row_offsets, col_indices, mask_values,
                     spk::Dtype::f32, x, y, y_layout, alpha, beta, out, batch, stride_values,
                     stride_x, stride_y, stride_out, stream, workspace, workspace_bytes);
}

sp_status_t sp_sddmm_softmax(int m, int k, int d, int nnz, const int *row_indices,
                             const int *row_offsets, const int *col_indices, int dtype,
                             const void *x, const void *y, float alpha, float *out, int batch,
                             long long stride_x, long long stride_y, long long stride_out,
                             sp_stream_t stream)
{
    spk::Dtype dt;
    if (!dtype_of(dtype, &dt)) return SP_ERROR_INVALID_VALUE;
    spk::SddmmArgs a;
    bool work = false;
    const sp_status_t st = sddmm_prepare(m, k, d, nnz, row_indices, row_offsets, col_indices,
                                         nullptr, dt, x, y, SP_Y_KD, alpha, 0.f, out, batch, 0,
                                         stride_x, stride_y, stride_out, &a, &work);
    if (st != SP_SUCCESS || !work) return st;
    a.softmax = true;
    return from_hip(spk::launch_sddmm(a, as_stream(stream)));
}

sp_status_t sp_sparse_attention(int m, int k, int d, int nnz, const int *row_indices,
                                const int *row_offsets, const int *col_indices, int dtype,
                                const void *q, const void *kmat, const void *v, float alpha,
                                float *out, int batch, long long stride_q, long long stride_k,
                                long long stride_v, long long stride_out, sp_stream_t stream)
{
    spk::Dtype dt;
    if (!dtype_of(dtype, &dt)) return SP_ERROR_INVALID_VALUE;
    if (m < 0 || k < 0 || d < 0 || nnz < 0 || batch < 0 || stride_q < 0 || stride_k < 0 ||
        stride_v < 0 || stride_out < 0)
        return SP_ERROR_INVALID_VALUE;
    if (m == 0 || batch == 0) return SP_SUCCESS;
    if (!need(row_offsets, m) || !need(col_indices, nnz) || out == nullptr ||
        !need(q, (long long)m * d) || !need(kmat, nnz > 0 ? (long long)k * d : 0) ||
        !need(v, nnz > 0 ? (long long)k * d : 0))
        return SP_ERROR_INVALID_VALUE;
    if (batch > 1 && stride_out < (long long)m * d) return SP_ERROR_INVALID_VALUE;
    spk::AttnArgs a;
    a.m = m;
    a.k_rows = k;
    a.d = d;
    a.batch = batch;
    a.row_indices = row_indices;
    a.row_offsets = row_offsets;
    a.col_indices = col_indices;
    a.q = q;
    a.k = kmat;
    a.v = v;
    a.alpha = alpha;
    a.out = out;
    a.stride_q = stride_q;
    a.stride_k = stride_k;
    a.stride_v = stride_v;
    a.stride_out = stride_out;
    a.dtype = dt;
    return from_hip(spk::launch_attention(a, as_stream(stream)));
}

sp_status_t sp_sddmm_ex(int m, int k, int d, int nnz, const int *row_indices,
                        const int *row_offsets, const int *col_indices, int dtype,
                        const void *x, const void *y, float alpha, float *out, int batch,
                        long long stride_x, long long stride_y, long long stride_out,
                        sp_stream_t stream)
{
    spk::Dtype dt;
    if (!dtype_of(dtype, &dt)) return SP_ERROR_INVALID_VALUE;
    return sddmm_any(m, k, d, nnz, row_indices, row_offsets, col_indices, nullptr, dt, x, y,
                     SP_Y_KD, alpha, 0.f, out, batch, 0, stride_x, stride_y, stride_out,
                     stream);
}

sp_status_t sp_sddmm_batched(int m, int k, int d, int nnz, const int *row_indices,
                             const int *row_offsets, const int *col_indices,
                             const float *x, const float *y, float alpha, float *out,
                             int batch, long long stride_x, long long stride_y,
                             long long stride_out, sp_stream_t stream)
{
    return sp_sddmm_general(m, k, d, nnz, row_indices, row_offsets, col_indices, nullptr, x,
                            y, SP_Y_KD, alpha, 0.f, out, batch, 0, stride_x, stride_y,
                            stride_out, nullptr, 0, stream);
}

sp_status_t sp_sddmm(int m, int k, int d, int nnz, const int *row_indices,
                     const int *row_offsets, const int *col_indices, const float *x,
                     const float *y, float *out, sp_stream_t stream)
{
    return sp_sddmm_batched(m, k, d, nnz, row_indices, row_offsets, col_indices, x, y,
                            1.f, out, 1, 0, 0, 0, stream);
}

sp_status_t sp_sddmm_balanced(int m, int k, int d, int nnz, const int *row_indices,
                              const int *row_offsets, const int *col_indices, const float *x,
                              const float *y, float *out, sp_stream_t stream)
{
    spk::SddmmArgs a;
    bool work = false;
    const sp_status_t st = sddmm_prepare(m, k, d, nnz, row_indices, row_offsets, col_indices,
                                         nullptr, spk::Dtype::f32, x, y, SP_Y_KD, 1.f, 0.f,
                                         out, 1, 0, 0, 0, 0, &a, &work);
    if (st != SP_SUCCESS || !work) return st;
    a.parts = 4;  // a workgroup of waves per row, each taking every 4th window of 64 entries
    return from_hip(spk::launch_sddmm(a, as_stream(stream)));
}

sp_status_t sp_csr_transpose_workspace(int m, int k, int nnz, size_t *bytes)
{
    if (m < 0 || k < 0 || nnz < 0 || bytes == nullptr) return SP_ERROR_INVALID_VALUE;
    *bytes = spk::transpose_workspace_bytes(nnz);
    return SP_SUCCESS;
}

sp_status_t sp_csr_transpose(int m, int k, int nnz, const int *row_offsets,
                             const int *col_indices, const float *values, int *t_row_offsets,
                             int *t_col_indices, float *t_values, int *t_perm, void *workspace,
                             size_t workspace_bytes, sp_stream_t stream)
{
    if (m < 0 || k < 0 || nnz < 0) return SP_ERROR_INVALID_VALUE;
    if (k == INT_MAX) return SP_ERROR_INVALID_VALUE;  // k + 1 offsets must be indexable
    if (!need(row_offsets, m) || t_row_offsets == nullptr || !need(col_indices, nnz) ||
        !need(t_col_indices, nnz) || (t_values != nullptr && !need(values, nnz)))
        return SP_ERROR_INVALID_VALUE;
    if (nnz > 0 && k == 0) return SP_ERROR_INVALID_VALUE;  // an entry needs a column
    if (nnz > 0 && (workspace == nullptr ||
                    workspace_bytes < spk::transpose_workspace_bytes(nnz)))
        return SP_ERROR_INVALID_VALUE;
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return SP_ERROR_INVALID_VALUE;
    return from_hip(spk::launch_csr_transpose(m, k, nnz, row_offsets, col_indices, values,
                                              t_row_offsets, t_col_indices, t_values, t_perm,
                                              workspace, as_stream(stream)));
}

sp_status_t sp_csr_transpose_values(int nnz, const int *t_perm, const float *values,
                                    float *t_values, sp_stream_t stream)
{
    if (nnz < 0) return SP_ERROR_INVALID_VALUE;
    if (!need(t_perm, nnz) || !need(values, nnz) || !need(t_values, nnz))
        return SP_ERROR_INVALID_VALUE;
    return from_hip(spk::launch_gather_values(nnz, t_perm, values, t_values, as_stream(stream)));
}

sp_status_t sp_csr_row_softmax(int m, int nnz, const int *row_indices,
                               const int *row_offsets, const float *in, float *out,
                               int batch, long long stride_in, long long stride_out,
                               sp_stream_t stream)
{
    if (m < 0 || nnz < 0 || batch < 0 || stride_in < 0 || stride_out < 0)
        return SP_ERROR_INVALID_VALUE;
    if (m == 0 || nnz == 0 || batch == 0) return SP_SUCCESS;
    if (!need(row_offsets, m) || in == nullptr || out == nullptr)
        return SP_ERROR_INVALID_VALUE;
    if (batch > 1 && stride_out < nnz) return SP_ERROR_INVALID_VALUE;
    return from_hip(spk::launch_row_softmax(m, row_indices, row_offsets, in, out, batch,
                                            stride_in, stride_out, as_stream(stream)));
}

}  // extern "C"
