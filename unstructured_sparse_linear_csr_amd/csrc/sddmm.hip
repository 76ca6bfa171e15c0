// CSR SDDMM for gfx950 ("Sparse GPU Kernels for Deep Learning", summary card,
// "Summary" and "Interesting ideas" I3).  The body for Y stored k x d, and the
// design notes for it, are in sddmm_rows.h; this file holds the kernel for Y
// stored d x k (the general form I3 leaves out) and the variant selection.
#include <algorithm>

#include "sp_device.h"
#include "sp_launch.h"
#include "sp_types.h"
#include "sddmm_rows.h"
#include "sp_plan.h"

namespace spk {

namespace {

using namespace sddmm_detail;

template <typename E, int kG, int kNv, int kVec, bool kSoftmax>
__global__ __launch_bounds__(kWave) void sddmm_kernel(SddmmParams p)
{
    sddmm_rows_body<E, kG, kNv, kVec, kSoftmax>(p, rows_work(p, blockIdx.x));
}

// A workgroup of kSplitParts waves per row slot, sharing the row's windows.
constexpr int kSplitParts = 4;
template <typename E, int kG, int kNv, int kVec>
__global__ __launch_bounds__(kSplitParts * kWave) void sddmm_split_kernel(SddmmParams p)
{
    sddmm_rows_body<E, kG, kNv, kVec, false, kSplitParts>(p, rows_work(p, blockIdx.x));
}

// Y stored d x k (the operand not transposed): Yop(c, l) = Y[l][c].  One wave
// per row slot as above, but lanes are dealt to entries, 64 at a time: for each
// l the wave gathers Y[l][c] of its 64 columns -- all within row l of Y, whose
// columns ascend with the lanes -- and multiplies by X[i][l], which every lane
// shares (a wave-uniform, scalar load).  Each lane sums its entry's d products
// in order with FMA; kU gathers are issued before their FMAs.  Idle lanes of a
// row's last pass gather column 0 (in bounds) and store nothing.
template <typename E, bool kBuf>
__global__ __launch_bounds__(kWave) void sddmm_cols_kernel(SddmmParams p)
{
    using V1 = GVec<E, 1>;
    constexpr unsigned kEb = Elem<E>::kBytes;
    constexpr int kU = 16;
    const long long w = xcd_work_index(p.batch, p.m);
    if (w < 0) return;
    const long long z = w / p.m;
    const int slot = (int)(w - z * p.m);
    const int lane = threadIdx.x;
    const int row = p.row_indices ? p.row_indices[slot] : slot;
    const int p0 = p.row_offsets[row];
    const int p1 = p.row_offsets[row + 1];
    const E *__restrict__ xr =
        static_cast<const E *>(p.x) + z * p.stride_x + (size_t)row * (size_t)p.d;
    const E *__restrict__ yz = static_cast<const E *>(p.y) + z * p.stride_y;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<E *>(yz), 0, (int)p.y_bytes, 0x00020000);
    const unsigned row_bytes = (unsigned)p.k * kEb;

    for (int base = p0; base < p1; base += kWave) {
        const int q = base + lane;
        const bool live = q < p1;
        const int c = live ? p.col_indices[q] : 0;
        float acc = 0.f;
        int l = 0;
        for (; l + kU <= p.d; l += kU) {
            float yv[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                if constexpr (kBuf)
                    V1::to_f32(V1::buf_load(rsrc, (unsigned)(l + u) * row_bytes +
                                                      (unsigned)c * kEb),
                               &yv[u]);
                else
                    yv[u] = Elem<E>::f32(yz[(size_t)(l + u) * (size_t)p.k + (size_t)c]);
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) acc = fmaf(Elem<E>::f32(xr[l + u]), yv[u], acc);
        }
        for (; l < p.d; ++l)
            acc = fmaf(Elem<E>::f32(xr[l]),
                       Elem<E>::f32(yz[(size_t)l * (size_t)p.k + (size_t)c]), acc);
        if (live) store_entry(p, z, q, acc);
    }
}

// out_z = in_z^T for a rows x cols matrix in_z (row-major, z = blockIdx.z):
// 32 x 32 tiles through LDS (one padding column, so the transposed reads hit
// distinct banks), 256 threads reading 4 rows each.  (c_base, r_base) is the
// first tile's corner, so that grids too large for one launch can be split.
template <typename E>
__global__ __launch_bounds__(256) void transpose_kernel(const E *__restrict__ in, E *__restrict__ out,
                                                        int rows, int cols, int r_base, int c_base,
                                                        long long stride_in, long long stride_out)
{
    constexpr int kT = 32;
    __shared__ E tile[kT][kT + 1];
    const E *iz = in + blockIdx.z * stride_in;
    E *oz = out + blockIdx.z * stride_out;
    const int c0 = c_base + (int)blockIdx.x * kT, r0 = r_base + (int)blockIdx.y * kT;
    const int tx = threadIdx.x % kT, ty = threadIdx.x / kT;  // ty in [0, 8)
#pragma unroll
    for (int i = 0; i < kT; i += 8) {
        const int r = r0 + ty + i, c = c0 + tx;
        if (r < rows && c < cols) tile[ty + i][tx] = iz[(size_t)r * cols + c];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kT; i += 8) {
        const int c = c0 + ty + i, r = r0 + tx;  // out row c, column r
        if (c < cols && r < rows) oz[(size_t)c * rows + r] = tile[tx][ty + i];
    }
}

template <typename E>
hipError_t launch_transpose(const void *in, void *out, int rows, int cols, long long stride_in,
                            long long stride_out, int batch, hipStream_t s)
{
    // Tiles per launch in each dimension: x, y and z stay within the grid limits.
    constexpr long long kMaxX = 1LL << 20, kMaxYZ = 65535;
    const long long tx = (cols + 31) / 32, ty = (rows + 31) / 32;
    for (long long z0 = 0; z0 < batch; z0 += kMaxYZ)
        for (long long y0 = 0; y0 < ty; y0 += kMaxYZ)
            for (long long x0 = 0; x0 < tx; x0 += kMaxX) {
                const dim3 grid((unsigned)std::min(kMaxX, tx - x0),
                                (unsigned)std::min(kMaxYZ, ty - y0),
                                (unsigned)std::min(kMaxYZ, (long long)batch - z0));
                hipLaunchKernelGGL((transpose_kernel<E>), grid, dim3(256), 0, s,
                                   static_cast<const E *>(in) + z0 * stride_in,
                                   static_cast<E *>(out) + z0 * stride_out, rows, cols,
                                   (int)(y0 * 32), (int)(x0 * 32), stride_in, stride_out);
                const hipError_t e = hipGetLastError();
                if (e != hipSuccess) return e;
            }
    return hipSuccess;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *dst, long long count,
                                                        long long stride)
{
    float *dz = dst + (long long)blockIdx.y * stride;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < count;
         i += (long long)gridDim.x * 256)
        dz[i] = 0.f;
}

template <typename E, int kG, int kNv, int kVec, bool kSm>
hipError_t launch_t(const SddmmParams &p, bool split, hipStream_t s)
{
    dim3 grid((unsigned)rows_grid(p));
    if constexpr (!kSm) {
        if (split) {
            hipLaunchKernelGGL((sddmm_split_kernel<E, kG, kNv, kVec>), grid,
                               dim3(kSplitParts * kWave), 0, s, p);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((sddmm_kernel<E, kG, kNv, kVec, kSm>), grid, dim3(kWave), 0, s, p);
    return hipGetLastError();
}

template <typename E, int kG, int kVec, bool kSm>
hipError_t launch_nv(int nv, const SddmmParams &p, bool split, hipStream_t s)
{
    switch (nv) {
    case 1: return launch_t<E, kG, 1, kVec, kSm>(p, split, s);
    case 2: return launch_t<E, kG, 2, kVec, kSm>(p, split, s);
    case 4: return launch_t<E, kG, 4, kVec, kSm>(p, split, s);
    case 8: return launch_t<E, kG, 8, kVec, kSm>(p, split, s);
    default: return launch_t<E, kG, 0, kVec, kSm>(p, split, s);
    }
}

template <typename E, int kVec, bool kSm>
hipError_t launch_g(int g, int nv, const SddmmParams &p, bool split, hipStream_t s)
{
    switch (g) {
    case 4: return launch_nv<E, 4, kVec, kSm>(nv, p, split, s);
    case 8: return launch_nv<E, 8, kVec, kSm>(nv, p, split, s);
    default: return launch_nv<E, 16, kVec, kSm>(nv, p, split, s);
    }
}

// Element type E: 16-byte vectors of kVec16 elements, or single elements;
// scores written as they are, or row-softmaxed.
template <typename E, int kVec16>
hipError_t launch_typed(bool vec, bool softmax, bool split, int g, int nv,
                        const SddmmParams &p, hipStream_t s)
{
    if (softmax)
        return vec ? launch_g<E, kVec16, true>(g, nv, p, false, s)
                   : launch_g<E, 1, true>(g, nv, p, false, s);
    return vec ? launch_g<E, kVec16, false>(g, nv, p, split, s)
               : launch_g<E, 1, false>(g, nv, p, split, s);
}

template <typename E>
hipError_t launch_cols(bool buf, const SddmmParams &p, hipStream_t s)
{
    const dim3 grid((unsigned)xcd_grid(p.batch, p.m));
    if (buf)
        hipLaunchKernelGGL((sddmm_cols_kernel<E, true>), grid, dim3(kWave), 0, s, p);
    else
        hipLaunchKernelGGL((sddmm_cols_kernel<E, false>), grid, dim3(kWave), 0, s, p);
    return hipGetLastError();
}

inline bool aligned16(const void *ptr)
{
    return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0;
}

}  // namespace

hipError_t launch_fill_zero(float *dst, long long count, hipStream_t stream)
{
    if (count <= 0) return hipSuccess;
    const long long blocks = std::min<long long>((count + 255) / 256, 65536);
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks, 1), dim3(256), 0,
                       stream, dst, count, 0LL);
    return hipGetLastError();
}

// Lanes per entry kG: the smallest of 4/8/16 covering the row's vectors (16
// beyond).  Vectors per lane kNv rounded up to 1/2/4/8; wider rows take the
// kNv == 0 loop.  d == 0 with no mask values and beta == 0 zero-fills every
// batch's outputs; otherwise the kernels run with empty dot products.
hipError_t plan_sddmm(const SddmmArgs &a, SddmmPlan *plan)
{
    plan->kind = SddmmPlan::kNothing;
    plan->dtype = a.dtype;
    plan->softmax = false;
    plan->split = false;
    plan->t_src = nullptr;
    plan->t_src_stride = 0;
    plan->t_batch = 0;
    if (a.m == 0 || a.nnz == 0) return hipSuccess;
    if (xcd_grid(a.batch, a.m) > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    // A row's 64-entry windows spread over a workgroup of waves (outputs are
    // bit-identical: an entry needs no combine step): on request, and by
    // default for one batch entry whose rows average 16 entries or more.  A
    // row of one window leaves the other waves nothing to do (they exit at
    // once), so uniform rows lose little while the longest rows of a
    // heavy-tailed structure no longer set the launch's duration (the card's
    // I4).  Batched problems keep one wave per row slot: their many row slots
    // already fill the GPU.  The softmax needs whole rows.
    const bool auto_split = a.batch == 1 && (long long)a.nnz >= 16LL * a.m;
    plan->split = !a.softmax && (a.parts > 1 || auto_split);
    SddmmParams &p = plan->p;
    p.m = a.m;
    p.batch = a.batch;
    p.d = a.d;
    p.k = a.k;
    p.nnz = a.nnz;
    p.row_indices = a.row_indices;
    p.row_offsets = a.row_offsets;
    p.col_indices = a.col_indices;
    p.mask_values = a.mask_values;
    p.x = a.x;
    p.y = a.y;
    p.alpha = a.alpha;
    p.beta = a.beta;
    p.out = a.out;
    p.stride_values = a.stride_values;
    p.stride_x = a.stride_x;
    p.stride_y = a.stride_y;
    p.stride_out = a.stride_out;
    const int eb = a.dtype == Dtype::f32 ? 4 : 2;  // bytes per element of X and Y
    const int vlen = 16 / eb;                        // elements per 16-byte vector
    // Buffer offsets into Y must stay below 2^31 (padding offsets lie beyond).
    const bool buf = (long long)a.k * (long long)a.d * eb <= (1LL << 31);
    p.y_bytes = buf ? (unsigned)((long long)a.k * a.d * eb) : 0u;
    plan->buf = buf;
    if (a.y_layout == 1 && a.workspace == nullptr) {
        plan->kind = SddmmPlan::kCols;
        return hipSuccess;
    }
    if (a.y_layout == 1) {
        // Y^T (k x d per batch entry, or one shared copy) into the workspace,
        // then the k x d kernels on it.
        plan->t_src = a.y;
        plan->t_src_stride = a.stride_y;
        plan->t_batch = a.stride_y == 0 ? 1 : a.batch;
        p.y = a.workspace;
        p.stride_y = a.stride_y == 0 ? 0 : (long long)a.k * a.d;
    }
    plan->softmax = a.softmax;
    if (a.d == 0 && a.mask_values == nullptr && a.beta == 0.f && !a.softmax) {
        plan->kind = SddmmPlan::kFill;
        return hipSuccess;
    }
    const bool vec = (a.d % vlen == 0) && aligned16(a.x) && aligned16(p.y) &&
                     (a.stride_x % vlen == 0) && (p.stride_y % vlen == 0);
    // Register-resident X and buffer gathers need valid offsets below Y's size
    // and padding offsets (>= 2^31) beyond it.
    const int kvec = vec ? vlen : 1;
    const int dv = (a.d + kvec - 1) / kvec;
    const int g = dv <= 4 ? 4 : dv <= 8 ? 8 : 16;
    const int need = (dv + g - 1) / g;
    int nv = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : 0;
    if (!buf) nv = 0;
    plan->kind = SddmmPlan::kRows;
    plan->vec = vec;
    plan->g = g;
    plan->nv = nv;
    return hipSuccess;
}

hipError_t run_sddmm(const SddmmPlan &plan, hipStream_t stream)
{
    const SddmmParams &p = plan.p;
    if (plan.t_src != nullptr && p.d > 0 && p.k > 0) {
        const long long stride_out = (long long)p.k * p.d;
        const hipError_t e =
            plan.dtype == Dtype::f32
                ? launch_transpose<float>(plan.t_src, const_cast<void *>(p.y), p.d, p.k,
                                          plan.t_src_stride, stride_out, plan.t_batch, stream)
                : launch_transpose<unsigned short>(plan.t_src, const_cast<void *>(p.y), p.d,
                                                   p.k, plan.t_src_stride, stride_out,
                                                   plan.t_batch, stream);
        if (e != hipSuccess) return e;
    }
    switch (plan.kind) {
    case SddmmPlan::kNothing:
        return hipSuccess;
    case SddmmPlan::kFill: {
        const long long blocks = std::min<long long>((p.nnz + 255) / 256, 65536);
        for (long long z0 = 0; z0 < p.batch; z0 += 65535) {  // batch entries on grid y
            const long long nz = std::min<long long>(65535, p.batch - z0);
            hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks, (unsigned)nz), dim3(256),
                               0, stream, p.out + z0 * p.stride_out, (long long)p.nnz,
                               p.stride_out);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    case SddmmPlan::kCols:
        switch (plan.dtype) {
        case Dtype::f16: return launch_cols<_Float16>(plan.buf, p, stream);
        case Dtype::bf16: return launch_cols<bf16>(plan.buf, p, stream);
        default: return launch_cols<float>(plan.buf, p, stream);
        }
    default:
        break;
    }
    const bool sm = plan.softmax, sp = plan.split;
    switch (plan.dtype) {
    case Dtype::f16:
        return launch_typed<_Float16, 8>(plan.vec, sm, sp, plan.g, plan.nv, p, stream);
    case Dtype::bf16: return launch_typed<bf16, 8>(plan.vec, sm, sp, plan.g, plan.nv, p, stream);
    default: return launch_typed<float, 4>(plan.vec, sm, sp, plan.g, plan.nv, p, stream);
    }
}

hipError_t launch_sddmm(const SddmmArgs &a, hipStream_t stream)
{
    SddmmPlan plan;
    const hipError_t e = plan_sddmm(a, &plan);
    return e != hipSuccess ? e : run_sddmm(plan, stream);
}

}  // namespace spk
