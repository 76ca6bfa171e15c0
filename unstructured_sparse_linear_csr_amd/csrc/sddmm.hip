// CSR SDDMM for gfx950: out[p] = alpha * dot(X[i], Y[col_indices[p]]) for each
// entry p of row i ("Sparse GPU Kernels for Deep Learning", summary card,
// "Summary" and "Interesting ideas" I3: the specialised form with no scaling
// by mask values and the second operand transposed, so that X and Y are both
// read by contiguous rows).
//
// Mapping.  One wavefront (= one workgroup) per mask row.  The wave is split
// into 64/kG groups of kG lanes; a group computes one entry's dot product at a
// time, each lane covering kNv vectors of kVec elements of the d-long rows
// (interleaved so that the group's loads of one Y row are contiguous).  The X
// row is loaded once into registers and reused for every entry of the row.
//
// Reduction.  The kG lane partials of an entry are summed with DPP moves inside
// a 16-lane row (quad swaps, half-row mirror, row mirror), fused into
// v_add_f32_dpp; no LDS round trip.  Entries are dealt to groups round-robin
// in windows of 64: at step s group g takes entry s*(64/kG) + g, and lane
// (g, s) keeps that entry's sum, so after a window every lane holds one result
// and the wave writes 64 consecutive outputs with one store.
//
// Staging.  The window's 64 column indices are read with one coalesced load and
// kept in LDS as Y-row offsets (bytes when k*d < 2^30).
//
// Summation order: each lane sums its elements in order with FMA, then the
// DPP tree adds the kG lane partials; deterministic run to run.
#include <algorithm>

#include "sp_device.h"
#include "sp_launch.h"

namespace spk {

namespace {

struct SddmmParams {
    int m, d, nnz;
    const int *row_indices;
    const int *row_offsets;
    const int *col_indices;
    const float *x;
    const float *y;
    float alpha;
    float *out;
    long long stride_x, stride_y, stride_out;
};

template <int kVec> struct DVec;
template <> struct DVec<4> {
    using T = float4;
    static __device__ __forceinline__ T zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
    static __device__ __forceinline__ float dot(const T &a, const T &b, float acc)
    {
        acc = fmaf(a.x, b.x, acc);
        acc = fmaf(a.y, b.y, acc);
        acc = fmaf(a.z, b.z, acc);
        return fmaf(a.w, b.w, acc);
    }
};
template <> struct DVec<1> {
    using T = float;
    static __device__ __forceinline__ T zero() { return 0.f; }
    static __device__ __forceinline__ float dot(const T &a, const T &b, float acc)
    {
        return fmaf(a, b, acc);
    }
};

// kNv > 0: the lane's kNv vectors of the X row live in registers.
// kNv == 0: any d; X and Y are both read from memory in a loop over d.
template <int kG, int kNv, int kVec, bool kOff32>
__global__ __launch_bounds__(kWave) void sddmm_kernel(SddmmParams p)
{
    using V = DVec<kVec>;
    using VecT = typename V::T;
    constexpr int kNg = kWave / kG;                          // entries per step
    constexpr int kU = kNv == 0 ? 1 : (kNv >= 8 ? 1 : 8 / kNv);  // steps in flight
    constexpr int kXv = kNv == 0 ? 1 : kNv;
    __shared__ int s_off[kWave];

    const int lane = threadIdx.x;
    const int g = lane / kG;
    const int gl = lane - g * kG;
    const int slot = blockIdx.x;
    const long long z = blockIdx.y;
    const int row = p.row_indices ? p.row_indices[slot] : slot;
    const int p0 = p.row_offsets[row];
    const int p1 = p.row_offsets[row + 1];
    if (p0 >= p1) return;  // one row per wave: uniform, before any barrier

    const float *__restrict__ xr_ptr = p.x + z * p.stride_x + (size_t)row * (size_t)p.d;
    const float *__restrict__ yz = p.y + z * p.stride_y;
    float *__restrict__ oz = p.out + z * p.stride_out;

    auto offset_of = [&](int col) -> int {
        if constexpr (kOff32)
            return (int)((unsigned)col * (unsigned)p.d * 4u);
        else
            return col;
    };
    auto load_y = [&](int off, int e) -> VecT {
        if constexpr (kOff32)
            return *reinterpret_cast<const VecT *>(
                reinterpret_cast<const char *>(yz) + ((unsigned)off + (unsigned)e * 4u));
        else
            return *reinterpret_cast<const VecT *>(yz + (size_t)off * (size_t)p.d + e);
    };

    VecT xr[kXv];
    if constexpr (kNv > 0) {
#pragma unroll
        for (int v = 0; v < kNv; ++v) {
            const int e = (v * kG + gl) * kVec;
            xr[v] = e < p.d ? *reinterpret_cast<const VecT *>(xr_ptr + e) : V::zero();
        }
    }

    for (int base = p0; base < p1; base += kWave) {
        const int cnt = min(kWave, p1 - base);
        s_off[lane] = lane < cnt ? offset_of(p.col_indices[base + lane]) : 0;
        __syncthreads();
        const int steps = (cnt + kNg - 1) / kNg;
        float res = 0.f;
        for (int s0 = 0; s0 < steps; s0 += kU) {
            float part[kU];
            if constexpr (kNv > 0) {
                VecT yv[kU][kNv];
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    const int j = (s0 + u) * kNg + g;
                    const bool valid = (s0 + u < steps) && (j < cnt);
                    const int off = s_off[valid ? j : 0];
#pragma unroll
                    for (int v = 0; v < kNv; ++v) {
                        const int e = (v * kG + gl) * kVec;
                        yv[u][v] = (valid && e < p.d) ? load_y(off, e) : V::zero();
                    }
                }
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    float acc = 0.f;
#pragma unroll
                    for (int v = 0; v < kNv; ++v) acc = V::dot(xr[v], yv[u][v], acc);
                    part[u] = acc;
                }
            } else {
                const int j = s0 * kNg + g;
                const bool valid = j < cnt;
                const int off = s_off[valid ? j : 0];
                float acc = 0.f;
                if (valid) {
                    for (int e = gl * kVec; e < p.d; e += kG * kVec)
                        acc = V::dot(*reinterpret_cast<const VecT *>(xr_ptr + e),
                                     load_y(off, e), acc);
                }
                part[0] = acc;
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const float sum = group_sum<kG>(part[u]);
                if (gl == s0 + u) res = sum;
            }
        }
        const int jo = gl * kNg + g;  // the entry whose sum this lane kept
        if (jo < cnt) oz[base + jo] = p.alpha * res;
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *dst, long long count,
                                                        long long stride)
{
    float *dz = dst + (long long)blockIdx.y * stride;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < count;
         i += (long long)gridDim.x * 256)
        dz[i] = 0.f;
}

template <int kG, int kNv, int kVec>
hipError_t launch_t(const SddmmParams &p, int batch, bool off32, hipStream_t s)
{
    dim3 grid((unsigned)p.m, (unsigned)batch);
    if (off32)
        hipLaunchKernelGGL((sddmm_kernel<kG, kNv, kVec, true>), grid, dim3(kWave), 0, s, p);
    else
        hipLaunchKernelGGL((sddmm_kernel<kG, kNv, kVec, false>), grid, dim3(kWave), 0, s, p);
    return hipGetLastError();
}

template <int kG, int kVec>
hipError_t launch_nv(int nv, const SddmmParams &p, int batch, bool off32, hipStream_t s)
{
    switch (nv) {
    case 1: return launch_t<kG, 1, kVec>(p, batch, off32, s);
    case 2: return launch_t<kG, 2, kVec>(p, batch, off32, s);
    case 4: return launch_t<kG, 4, kVec>(p, batch, off32, s);
    case 8: return launch_t<kG, 8, kVec>(p, batch, off32, s);
    default: return launch_t<kG, 0, kVec>(p, batch, off32, s);
    }
}

template <int kVec>
hipError_t launch_g(int g, int nv, const SddmmParams &p, int batch, bool off32,
                    hipStream_t s)
{
    switch (g) {
    case 4: return launch_nv<4, kVec>(nv, p, batch, off32, s);
    case 8: return launch_nv<8, kVec>(nv, p, batch, off32, s);
    default: return launch_nv<16, kVec>(nv, p, batch, off32, s);
    }
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
// kNv == 0 loop.  d == 0 zero-fills every batch's outputs.
hipError_t launch_sddmm(const SddmmArgs &a, hipStream_t stream)
{
    if (a.m == 0 || a.nnz == 0) return hipSuccess;
    if (a.batch > 65535) return hipErrorInvalidConfiguration;
    if (a.d == 0) {
        const long long blocks = std::min<long long>((a.nnz + 255) / 256, 65536);
        hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks, (unsigned)a.batch),
                           dim3(256), 0, stream, a.out, (long long)a.nnz, a.stride_out);
        return hipGetLastError();
    }
    const bool vec = (a.d % 4 == 0) && aligned16(a.x) && aligned16(a.y) &&
                     (a.stride_x % 4 == 0) && (a.stride_y % 4 == 0);
    const bool off32 = (long long)a.k * (long long)a.d < (1LL << 30);
    const int kvec = vec ? 4 : 1;
    const int dv = (a.d + kvec - 1) / kvec;
    const int g = dv <= 4 ? 4 : dv <= 8 ? 8 : 16;
    const int need = (dv + g - 1) / g;
    const int nv = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : 0;

    SddmmParams p;
    p.m = a.m;
    p.d = a.d;
    p.nnz = a.nnz;
    p.row_indices = a.row_indices;
    p.row_offsets = a.row_offsets;
    p.col_indices = a.col_indices;
    p.x = a.x;
    p.y = a.y;
    p.alpha = a.alpha;
    p.out = a.out;
    p.stride_x = a.stride_x;
    p.stride_y = a.stride_y;
    p.stride_out = a.stride_out;
    return vec ? launch_g<4>(g, nv, p, a.batch, off32, stream)
               : launch_g<1>(g, nv, p, a.batch, off32, stream);
}

}  // namespace spk
