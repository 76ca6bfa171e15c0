// Measured ceilings for the roofline figures: how fast this GPU streams a
// large array from HBM with plain 16-byte loads, how fast it gathers whole
// rows of an L2-resident matrix at random (the access pattern of the SpMM and
// SDDMM kernels, without their arithmetic), and what an empty launch costs.
// These are measurement aids, not part of the sparse kernels' interface.
#include <hip/hip_runtime.h>

namespace {

constexpr unsigned kOutOfRange = 0x80000000u;  // buffer offset that reads as zero

// Each thread sums kUnroll 16-byte loads per trip of a grid-stride loop over
// n4 vectors, then writes one float (so no load is optimised away).
template <int kUnroll>
__global__ __launch_bounds__(256) void stream_read_kernel(const float4 *__restrict__ a,
                                                          long long n4, float *__restrict__ out)
{
    float s = 0.f;
    const long long stride = (long long)gridDim.x * 256;
    long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < n4; i += kUnroll * stride) {
        float4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = a[i + u * stride];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) s += (v[u].x + v[u].y) + (v[u].z + v[u].w);
    }
    for (; i < n4; i += stride) {
        const float4 v = a[i];
        s += (v.x + v.y) + (v.z + v.w);
    }
    out[(long long)blockIdx.x * 256 + threadIdx.x] = s;
}

// The same over two arrays read side by side: each trip loads kUnroll / 2
// vectors at the same positions of a and of b -- the access pattern of a CSR
// whose column-index and value arrays are streamed together.
template <int kUnroll>
__global__ __launch_bounds__(256) void stream_read2_kernel(const float4 *__restrict__ a,
                                                           const float4 *__restrict__ b,
                                                           long long n4, float *__restrict__ out)
{
    constexpr int kHalf = kUnroll / 2;
    float s = 0.f;
    const long long stride = (long long)gridDim.x * 256;
    long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    for (; i + (kHalf - 1) * stride < n4; i += kHalf * stride) {
        float4 va[kHalf], vb[kHalf];
#pragma unroll
        for (int u = 0; u < kHalf; ++u) {
            va[u] = a[i + u * stride];
            vb[u] = b[i + u * stride];
        }
#pragma unroll
        for (int u = 0; u < kHalf; ++u)
            s += ((va[u].x + va[u].y) + (va[u].z + va[u].w)) +
                 ((vb[u].x + vb[u].y) + (vb[u].z + vb[u].w));
    }
    for (; i < n4; i += stride) {
        const float4 va = a[i], vb = b[i];
        s += ((va.x + va.y) + (va.z + va.w)) + ((vb.x + vb.y) + (vb.z + vb.w));
    }
    out[(long long)blockIdx.x * 256 + threadIdx.x] = s;
}

// One wave per workgroup gathers per_wave rows of 1 KB (64 lanes x 16 bytes)
// of B at the byte offsets offs[wave * per_wave + j], kUnroll rows in flight,
// through a buffer resource as the sparse kernels do.
template <int kUnroll>
__global__ __launch_bounds__(64) void row_gather_kernel(const unsigned *__restrict__ offs,
                                                        int per_wave, const float *b,
                                                        unsigned b_bytes, float *__restrict__ out)
{
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(b), 0, (int)b_bytes, 0x00020000);
    const unsigned *mine = offs + (size_t)blockIdx.x * per_wave;
    const unsigned lane_bytes = threadIdx.x * 16u;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int j = 0; j < per_wave; j += kUnroll) {
        float4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const unsigned off = j + u < per_wave ? mine[j + u] + lane_bytes : kOutOfRange;
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
            v[u] = make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]),
                               __uint_as_float(x[2]), __uint_as_float(x[3]));
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            a0 += v[u].x;
            a1 += v[u].y;
            a2 += v[u].z;
            a3 += v[u].w;
        }
    }
    out[(size_t)blockIdx.x * 64 + threadIdx.x] = (a0 + a1) + (a2 + a3);
}

__global__ void empty_kernel() {}

}  // namespace

extern "C" {

// out: float[blocks * 256].  Returns a hipError_t code.
int sp_probe_stream_read(const void *a, long long bytes, int blocks, float *out, void *stream)
{
    if (a == nullptr || out == nullptr || bytes < 16 || blocks <= 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_read_kernel<8>, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const float4 *>(a),
                       bytes / 16, out);
    return (int)hipGetLastError();
}

// a and b: bytes_each bytes each (whole 16-byte vectors are read);
// out: float[blocks * 256].
int sp_probe_stream_read2(const void *a, const void *b, long long bytes_each, int blocks,
                          float *out, void *stream)
{
    if (a == nullptr || b == nullptr || out == nullptr || bytes_each < 16 || blocks <= 0)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_read2_kernel<8>, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const float4 *>(a),
                       static_cast<const float4 *>(b), bytes_each / 16, out);
    return (int)hipGetLastError();
}

// offs: waves * per_wave byte offsets of 1 KB rows, each + 1024 <= b_bytes
// (the caller's contract); out: float[waves * 64].
int sp_probe_row_gather(const unsigned *offs, int waves, int per_wave, const float *b,
                        unsigned b_bytes, float *out, void *stream)
{
    if (offs == nullptr || b == nullptr || out == nullptr || waves <= 0 || per_wave <= 0 ||
        b_bytes < 1024 || b_bytes > 0x7fffffffu)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(row_gather_kernel<8>, dim3((unsigned)waves), dim3(64), 0,
                       static_cast<hipStream_t>(stream), offs, per_wave, b, b_bytes, out);
    return (int)hipGetLastError();
}

int sp_probe_empty(int blocks, void *stream)
{
    if (blocks <= 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(empty_kernel, dim3((unsigned)blocks), dim3(64), 0,
                       static_cast<hipStream_t>(stream));
    return (int)hipGetLastError();
}

}  // extern "C"
