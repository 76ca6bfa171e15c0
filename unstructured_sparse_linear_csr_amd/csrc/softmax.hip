// Row softmax over the entries of a CSR matrix: for each row, p = exp(s - max)
// / sum exp(s - max) over that row's entries.  This is the step between SDDMM
// and SpMM in sparse attention ("Sparse GPU Kernels for Deep Learning",
// summary card, "Interesting ideas" I3: the SDDMM form that sparse attention
// needs); with it the attention pair runs entirely on the device.
//
// Mapping.  One wavefront per (batch entry, row).  Rows of up to kHeld entries
// keep their scores in registers (one read, one write); longer rows are read
// three times (max, sum, scale).  Max and sum are wave-wide reductions; each
// lane sums its own entries in order first, so results are deterministic.
// Arithmetic is fp32 with the accurate expf.  in == out is allowed: each wave
// reads its row completely before writing it.
#include <algorithm>

#include "sp_device.h"
#include "sp_launch.h"

namespace spk {

namespace {

constexpr int kHeldPerLane = 4;
constexpr int kHeld = kHeldPerLane * kWave;

struct SoftmaxParams {
    int m, batch;
    const int *row_indices;
    const int *row_offsets;
    const float *in;
    float *out;
    long long stride_in, stride_out;
};

__global__ __launch_bounds__(kWave) void row_softmax_kernel(SoftmaxParams p)
{
    const long long w = xcd_work_index(p.batch, p.m);
    if (w < 0) return;
    const long long z = w / p.m;
    const int slot = (int)(w - z * p.m);
    const int row = p.row_indices ? p.row_indices[slot] : slot;
    const int p0 = p.row_offsets[row];
    const int p1 = p.row_offsets[row + 1];
    const int len = p1 - p0;
    if (len <= 0) return;
    const float *in = p.in + z * p.stride_in + p0;
    float *out = p.out + z * p.stride_out + p0;
    const int lane = threadIdx.x;

    if (len <= kHeld) {
        float sv[kHeldPerLane];
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < kHeldPerLane; ++t) {
            const int j = t * kWave + lane;
            sv[t] = j < len ? in[j] : -INFINITY;
            mx = fmaxf(mx, sv[t]);
        }
        mx = wave_max(mx);
        float sum = 0.f;
#pragma unroll
        for (int t = 0; t < kHeldPerLane; ++t) {
            const int j = t * kWave + lane;
            sv[t] = j < len ? expf(sv[t] - mx) : 0.f;
            sum += sv[t];
        }
        sum = wave_sum(sum);
        const float inv = 1.f / sum;
#pragma unroll
        for (int t = 0; t < kHeldPerLane; ++t) {
            const int j = t * kWave + lane;
            if (j < len) out[j] = sv[t] * inv;
        }
    } else {
        float mx = -INFINITY;
        for (int j = lane; j < len; j += kWave) mx = fmaxf(mx, in[j]);
        mx = wave_max(mx);
        float sum = 0.f;
        for (int j = lane; j < len; j += kWave) sum += expf(in[j] - mx);
        sum = wave_sum(sum);
        const float inv = 1.f / sum;
        // reads of entry j precede its write within the same lane
        for (int j = lane; j < len; j += kWave) out[j] = expf(in[j] - mx) * inv;
    }
}

}  // namespace

hipError_t launch_row_softmax(int m, const int *row_indices, const int *row_offsets,
                              const float *in, float *out, int batch, long long stride_in,
                              long long stride_out, hipStream_t stream)
{
    if (m == 0 || batch == 0) return hipSuccess;
    if (xcd_grid(batch, m) > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    SoftmaxParams p;
    p.m = m;
    p.batch = batch;
    p.row_indices = row_indices;
    p.row_offsets = row_offsets;
    p.in = in;
    p.out = out;
    p.stride_in = stride_in;
    p.stride_out = stride_out;
    hipLaunchKernelGGL(row_softmax_kernel, dim3((unsigned)xcd_grid(batch, m)), dim3(kWave), 0,
                       stream, p);
    return hipGetLastError();
}

}  // namespace spk
