// Row softmax over the entries of a CSR matrix: for each row, p = exp(s - max)
// / sum exp(s - max) over that row's entries.  This is the step between SDDMM
// and SpMM in sparse attention ("Sparse GPU Kernels for Deep Learning",
// summary card, "Interesting ideas" I3: the SDDMM form that sparse attention
// needs); with it the attention pair runs entirely on the device.
//
// Mapping.  kSmLanes = 16 lanes per (batch entry, row), four rows per
// wavefront, so a wave's dependent chain (offsets, scores, max, sum, write)
// serves four rows at once.  Rows of up to kHeld entries keep their scores in
// registers (one read, one write); longer rows are read three times (max,
// sum, scale).  Max and sum are reductions over the row's 16 lanes by DPP
// inside one 16-lane row of the wave (no LDS); each lane first combines its
// own entries in order, so results are deterministic and do not depend on
// which wave or lane group a row lands in.  Arithmetic is fp32 with the
// accurate expf.  in == out is allowed: each row is read completely before
// it is written.
#include <algorithm>

#include "sp_device.h"
#include "sp_launch.h"

namespace spk {

namespace {

constexpr int kSmLanes = 16;                    // lanes per row (one DPP row)
constexpr int kSmRows = kWave / kSmLanes;       // rows per wave
constexpr int kHeldPerLane = 8;
constexpr int kHeld = kHeldPerLane * kSmLanes;  // entries held in registers

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
    const long long groups = ((long long)p.m + kSmRows - 1) / kSmRows;
    const long long w = xcd_work_index(p.batch, groups);
    if (w < 0) return;
    const long long z = w / groups;
    const int lane = threadIdx.x;
    const int gl = lane % kSmLanes;  // lane within the row's group
    const long long slot_ll = (w - z * groups) * kSmRows + lane / kSmLanes;
    // Groups leave independently: every cross-lane step below stays inside
    // one group's 16-lane DPP row.
    if (slot_ll >= p.m) return;
    const int slot = (int)slot_ll;
    const int row = p.row_indices ? p.row_indices[slot] : slot;
    const int p0 = p.row_offsets[row];
    const int p1 = p.row_offsets[row + 1];
    const int len = p1 - p0;
    if (len <= 0) return;
    const float *in = p.in + z * p.stride_in + p0;
    float *out = p.out + z * p.stride_out + p0;

    if (len <= kHeld) {
        float sv[kHeldPerLane];
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < kHeldPerLane; ++t) {
            const int j = t * kSmLanes + gl;
            sv[t] = j < len ? in[j] : -INFINITY;
            mx = fmaxf(mx, sv[t]);
        }
        mx = group_reduce<kSmLanes>(mx, OpMax{});
        float sum = 0.f;
#pragma unroll
        for (int t = 0; t < kHeldPerLane; ++t) {
            if (t * kSmLanes < len) {  // uniform over the group
                const int j = t * kSmLanes + gl;
                sv[t] = j < len ? expf(sv[t] - mx) : 0.f;
                sum += sv[t];
            }
        }
        sum = group_reduce<kSmLanes>(sum, OpAdd{});
        const float inv = 1.f / sum;
#pragma unroll
        for (int t = 0; t < kHeldPerLane; ++t) {
            const int j = t * kSmLanes + gl;
            if (j < len) out[j] = sv[t] * inv;
        }
    } else {
        float mx = -INFINITY;
        for (int j = gl; j < len; j += kSmLanes) mx = fmaxf(mx, in[j]);
        mx = group_reduce<kSmLanes>(mx, OpMax{});
        float sum = 0.f;
        for (int j = gl; j < len; j += kSmLanes) sum += expf(in[j] - mx);
        sum = group_reduce<kSmLanes>(sum, OpAdd{});
        const float inv = 1.f / sum;
        // reads of entry j precede its write within the same lane
        for (int j = gl; j < len; j += kSmLanes) out[j] = expf(in[j] - mx) * inv;
    }
}

}  // namespace

hipError_t launch_row_softmax(int m, const int *row_indices, const int *row_offsets,
                              const float *in, float *out, int batch, long long stride_in,
                              long long stride_out, hipStream_t stream)
{
    if (m == 0 || batch == 0) return hipSuccess;
    const long long groups = ((long long)m + kSmRows - 1) / kSmRows;
    if (xcd_grid(batch, groups) > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    SoftmaxParams p;
    p.m = m;
    p.batch = batch;
    p.row_indices = row_indices;
    p.row_offsets = row_offsets;
    p.in = in;
    p.out = out;
    p.stride_in = stride_in;
    p.stride_out = stride_out;
    hipLaunchKernelGGL(row_softmax_kernel, dim3((unsigned)xcd_grid(batch, groups)), dim3(kWave),
                       0, stream, p);
    return hipGetLastError();
}

}  // namespace spk
