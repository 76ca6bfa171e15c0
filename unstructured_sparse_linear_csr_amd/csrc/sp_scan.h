// One workgroup's exclusive prefix sum of int row lengths into CSR row
// offsets, shared by the CSR-build kernels.
#pragma once

#include "sp_device.h"

namespace spk {

// out[0] = 0 and out[i+1] = in[0] + ... + in[i] for i < m, computed by one
// workgroup of kThreads threads walking the array tile by tile with a running
// carry.  Each thread reads its own elements before the barrier and writes the
// same positions after it, so `in` may alias `out + 1` (the in-place form used
// after counting).
template <int kThreads>
__device__ void exclusive_scan_block(int m, const int *in, int *out)
{
    constexpr int kPer = 4;
    constexpr int kTile = kThreads * kPer;
    constexpr int kWaves = kThreads / kWave;
    __shared__ int wave_total[kWaves];
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    if (tid == 0) out[0] = 0;
    int carry = 0;
    for (int base = 0; base < m; base += kTile) {
        const int i0 = base + tid * kPer;
        int v[kPer];
#pragma unroll
        for (int t = 0; t < kPer; ++t) v[t] = (i0 + t < m) ? in[i0 + t] : 0;
#pragma unroll
        for (int t = 1; t < kPer; ++t) v[t] += v[t - 1];
        const int mine = v[kPer - 1];
        const int incl = wave_inclusive_sum(mine, lane);
        if (lane == kWave - 1) wave_total[wave] = incl;
        __syncthreads();
        int before = 0, tile_total = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int t = wave_total[w];
            before += (w < wave) ? t : 0;
            tile_total += t;
        }
        const int excl = carry + before + incl - mine;
#pragma unroll
        for (int t = 0; t < kPer; ++t)
            if (i0 + t < m) out[i0 + t + 1] = excl + v[t];
        carry += tile_total;
        __syncthreads();
    }
}

}  // namespace spk
