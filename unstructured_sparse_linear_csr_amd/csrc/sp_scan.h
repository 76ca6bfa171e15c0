// One workgroup's exclusive prefix sum of int row lengths into CSR row
// offsets, shared by the CSR-build kernels.
#pragma once

#include "sp_device.h"

namespace spk {

// out[0] = 0 and out[i+1] = in[0] + ... + in[i] for i < m, computed by one
// workgroup of kThreads threads walking the array tile by tile with a running
// carry.  Element j * kThreads + tid of a tile belongs to thread tid, so every
// load and store instruction is coalesced; the tile's kPer columns are
// scanned across the threads (a DPP scan per wave, the waves' totals through
// LDS) and the next tile's loads are in flight meanwhile.  Each thread reads
// its own elements before the barrier and writes the same positions after it,
// and a tile's reads never touch the positions the tile before it writes, so
// `in` may alias `out + 1` (the in-place form used after counting).
template <int kThreads>
__device__ void exclusive_scan_block(int m, const int *in, int *out)
{
    // 2,048 elements per tile up to 1,024 threads: each thread then reads
    // kPer * kWaves = 32 wave totals per tile
    constexpr int kPer = kThreads >= 1024 ? 2 : kThreads >= 512 ? 4 : 8;
    constexpr int kTile = kThreads * kPer;
    constexpr int kWaves = kThreads / kWave;
    __shared__ int wave_total[kPer][kWaves];
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    if (tid == 0) out[0] = 0;
    // 64-bit positions: m may come within a tile of 2^31 - 1
    auto load = [&](long long base, int (&v)[kPer]) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const long long i = base + j * kThreads + tid;
            v[j] = i < m ? in[i] : 0;
        }
    };
    int v[kPer];
    load(0, v);
    int carry = 0;
    for (long long base = 0; base < m; base += kTile) {
        int nv[kPer];
        load(base + kTile, nv);
        int incl[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            incl[j] = wave_inclusive_sum(v[j]);
            if (lane == kWave - 1) wave_total[j][wave] = incl[j];
        }
        __syncthreads();
        // before[j]: everything ahead of element (j, tid) in the tile
        int run = carry;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            int ahead = 0, col = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const int t = wave_total[j][w];
                ahead += (w < wave) ? t : 0;
                col += t;
            }
            const long long i = base + j * kThreads + tid;
            if (i < m) out[i + 1] = run + ahead + incl[j];
            run += col;
        }
        carry = run;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kPer; ++j) v[j] = nv[j];
    }
}

}  // namespace spk
