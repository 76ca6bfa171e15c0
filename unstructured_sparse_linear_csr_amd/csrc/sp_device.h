// Device-side helpers shared by the gfx950 kernels of this library.
//
// Every kernel here is written for wave64 (CDNA): one wavefront is one
// workgroup unless stated otherwise, so a workgroup barrier is a wave barrier
// and orders the wave's LDS staging.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spk {

constexpr int kWave = 64;

// DPP lane-permute controls (GCN/CDNA DPP encodings).
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kDppRowMirror = 0x140;     // lane i <- lane 15-i within 16

template <int kCtrl>
__device__ __forceinline__ float dpp_read(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(
        0, __float_as_int(v), kCtrl, 0xF, 0xF, true));
}

// Sum over aligned groups of kLanes consecutive lanes (kLanes in 1, 2, 4, 8,
// 16); every lane of a group receives the group's sum.  Uses only DPP moves
// inside a 16-lane row, fused by the compiler into v_add_f32_dpp.  All lanes
// of each group must be active.
template <int kLanes>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert(kLanes == 1 || kLanes == 2 || kLanes == 4 || kLanes == 8 ||
                      kLanes == 16, "group must fit a DPP row");
    if constexpr (kLanes >= 2) v += dpp_read<kDppQuadXor1>(v);
    if constexpr (kLanes >= 4) v += dpp_read<kDppQuadXor2>(v);
    if constexpr (kLanes >= 8) v += dpp_read<kDppRowHalfMirror>(v);
    if constexpr (kLanes >= 16) v += dpp_read<kDppRowMirror>(v);
    return v;
}

// Wave-wide inclusive prefix sum of an int (Hillis-Steele over 64 lanes).
__device__ __forceinline__ int wave_inclusive_sum(int v, int lane)
{
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int up = __shfl_up(v, off, kWave);
        if (lane >= off) v += up;
    }
    return v;
}

// Bit mask of the lanes below `lane` (for ballot-based compaction).
__device__ __forceinline__ uint64_t lanes_below(int lane)
{
    return lane == 0 ? 0ull : (~0ull >> (kWave - lane));
}

}  // namespace spk
