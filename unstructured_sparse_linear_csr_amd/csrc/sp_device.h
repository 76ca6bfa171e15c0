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

// Sum over the lanes of the wave congruent to this lane modulo kStride (1, 2,
// 4, 8 or 16); every lane receives its class's sum.  Rotations inside each
// 16-lane row (DPP row_ror, fused into v_add_f32_dpp) sum a row's lanes of
// the class; gfx950's v_permlane16_swap then pairs each row with its
// neighbour, and v_permlane32_swap the two wave halves.  Every lane of a pair
// adds (lower half) + (upper half), so the order is fixed and the results are
// deterministic; no LDS traffic.  All 64 lanes must be active.
constexpr int kDppRowRor1 = 0x121;  // lane i <- lane (i - 1) mod 16 within a row
constexpr int kDppRowRor2 = 0x122;
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

__device__ __forceinline__ float swap_pair_sum(float v, bool halves)
{
    const unsigned u = __float_as_uint(v);
    const auto p = halves ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                          : __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

template <int kStride>
__device__ __forceinline__ float strided_wave_sum(float v)
{
    static_assert(kStride == 1 || kStride == 2 || kStride == 4 || kStride == 8 ||
                      kStride == 16, "stride must divide a DPP row");
    if constexpr (kStride <= 1) v += dpp_read<kDppRowRor1>(v);
    if constexpr (kStride <= 2) v += dpp_read<kDppRowRor2>(v);
    if constexpr (kStride <= 4) v += dpp_read<kDppRowRor4>(v);
    if constexpr (kStride <= 8) v += dpp_read<kDppRowRor8>(v);
    v = swap_pair_sum(v, false);
    return swap_pair_sum(v, true);
}

// Keeps the compiler from moving any instruction across this point (memory
// operations at the IR level, everything in the machine scheduler).  Used
// after a batch of prefetch gathers so that they stay issued ahead of the
// arithmetic on the previous batch: otherwise the scheduler interleaves the
// two to shorten register lifetimes, the two buffers share registers, and
// every batch waits for all outstanding gathers.
__device__ __forceinline__ void keep_issued_above()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Wave-wide maximum and sum of a float, the same value in every lane (a
// butterfly over the 64 lanes: a fixed order, so results are deterministic).
__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) v += __shfl_xor(v, o);
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

// Workgroups of a launch are dealt to the chip's 8 XCDs round-robin, and
// each XCD has its own L2.  A launch whose work splits into `outer` independent
// units (batch entries times column tiles), each of `inner` row blocks, can
// keep each unit's operands (a tile's B slice, a batch entry's dense
// matrices) in one L2 instead of all eight: with outer >= 8, launch slot i is
// mapped so that each XCD takes one contiguous range of the outer-major work
// order.  With fewer outer units the identity order is kept: consecutive
// slots (rows in swizzled order, longest first) then spread over all XCDs,
// which is what load balance needs.  The mapping only affects locality and
// balance, never results.
constexpr int kXcds = 8;
__host__ __device__ inline bool xcd_remap(long long outer) { return outer >= kXcds; }
__host__ __device__ inline long long xcd_grid(long long outer, long long inner)
{
    const long long units = outer * inner;
    return xcd_remap(outer) ? (units + kXcds - 1) / kXcds * kXcds : units;
}
// The work index of workgroup `block` of a launch of xcd_grid(outer, inner)
// workgroups, or -1 for a padding slot.
__device__ __forceinline__ long long xcd_work_index_of(long long block, long long outer,
                                                       long long inner)
{
    const long long units = outer * inner;
    if (!xcd_remap(outer)) return block;
    const long long per = (units + kXcds - 1) / kXcds;
    const long long w = (block % kXcds) * per + block / kXcds;
    return w < units ? w : -1;
}
// The work index of this workgroup, or -1 for a padding slot.
__device__ __forceinline__ long long xcd_work_index(long long outer, long long inner)
{
    return xcd_work_index_of(blockIdx.x, outer, inner);
}

// Bit mask of the lanes below `lane` (for ballot-based compaction).
__device__ __forceinline__ uint64_t lanes_below(int lane)
{
    return lane == 0 ? 0ull : (~0ull >> (kWave - lane));
}

}  // namespace spk
