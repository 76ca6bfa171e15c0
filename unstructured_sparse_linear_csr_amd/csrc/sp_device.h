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

// 32-bit values travel through the lane-permute builtins as their bits.
template <class T> __device__ __forceinline__ unsigned to_bits(T v)
{
    static_assert(sizeof(T) == 4, "32-bit lane values");
    return __builtin_bit_cast(unsigned, v);
}
template <class T> __device__ __forceinline__ T from_bits(unsigned u)
{
    return __builtin_bit_cast(T, u);
}

template <int kCtrl, class T>
__device__ __forceinline__ T dpp_read(T v)
{
    return from_bits<T>((unsigned)__builtin_amdgcn_update_dpp(
        0, (int)to_bits(v), kCtrl, 0xF, 0xF, true));
}

// gfx950's lane swaps: v_permlane16_swap exchanges the odd 16-lane rows of one
// copy of v with the even rows of another, v_permlane32_swap the upper wave
// half of one with the lower half of the other.  Each lane then holds its own
// value and its partner's as (lower, upper) in the same order in both lanes,
// so op(lower, upper) is the same in both.
template <bool kHalves, class T, class Op>
__device__ __forceinline__ T swap_combine(T v, Op op)
{
    const unsigned u = to_bits(v);
    if constexpr (kHalves) {
        const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return op(from_bits<T>(p[0]), from_bits<T>(p[1]));
    } else {
        const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        return op(from_bits<T>(p[0]), from_bits<T>(p[1]));
    }
}

struct OpAdd {
    template <class T> __device__ T operator()(T a, T b) const { return a + b; }
};
struct OpMax {
    __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
    __device__ int operator()(int a, int b) const { return max(a, b); }
};

// Reduction over aligned groups of kLanes consecutive lanes (1 ... 64); every
// lane of a group receives the same result.  A butterfly whose every step
// joins two lanes holding equal values (quad swaps, then the 8- and 16-lane
// mirrors by DPP, fused by the compiler into v_add_f32_dpp and the like; then
// the row and half-wave swaps), with a commutative op: every lane computes
// the same result in a fixed order, so results are deterministic.  No LDS
// traffic.  Every lane of each group must be active; lanes of other groups
// need not be (every source lane lies in the reading lane's own group).
template <int kLanes, class T, class Op>
__device__ __forceinline__ T group_reduce(T v, Op op)
{
    static_assert(kLanes == 1 || kLanes == 2 || kLanes == 4 || kLanes == 8 || kLanes == 16 ||
                      kLanes == 32 || kLanes == 64, "group of 1 ... 64 lanes");
    if constexpr (kLanes >= 2) v = op(v, dpp_read<kDppQuadXor1>(v));
    if constexpr (kLanes >= 4) v = op(v, dpp_read<kDppQuadXor2>(v));
    if constexpr (kLanes >= 8) v = op(v, dpp_read<kDppRowHalfMirror>(v));
    if constexpr (kLanes >= 16) v = op(v, dpp_read<kDppRowMirror>(v));
    if constexpr (kLanes >= 32) v = swap_combine<false>(v, op);
    if constexpr (kLanes >= 64) v = swap_combine<true>(v, op);
    return v;
}

// Sum over aligned groups of kLanes consecutive lanes (kLanes in 1, 2, 4, 8,
// 16: DPP moves inside a 16-lane row only).
template <int kLanes>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert(kLanes <= 16, "group must fit a DPP row");
    return group_reduce<kLanes>(v, OpAdd{});
}

// Reduction over the lanes of the wave congruent to this lane modulo kStride
// (1 ... 64); every lane receives its class's result (for a sum, lanes of a
// class may differ in rounding: each adds in its own order).  Rotations
// inside each 16-lane row (DPP row_ror) combine a row's lanes of the class,
// then the row and half-wave swaps.  Fixed order, deterministic, no LDS
// traffic.  All 64 lanes must be active.
constexpr int kDppRowRor1 = 0x121;  // lane i <- lane (i - 1) mod 16 within a row
constexpr int kDppRowRor2 = 0x122;
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

template <int kStride, class T, class Op>
__device__ __forceinline__ T strided_wave_reduce(T v, Op op)
{
    static_assert(kStride == 1 || kStride == 2 || kStride == 4 || kStride == 8 ||
                      kStride == 16 || kStride == 32 || kStride == 64,
                  "stride of 1 ... 64 lanes");
    if constexpr (kStride <= 1) v = op(v, dpp_read<kDppRowRor1>(v));
    if constexpr (kStride <= 2) v = op(v, dpp_read<kDppRowRor2>(v));
    if constexpr (kStride <= 4) v = op(v, dpp_read<kDppRowRor4>(v));
    if constexpr (kStride <= 8) v = op(v, dpp_read<kDppRowRor8>(v));
    if constexpr (kStride <= 16) v = swap_combine<false>(v, op);
    if constexpr (kStride <= 32) v = swap_combine<true>(v, op);
    return v;
}

template <int kStride>
__device__ __forceinline__ float strided_wave_sum(float v)
{
    return strided_wave_reduce<kStride>(v, OpAdd{});
}

// Keeps the compiler from moving any instruction across this point (memory
// operations at the IR level, everything in the machine scheduler).  Used
// after a batch of prefetch gathers so that they stay issued ahead of the
// arithmetic on the previous batch: otherwise the scheduler interleaves the
// two to shorten register lifetimes, the two buffers share registers, and
// every batch waits for all outstanding gathers.
// A value of T (4, 8 or 16 bytes) read from 32-bit LDS address `addr`: the
// address stays an LDS one, so the read is a single ds_read with no generic-
// to-LDS conversion, and the address arithmetic before it can fold the base.
template <class T> __device__ __forceinline__ T lds_read(unsigned addr)
{
    static_assert(sizeof(T) % 4 == 0 && sizeof(T) <= 16, "4 to 16 bytes");
    using W = unsigned __attribute__((ext_vector_type(sizeof(T) / 4)));
    const W w = *(const __attribute__((address_space(3))) W *)(size_t)addr;
    T t;
    __builtin_memcpy(&t, &w, sizeof(T));
    return t;
}

// The 32-bit LDS address of a pointer into LDS.
template <class T> __device__ __forceinline__ unsigned lds_address(const T *p)
{
    return (unsigned)(size_t)(const __attribute__((address_space(3))) T *)p;
}

__device__ __forceinline__ void keep_issued_above()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Wave-wide maximum and sum of a float, the same value in every lane.
__device__ __forceinline__ float wave_max(float v) { return group_reduce<kWave>(v, OpMax{}); }
__device__ __forceinline__ float wave_sum(float v) { return group_reduce<kWave>(v, OpAdd{}); }

// Wave-wide inclusive prefix sum of an int: Hillis-Steele inside each 16-lane
// row by DPP row shifts (lanes shifted in from outside the row read 0), then
// each row adds the running total of the rows before it, broadcast from lane
// 15 (rows 1 and 3) and lane 31 (rows 2 and 3).  No LDS traffic.  All 64
// lanes must be active.
constexpr int kDppRowShr1 = 0x111;      // lane i <- lane i-1 within a row (0 at the row start)
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;   // lane 15 of each row to the next row
constexpr int kDppRowBcast31 = 0x143;   // lane 31 to rows 2 and 3

__device__ __forceinline__ int wave_inclusive_sum(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr1, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr2, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr4, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr8, 0xF, 0xF, true);
    // rows outside the row mask keep the old value, 0
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast15, 0xA, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast31, 0xC, 0xF, false);
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
