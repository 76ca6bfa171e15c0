// The wide-B CSR SpMM body (one wavefront per output strip), shared by the
// SpMM launch and the launch that runs an SpMM and an SDDMM together.
//
// CSR SpMM for gfx950: C = A * B with A sparse (CSR) and B, C dense row-major
// ("Sparse GPU Kernels for Deep Learning", summary card, "Summary": SpMM on
// plain CSR using 1-D tiling, vector memory access on misaligned sparse data,
// and load balancing decoupled from the parallelisation).
//
// Mapping.  One wavefront (= one workgroup) owns a 1-D output strip: kRpw
// consecutive work slots (rows in row_indices order) by one column tile of
// kLpr * kVec columns.  Each slot is served by a group of kLpr lanes; a lane
// owns kVec adjacent output columns and keeps their sums in registers, so C is
// written exactly once, with no atomics and no split over k.
//
// Staging.  A group copies its row's (B-row offset, value) pairs into LDS one
// window of kEpl * kLpr entries at a time.  On the vector path each lane reads
// 16-byte segments of col_indices and values with dwordx4 loads, starting from
// the row's first entry rounded down to a multiple of 4; slots before the
// row's start (the misaligned prefix) or after its end become padding.  A
// segment that holds no entry of the row is not loaded.
//
// Gathers.  B is read through a buffer resource: a padding slot carries an
// offset beyond the resource's range, for which the hardware returns zeros
// without touching memory, and its value is 0.  Every gather is therefore
// unconditional, batches of kU gathers are issued back to back, and the next
// batch is in flight while the current one is summed (two register buffers).
// Loop bounds are wave-uniform: a group whose row is done reads padding, so
// multi-row waves never diverge.  B larger than 2 GiB takes the same kernel
// with 64-bit addresses and per-slot predicates instead.
//
// Order of summation: entries of a row in CSR order, sequentially, with fused
// multiply-add (a padding slot adds 0 * 0) -- deterministic, and identical
// whatever row order is used.
#pragma once

#include "sp_device.h"
#include "sp_types.h"

namespace spk {
namespace spmm_detail {

#ifndef SP_SPMM_UNROLL
#define SP_SPMM_UNROLL 4
#endif
#ifndef SP_SPMM_ENTRIES_PER_LANE
#define SP_SPMM_ENTRIES_PER_LANE 4
#endif
constexpr int kU = SP_SPMM_UNROLL;                // gathers per batch
constexpr int kEpl = SP_SPMM_ENTRIES_PER_LANE;    // staged entries per lane per window
constexpr unsigned kOutOfRange = 0x80000000u;     // buffer offset that reads as zero
static_assert(kEpl % 4 == 0, "segments of 4 entries");

struct SpmmParams {
    int m, n, nnz, row_blocks, tiles, batch;
    unsigned b_bytes;    // bytes of one B operand (buffer path)
    unsigned csr_bytes;  // bytes of col_indices (= of one values array), narrow kernel
    unsigned c_bytes;    // LDS kernel: bytes of C (stored through a buffer resource)
    // LDS kernel: B's columns in slices of lds_slice_n, one slice per
    // workgroup (lds_slices = 1: all of B); k = rows of B
    int k, lds_slices, lds_slice_n;
    const int *row_indices;
    const int *row_offsets;
    const int *col_indices;
    const void *values;  // element type of the kernel instance (fp32 elsewhere)
    const void *b;
    float *c;
    long long stride_values, stride_b, stride_c;
};

// kBuf: B < 2 GiB, gathers through a buffer resource with byte offsets.
// Otherwise: 64-bit addressing, staged offsets are columns, padding has value
// 0 and column -1 and is skipped by a predicate.  E is the element type of
// the values and of B (fp32, fp16 or bf16); values are widened to fp32 when
// staged and B elements when gathered, so all arithmetic is fp32.
// Staging barrier between windows: the workgroup's when a workgroup is one
// wave, or only the wave's own (LDS operations of a wave complete in program
// order, so a compiler barrier suffices) when several waves of a workgroup
// run different numbers of windows over private staging regions.
template <bool kWaveSync>
__device__ __forceinline__ void window_sync()
{
    if constexpr (kWaveSync) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
        __syncthreads();
    }
}

// acc += sum over entries q in [p0, p1) of value(q) * B[col(q)][col0 ...],
// for this lane's kVec columns starting at col0 (col_ok: the lane owns
// columns), in entry order, through the staging region g_off / g_val of the
// lane's group (kLpr lanes).  p0 and p1 may delimit any part of a row.
template <typename E, int kLpr, int kVec, bool kVecCsr, bool kBuf, bool kWaveSync>
__device__ __forceinline__ void wide_accumulate(const SpmmParams &p, const E *__restrict__ vals,
                                                const E *__restrict__ bz, int p0, int p1,
                                                int gl, int col0, bool col_ok, int *g_off,
                                                float *g_val, float *acc)
{
    using V = GVec<E, kVec>;
    using VecT = typename V::T;
    constexpr unsigned kEb = Elem<E>::kBytes;
    constexpr int kChunk = kEpl * kLpr;      // entries per row per window
    constexpr int kPad = kBuf ? (int)kOutOfRange : -1;
    // Lanes past the last column read only out-of-range (zero) data.
    const unsigned lane_bytes = col_ok ? (unsigned)col0 * kEb : kOutOfRange;
    for (int j = gl; j < kU; j += kLpr) {
        g_off[kChunk + j] = kPad;
        g_val[kChunk + j] = 0.f;
    }

    __amdgpu_buffer_rsrc_t rsrc;
    if constexpr (kBuf)
        rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<E *>(bz), 0, p.b_bytes,
                                                 0x00020000);

    auto offset_of = [&](int idx, int col) -> int {
        const bool in = idx >= p0 && idx < p1;
        if constexpr (kBuf)
            return in ? (int)((unsigned)col * (unsigned)p.n * kEb) : kPad;
        else
            return in ? col : kPad;
    };
    auto value_of = [&](int idx, float v) -> float {
        return (idx >= p0 && idx < p1) ? v : 0.f;
    };
    auto gather = [&](int off) -> VecT {
        if constexpr (kBuf) {
            return V::buf_load(rsrc, (unsigned)off + lane_bytes);
        } else {
            if (off < 0 || !col_ok) return V::zero();
            return V::load(bz + (size_t)off * (size_t)p.n + col0);
        }
    };
    // kU staged entries starting at slot j (a multiple of 4): 16-byte
    // broadcast reads of both arrays.
    auto read_batch = [&](int j, int (&off)[kU], float (&val)[kU]) {
#pragma unroll
        for (int u = 0; u < kU; u += 4) {
            const int4 o4 = *reinterpret_cast<const int4 *>(g_off + j + u);
            const float4 v4 = *reinterpret_cast<const float4 *>(g_val + j + u);
            off[u] = o4.x; off[u + 1] = o4.y; off[u + 2] = o4.z; off[u + 3] = o4.w;
            val[u] = v4.x; val[u + 1] = v4.y; val[u + 2] = v4.z; val[u + 3] = v4.w;
        }
    };

    int win = kVecCsr ? (p0 & ~3) : p0;
    for (;;) {
        const bool more = win < p1;
        if (!__any(more)) break;  // wave-uniform: every lane reaches the barriers
        // ---- stage one window (padding outside [p0, p1))
        if constexpr (kVecCsr) {
#pragma unroll
            for (int sg = 0; sg < kEpl / 4; ++sg) {
                const int slot0 = (sg * kLpr + gl) * 4;
                const int e = win + slot0;
                int cc[4] = {0, 0, 0, 0};
                float vv[4] = {0.f, 0.f, 0.f, 0.f};
                if (e < p1 && e + 4 > p0) {
                    if (e + 4 <= p.nnz) {
                        const int4 c4 = *reinterpret_cast<const int4 *>(p.col_indices + e);
                        cc[0] = c4.x; cc[1] = c4.y; cc[2] = c4.z; cc[3] = c4.w;
                        load4_f32<E>(vals + e, vv);
                    } else {
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            if (e + t < p.nnz) {
                                cc[t] = p.col_indices[e + t];
                                vv[t] = Elem<E>::f32(vals[e + t]);
                            }
                        }
                    }
                }
                *reinterpret_cast<int4 *>(g_off + slot0) =
                    make_int4(offset_of(e, cc[0]), offset_of(e + 1, cc[1]),
                              offset_of(e + 2, cc[2]), offset_of(e + 3, cc[3]));
                *reinterpret_cast<float4 *>(g_val + slot0) =
                    make_float4(value_of(e, vv[0]), value_of(e + 1, vv[1]),
                                value_of(e + 2, vv[2]), value_of(e + 3, vv[3]));
            }
        } else {
#pragma unroll
            for (int t = 0; t < kEpl; ++t) {
                const int idx = win + t * kLpr + gl;
                const bool in = idx < p1;
                g_off[t * kLpr + gl] = offset_of(idx, in ? p.col_indices[idx] : 0);
                g_val[t * kLpr + gl] = value_of(idx, in ? Elem<E>::f32(vals[idx]) : 0.f);
            }
        }
        window_sync<kWaveSync>();
        // ---- gather and accumulate: double-buffered batches of kU slots.
        // Slots [0, wend) of the window cover every group's live entries.
        const int my_end = min(p1 - win, kChunk);
        const int wend = strided_wave_reduce<kLpr>(my_end, OpMax{});
        VecT bufa[kU], bufb[kU];
        int offa[kU], offb[kU];
        float vala[kU], valb[kU];
        // Each batch's staged entries are read right after the arithmetic
        // that frees their registers, and the loop body is one basic block
        // (two batches per trip, the second possibly all padding): the
        // compiler's wait counts are then exact and the next batch's gathers
        // are issued before the current batch is waited for.  Batches past
        // the window are the kU padding slots (min(., kChunk)).
        read_batch(0, offa, vala);
#pragma unroll
        for (int u = 0; u < kU; ++u) bufa[u] = gather(offa[u]);
        read_batch(min(kU, kChunk), offb, valb);
        int j = 0;
        do {
#pragma unroll
            for (int u = 0; u < kU; ++u) bufb[u] = gather(offb[u]);
            keep_issued_above();
#pragma unroll
            for (int u = 0; u < kU; u += 2) V::fma2(vala[u], vala[u + 1], bufa[u], bufa[u + 1], acc);
            read_batch(min(j + 2 * kU, kChunk), offa, vala);
#pragma unroll
            for (int u = 0; u < kU; ++u) bufa[u] = gather(offa[u]);
            keep_issued_above();
#pragma unroll
            for (int u = 0; u < kU; u += 2) V::fma2(valb[u], valb[u + 1], bufb[u], bufb[u + 1], acc);
            read_batch(min(j + 3 * kU, kChunk), offb, valb);
            j += 2 * kU;
        } while (j < wend);
        window_sync<kWaveSync>();
        win += kChunk;
    }
}

template <typename E, int kLpr, int kVec, bool kVecCsr, bool kBuf>
__device__ __forceinline__ void spmm_wide_body(const SpmmParams &p, long long w)
{
    using V = GVec<E, kVec>;
    constexpr int kRpw = kWave / kLpr;       // rows per wave
    constexpr int kChunk = kEpl * kLpr;      // entries per row per window
    // A group's slots: the window, kU padding slots read by the prefetch, and
    // 4 more so that the groups' regions start 12 words apart modulo the 64
    // LDS banks (their broadcast reads then never share a bank).
    constexpr int kPitch = kChunk + kU + 4;
    static_assert(kPitch % 4 == 0 && kU % 4 == 0, "16-byte aligned batches");
    static_assert(kChunk % kU == 0, "batches never straddle the window end");
    // Staged entries, one array per field so that each lane's staging writes
    // are 16 contiguous bytes: B-row byte offset (kBuf) or column, and value.
    __shared__ __align__(16) int s_off[kRpw * kPitch];
    __shared__ __align__(16) float s_val[kRpw * kPitch];

    if (w < 0) return;
    const long long per_z = (long long)p.tiles * p.row_blocks;
    const long long z = w / per_z;
    const int tile = (int)((w - z * per_z) / p.row_blocks);
    const int rb = (int)(w - z * per_z - (long long)tile * p.row_blocks);

    const int lane = threadIdx.x;
    const int grp = kRpw == 1 ? 0 : lane / kLpr;
    const int gl = kRpw == 1 ? lane : lane - grp * kLpr;
    const E *__restrict__ vals = static_cast<const E *>(p.values) + z * p.stride_values;
    const E *__restrict__ bz = static_cast<const E *>(p.b) + z * p.stride_b;
    float *__restrict__ cz = p.c + z * p.stride_c;

    const int slot = rb * kRpw + grp;
    const bool has_row = slot < p.m;
    const int row = has_row ? (p.row_indices ? p.row_indices[slot] : slot) : 0;
    const int p0 = has_row ? p.row_offsets[row] : 0;
    const int p1 = has_row ? p.row_offsets[row + 1] : 0;
    const int col0 = (tile * kLpr + gl) * kVec;
    const bool col_ok = col0 < p.n;  // vector path: n % kVec == 0, so the whole vector is in range
    int *g_off = s_off + grp * kPitch;
    float *g_val = s_val + grp * kPitch;
    float acc[kVec];
#pragma unroll
    for (int t = 0; t < kVec; ++t) acc[t] = 0.f;

    wide_accumulate<E, kLpr, kVec, kVecCsr, kBuf, false>(p, vals, bz, p0, p1, gl, col0, col_ok,
                                                         g_off, g_val, acc);
    if (has_row && col_ok) V::store(cz + (size_t)row * (size_t)p.n + col0, acc);
}

// Workgroups of the wide launch, and the work index of workgroup `block`.
inline long long wide_grid(const SpmmParams &p)
{
    return xcd_grid((long long)p.batch * p.tiles, p.row_blocks);
}
__device__ __forceinline__ long long wide_work(const SpmmParams &p, long long block)
{
    return xcd_work_index_of(block, (long long)p.batch * p.tiles, p.row_blocks);
}

}  // namespace spmm_detail
}  // namespace spk
