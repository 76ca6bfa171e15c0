// The SDDMM body for Y stored k x d (one wavefront per mask row), shared by
// the SDDMM launch and the launch that runs an SpMM and an SDDMM together.
//
// CSR SDDMM for gfx950: out[p] = alpha * dot(X[i], Y[col_indices[p]]) for each
// entry p of row i ("Sparse GPU Kernels for Deep Learning", summary card,
// "Summary" and "Interesting ideas" I3: the specialised form with no scaling
// by mask values and the second operand transposed, so that X and Y are both
// read by contiguous rows).  The general form I3 leaves out is an epilogue of
// the same kernels (scaling by the mask's values, out = ... + beta * out) and,
// for Y stored d x k, a second kernel that deals lanes to entries.
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
// Long rows.  With kParts > 1, each row slot gets a workgroup of kParts waves
// and wave j takes the row's windows j, j + kParts, j + 2 kParts, ...: an
// entry's output never depends on other entries, so windows need no combine
// step, and a row of many windows no longer runs in one wave.  Each wave loads
// the X row itself, stages in its own LDS region and syncs only itself; waves
// without a window leave at once.  The arithmetic of every entry is the same
// for any kParts (bit-identical outputs).
//
// Summation order: each lane sums its elements in order with FMA (16-bit
// types: by pairs, v_dot2c_f32_bf16 / _f16), then the DPP tree adds the kG
// lane partials; deterministic run to run.
#pragma once

#include "sp_device.h"
#include "sp_types.h"

namespace spk {
namespace sddmm_detail {

struct SddmmParams {
    int m, d, nnz, batch;
    const int *row_indices;
    const int *row_offsets;
    const int *col_indices;
    const float *mask_values;  // NULL: scale by alpha only
    const void *x;             // element type of the kernel instance
    const void *y;
    int k;
    float alpha, beta;
    unsigned y_bytes;  // bytes of one Y operand (buffer path)
    float *out;
    long long stride_values, stride_x, stride_y, stride_out;
};

// out[q] = alpha * v_q * dot + beta * out[q] for the entry q a lane finished.
// beta == 0 leaves out unread (it may hold anything, NaN included).
__device__ __forceinline__ void store_entry(const SddmmParams &p, long long z, int q, float dot)
{
    float scale = p.alpha;
    if (p.mask_values) scale *= p.mask_values[z * p.stride_values + q];
    float *o = p.out + z * p.stride_out + q;
    float r = scale * dot;
    if (p.beta != 0.f) r = fmaf(p.beta, *o, r);
    *o = r;
}

#ifndef SP_SDDMM_LOADS_PER_BATCH
#define SP_SDDMM_LOADS_PER_BATCH 2
#endif
constexpr unsigned kOutOfRange = 0x80000000u;  // buffer offset that reads as zero

// kNv > 0 (Y < 2 GiB): the lane's kNv vectors of the X row live in registers
// (as loaded); Y rows are gathered through a buffer resource, and window
// slots past the row's end carry an out-of-range offset that reads as zeros,
// so steps are issued in unconditional double-buffered batches of kU.
// kNv == 0: any d and any Y size; X and Y are read with 64-bit addresses in a
// loop over d, one step at a time.  E is the element type of X and Y (fp32,
// fp16 or bf16); products and sums are fp32 (V::dot).
//
// kSoftmax: the row softmax of the scaled scores is applied before they are
// written (out = softmax over the row's entries of alpha * X Y^T), the step
// between the scores and their weighted sum in sparse attention.  The wave
// holds its row's scores (one per lane per window of 64) in registers for up
// to kHeldWindows windows and parks later windows' scores in `out`; after the
// last window it reduces the row maximum and the sum of exp(s - max) across
// the wave (butterflies, fixed order) and writes exp(s - max) / sum.
// The staging barrier between windows: the workgroup's when it is one wave,
// else only the wave's own (its LDS operations complete in program order; the
// fences keep the compiler from moving them across).
template <int kParts>
__device__ __forceinline__ void rows_sync()
{
    if constexpr (kParts == 1) {
        __syncthreads();
    } else {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// kWaves: the waves of the workgroup, each with its own staging region and a
// wave-local sync (kParts of them split a row's windows; with kParts = 1 and
// kWaves > 1 each wave walks rows of its own, as the panel-union kernel's
// per-row fallback does).
template <typename E, int kG, int kNv, int kVec, bool kSoftmax = false, int kParts = 1,
          int kWaves = kParts>
__device__ __forceinline__ void sddmm_rows_body(const SddmmParams &p, long long w)
{
    static_assert(kParts == 1 || kParts == kWaves, "split rows use every wave");
    static_assert(!(kSoftmax && kParts > 1), "the row softmax needs the whole row in one wave");
    using V = GVec<E, kVec>;
    using VecT = typename V::T;
    constexpr unsigned kEb = Elem<E>::kBytes;
    constexpr int kNg = kWave / kG;  // entries per step
    constexpr int kU = kNv == 0 ? 1
                                : (SP_SDDMM_LOADS_PER_BATCH / kNv > 0 ? SP_SDDMM_LOADS_PER_BATCH / kNv : 1);
    constexpr int kXv = kNv == 0 ? 1 : kNv;
    // The window's 64 entries, then padding for the prefetch of up to two
    // batches past the last step.
    constexpr int kSlots = kWave + 2 * kU * kNg;
    __shared__ unsigned s_off_all[kWaves][kSlots];

    constexpr int kHeldWindows = 4;
    float held[kHeldWindows];
    float row_max = -INFINITY;
    int window = 0;

    if (w < 0) return;
    const long long z = w / p.m;
    const int slot = (int)(w - z * p.m);
    const int part = kParts == 1 ? 0 : (int)threadIdx.x / kWave;  // this wave's windows
    const int region = kWaves == 1 ? 0 : (int)threadIdx.x / kWave;  // its staging
    const int lane = kWaves == 1 ? (int)threadIdx.x : (int)threadIdx.x % kWave;
    unsigned *s_off = s_off_all[region];
    const int g = lane / kG;
    const int gl = lane - g * kG;
    const int row = p.row_indices ? p.row_indices[slot] : slot;
    const int p0 = p.row_offsets[row];
    const int p1 = p.row_offsets[row + 1];
    // this wave's windows: part, part + kParts, ... of the row's nwin
    const int nwin = (int)(((long long)p1 - p0 + kWave - 1) / kWave);
    if (part >= nwin) return;  // one row per wave: uniform, before any barrier

    const E *__restrict__ xr_ptr =
        static_cast<const E *>(p.x) + z * p.stride_x + (size_t)row * (size_t)p.d;
    const E *__restrict__ yz = static_cast<const E *>(p.y) + z * p.stride_y;
    float *__restrict__ oz = p.out + z * p.stride_out;

    // The score of entry q, kept by this lane, in window `window` of the row.
    auto emit = [&](int q, float res) {
        if constexpr (kSoftmax) {
            const float s = p.alpha * res;
            row_max = fmaxf(row_max, s);
#pragma unroll
            for (int t = 0; t < kHeldWindows; ++t)
                if (t == window) held[t] = s;
            if (window >= kHeldWindows) oz[q] = s;
        } else {
            store_entry(p, z, q, res);
        }
    };

    if constexpr (kNv == 0) {
        __shared__ int s_col_all[kWaves][kWave];
        int *s_col = s_col_all[region];
        for (int wi = part; wi < nwin; wi += kParts) {
            const int base = p0 + wi * kWave;
            const int cnt = min(kWave, p1 - base);
            s_col[lane] = lane < cnt ? p.col_indices[base + lane] : 0;
            rows_sync<kWaves>();
            const int steps = (cnt + kNg - 1) / kNg;
            float res = 0.f;
            for (int s = 0; s < steps; ++s) {
                const int j = s * kNg + g;
                float acc = 0.f;
                if (j < cnt) {
                    const E *yr = yz + (size_t)s_col[j] * (size_t)p.d;
                    for (int e = gl * kVec; e < p.d; e += kG * kVec) {
                        acc = V::dot(V::load(xr_ptr + e), V::load(yr + e), acc);
                    }
                }
                const float sum = group_sum<kG>(acc);
                if (gl == s) res = sum;
            }
            const int jo = gl * kNg + g;
            if (jo < cnt) emit(base + jo, res);
            rows_sync<kWaves>();
            ++window;
        }
    } else {
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<E *>(yz), 0, (int)p.y_bytes, 0x00020000);
        VecT xr[kXv];
        unsigned lane_off[kXv];
#pragma unroll
        for (int v = 0; v < kNv; ++v) {
            const int e = (v * kG + gl) * kVec;
            xr[v] = e < p.d ? V::load(xr_ptr + e) : V::zero();
            lane_off[v] = e < p.d ? (unsigned)e * kEb : kOutOfRange;
        }
        for (int t = kWave + lane; t < kSlots; t += kWave) s_off[t] = kOutOfRange;

        auto load_batch = [&](int s0, VecT (&yv)[kU][kXv]) {
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const unsigned off = s_off[(s0 + u) * kNg + g];
#pragma unroll
                for (int v = 0; v < kNv; ++v) yv[u][v] = V::buf_load(rsrc, off + lane_off[v]);
            }
        };
        auto reduce_batch = [&](int s0, const VecT (&yv)[kU][kXv], float &res) {
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                float acc = 0.f;
#pragma unroll
                for (int v = 0; v < kNv; ++v) acc = V::dot(xr[v], yv[u][v], acc);
                const float sum = group_sum<kG>(acc);
                if (gl == s0 + u) res = sum;
            }
        };

        for (int wi = part; wi < nwin; wi += kParts) {
            const int base = p0 + wi * kWave;
            const int cnt = min(kWave, p1 - base);
            s_off[lane] = lane < cnt
                              ? (unsigned)p.col_indices[base + lane] * (unsigned)p.d * kEb
                              : kOutOfRange;
            rows_sync<kWaves>();
            const int steps = (cnt + kNg - 1) / kNg;
            float res = 0.f;
            // A window has at most kG steps, so its batches are unrolled into
            // straight-line code (exact wait counts: no loop back edge).
            constexpr int kBatches = (kG + kU - 1) / kU;
            VecT ya[kU][kXv], yb[kU][kXv];
            load_batch(0, ya);
#pragma unroll
            for (int bt = 0; bt < kBatches; bt += 2) {
                if (bt * kU >= steps) break;
                load_batch((bt + 1) * kU, yb);
                keep_issued_above();
                reduce_batch(bt * kU, ya, res);
                if ((bt + 1) * kU >= steps) break;
                load_batch((bt + 2) * kU, ya);
                keep_issued_above();
                reduce_batch((bt + 1) * kU, yb, res);
            }
            const int jo = gl * kNg + g;  // the entry whose sum this lane kept
            if (jo < cnt) emit(base + jo, res);
            rows_sync<kWaves>();
            ++window;
        }
    }
    if constexpr (kSoftmax) {
        // window t of the row holds entries p0 + 64 t ...; this lane's is jo
        const int jo = gl * kNg + g;
        auto live = [&](int t) { return jo < min(kWave, p1 - p0 - t * kWave); };
        const float mx = wave_max(row_max);
        float sum = 0.f;
#pragma unroll
        for (int t = 0; t < kHeldWindows; ++t) {
            const float e = (t < window && live(t)) ? expf(held[t] - mx) : 0.f;
            held[t] = e;
            sum += e;
        }
        for (int t = kHeldWindows; t < window; ++t)
            if (live(t)) sum += expf(oz[p0 + t * kWave + jo] - mx);
        const float inv = 1.f / wave_sum(sum);
#pragma unroll
        for (int t = 0; t < kHeldWindows; ++t)
            if (t < window && live(t)) oz[p0 + t * kWave + jo] = held[t] * inv;
        for (int t = kHeldWindows; t < window; ++t)
            if (live(t)) {
                const int q = p0 + t * kWave + jo;
                oz[q] = expf(oz[q] - mx) * inv;
            }
    }
}

// Workgroups of the row launch, and the work index of workgroup `block`.
inline long long rows_grid(const SddmmParams &p)
{
    return xcd_grid(p.batch, p.m);
}
__device__ __forceinline__ long long rows_work(const SddmmParams &p, long long block)
{
    return xcd_work_index_of(block, p.batch, p.m);
}

}  // namespace sddmm_detail
}  // namespace spk
