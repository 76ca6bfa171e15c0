// Sparse attention in one pass: O = softmax(alpha * Q K^T at the mask) V,
// row by row ("Sparse GPU Kernels for Deep Learning", summary card,
// "Interesting ideas" I3: the SDDMM form that sparse attention needs; the
// attention is SDDMM -> row softmax -> SpMM).  Neither the scores nor the
// probabilities are written: one wavefront per (batch entry, query row) walks
// the row's entries in windows of 64 and, per window,
//   1. computes the 64 scores as the SDDMM row kernel does (kG lanes per
//      entry, the Q row in registers, K rows gathered with buffer loads,
//      partials summed by DPP within 16-lane rows);
//   2. folds them into the row's running maximum mx and running sum
//      l = sum exp(s - mx) (when mx grows, l and the output accumulators are
//      multiplied by exp(mx_old - mx_new): the online form of the softmax);
//   3. stages exp(s - mx) and the V-row offsets of the window in LDS and
//      accumulates sum_j exp(s_j - mx) V[col_j] with lanes over (entry slot,
//      16-byte vector of the V row) -- the narrow SpMM mapping.
// After the last window the entry slots' partial sums are added across lanes
// (DPP rotations and lane swaps) and divided by l.  Every reduction has a fixed order: deterministic.  Rows
// without entries produce zero rows (as the three-kernel pipeline does).
//
// Head dimensions: Q, K and V rows have the same length d, a multiple of one
// 16-byte vector, with d / (elements per vector) in {8, 16, 32, 64} (fp32: d =
// 32, 64, 128, 256; fp16 and bf16: 64, 128, 256, 512).
#include <algorithm>

#include "sp_device.h"
#include "sp_launch.h"
#include "sp_types.h"

namespace spk {

namespace {

constexpr unsigned kOutOfRange = 0x80000000u;  // buffer offset that reads as zero

// Waves per workgroup, each its own query row: kAttnWaves consecutive slots
// (in the row order) run on one CU, so rows that share most of their keys --
// a banded mask's neighbouring rows -- find those K and V rows in the CU's
// L1 cache.  Each wave has its own LDS staging region and syncs only itself.
#ifndef SP_ATTN_WAVES
#define SP_ATTN_WAVES 4
#endif
constexpr int kAttnWaves = SP_ATTN_WAVES;

// Orders a wave's own LDS writes before its lanes read them (the LDS
// operations of one wave complete in program order; the fences keep the
// compiler from moving them across).
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct AttnParams {
    int m, d, batch;
    const int *row_indices;
    const int *row_offsets;
    const int *col_indices;
    const void *q, *k, *v;
    float alpha;
    unsigned kv_bytes;  // bytes of one K (= one V) operand
    float *out;
    long long stride_q, stride_k, stride_v, stride_out;
};

template <typename E, int kDv>
__global__ __launch_bounds__(kAttnWaves * kWave) void attention_kernel(AttnParams p)
{
    constexpr int kVec = 16 / Elem<E>::kBytes;   // elements per 16-byte vector
    using V = GVec<E, kVec>;
    using VecT = typename V::T;
    constexpr unsigned kEb = Elem<E>::kBytes;
    // score phase: kG lanes per entry, kNv vectors each, kNg entries per step
    constexpr int kG = kDv <= 8 ? 8 : 16;
    constexpr int kNv = kDv / kG;
    constexpr int kNg = kWave / kG;
#ifndef SP_ATTN_SCORE_LOADS
#define SP_ATTN_SCORE_LOADS 2
#endif
    constexpr int kU = SP_ATTN_SCORE_LOADS / kNv > 0 ? SP_ATTN_SCORE_LOADS / kNv : 1;  // steps per batch
    constexpr int kBatches = (kG + kU - 1) / kU;
    // P.V phase: kDv lanes per entry (one vector each), kSl entries per step
    constexpr int kSl = kWave / kDv;
    constexpr int kUv = kDv <= 16 ? 2 : kDv / 8; // P.V steps per batch (at most 8 batches)
    constexpr int kVB = (kDv + kUv - 1) / kUv;   // P.V batches of a full window
    static_assert(kNv * kG == kDv, "score lanes cover the row");
    // windows plus the padding read by the prefetch of up to two batches
    constexpr int kVPad = 3 * kUv * kSl;
    __shared__ unsigned s_koff_all[kAttnWaves][kWave + 2 * kU * kNg];
    __shared__ unsigned s_voff_all[kAttnWaves][kWave + kVPad];
    __shared__ float s_e_all[kAttnWaves][kWave + kVPad];

    // workgroup: kAttnWaves consecutive slots of one batch entry
    const long long groups = ((long long)p.m + kAttnWaves - 1) / kAttnWaves;
    const long long w = xcd_work_index(p.batch, groups);
    if (w < 0) return;
    const long long z = w / groups;
    const int wave = threadIdx.x / kWave;
    const long long slot_ll = (w - z * groups) * kAttnWaves + wave;
    if (slot_ll >= p.m) return;  // no workgroup barrier follows
    const int slot = (int)slot_ll;
    const int lane = threadIdx.x - wave * kWave;
    unsigned *s_koff = s_koff_all[wave];
    unsigned *s_voff = s_voff_all[wave];
    float *s_e = s_e_all[wave];
    const int row = p.row_indices ? p.row_indices[slot] : slot;
    const int p0 = p.row_offsets[row];
    const int p1 = p.row_offsets[row + 1];
    const int d = p.d;
    float *__restrict__ orow = p.out + z * p.stride_out + (size_t)row * (size_t)d;

    // P.V lanes: entry slot sl, vector vv of the V row
    const int sl = lane / kDv;
    const int vv = lane - sl * kDv;
    if (p0 >= p1) {
        if (sl == 0) {
            float zero[kVec];
#pragma unroll
            for (int t = 0; t < kVec; ++t) zero[t] = 0.f;
            V::store(orow + vv * kVec, zero);
        }
        return;
    }

    const E *qz = static_cast<const E *>(p.q) + z * p.stride_q + (size_t)row * (size_t)d;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<E *>(static_cast<const E *>(p.k) + z * p.stride_k), 0, (int)p.kv_bytes,
        0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<E *>(static_cast<const E *>(p.v) + z * p.stride_v), 0, (int)p.kv_bytes,
        0x00020000);

    // score lanes: group g, lane gl within it
    const int g = lane / kG;
    const int gl = lane - g * kG;
    VecT qv[kNv];
    unsigned lane_koff[kNv];
#pragma unroll
    for (int u = 0; u < kNv; ++u) {
        const int e = (u * kG + gl) * kVec;
        qv[u] = V::load(qz + e);
        lane_koff[u] = (unsigned)e * kEb;
    }
    const unsigned lane_voff = (unsigned)vv * 16u;
    const unsigned row_bytes = (unsigned)d * kEb;
    for (int t = kWave + lane; t < kWave + 2 * kU * kNg; t += kWave) s_koff[t] = kOutOfRange;
    for (int t = kWave + lane; t < kWave + kVPad; t += kWave) {
        s_voff[t] = kOutOfRange;
        s_e[t] = 0.f;
    }

    auto load_k = [&](int s0, VecT (&kb)[kU][kNv]) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const unsigned off = s_koff[(s0 + u) * kNg + g];
#pragma unroll
            for (int c = 0; c < kNv; ++c) kb[u][c] = V::buf_load(rk, off + lane_koff[c]);
        }
    };
    auto score_batch = [&](int s0, const VecT (&kb)[kU][kNv], float &res) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < kNv; ++c) acc = V::dot(qv[c], kb[u][c], acc);
            const float sum = group_sum<kG>(acc);
            if (gl == s0 + u) res = sum;
        }
    };

    float o[kVec];
#pragma unroll
    for (int t = 0; t < kVec; ++t) o[t] = 0.f;
    float mx = -INFINITY;  // running row maximum (wave-uniform)
    float l = 0.f;         // running sum of exp(s - mx) (wave-uniform)

    for (int base = p0; base < p1; base += kWave) {
        const int cnt = min(kWave, p1 - base);
        const int col = lane < cnt ? p.col_indices[base + lane] : 0;
        s_koff[lane] = lane < cnt ? (unsigned)col * row_bytes : kOutOfRange;
        wave_lds_sync();
        // ---- 1. scores of the window: lane (g, gl) keeps entry gl * kNg + g
        const int steps = (cnt + kNg - 1) / kNg;
        float res = 0.f;
        VecT ka[kU][kNv], kb[kU][kNv];
        load_k(0, ka);
#pragma unroll
        for (int bt = 0; bt < kBatches; bt += 2) {
            if (bt * kU >= steps) break;
            load_k((bt + 1) * kU, kb);
            keep_issued_above();
            score_batch(bt * kU, ka, res);
            if ((bt + 1) * kU >= steps) break;
            load_k((bt + 2) * kU, ka);
            keep_issued_above();
            score_batch((bt + 1) * kU, kb, res);
        }
        const int jo = gl * kNg + g;
        const bool live = jo < cnt;
        const float s = live ? p.alpha * res : -INFINITY;
        // ---- 2. online softmax statistics
        const float mx_new = fmaxf(mx, wave_max(s));
        const float rescale = expf(mx - mx_new);  // 0 on the first window
        const float e = live ? expf(s - mx_new) : 0.f;
        l = l * rescale + wave_sum(e);
        mx = mx_new;
#pragma unroll
        for (int t = 0; t < kVec; ++t) o[t] *= rescale;
        // ---- 3. weighted V rows of the window
        s_e[jo] = e;
        s_voff[lane] = lane < cnt ? (unsigned)col * row_bytes : kOutOfRange;
        wave_lds_sync();
        // Batches of kUv steps, double-buffered and unrolled like the score
        // phase; slots past the window read zeros with weight 0.
        const int vsteps = (cnt + kSl - 1) / kSl;
        auto load_v = [&](int t0, VecT (&vb)[kUv], float (&ev)[kUv]) {
#pragma unroll
            for (int u = 0; u < kUv; ++u) {
                const int j = (t0 + u) * kSl + sl;
                ev[u] = s_e[j];
                vb[u] = V::buf_load(rv, s_voff[j] + lane_voff);
            }
        };
        auto add_v = [&](const VecT (&vb)[kUv], const float (&ev)[kUv]) {
#pragma unroll
            for (int u = 0; u < kUv; ++u) V::fma(ev[u], vb[u], o);
        };
        VecT va[kUv], vb2[kUv];
        float ea[kUv], eb2[kUv];
        load_v(0, va, ea);
#pragma unroll
        for (int bt = 0; bt < kVB; bt += 2) {
            if (bt * kUv >= vsteps) break;
            load_v((bt + 1) * kUv, vb2, eb2);
            keep_issued_above();
            add_v(va, ea);
            if ((bt + 1) * kUv >= vsteps) break;
            load_v((bt + 2) * kUv, va, ea);
            keep_issued_above();
            add_v(vb2, eb2);
        }
        wave_lds_sync();
    }
    // entry slots' partial sums, then the normalisation
#pragma unroll
    for (int t = 0; t < kVec; ++t) o[t] = strided_wave_sum<kDv>(o[t]);
    const float inv = 1.f / l;
#pragma unroll
    for (int t = 0; t < kVec; ++t) o[t] *= inv;
    if (sl == 0) V::store(orow + vv * kVec, o);
}

template <typename E, int kDv>
hipError_t launch_t(const AttnParams &p, hipStream_t s)
{
    const long long groups = ((long long)p.m + kAttnWaves - 1) / kAttnWaves;
    hipLaunchKernelGGL((attention_kernel<E, kDv>), dim3((unsigned)xcd_grid(p.batch, groups)),
                       dim3(kAttnWaves * kWave), 0, s, p);
    return hipGetLastError();
}

template <typename E>
hipError_t launch_e(int dv, const AttnParams &p, hipStream_t s)
{
    switch (dv) {
    case 8: return launch_t<E, 8>(p, s);
    case 16: return launch_t<E, 16>(p, s);
    case 32: return launch_t<E, 32>(p, s);
    default: return launch_t<E, 64>(p, s);
    }
}

inline bool aligned16(const void *ptr)
{
    return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0;
}

}  // namespace

hipError_t launch_attention(const AttnArgs &a, hipStream_t stream)
{
    if (a.m == 0 || a.batch == 0) return hipSuccess;
    const int eb = a.dtype == Dtype::f32 ? 4 : 2;
    const int vlen = 16 / eb;
    const int dv = a.d / vlen;
    const bool shape_ok = a.d % vlen == 0 && (dv == 8 || dv == 16 || dv == 32 || dv == 64);
    const bool layout_ok = aligned16(a.q) && aligned16(a.k) && aligned16(a.v) &&
                           aligned16(a.out) && a.stride_q % vlen == 0 &&
                           a.stride_k % vlen == 0 && a.stride_v % vlen == 0 &&
                           a.stride_out % 4 == 0;
    const bool size_ok = (long long)a.k_rows * a.d * eb <= (1LL << 31);
    if (!shape_ok || !layout_ok || !size_ok) return hipErrorInvalidConfiguration;
    if (xcd_grid(a.batch, a.m) > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    AttnParams p;
    p.m = a.m;
    p.d = a.d;
    p.batch = a.batch;
    p.row_indices = a.row_indices;
    p.row_offsets = a.row_offsets;
    p.col_indices = a.col_indices;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.alpha = a.alpha;
    p.kv_bytes = (unsigned)((long long)a.k_rows * a.d * eb);
    p.out = a.out;
    p.stride_q = a.stride_q;
    p.stride_k = a.stride_k;
    p.stride_v = a.stride_v;
    p.stride_out = a.stride_out;
    switch (a.dtype) {
    case Dtype::f16: return launch_e<_Float16>(dv, p, stream);
    case Dtype::bf16: return launch_e<bf16>(dv, p, stream);
    default: return launch_e<float>(dv, p, stream);
    }
}

}  // namespace spk
