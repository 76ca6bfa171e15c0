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
//
// Batches whose heads are small enough (fp32 d = 32 or 64, 16-bit d = 64) take
// attention_union_kernel below instead: panels of 16 query rows walked in
// 16-key tiles of their key union on matrix cores, with the per-row walk
// above (attention_row) for panels that share few keys.
#include <algorithm>

#include "sp_device.h"
#include "sp_launch.h"
#include "sp_types.h"
#include "panel_union.h"

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
    int k_rows;         // rows of K and V
    float *out;
    long long stride_q, stride_k, stride_v, stride_out;
};

#ifndef SP_ATTN_SCORE_LOADS
#define SP_ATTN_SCORE_LOADS 2
#endif
// The shape of one row's walk for element type E and kDv 16-byte vectors per
// row, and the sizes of its per-wave LDS staging.
template <typename E, int kDv> struct AttnShape {
    static constexpr int kVec = 16 / Elem<E>::kBytes;   // elements per 16-byte vector
    static constexpr unsigned kEb = Elem<E>::kBytes;
    // score phase: kG lanes per entry, kNv vectors each, kNg entries per step
    static constexpr int kG = kDv <= 8 ? 8 : 16;
    static constexpr int kNv = kDv / kG;
    static constexpr int kNg = kWave / kG;
    static constexpr int kU = SP_ATTN_SCORE_LOADS / kNv > 0 ? SP_ATTN_SCORE_LOADS / kNv : 1;
    static constexpr int kBatches = (kG + kU - 1) / kU;
    // P.V phase: kDv lanes per entry (one vector each), kSl entries per step
    static constexpr int kSl = kWave / kDv;
    static constexpr int kUv = kDv <= 16 ? 2 : kDv / 8;  // P.V steps per batch (at most 8 batches)
    static constexpr int kVB = (kDv + kUv - 1) / kUv;    // P.V batches of a full window
    static_assert(kNv * kG == kDv, "score lanes cover the row");
    // windows plus the padding read by the prefetch of up to two batches
    static constexpr int kVPad = 3 * kUv * kSl;
    static constexpr int kKoff = kWave + 2 * kU * kNg;   // words of the K-offset staging
    static constexpr int kVoff = kWave + kVPad;          // words of the V-offset / weight staging
};

// One wave's walk of one query row (batch entry z) through its own staging
// regions s_koff, s_voff and s_e (AttnShape sizes); writes the output row.
template <typename E, int kDv>
__device__ __forceinline__ void attention_row(const AttnParams &p, long long z, int row,
                                              int lane, unsigned *s_koff, unsigned *s_voff,
                                              float *s_e)
{
    using S = AttnShape<E, kDv>;
    constexpr int kVec = S::kVec;
    using V = GVec<E, kVec>;
    using VecT = typename V::T;
    constexpr unsigned kEb = S::kEb;
    constexpr int kG = S::kG, kNv = S::kNv, kNg = S::kNg, kU = S::kU, kBatches = S::kBatches;
    constexpr int kSl = S::kSl, kUv = S::kUv, kVB = S::kVB, kVPad = S::kVPad;
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
__global__ __launch_bounds__(kAttnWaves * kWave) void attention_kernel(AttnParams p)
{
    using S = AttnShape<E, kDv>;
    __shared__ unsigned s_koff_all[kAttnWaves][S::kKoff];
    __shared__ unsigned s_voff_all[kAttnWaves][S::kVoff];
    __shared__ float s_e_all[kAttnWaves][S::kVoff];
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
    const int row = p.row_indices ? p.row_indices[slot] : slot;
    attention_row<E, kDv>(p, z, row, lane, s_koff_all[wave], s_voff_all[wave], s_e_all[wave]);
}

// Batched fp32 attention (d = 32 or 64) over a mask whose neighbouring rows
// share most of their keys (sparse attention's band).  A workgroup takes a
// panel of 16 consecutive query rows and 4 batch entries and forms the panel's
// key union once (panel_union.h); each wave then walks its batch entry's
// union in 16-key tiles, the online softmax of the walk above on matrix cores:
//   1. S = Q[panel] K[tile]^T with v_mfma_f32_16x16x4f32 (lane l holds, of
//      Q's row l % 16 and of key 16 T + l % 16, elements 16 v + 4 (l / 16)
//      ... + 3, as in the panel-union SDDMM), scaled by alpha; keys a row
//      does not have become -Inf;
//   2. per row (lanes of one 16-lane group hold the same four rows): the
//      tile's maximum and the running maximum mx, the running sum l of
//      exp(s - mx), and the rescaling of l and the output accumulators by
//      exp(mx_old - mx_new) when mx grows;
//   3. the weights exp(s - mx) go through a 16 x 16 LDS tile into the A
//      operand's layout (row l % 16, key 4 st + l / 16), and
//      O += P[panel, tile] V[tile] with four (d = 64) or two (d = 32) MFMAs
//      per step of 4 keys, lane l's accumulators holding
//      O[4 (l / 16) + r][kNc (l % 16) + c], as in the panel-union SpMM.
// After the last tile O is divided by l (rows without entries stay zero) and
// leaves as one vector store per row.  Panels whose union is too wide for
// their entry count run attention_row on their rows; so does a wave that
// loads a V value that is not finite (a tile multiplies the zero weights of
// absent keys by V rows: 0 x Inf would be NaN where the row's result is
// finite), its stores replacing the tile's.  Sums and maxima are taken in a
// fixed order: deterministic, rounding in the MFMA's order.
namespace pu = panel_union;

// At least 4 waves per SIMD: the walk loads each tile just before it is used
// (no second tile in flight), which keeps it near 90 VGPRs; the other resident
// waves hide the loads.  With a tile prefetched, 168 VGPRs allowed two waves per
// SIMD and the walk ran 18 % slower.
template <typename E, int kD>
__global__ __launch_bounds__(pu::kThreads, 4) void attention_union_kernel(AttnParams p)
{
    typedef float f4 __attribute__((ext_vector_type(4)));
    constexpr int kVecE = 16 / (int)Elem<E>::kBytes;  // elements per 16-byte vector
    constexpr unsigned kEb = Elem<E>::kBytes;
    constexpr int kS = kD / 4;     // score MFMA steps per tile: elements of d per lane
    constexpr int kNc = kD / 16;   // output columns per lane, one accumulator each
    constexpr int kDv = kD / kVecE;  // 16-byte vectors per row (the per-row walk)
    static_assert(kS % kVecE == 0, "whole vectors per lane");
    using Sh = AttnShape<E, kDv>;
    constexpr int kPp = 17;        // pitch of the weight tile (odd: the transposed read is spread over banks)
    __shared__ pu::Shared s;
    __shared__ float s_p[pu::kWaves][16 * kPp];
    __shared__ unsigned s_koff_all[pu::kWaves][Sh::kKoff];
    __shared__ unsigned s_voff_all[pu::kWaves][Sh::kVoff];
    __shared__ float s_e_all[pu::kWaves][Sh::kVoff];
    extern __shared__ unsigned s_dyn[];
    pu::Panel pp;
    if (!pu::panel_of(p.m, p.batch, p.row_offsets, pp)) return;
    // an empty panel stores zero rows through the tile path (no tiles)
    const int nu = pp.pn > 0 ? pu::build(p.row_offsets, p.col_indices, p.k_rows, pp, s, s_dyn) : 0;
    // (uniform in the wave; the buffer resources below depend on it)
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int z = pp.hg * pu::kWaves + wave;
    if (z >= p.batch) return;
    auto per_row = [&]() {
#pragma unroll 1
        for (int i = 0; i < pp.nr; ++i)
            attention_row<E, kDv>(p, z, pp.r0 + i, lane, s_koff_all[wave], s_voff_all[wave],
                                  s_e_all[wave]);
    };
    if (nu < 0) {
        per_row();
        return;
    }

    const int ntiles = (nu + 15) / 16;
    const unsigned rowbytes = (unsigned)kD * kEb;      // a row of Q, K or V
    const unsigned orowbytes = (unsigned)kD * 4u;      // a row of the fp32 output
    float *oz = p.out + z * p.stride_out;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<E *>(static_cast<const E *>(p.q) + z * p.stride_q), 0,
        (int)((unsigned)p.m * rowbytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<E *>(static_cast<const E *>(p.k) + z * p.stride_k), 0, (int)p.kv_bytes,
        0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<E *>(static_cast<const E *>(p.v) + z * p.stride_v), 0, (int)p.kv_bytes,
        0x00020000);
    const __amdgpu_buffer_rsrc_t ro =
        __builtin_amdgcn_make_buffer_rsrc(oz, 0, (int)((unsigned)p.m * orowbytes), 0x00020000);
    const int jl = lane % 16;  // the lane's Q row and key of a tile; its output column group
    const int q = lane / 16;   // the lane's 16-byte piece of each 64-byte block of d; key of a step
    float *tp = s_p[wave];

    // The lane's kS elements of a Q or K row: vector v holds elements
    // 4 kVecE v + kVecE q ... + kVecE - 1, so the four lanes of a row read 64
    // contiguous bytes per instruction; step kVecE v + s multiplies element
    // 4 kVecE v + kVecE q + s of both.
    auto lane_elem_bytes = [&](int v) { return (unsigned)(4 * kVecE * v + kVecE * q) * kEb; };
    float xa[kS];
    {
        const unsigned base = jl < pp.nr ? (unsigned)(pp.r0 + jl) * rowbytes : kOutOfRange;
#pragma unroll
        for (int v = 0; v < kS / kVecE; ++v)
            load_widen<E, kVecE>(rq, base + lane_elem_bytes(v), &xa[kVecE * v]);
    }
    struct Tile {
        float k[kS];        // key 16 T + jl: the lane's elements
        float v[4][kNc];    // keys 16 T + 4 st + q: the lane's output columns
    };
    auto load = [&](int T, Tile &t) {
        {
            const int u = 16 * T + jl;
            const unsigned col = (unsigned)s.ucol[min(u, pu::kMaxCols - 1)];
            const unsigned base = u < nu ? col * rowbytes : kOutOfRange;
#pragma unroll
            for (int v = 0; v < kS / kVecE; ++v)
                load_widen<E, kVecE>(rk, base + lane_elem_bytes(v), &t.k[kVecE * v]);
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int u = 16 * T + 4 * st + q;
            const unsigned col = (unsigned)s.ucol[min(u, pu::kMaxCols - 1)];
            const unsigned off = (u < nu ? col * rowbytes : kOutOfRange) + (unsigned)(kNc * jl) * kEb;
            load_widen<E, kNc>(rv, off, t.v[st]);
        }
    };
    f4 o[kNc];
#pragma unroll
    for (int c = 0; c < kNc; ++c) o[c] = f4{0.f, 0.f, 0.f, 0.f};
    float mx[4], l[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        mx[r] = -INFINITY;
        l[r] = 0.f;
    }
    bool finite = true;
    auto process = [&](int T, const Tile &t) {
        f4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < kS; ++i)
            sc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[i], t.k[i], sc, 0, 0, 0);
        const int u = 16 * T + jl;
        const int uc = min(u, pu::kMaxCols - 1);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool present = u < nu && s.emap[(4 * q + r) * pu::kEmapStride + uc] != 0;
            const float sv = present ? p.alpha * sc[r] : -INFINITY;
            const float mnew = fmaxf(mx[r], group_reduce<16>(sv, OpMax{}));
            const float c = mnew == -INFINITY ? 1.f : expf(mx[r] - mnew);
            const float e = present ? expf(sv - mnew) : 0.f;
            l[r] = l[r] * c + group_sum<16>(e);
            mx[r] = mnew;
#pragma unroll
            for (int cc = 0; cc < kNc; ++cc) o[cc][r] *= c;
            tp[(4 * q + r) * kPp + jl] = e;
        }
        wave_lds_sync();
        float a[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) a[st] = tp[jl * kPp + 4 * st + q];
        wave_lds_sync();
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int cc = 0; cc < kNc; ++cc) {
                finite = finite && __builtin_isfinite(t.v[st][cc]);
                o[cc] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[st], t.v[st][cc], o[cc], 0, 0, 0);
            }
    };
    for (int T = 0; T < ntiles; ++T) {
        Tile t;
        load(T, t);
        process(T, t);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 4 * q + r;
        const float inv = l[r] > 0.f ? 1.f / l[r] : 0.f;
        const unsigned off =
            row < pp.nr ? (unsigned)(pp.r0 + row) * orowbytes + (unsigned)(kNc * jl) * 4u
                        : kOutOfRange;
        if constexpr (kNc == 4) {
            typedef unsigned u4 __attribute__((ext_vector_type(4)));
            const u4 x = {__float_as_uint(o[0][r] * inv), __float_as_uint(o[1][r] * inv),
                          __float_as_uint(o[2][r] * inv), __float_as_uint(o[3][r] * inv)};
            __builtin_amdgcn_raw_buffer_store_b128(x, ro, (int)off, 0, 0);
        } else {
            typedef unsigned u2 __attribute__((ext_vector_type(2)));
            const u2 x = {__float_as_uint(o[0][r] * inv), __float_as_uint(o[1][r] * inv)};
            __builtin_amdgcn_raw_buffer_store_b64(x, ro, (int)off, 0, 0);
        }
    }
    // a V value that is not finite among this wave's union rows: the per-row
    // walk replaces what the tiles stored (same wave, so the stores stay in order)
    if (__builtin_amdgcn_ballot_w64(!finite) != 0) per_row();
}

template <typename E, int kD>
hipError_t launch_union_t(const AttnParams &p, hipStream_t s)
{
    hipLaunchKernelGGL((attention_union_kernel<E, kD>), dim3((unsigned)pu::grid(p.m, p.batch)),
                       dim3(pu::kThreads), pu::dynamic_lds(p.k_rows), s, p);
    return hipGetLastError();
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
    p.k_rows = a.k_rows;
    p.out = a.out;
    p.stride_q = a.stride_q;
    p.stride_k = a.stride_k;
    p.stride_v = a.stride_v;
    p.stride_out = a.stride_out;
    // Batches of fp32 heads of 32 or 64, or 16-bit heads of 64, on up to
    // 65,536 keys: the panel-union kernel, which runs the per-row walk on
    // panels whose rows share few keys.
    if ((a.d == 64 || (a.d == 32 && a.dtype == Dtype::f32)) && a.batch >= 2 &&
        a.k_rows <= pu::kMaxK && (long long)a.m * a.d * 4 < (1LL << 31) &&
        pu::grid(a.m, a.batch) <= 0x7fffffffLL) {
        switch (a.dtype) {
        case Dtype::f16: return launch_union_t<_Float16, 64>(p, stream);
        case Dtype::bf16: return launch_union_t<bf16, 64>(p, stream);
        default:
            return a.d == 32 ? launch_union_t<float, 32>(p, stream)
                             : launch_union_t<float, 64>(p, stream);
        }
    }
    switch (a.dtype) {
    case Dtype::f16: return launch_e<_Float16>(dv, p, stream);
    case Dtype::bf16: return launch_e<bf16>(dv, p, stream);
    default: return launch_e<float>(dv, p, stream);
    }
}

}  // namespace spk
