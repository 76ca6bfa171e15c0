// CSR SpMM for gfx950: C = A * B with A sparse (CSR) and B, C dense row-major
// ("Sparse GPU Kernels for Deep Learning", summary card, "Summary").  The wide
// kernel's body, and the design notes for it, are in spmm_wide.h; this file
// holds the narrow-B, streaming, balanced, row-split and panel-union (batched
// panels as matrix-core tiles over their column union, panel_union.h) kernels
// and the variant selection.
#include <algorithm>
#include <type_traits>

#include "sp_device.h"
#include "sp_launch.h"
#include "sp_types.h"
#include "sp_plan.h"
#include "spmm_panel.h"
#include "spmm_wide.h"
#include "panel_union.h"

namespace spk {

namespace {

using namespace spmm_detail;
template <int kVec> using Vec = GVec<float, kVec>;

template <typename E, int kLpr, int kVec, bool kVecCsr, bool kBuf>
__global__ __launch_bounds__(kWave) void spmm_kernel(SpmmParams p)
{
    spmm_wide_body<E, kLpr, kVec, kVecCsr, kBuf>(p, wide_work(p, blockIdx.x));
}

#ifndef SP_PANEL_MIN_REUSE
#define SP_PANEL_MIN_REUSE 4.0
#endif
constexpr double kPanelMinReuse = SP_PANEL_MIN_REUSE;

// B staged in LDS per row panel (spmm_panel.h).  Column tiles are the outer
// units of the XCD order, so the workgroups sharing a tile share an L2.  Two
// shapes, both 128-column tiles of 16 lanes x 8 columns per row and 8 waves:
//   kPanelMany: panels of 64 rows, chunks of 128 B rows in two buffers -- for
//     problems with many column tiles (the ResNet-50 1x1 layer: 49 tiles);
//   kPanelFew: panels of 32 rows, chunks of 224 B rows in one buffer with
//     128-entry windows -- for one or two tiles over many rows (the LSTM layer),
//     where 64-row panels would leave half the CUs idle.
using PanelMany = PanelShape<16, 2, 8, 2, 4, 128, 2>;
using PanelFew = PanelShape<16, 2, 8, 1, 8, 224, 1>;

template <class S, int kLpr, int kVecs, int kWaves, int kRounds, int kEpl, int kKc, int kBufs>
__global__ __launch_bounds__(S::kThreads) void spmm_panel_kernel(SpmmParams p, PanelParams q)
{
    spmm_panel_body<kLpr, kVecs, kWaves, kRounds, kEpl, kKc, kBufs>(
        p, q, xcd_work_index(q.tiles, q.panels));
}

template <class S> struct PanelKernel;
template <> struct PanelKernel<PanelMany> {
    static constexpr auto fn = &spmm_panel_kernel<PanelMany, 16, 2, 8, 2, 4, 128, 2>;
};
template <> struct PanelKernel<PanelFew> {
    static constexpr auto fn = &spmm_panel_kernel<PanelFew, 16, 2, 8, 1, 8, 224, 1>;
};

template <class S>
hipError_t launch_panel_t(const SpmmParams &p, const PanelParams &q, hipStream_t s)
{
    const size_t lds = S::lds_bytes(q.chunks);
    const auto fn = PanelKernel<S>::fn;
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3((unsigned)xcd_grid(q.tiles, q.panels)), dim3(S::kThreads), lds, s,
                       p, q);
    return hipGetLastError();
}

// The panel shape for an m x k by k x n problem with nnz entries on a GPU of
// `cus` compute units and `lds_max` bytes of LDS per workgroup: the first of
// kPanelMany, kPanelFew whose launch gives every CU a workgroup and whose
// panels touch each staged B row at least kPanelMinReuse times on average
// (rows per panel x density); 0 when neither does.
template <class S>
bool panel_fits(const SpmmArgs &a, int cus, int lds_max, PanelParams *q)
{
    const int chunks = (a.k + S::kKcRows - 1) / S::kKcRows;
    const long long panels = ((long long)a.m + S::kRows - 1) / S::kRows;
    const long long tiles = ((long long)a.n + S::kT - 1) / S::kT;
    if (a.n < S::kT || tiles * panels < cus || (long long)lds_max < (long long)S::lds_bytes(chunks))
        return false;
    if ((double)std::min(a.m, S::kRows) * a.nnz < kPanelMinReuse * (double)a.m * (double)a.k)
        return false;
    if (tiles * panels > 0x7fffffffLL) return false;
    q->k = a.k;
    q->chunks = chunks;
    q->panels = (int)panels;
    q->tiles = (int)tiles;
    return true;
}

// Wide B with balanced waves (64 lanes per row, one column tile of 64 kVec
// columns per workgroup).  A workgroup of kBalWaves waves takes kBalWaves
// rows chosen in serpentine order over the work slots -- g, 2G-1-g, 2G+g,
// 4G-1-g for group g of G -- so that, in the swizzled order (rows by nonzero
// count, longest first), each group pairs long rows with short ones.  A group
// whose longest row holds at most kBalSkew times the group's mean row length
// runs one row per wave, exactly as the wide kernel does (same staging, same
// summation).  Otherwise the group's entries, taken as one sequence (row after
// row), are cut into kBalWaves equal parts, one per wave; a wave accumulates
// each row piece of its part (the wide kernel's staging and gathers, with a
// wave-local barrier since the waves run different numbers of windows) and
// leaves the partial sums in LDS; then wave j adds row j's partial sums in
// wave order and writes the row.  Every wave thus streams about the group's
// mean row length, and the longest row no longer sets the launch's duration.
// Summation: in entry order within a piece, pieces in order; deterministic for
// a given row order.
constexpr int kBalWaves = 4;
constexpr int kBalSkewNum = 3, kBalSkewDen = 2;  // kBalSkew = 1.5

template <typename E, int kVec, bool kVecCsr, bool kBuf>
__global__ __launch_bounds__(kBalWaves * kWave) void spmm_balanced_kernel(SpmmParams p)
{
    using V = GVec<E, kVec>;
    constexpr int kChunk = kEpl * kWave;
    constexpr int kPitch = kChunk + kU + 4;
    __shared__ __align__(16) int s_off[kBalWaves * kPitch];
    __shared__ __align__(16) float s_val[kBalWaves * kPitch];
    __shared__ __align__(16) float s_part[kBalWaves][kBalWaves][kWave * kVec];
    __shared__ int s_row[kBalWaves], s_p0[kBalWaves], s_len[kBalWaves];

    const int groups = p.row_blocks;
    const long long w = xcd_work_index((long long)p.batch * p.tiles, groups);
    if (w < 0) return;  // uniform over the workgroup
    const long long per_z = (long long)p.tiles * groups;
    const long long z = w / per_z;
    const int tile = (int)((w - z * per_z) / groups);
    const int g = (int)(w - z * per_z - (long long)tile * groups);
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x - wave * kWave;

    if (lane == 0) {
        const int half = wave >> 1;
        const int slot = (wave & 1) ? half * 2 * groups + 2 * groups - 1 - g
                                    : half * 2 * groups + g;
        int row = -1, p0 = 0, len = 0;
        if (slot < p.m) {
            row = p.row_indices ? p.row_indices[slot] : slot;
            p0 = p.row_offsets[row];
            len = p.row_offsets[row + 1] - p0;
        }
        s_row[wave] = row;
        s_p0[wave] = p0;
        s_len[wave] = len;
    }
    __syncthreads();
    int cum[kBalWaves + 1];
    int longest = 0;
    cum[0] = 0;
#pragma unroll
    for (int j = 0; j < kBalWaves; ++j) {
        cum[j + 1] = cum[j] + s_len[j];
        longest = max(longest, s_len[j]);
    }
    const long long total = cum[kBalWaves];
    auto part_lo = [&](int v) { return (int)(total * v / kBalWaves); };

    const E *__restrict__ vals = static_cast<const E *>(p.values) + z * p.stride_values;
    const E *__restrict__ bz = static_cast<const E *>(p.b) + z * p.stride_b;
    const int col0 = (tile * kWave + lane) * kVec;
    const bool col_ok = col0 < p.n;
    float *cz = p.c + z * p.stride_c;
    // Rows of similar length (uniform over the workgroup): one row per wave.
    if ((long long)kBalWaves * kBalSkewDen * longest <= (long long)kBalSkewNum * total) {
        const int row = s_row[wave];
        if (row < 0) return;
        float acc[kVec];
#pragma unroll
        for (int t = 0; t < kVec; ++t) acc[t] = 0.f;
        wide_accumulate<E, kWave, kVec, kVecCsr, kBuf, true>(
            p, vals, bz, s_p0[wave], s_p0[wave] + s_len[wave], lane, col0, col_ok,
            s_off + wave * kPitch, s_val + wave * kPitch, acc);
        if (col_ok) V::store(cz + (size_t)row * (size_t)p.n + col0, acc);
        return;
    }
    const int lo_w = part_lo(wave), hi_w = part_lo(wave + 1);
#pragma unroll
    for (int j = 0; j < kBalWaves; ++j) {
        const int lo = max(lo_w, cum[j]), hi = min(hi_w, cum[j + 1]);
        if (lo >= hi) continue;  // uniform over the wave
        float acc[kVec];
#pragma unroll
        for (int t = 0; t < kVec; ++t) acc[t] = 0.f;
        wide_accumulate<E, kWave, kVec, kVecCsr, kBuf, true>(
            p, vals, bz, s_p0[j] + lo - cum[j], s_p0[j] + hi - cum[j], lane, col0, col_ok,
            s_off + wave * kPitch, s_val + wave * kPitch, acc);
#pragma unroll
        for (int t = 0; t < kVec; ++t) s_part[j][wave][lane * kVec + t] = acc[t];
    }
    __syncthreads();
    const int row = s_row[wave];
    if (row < 0 || !col_ok) return;
    float acc[kVec];
#pragma unroll
    for (int t = 0; t < kVec; ++t) acc[t] = 0.f;
#pragma unroll
    for (int v = 0; v < kBalWaves; ++v) {
        const int lo = max(part_lo(v), cum[wave]), hi = min(part_lo(v + 1), cum[wave + 1]);
        if (lo < hi) {
#pragma unroll
            for (int t = 0; t < kVec; ++t) acc[t] += s_part[wave][v][lane * kVec + t];
        }
    }
    V::store(cz + (size_t)row * (size_t)p.n + col0, acc);
}

// Few, long rows: the wide launch would leave most SIMDs with one wave or
// none.  Each row's entries are cut into kSplitWaves equal parts, taken by the
// kSplitWaves waves of a workgroup (each wave laid out as the wide kernel,
// kLpr lanes per row, over its part); wave 0 then adds the parts' partial
// sums in part order from LDS and writes the rows.  Summation: entry order
// within a part, parts in order; deterministic.
constexpr int kSplitWaves = 4;
constexpr int kSplitMinLength = 256;  // mean entries per row for the split kernel
constexpr int kSimdsPerCu = 4;

template <typename E, int kLpr, int kVec>
__global__ __launch_bounds__(kSplitWaves * kWave) void spmm_split_kernel(SpmmParams p)
{
    using V = GVec<E, kVec>;
    constexpr int kRpw = kWave / kLpr;
    constexpr int kChunk = kEpl * kLpr;
    constexpr int kPitch = kChunk + kU + 4;
    __shared__ __align__(16) int s_off[kSplitWaves * kRpw * kPitch];
    __shared__ __align__(16) float s_val[kSplitWaves * kRpw * kPitch];
    __shared__ __align__(16) float s_part[kSplitWaves][kWave * kVec];

    const long long w = wide_work(p, blockIdx.x);
    if (w < 0) return;  // uniform over the workgroup
    const long long per_z = (long long)p.tiles * p.row_blocks;
    const long long z = w / per_z;
    const int tile = (int)((w - z * per_z) / p.row_blocks);
    const int rb = (int)(w - z * per_z - (long long)tile * p.row_blocks);
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x - wave * kWave;
    const int grp = kRpw == 1 ? 0 : lane / kLpr;
    const int gl = kRpw == 1 ? lane : lane - grp * kLpr;
    const E *__restrict__ vals = static_cast<const E *>(p.values) + z * p.stride_values;
    const E *__restrict__ bz = static_cast<const E *>(p.b) + z * p.stride_b;

    const int slot = rb * kRpw + grp;
    const bool has_row = slot < p.m;
    const int row = has_row ? (p.row_indices ? p.row_indices[slot] : slot) : 0;
    const int p0 = has_row ? p.row_offsets[row] : 0;
    const int p1 = has_row ? p.row_offsets[row + 1] : 0;
    const long long len = p1 - p0;
    const int q0 = p0 + (int)(len * wave / kSplitWaves);
    const int q1 = p0 + (int)(len * (wave + 1) / kSplitWaves);
    const int col0 = (tile * kLpr + gl) * kVec;
    const bool col_ok = col0 < p.n;
    float acc[kVec];
#pragma unroll
    for (int t = 0; t < kVec; ++t) acc[t] = 0.f;
    wide_accumulate<E, kLpr, kVec, true, true, true>(p, vals, bz, q0, q1, gl, col0, col_ok,
                                                     s_off + (wave * kRpw + grp) * kPitch,
                                                     s_val + (wave * kRpw + grp) * kPitch, acc);
#pragma unroll
    for (int t = 0; t < kVec; ++t) s_part[wave][lane * kVec + t] = acc[t];
    __syncthreads();
    if (wave != 0 || !has_row || !col_ok) return;
#pragma unroll
    for (int t = 0; t < kVec; ++t) acc[t] = 0.f;
#pragma unroll
    for (int v = 0; v < kSplitWaves; ++v) {
#pragma unroll
        for (int t = 0; t < kVec; ++t) acc[t] += s_part[v][lane * kVec + t];
    }
    float *cz = p.c + z * p.stride_c;
    V::store(cz + (size_t)row * (size_t)p.n + col0, acc);
}

// Narrow B (n of at most 16 columns): the lane-over-columns mapping above
// would leave most of a row group idle, so here the lanes of one wave split
// a row's entries instead.  Lane (s, v) handles entries s, s + kS, s + 2kS, ...
// of the row (kS = 64 / kE entry slots) and the v-th vector of kVec columns
// of B (kE vectors cover the row of B).  Column indices and values are read
// through buffer resources (out-of-range past the row's end: zeros, no
// traffic); each lane sums its entries in order, then the kS partial sums of
// each column vector are added across lanes (DPP rotations inside 16-lane
// rows, then lane swaps between rows and between wave halves).
// Deterministic; a different (tree) order from the wide kernel.
// Batched fp32 SpMM over a structure whose neighbouring rows share most of
// their columns (sparse attention's P V: 32 heads, one mask).  A workgroup
// takes a panel of 16 consecutive rows and 4 batch entries and forms the
// panel's column union once (panel_union.h); each wave then computes its batch
// entry's C[panel] = A[panel, union] B[union] with v_mfma_f32_16x16x4f32, every
// union row of B loaded once per panel instead of once per entry.  Per
// 64-column block of C and per step of 4 union slots, lane l supplies
// A[row l % 16][slot 4 st + l / 16] (the entry map gives the entry, a buffer
// load its value; 0 where the row has no entry) and B[union row 4 st + l / 16]
// [4 (l % 16) ... + 3]; the four MFMAs of a step take one of those columns
// each, so lane l's accumulators hold C[4 (l / 16) + r][4 (l % 16) + c] and
// leave as one 16-byte store per row.  A tile multiplies the zeros of absent
// entries by B rows: a B value that is not finite would make 0 x Inf = NaN
// where the per-entry result is finite, so a wave that loads one redoes its
// panel on the per-entry path.  Panels whose union is too wide for their entry
// count take that path too: the wide kernel's accumulation (wide_accumulate)
// on the panel's rows, bit-identical to the wide kernel.  Tile sums round in
// the MFMA's order, within the same bound.
namespace pu = panel_union;

// Waves per SIMD the union SpMM asks the compiler for.  Its tiles are loaded
// just before use (no second tile in flight), so more resident waves hide the
// loads: 8 for fp32 at n = 64 (attention's P V; 12 % faster than without a
// bound, 1 VGPR spilled on the per-entry path), 6 elsewhere (8 would spill
// the 16-bit per-entry paths).
template <typename E, int kLpr>
constexpr int union_spmm_waves()
{
    return (sizeof(E) == 4 && kLpr == 16) ? 8 : 6;
}

template <typename E, int kLpr, bool kVecCsr>
__global__ __launch_bounds__(pu::kThreads, (union_spmm_waves<E, kLpr>())) void spmm_union_kernel(
    SpmmParams p)
{
    typedef float f4 __attribute__((ext_vector_type(4)));
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    constexpr int kVec = 16 / (int)Elem<E>::kBytes;  // elements per 16-byte vector
    constexpr unsigned kEb = Elem<E>::kBytes;
    using VE = GVec<E, kVec>;
    constexpr int kBlocks = kLpr * kVec / 64;  // 64-column blocks of C: n = kLpr kVec
    constexpr int kRpw = kWave / kLpr;  // rows per wave on the per-entry path
    constexpr int kChunk = kEpl * kLpr;
    constexpr int kPitch = kChunk + kU + 4;
    __shared__ pu::Shared s;
    __shared__ __align__(16) int s_off[pu::kWaves * kRpw * kPitch];
    __shared__ __align__(16) float s_val[pu::kWaves * kRpw * kPitch];
    extern __shared__ unsigned s_dyn[];
    pu::Panel pp;
    if (!pu::panel_of(p.m, p.batch, p.row_offsets, pp)) return;
    // an empty panel stores zeros through the tile path (no tiles)
    const int nu = pp.pn > 0 ? pu::build(p.row_offsets, p.col_indices, p.k, pp, s, s_dyn) : 0;
    // (uniform in the wave; the buffer resources below depend on it)
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int z = pp.hg * pu::kWaves + wave;
    if (z >= p.batch) return;
    const E *vals = static_cast<const E *>(p.values) + z * p.stride_values;
    const E *bz = static_cast<const E *>(p.b) + z * p.stride_b;
    float *cz = p.c + z * p.stride_c;

    auto per_entry = [&]() {
        const int grp = lane / kLpr, gl = lane % kLpr;
        int *g_off = s_off + (wave * kRpw + grp) * kPitch;
        float *g_val = s_val + (wave * kRpw + grp) * kPitch;
#pragma unroll 1
        for (int u = 0; u < pu::kRows / kRpw; ++u) {
            const int slot = u * kRpw + grp;
            const bool has = slot < pp.nr;
            const int row = pp.r0 + (has ? slot : 0);
            const int p0 = has ? p.row_offsets[row] : 0;
            const int p1 = has ? p.row_offsets[row + 1] : 0;
            float acc[kVec];
#pragma unroll
            for (int t = 0; t < kVec; ++t) acc[t] = 0.f;
            wide_accumulate<E, kLpr, kVec, kVecCsr, true, true>(p, vals, bz, p0, p1, gl,
                                                                kVec * gl, true, g_off, g_val, acc);
            if (has) VE::store(cz + (size_t)row * (size_t)p.n + kVec * gl, acc);
        }
    };
    if (nu < 0) {
        per_entry();
        return;
    }

    const int ntiles = (nu + 15) / 16;
    const unsigned rowbytes = (unsigned)p.n * kEb;   // a row of B
    const unsigned crowbytes = (unsigned)p.n * 4u;   // a row of the fp32 C
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<E *>(vals), 0, (int)p.csr_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<E *>(bz), 0, (int)p.b_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rc =
        __builtin_amdgcn_make_buffer_rsrc(cz, 0, (int)p.c_bytes, 0x00020000);
    const int jl = lane % 16;  // the lane's row of A, column group of B and C
    const int q = lane / 16;   // the lane's union slot within a step
    struct Tile {
        float a[4];
        float b[4][4];
    };
    bool finite = true;
#pragma unroll 1
    for (int cb = 0; cb < kBlocks; ++cb) {
        const unsigned col = (unsigned)(64 * cb + 4 * jl);  // the lane's first column of C
        auto load = [&](int T, Tile &t) {
            // the step's map entries and union columns first (clamped slots,
            // so every read is in bounds; slots past the union are not used)
            unsigned idx[4], ucol[4];
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int uc = min(16 * T + 4 * st + q, pu::kMaxCols - 1);
                idx[st] = s.emap[jl * pu::kEmapStride + uc];
                ucol[st] = (unsigned)s.ucol[uc];
            }
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const bool ok = 16 * T + 4 * st + q < nu;
                const unsigned vo =
                    ok && idx[st] ? (unsigned)(pp.e0 + (int)idx[st] - 1) * kEb : kOutOfRange;
                if constexpr (__is_same(E, float)) {
                    t.a[st] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rv, (int)vo, 0, 0));
                } else {
                    const unsigned short h = __builtin_amdgcn_raw_buffer_load_b16(rv, (int)vo, 0, 0);
                    t.a[st] = Elem<E>::lo(h);
                }
                const unsigned base = ok ? ucol[st] * rowbytes : kOutOfRange;
                load_widen<E, 4>(rb, base + col * kEb | (base & kOutOfRange), t.b[st]);
            }
        };
        f4 acc[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = f4{0.f, 0.f, 0.f, 0.f};
        auto mma = [&](const Tile &t) {
#pragma unroll
            for (int st = 0; st < 4; ++st) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    finite = finite && __builtin_isfinite(t.b[st][c]);
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(t.a[st], t.b[st][c], acc[c], 0,
                                                                  0, 0);
                }
            }
        };
        for (int T = 0; T < ntiles; ++T) {
            Tile t;
            load(T, t);
            mma(t);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 4 * q + r;
            const unsigned off =
                row < pp.nr ? (unsigned)(pp.r0 + row) * crowbytes + col * 4u : kOutOfRange;
            const u4 ov = {__float_as_uint(acc[0][r]), __float_as_uint(acc[1][r]),
                           __float_as_uint(acc[2][r]), __float_as_uint(acc[3][r])};
            __builtin_amdgcn_raw_buffer_store_b128(ov, rc, (int)off, 0, 0);
        }
    }
    // a non-finite B value in this wave's union rows: the per-entry sums
    // replace what the tiles stored (same wave, so the stores stay in order)
    if (__builtin_amdgcn_ballot_w64(!finite) != 0) per_entry();
}

template <int kE, int kVec>
__global__ __launch_bounds__(kWave) void spmm_narrow_kernel(SpmmParams p)
{
    using V = Vec<kVec>;
    using VecT = typename V::T;
    constexpr int kS = kWave / kE;  // entries per step
    constexpr int kSteps = 8;       // steps per batch (CSR loads, then gathers)
    const long long w = xcd_work_index(p.batch, p.m);
    if (w < 0) return;
    const long long z = w / p.m;
    const int slot = (int)(w - z * p.m);
    const int lane = threadIdx.x;
    const int s = lane / kE;
    const int v = lane - s * kE;
    const int row = p.row_indices ? p.row_indices[slot] : slot;
    const int p0 = p.row_offsets[row];
    const int p1 = p.row_offsets[row + 1];
    const float *vals = static_cast<const float *>(p.values) + z * p.stride_values;
    const float *bz = static_cast<const float *>(p.b) + z * p.stride_b;
    float *cz = p.c + z * p.stride_c;
    const int col0 = v * kVec;
    const bool col_ok = col0 < p.n;
    const unsigned lane_bytes = col_ok ? (unsigned)col0 * 4u : kOutOfRange;
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(bz), 0, (int)p.b_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int *>(p.col_indices), 0, (int)p.csr_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(vals), 0, (int)p.csr_bytes, 0x00020000);

    float acc[kVec];
#pragma unroll
    for (int t = 0; t < kVec; ++t) acc[t] = 0.f;
    for (int base = p0; base < p1; base += kS * kSteps) {  // wave-uniform bound
        unsigned coff[kSteps];
        int cc[kSteps];
        float vv[kSteps];
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            const int idx = base + u * kS + s;
            coff[u] = idx < p1 ? (unsigned)idx * 4u : kOutOfRange;
        }
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            cc[u] = (int)__builtin_amdgcn_raw_buffer_load_b32(rc, (int)coff[u], 0, 0);
            vv[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rv, (int)coff[u], 0, 0));
        }
        VecT bv[kSteps];
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            const unsigned off = coff[u] == kOutOfRange
                                     ? kOutOfRange
                                     : (unsigned)cc[u] * (unsigned)p.n * 4u + lane_bytes;
            bv[u] = V::buf_load(rb, off);
        }
#pragma unroll
        for (int u = 0; u < kSteps; ++u) V::fma(vv[u], bv[u], acc);
    }
#pragma unroll
    for (int t = 0; t < kVec; ++t) acc[t] = strided_wave_sum<kE>(acc[t]);
    if (s == 0 && col_ok) V::store(cz + (size_t)row * (size_t)p.n + col0, acc);
}

// Narrow B that fits in LDS, with many entries per B element: the streaming
// regime, where the CSR arrays (8 bytes per entry) are the traffic that must
// reach HBM speed.  One 1024-thread workgroup per CU copies B into LDS once;
// its 16 waves then take rows (in row_indices order, round-robin over all
// waves of the launch).  When all of B does not fit, B is cut into S column
// slices that do: the grid is S groups of workgroups, each holding one slice
// and taking every row for that slice's columns of C, and the S workgroups
// that take the same rows are launched on the same XCD (block ids 8 apart)
// at the same time, so the second and later reads of those rows' CSR entries
// come from that XCD's L2 rather than HBM.  Lanes split a row's entries in 16-byte segments of 4
// (lane (s, v): segments s, s + kS, ...; the kE lanes of a segment cover the
// kE column vectors of B), and each segment's column indices and values are
// read with one dwordx4 buffer load each, starting from the row's first entry
// rounded down to a multiple of 4 (entries outside the row are skipped).  With
// the LDS holding B, only 16 waves fit on a CU, so the 16-byte reads are what
// keeps enough bytes in flight to stream from HBM.  Batches are issued
// unconditionally and double-buffered across row boundaries: the wave walks
// its (row, batch) pairs as one sequence, and the metadata of its next 64 rows
// sits one row per lane in registers (read with readlane), so a row change
// costs no memory operation.  The array's last segment, if it extends past
// nnz, is read from the last 4 entries instead (positions before the segment's
// first entry are skipped), so no load is ever partly out of range.  A zero
// vector stored after B in LDS
// stands in for the entries of a segment that lie outside the row (with value
// 0): every entry slot is one unconditional LDS read and FMA, adding +0
// exactly, with no branch, so a batch's reads are all issued before its FMAs.
// E is the element type of the values and of B: fp16 and bf16 B is widened
// to fp32 as it is copied into LDS (the LDS layout, reads and FMAs are those of
// fp32), or, with kVec == 8, kept 16-bit there (8 elements per 16-byte vector,
// widened at the FMA: half the LDS, so fewer column slices); a segment's four
// 16-bit values are read with one 8-byte buffer load and widened when
// consumed: the CSR then streams 6 bytes per entry
// instead of 8.  In the 16-bit form every segment, the array's last included,
// is read from its own first entry: its 4-byte words past the end of the
// column array (or past the value array rounded up to whole words) are out of
// the buffer's range and read as zeros.
constexpr int kLdsThreads = 1024;
constexpr int kLdsWaves = kLdsThreads / kWave;
constexpr unsigned kLdsMaxB = 128u * 1024u;

template <typename E, int kE, int kVec>
__global__ __launch_bounds__(kLdsThreads) void spmm_lds_kernel(SpmmParams p)
{
    constexpr unsigned kEb = Elem<E>::kBytes;
    // B in LDS: fp32 vectors of kVec (fp32 B, or 16-bit B widened on the copy),
    // or -- kVec == 8 -- 16-bit B as it is, 8 elements per 16-byte vector,
    // widened at the FMA
    constexpr bool kRaw16 = kEb == 2 && kVec == 8;
    using V = std::conditional_t<kRaw16, GVec<E, 8>, Vec<kVec == 8 ? 4 : kVec>>;
    using VecT = typename V::T;
    constexpr int kS = kWave / kE;  // segment slots per step
    constexpr int kSteps = 4;       // steps per batch
    constexpr int kBatch = kSteps * kS * 4;  // entries per batch
    extern __shared__ __align__(16) float s_b[];

    // ---- this workgroup's slice and row group
    const int n_slices = p.lds_slices;
    const int groups = (int)gridDim.x / n_slices;
    int slice = 0, group = (int)blockIdx.x;
    if (n_slices > 1) {  // gridDim.x is a multiple of 8 * n_slices
        slice = (int)(blockIdx.x / 8) % n_slices;
        group = (int)(blockIdx.x / (8 * n_slices)) * 8 + (int)(blockIdx.x % 8);
    }
    const int col_base = slice * p.lds_slice_n;
    const int width = min(p.lds_slice_n, p.n - col_base);  // columns of this slice
    const int wv = width / kVec;                            // vectors per B row in LDS

    // ---- B's slice into LDS, k x width row-major
    const int tid = threadIdx.x;
    VecT *s_bv = reinterpret_cast<VecT *>(s_b);
    const int total = p.k * wv;
    if (tid == 0) s_bv[total] = VecT{};  // the zero vector
    if constexpr (kEb == 2 && !kRaw16) {
        // 16-bit B: vector i of the slice holds B[r][col .. col + kVec) widened
        const E *__restrict__ b16 = static_cast<const E *>(p.b);
        for (int i = tid; i < total; i += kLdsThreads) {
            const int r = i / wv;
            const E *src = b16 + (size_t)r * p.n + col_base + (i - r * wv) * kVec;
            if constexpr (kVec == 4) {
                const uint2 u = *reinterpret_cast<const uint2 *>(src);  // 8-byte aligned
                s_bv[i] = make_float4(Elem<E>::lo(u.x), Elem<E>::hi(u.x), Elem<E>::lo(u.y),
                                      Elem<E>::hi(u.y));
            } else {
                s_bv[i] = Elem<E>::f32(*src);
            }
        }
    } else if (n_slices == 1) {
        const VecT *__restrict__ bsrc = static_cast<const VecT *>(p.b);
        for (int i = tid; i < total; i += kLdsThreads) s_bv[i] = bsrc[i];
    } else {
        const VecT *__restrict__ bsrc = static_cast<const VecT *>(p.b);
        const int nv_all = p.n / kVec, vbase = col_base / kVec;
        for (int i = tid; i < total; i += kLdsThreads) {
            const int r = i / wv;
            s_bv[i] = bsrc[(size_t)r * nv_all + vbase + (i - r * wv)];
        }
    }
    __syncthreads();

    const int lane = tid % kWave;
    const int s = lane / kE;
    const int v = lane - s * kE;
    const int col0 = v * kVec;
    const bool col_ok = col0 < width;
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int *>(p.col_indices), 0, (int)p.csr_bytes, 0x00020000);
    // 16-bit values: the range is rounded up to whole dwords (the array's last
    // dword may hold one value and 2 bytes beyond it, within the same page)
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(p.values), 0,
        (int)(kEb == 4 ? p.csr_bytes : (p.csr_bytes / 2u + 3u) & ~3u), 0x00020000);
    const int last4 = p.nnz - 4;  // first entry of the array's last full segment (nnz >= 4)

    const int *__restrict__ order = p.row_indices;
    const int *__restrict__ offsets = p.row_offsets;
    const int stride = groups * kLdsWaves;
    // wave-uniform (scalar), so that every branch on the rows is a scalar one
    const int first = __builtin_amdgcn_readfirstlane(group * kLdsWaves + tid / kWave);
    if (first >= p.m) return;  // no LDS barrier follows
    const int rows_of_wave = (p.m - first + stride - 1) / stride;

    int meta_row = 0, meta_p0 = 0, meta_p1 = 0, meta_base = 0;
    // Row metadata of 64 of the wave's rows, one per lane; the loads are
    // unconditional, from valid addresses (row_offsets stands in for a missing
    // row order), so no branch surrounds them.
    auto load_meta = [&](int t0) {
        const int t = t0 + lane;
        const bool ok = t < rows_of_wave;
        const int sl = ok ? first + t * stride : first;
        const int o = (order ? order : offsets)[sl];
        const int row = order ? o : sl;
        const int q0 = offsets[row];
        const int q1 = offsets[row + 1];
        meta_row = ok ? row : 0;
        meta_p0 = ok ? q0 : 0;
        meta_p1 = ok ? q1 : 0;
        meta_base = __builtin_amdgcn_readfirstlane(t0);
    };
    struct Batch {
        int t, row, p0, p1, base;  // base: first entry of the batch (a multiple of 4)
    };
    // Batch fields are wave-uniform (scalar registers), so the choices below
    // are scalar branches: a divergent branch around the metadata loads would
    // make the compiler wait for every load in flight where it joins.
    auto uniform = [](Batch b) -> Batch {
        return {__builtin_amdgcn_readfirstlane(b.t), __builtin_amdgcn_readfirstlane(b.row),
                __builtin_amdgcn_readfirstlane(b.p0), __builtin_amdgcn_readfirstlane(b.p1),
                __builtin_amdgcn_readfirstlane(b.base)};
    };
    auto row_batch = [&](int t) -> Batch {
        if (t - meta_base >= kWave) load_meta(t);
        const int j = t - meta_base;
        const int p0 = __builtin_amdgcn_readlane(meta_p0, j);
        return uniform({t, __builtin_amdgcn_readlane(meta_row, j), p0,
                        __builtin_amdgcn_readlane(meta_p1, j), p0 & ~3});
    };
    auto next_of = [&](const Batch &cur) -> Batch {
        if (cur.base + kBatch < cur.p1)
            return uniform({cur.t, cur.row, cur.p0, cur.p1, cur.base + kBatch});
        if (cur.t + 1 >= rows_of_wave) return uniform({rows_of_wave, -1, 0, 0, 0});  // empty
        return row_batch(cur.t + 1);
    };

    struct Seg {
        int4 c;
        float4 v;
    };
    auto load = [&](const Batch &b, Seg (&sg)[kSteps]) {
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            const int e = b.base + (u * kS + s) * 4;
            const bool any = e < b.p1;
            // fp32: the array's last segment is read from its last 4 entries;
            // 16-bit: from the segment's own start, its dwords past the end
            // reading as zeros (range-checked per dword)
            const unsigned off = !any ? kOutOfRange
                                      : (unsigned)(kEb == 2 ? e : min(e, last4)) * 4u;
            const auto c4 = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)off, 0, 0);
            sg[u].c = make_int4((int)c4[0], (int)c4[1], (int)c4[2], (int)c4[3]);
            if constexpr (kEb == 4) {
                const auto v4 = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)off, 0, 0);
                sg[u].v = make_float4(__uint_as_float(v4[0]), __uint_as_float(v4[1]),
                                      __uint_as_float(v4[2]), __uint_as_float(v4[3]));
            } else {
                // the four raw 16-bit values in two dwords, widened only when
                // consumed (so that no instruction here waits for the load)
                const auto v2 = __builtin_amdgcn_raw_buffer_load_b64(
                    rv, (int)(off == kOutOfRange ? kOutOfRange : off / 2u), 0, 0);
                sg[u].v = make_float4(__uint_as_float(v2[0]), __uint_as_float(v2[1]), 0.f, 0.f);
            }
        }
    };
    const unsigned row_bytes = (unsigned)wv * sizeof(VecT);   // one row of B in LDS
    // 32-bit LDS addresses of this lane's vector in B's first row and of the
    // zero vector, so that each entry's address is one multiply-add
    const unsigned lds_b = lds_address(s_bv);
    const unsigned lds_lane = lds_b + (unsigned)v * sizeof(VecT);
    const unsigned lds_zero = lds_b + (unsigned)total * sizeof(VecT);
    auto consume = [&](const Batch &b, const Seg (&sg)[kSteps], float *acc) {
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            const int e = b.base + (u * kS + s) * 4;
            // The segment was loaded from entry e_ld: e, or (fp32) last4 for the
            // array's final segment (whose positions before e belong to the
            // segment before it; e + 4 > nnz exactly when e > last4).
            // Position t holds entry e_ld + t, which is this lane's when
            // lo <= e_ld + t < p1 with lo = max(p0, e); an idle lane (no
            // column vector) takes none.
            const int e_ld = kEb == 2 ? e : min(e, last4);
            const int lo = max(b.p0, e);
            const unsigned span = (col_ok && b.p1 > lo) ? (unsigned)(b.p1 - lo) : 0u;
            const int d = e_ld - lo;
            const int cs[4] = {sg[u].c.x, sg[u].c.y, sg[u].c.z, sg[u].c.w};
            float vs[4] = {sg[u].v.x, sg[u].v.y, sg[u].v.z, sg[u].v.w};
            if constexpr (kEb == 2) {
                const unsigned w0 = __float_as_uint(sg[u].v.x), w1 = __float_as_uint(sg[u].v.y);
                vs[0] = Elem<E>::lo(w0);
                vs[1] = Elem<E>::hi(w0);
                vs[2] = Elem<E>::lo(w1);
                vs[3] = Elem<E>::hi(w1);
            }
            VecT bv[4];
            float val[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bool in_row = (unsigned)(d + t) < span;
                // Address of row col of B, this lane's vector (or of the zero
                // vector); 16-byte aligned, so the read is one ds_read_b128.
                const unsigned a =
                    in_row ? __umul24((unsigned)cs[t], row_bytes) + lds_lane : lds_zero;
                val[t] = in_row ? vs[t] : 0.f;
                bv[t] = lds_read<VecT>(a);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) V::fma(val[t], bv[t], acc);
        }
    };
    float acc[kVec];
#pragma unroll
    for (int t = 0; t < kVec; ++t) acc[t] = 0.f;
    // C is written through a buffer resource: a lane that does not hold the
    // row's sum stores to an out-of-range offset, which the hardware drops.
    // A store under a branch would leave the compiler unsure how many memory
    // operations are in flight, and it would then wait for all of them at
    // the top of every batch, draining the loads kept in flight.
    const __amdgpu_buffer_rsrc_t rcs =
        __builtin_amdgcn_make_buffer_rsrc(p.c, 0, (int)p.c_bytes, 0x00020000);
    auto finish_row = [&](int r) {
#pragma unroll
        for (int t = 0; t < kVec; ++t) acc[t] = strided_wave_sum<kE>(acc[t]);
        const unsigned off =
            s == 0 && col_ok ? (unsigned)(((size_t)r * (size_t)p.n + col_base + col0) * 4u)
                             : kOutOfRange;
        if constexpr (kVec == 1) {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[0]), rcs, (int)off, 0, 0);
        } else {
#pragma unroll
            for (int h = 0; h < kVec / 4; ++h) {
                const unsigned v4 __attribute__((ext_vector_type(4))) = {
                    __float_as_uint(acc[4 * h]), __float_as_uint(acc[4 * h + 1]),
                    __float_as_uint(acc[4 * h + 2]), __float_as_uint(acc[4 * h + 3])};
                __builtin_amdgcn_raw_buffer_store_b128(v4, rcs, (int)(off + 16u * h), 0, 0);
            }
        }
#pragma unroll
        for (int t = 0; t < kVec; ++t) acc[t] = 0.f;
    };

    meta_base = __builtin_amdgcn_readfirstlane(meta_base);
    load_meta(0);
    Batch cur = row_batch(0);
    Seg sa[kSteps], sb[kSteps];
    load(cur, sa);
    // One exit, at the end: a second exit after the first half would give the
    // loop header an edge on which the first half's loads are still pending,
    // and the compiler would then wait for every load in flight at the top of
    // each iteration.  When the first half reaches the empty batch, the second
    // half runs on it as a no-op (out-of-range loads, zero terms, no row end).
    for (;;) {
        // Issued unconditionally (an empty next batch is all out of range),
        // which keeps the compiler's wait counts exact.
        const Batch nb = next_of(cur);
        load(nb, sb);
        keep_issued_above();
        consume(cur, sa, acc);
        if (nb.t != cur.t) finish_row(cur.row);
        cur = nb;
        const Batch na = next_of(cur);
        load(na, sa);
        keep_issued_above();
        consume(cur, sb, acc);
        if (na.t != cur.t) finish_row(cur.row);
        if (na.row < 0) break;
        cur = na;
    }
}

template <typename E, int kE, int kVec>
hipError_t launch_lds_t(const SpmmParams &p, int blocks, hipStream_t s)
{
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&spmm_lds_kernel<E, kE, kVec>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kLdsMaxB + 16u));
    if (e != hipSuccess) return e;
    // B's slice and the zero vector
    // B's slice and the zero vector, fp32 in LDS (or 16-bit B kept 16-bit: kVec 8)
    constexpr size_t kLdsEb = (Elem<E>::kBytes == 2 && kVec == 8) ? 2u : 4u;
    const size_t lds_bytes = ((size_t)p.k * (size_t)p.lds_slice_n + kVec) * kLdsEb;
    hipLaunchKernelGGL((spmm_lds_kernel<E, kE, kVec>), dim3(blocks), dim3(kLdsThreads),
                       lds_bytes, s, p);
    return hipGetLastError();
}

template <typename E, int kVec>
hipError_t launch_lds(int e, const SpmmParams &p, int blocks, hipStream_t s)
{
    switch (e) {
    case 1: return launch_lds_t<E, 1, kVec>(p, blocks, s);
    case 2: return launch_lds_t<E, 2, kVec>(p, blocks, s);
    default: return launch_lds_t<E, 4, kVec>(p, blocks, s);
    }
}

template <int kE, int kVec>
hipError_t launch_narrow_t(const SpmmParams &p, hipStream_t s)
{
    dim3 grid((unsigned)xcd_grid(p.batch, p.m));
    hipLaunchKernelGGL((spmm_narrow_kernel<kE, kVec>), grid, dim3(kWave), 0, s, p);
    return hipGetLastError();
}

template <int kVec>
hipError_t launch_narrow(int e, const SpmmParams &p, hipStream_t s)
{
    switch (e) {
    case 1: return launch_narrow_t<1, kVec>(p, s);
    case 2: return launch_narrow_t<2, kVec>(p, s);
    default: return launch_narrow_t<4, kVec>(p, s);
    }
}

template <typename E, int kLpr, int kVec, bool kVecCsr, bool kBuf>
hipError_t launch_t(const SpmmParams &p, hipStream_t s)
{
    dim3 grid((unsigned)wide_grid(p));
    hipLaunchKernelGGL((spmm_kernel<E, kLpr, kVec, kVecCsr, kBuf>), grid, dim3(kWave), 0, s, p);
    return hipGetLastError();
}

template <typename E, int kLpr, int kVec>
hipError_t launch_csr(const SpmmParams &p, bool vec_csr, bool buf, hipStream_t s)
{
    if (vec_csr)
        return buf ? launch_t<E, kLpr, kVec, true, true>(p, s)
                   : launch_t<E, kLpr, kVec, true, false>(p, s);
    return buf ? launch_t<E, kLpr, kVec, false, true>(p, s)
               : launch_t<E, kLpr, kVec, false, false>(p, s);
}

template <typename E, int kVec>
hipError_t launch_lpr(int lpr, const SpmmParams &p, bool vec_csr, bool buf, hipStream_t s)
{
    switch (lpr) {
    case 8: return launch_csr<E, 8, kVec>(p, vec_csr, buf, s);
    case 16: return launch_csr<E, 16, kVec>(p, vec_csr, buf, s);
    case 32: return launch_csr<E, 32, kVec>(p, vec_csr, buf, s);
    default: return launch_csr<E, 64, kVec>(p, vec_csr, buf, s);
    }
}

// The wide kernel for element type E: 16-byte vectors (kVec16 elements) or
// single elements.
template <typename E, int kVec16>
hipError_t launch_wide(bool vec, int lpr, const SpmmParams &p, bool vec_csr, bool buf,
                       hipStream_t s)
{
    return vec ? launch_lpr<E, kVec16>(lpr, p, vec_csr, buf, s)
               : launch_lpr<E, 1>(lpr, p, vec_csr, buf, s);
}

template <typename E, int kVec>
hipError_t launch_split(int lpr, const SpmmParams &p, hipStream_t s)
{
    const dim3 grid((unsigned)wide_grid(p));
    const dim3 block(kSplitWaves * kWave);
    switch (lpr) {
    case 8: hipLaunchKernelGGL((spmm_split_kernel<E, 8, kVec>), grid, block, 0, s, p); break;
    case 16: hipLaunchKernelGGL((spmm_split_kernel<E, 16, kVec>), grid, block, 0, s, p); break;
    case 32: hipLaunchKernelGGL((spmm_split_kernel<E, 32, kVec>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((spmm_split_kernel<E, 64, kVec>), grid, block, 0, s, p); break;
    }
    return hipGetLastError();
}

template <typename E, int kLpr, bool kVecCsr>
hipError_t launch_union_t(const SpmmParams &p, hipStream_t s)
{
    hipLaunchKernelGGL((spmm_union_kernel<E, kLpr, kVecCsr>),
                       dim3((unsigned)pu::grid(p.m, p.batch)), dim3(pu::kThreads),
                       pu::dynamic_lds(p.k), s, p);
    return hipGetLastError();
}

// lpr: the wide kernel's lanes per row for n (n = lpr * elements per vector)
template <typename E, int kL0>
hipError_t launch_union_e(int lpr, bool vec_csr, const SpmmParams &p, hipStream_t s)
{
    if (lpr == kL0)
        return vec_csr ? launch_union_t<E, kL0, true>(p, s) : launch_union_t<E, kL0, false>(p, s);
    if (lpr == 2 * kL0)
        return vec_csr ? launch_union_t<E, 2 * kL0, true>(p, s)
                       : launch_union_t<E, 2 * kL0, false>(p, s);
    return vec_csr ? launch_union_t<E, 4 * kL0, true>(p, s)
                   : launch_union_t<E, 4 * kL0, false>(p, s);
}

hipError_t launch_union(Dtype dtype, int lpr, bool vec_csr, const SpmmParams &p, hipStream_t s)
{
    switch (dtype) {
    case Dtype::f16: return launch_union_e<_Float16, 8>(lpr, vec_csr, p, s);
    case Dtype::bf16: return launch_union_e<bf16, 8>(lpr, vec_csr, p, s);
    default: return launch_union_e<float, 16>(lpr, vec_csr, p, s);
    }
}

template <typename E, int kVec>
hipError_t launch_balanced(const SpmmParams &p, bool vec_csr, bool buf, hipStream_t s)
{
    const dim3 grid((unsigned)xcd_grid((long long)p.batch * p.tiles, p.row_blocks));
    const dim3 block(kBalWaves * kWave);
    if (vec_csr) {
        if (buf)
            hipLaunchKernelGGL((spmm_balanced_kernel<E, kVec, true, true>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((spmm_balanced_kernel<E, kVec, true, false>), grid, block, 0, s, p);
    } else {
        if (buf)
            hipLaunchKernelGGL((spmm_balanced_kernel<E, kVec, false, true>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((spmm_balanced_kernel<E, kVec, false, false>), grid, block, 0, s, p);
    }
    return hipGetLastError();
}

// The current device's compute units and LDS bytes per workgroup (false if
// they cannot be queried; variant selection then keeps the default kernels).
bool device_limits(int *cus, int *lds_max)
{
    int device = 0;
    return hipGetDevice(&device) == hipSuccess &&
           hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, device) ==
               hipSuccess &&
           hipDeviceGetAttribute(lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, device) ==
               hipSuccess;
}

inline bool aligned(const void *ptr, unsigned bytes)
{
    return (reinterpret_cast<uintptr_t>(ptr) & (bytes - 1u)) == 0;
}
inline bool aligned16(const void *ptr) { return aligned(ptr, 16); }

}  // namespace

// Lanes per row: the smallest of 8/16/32/64 that covers the row's vectors,
// else 64 with several column tiles.  A grid that would not fit the launch
// limits returns hipErrorInvalidConfiguration without launching.  fp16 and
// bf16 operands take the wide kernel with 8-element vectors (or single
// elements) for every width.
hipError_t plan_spmm(const SpmmArgs &a, SpmmPlan *plan)
{
    const bool f32 = a.dtype == Dtype::f32;
    const int eb = f32 ? 4 : 2;   // bytes per element of values and B
    const int vlen = 16 / eb;     // elements per 16-byte vector
    const bool vec = (a.n % vlen == 0) && aligned16(a.b) && aligned16(a.c) &&
                     (a.stride_b % vlen == 0) && (a.stride_c % 4 == 0);
    const bool vec_csr = aligned16(a.col_indices) && aligned(a.values, 4u * eb) &&
                         (a.stride_values % 4 == 0);
    // Valid offsets stay below B's size and padding offsets (>= 2^31) beyond it.
    const bool buf = (long long)a.k * (long long)a.n * eb <= (1LL << 31);
    const int kvec = vec ? vlen : 1;
    const int nv = (a.n + kvec - 1) / kvec;
    const int lpr = nv <= 8 ? 8 : nv <= 16 ? 16 : nv <= 32 ? 32 : 64;
    const int rpw = kWave / lpr;
    const int tiles = (nv + lpr - 1) / lpr;
    const long long row_blocks = ((long long)a.m + rpw - 1) / rpw;
    if (xcd_grid((long long)a.batch * tiles, row_blocks) > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;

    // Narrow B: lanes over entries (needs the buffer paths for B and the CSR).
    const bool narrow = f32 && buf && nv <= 4 && (long long)a.nnz * 4 <= (1LL << 31);
    // The LDS (streaming) kernel: fp32 as the narrow kernel.  16-bit B stays
    // 16-bit in LDS, 8 elements per 16-byte vector, when n % 8 == 0 and B and C
    // are 16-byte aligned; otherwise it is widened into LDS as fp32 vectors of
    // 4 (n % 4 == 0, B 8-byte aligned) or single elements.  lds_eb: bytes per
    // element of B in LDS.
    int lds_kvec = kvec, lds_nv = nv, lds_eb = 4;
    bool lds_ok = narrow;
    if (!f32) {
        if (a.n % 8 == 0 && aligned16(a.b) && aligned16(a.c) && a.stride_b % 8 == 0) {
            lds_kvec = 8;
            lds_eb = 2;
        } else {
            // C is stored in fp32 vectors of 4 as well
            lds_kvec = (a.n % 4 == 0 && aligned(a.b, 8) && a.stride_b % 4 == 0 &&
                        aligned16(a.c) && a.stride_c % 4 == 0) ? 4 : 1;
        }
        lds_nv = (a.n + lds_kvec - 1) / lds_kvec;
        lds_ok = buf && lds_nv <= 4 && (long long)a.nnz * 4 <= (1LL << 31);
    }
    if (narrow && xcd_grid(a.batch, a.m) > 0x7fffffffLL) return hipErrorInvalidConfiguration;

    SpmmParams &p = plan->p;
    p.m = a.m;
    p.n = a.n;
    p.nnz = a.nnz;
    p.row_blocks = (int)row_blocks;
    p.tiles = tiles;
    p.batch = a.batch;
    p.b_bytes = buf ? (unsigned)((long long)a.k * a.n * eb) : 0u;
    p.csr_bytes = (narrow || lds_ok) ? (unsigned)((long long)a.nnz * 4) : 0u;
    p.k = a.k;
    p.lds_slices = 1;
    p.lds_slice_n = a.n;
    p.row_indices = a.row_indices;
    p.row_offsets = a.row_offsets;
    p.col_indices = a.col_indices;
    p.values = a.values;
    p.b = a.b;
    p.c = a.c;
    p.stride_values = a.stride_values;
    p.stride_b = a.stride_b;
    p.stride_c = a.stride_c;
    plan->dtype = a.dtype;
    plan->vec = vec;
    plan->vec_csr = vec_csr;
    plan->buf = buf;
    plan->lpr = lpr;
    plan->e = nv <= 1 ? 1 : nv <= 2 ? 2 : 4;
    plan->blocks = 0;
    plan->kind = SpmmPlan::kWide;
    // The balanced kernel (groups of kBalWaves rows in place of row blocks): on
    // request; and by default for one batch entry in a given row order -- the
    // swizzled order of the card's I4 is what makes its serpentine groups pair
    // long rows with short ones -- unless the problem is a few long rows.
    const bool balance_ok = lpr == kWave;
    if (balance_ok && a.balanced) {
        plan->kind = SpmmPlan::kBalanced;
    } else if (vec_csr && buf && (long long)a.nnz >= kSplitMinLength * (long long)a.m) {
        // Few, long rows: fewer than two waves per SIMD in the wide launch.
        int cus = 0, lds_max = 0;
        if (device_limits(&cus, &lds_max) &&
            (long long)a.batch * tiles * row_blocks < 2LL * kSimdsPerCu * cus)
            plan->kind = SpmmPlan::kSplit;
    }
    if (plan->kind == SpmmPlan::kWide && balance_ok && a.auto_balance &&
        a.row_indices != nullptr && a.batch == 1)
        plan->kind = SpmmPlan::kBalanced;
    if (plan->kind == SpmmPlan::kBalanced)
        p.row_blocks = (int)(((long long)a.m + kBalWaves - 1) / kBalWaves);
    // B shared in LDS by a panel of rows: fp32 vector paths, one batch entry.
    if (f32 && vec && vec_csr && a.batch == 1 && a.k > 0 && a.m > 0 && !a.balanced) {
        int cus = 0, lds_max = 0;
        if (device_limits(&cus, &lds_max)) {
            if (panel_fits<PanelMany>(a, cus, lds_max, &plan->q)) {
                plan->kind = SpmmPlan::kPanel;
                plan->panel = 0;
            } else if (panel_fits<PanelFew>(a, cus, lds_max, &plan->q)) {
                plan->kind = SpmmPlan::kPanel;
                plan->panel = 1;
            }
        }
    }
    // Batched problems of 64, 128 or 256 columns on up to 65,536 rows of B: the
    // panel-union kernel, which falls back to the wide kernel's accumulation
    // panel by panel where rows share few columns.
    if (plan->kind == SpmmPlan::kWide && vec && buf && a.batch >= 2 && a.k <= pu::kMaxK &&
        (a.n == 64 || a.n == 128 || a.n == 256) && (long long)a.m * a.n * 4 < (1LL << 31) &&
        (long long)a.nnz * eb < (1LL << 31) && pu::grid(a.m, a.batch) <= 0x7fffffffLL) {
        plan->kind = SpmmPlan::kUnion;
        p.c_bytes = (unsigned)((long long)a.m * a.n * 4);
        p.csr_bytes = (unsigned)((long long)a.nnz * eb);
    }
    if (narrow) plan->kind = SpmmPlan::kNarrow;
    if (lds_ok) {
        // B in LDS when it fits and every CU has at least as many entries to
        // stream as it copies B elements (nnz >= CUs * k * n).
        int cus = 0, lds_max = 0;
        if (!device_limits(&cus, &lds_max)) cus = 0;
        // B, or when it does not fit, S column slices of B: the widest
        // slice (in vectors of kvec columns) that fits, then the S slices
        // evened out.  Every group of S workgroups (one per CU) must stream at
        // least as many entries as each copies B elements: nnz >= (CUs / S)
        // * k * slice columns.
        const long long lds_cap = std::min<long long>(kLdsMaxB, lds_max - 16);
        const long long row_bytes = (long long)a.k * lds_kvec * lds_eb;  // one vector column of B
        long long slice_v = row_bytes > 0 ? std::min<long long>(lds_nv, lds_cap / row_bytes) : 0;
        const int slices = slice_v > 0 ? (int)((lds_nv + slice_v - 1) / slice_v) : 0;
        if (slices > 0) slice_v = (lds_nv + slices - 1) / slices;
        const int groups = slices > 1 ? cus / slices / 8 * 8 : cus;
        const long long c_bytes = (long long)a.m * a.n * 4;  // C through a buffer resource
        if (a.batch == 1 && cus > 0 && vec_csr && a.nnz >= 4 && slices > 0 && groups > 0 &&
            c_bytes < (1LL << 31) &&
            (long long)a.nnz >= (long long)groups * a.k * slice_v * lds_kvec) {
            p.c_bytes = (unsigned)c_bytes;
            const long long want = ((long long)a.m + kLdsWaves - 1) / kLdsWaves;
            long long g = want < groups ? want : groups;
            if (slices > 1) g = (g + 7) / 8 * 8;  // whole XCD rounds
            plan->kind = SpmmPlan::kLds;
            plan->vec = lds_kvec == 4;
            plan->lds_kvec = lds_kvec;
            plan->blocks = (int)(g * slices);
            plan->e = slice_v <= 1 ? 1 : slice_v <= 2 ? 2 : 4;
            p.lds_slices = slices;
            p.lds_slice_n = (int)(slice_v * lds_kvec);
        }
    }
    return hipSuccess;
}

hipError_t run_spmm(const SpmmPlan &plan, hipStream_t stream)
{
    const SpmmParams &p = plan.p;
    switch (plan.kind) {
    case SpmmPlan::kUnion:
        return launch_union(plan.dtype, plan.lpr, plan.vec_csr, p, stream);
    case SpmmPlan::kPanel:
        return plan.panel == 0 ? launch_panel_t<PanelMany>(p, plan.q, stream)
                               : launch_panel_t<PanelFew>(p, plan.q, stream);
    case SpmmPlan::kLds:
        switch (plan.dtype) {
        case Dtype::f16:
            return plan.lds_kvec == 8 ? launch_lds<_Float16, 8>(plan.e, p, plan.blocks, stream)
                   : plan.vec         ? launch_lds<_Float16, 4>(plan.e, p, plan.blocks, stream)
                                      : launch_lds<_Float16, 1>(plan.e, p, plan.blocks, stream);
        case Dtype::bf16:
            return plan.lds_kvec == 8 ? launch_lds<bf16, 8>(plan.e, p, plan.blocks, stream)
                   : plan.vec         ? launch_lds<bf16, 4>(plan.e, p, plan.blocks, stream)
                                      : launch_lds<bf16, 1>(plan.e, p, plan.blocks, stream);
        default:
            return plan.vec ? launch_lds<float, 4>(plan.e, p, plan.blocks, stream)
                            : launch_lds<float, 1>(plan.e, p, plan.blocks, stream);
        }
    case SpmmPlan::kNarrow:
        return plan.vec ? launch_narrow<4>(plan.e, p, stream)
                        : launch_narrow<1>(plan.e, p, stream);
    case SpmmPlan::kSplit:
        switch (plan.dtype) {
        case Dtype::f16:
            return plan.vec ? launch_split<_Float16, 8>(plan.lpr, p, stream)
                            : launch_split<_Float16, 1>(plan.lpr, p, stream);
        case Dtype::bf16:
            return plan.vec ? launch_split<bf16, 8>(plan.lpr, p, stream)
                            : launch_split<bf16, 1>(plan.lpr, p, stream);
        default:
            return plan.vec ? launch_split<float, 4>(plan.lpr, p, stream)
                            : launch_split<float, 1>(plan.lpr, p, stream);
        }
    case SpmmPlan::kBalanced:
        switch (plan.dtype) {
        case Dtype::f16:
            return plan.vec ? launch_balanced<_Float16, 8>(p, plan.vec_csr, plan.buf, stream)
                            : launch_balanced<_Float16, 1>(p, plan.vec_csr, plan.buf, stream);
        case Dtype::bf16:
            return plan.vec ? launch_balanced<bf16, 8>(p, plan.vec_csr, plan.buf, stream)
                            : launch_balanced<bf16, 1>(p, plan.vec_csr, plan.buf, stream);
        default:
            return plan.vec ? launch_balanced<float, 4>(p, plan.vec_csr, plan.buf, stream)
                            : launch_balanced<float, 1>(p, plan.vec_csr, plan.buf, stream);
        }
    default:
        break;
    }
    switch (plan.dtype) {
    case Dtype::f16:
        return launch_wide<_Float16, 8>(plan.vec, plan.lpr, p, plan.vec_csr, plan.buf, stream);
    case Dtype::bf16:
        return launch_wide<bf16, 8>(plan.vec, plan.lpr, p, plan.vec_csr, plan.buf, stream);
    default:
        return launch_wide<float, 4>(plan.vec, plan.lpr, p, plan.vec_csr, plan.buf, stream);
    }
}

const char *spmm_kernel_name(const SpmmArgs &a)
{
    SpmmPlan plan;
    if (plan_spmm(a, &plan) != hipSuccess) return "unsupported";
    switch (plan.kind) {
    case SpmmPlan::kWide: return "wide";
    case SpmmPlan::kNarrow: return "narrow";
    case SpmmPlan::kLds: return "lds";
    case SpmmPlan::kBalanced: return "balanced";
    case SpmmPlan::kSplit: return "split";
    case SpmmPlan::kPanel: return "panel";
    case SpmmPlan::kUnion: return "panel_union";
    }
    return "unknown";
}

hipError_t launch_spmm(const SpmmArgs &a, hipStream_t stream)
{
    SpmmPlan plan;
    const hipError_t e = plan_spmm(a, &plan);
    return e != hipSuccess ? e : run_spmm(plan, stream);
}

}  // namespace spk
