// CSR SDDMM for gfx950 ("Sparse GPU Kernels for Deep Learning", summary card,
// "Summary" and "Interesting ideas" I3).  The body for Y stored k x d, and the
// design notes for it, are in sddmm_rows.h; this file holds the kernels that
// walk several short rows per wave and that compute batched panels as matrix-
// core tiles over their column union (panel_union.h), the kernels for Y stored
// d x k (the general form I3 leaves out), and the variant selection.
#include <algorithm>

#include "sp_device.h"
#include "sp_launch.h"
#include "sp_types.h"
#include "sddmm_rows.h"
#include "panel_union.h"
#include "sp_plan.h"

namespace spk {

namespace {

using namespace sddmm_detail;

template <typename E, int kG, int kNv, int kVec, bool kSoftmax>
__global__ __launch_bounds__(kWave) void sddmm_kernel(SddmmParams p)
{
    sddmm_rows_body<E, kG, kNv, kVec, kSoftmax>(p, rows_work(p, blockIdx.x));
}

// A workgroup of kSplitParts waves per row slot, sharing the row's windows.
constexpr int kSplitParts = 4;
template <typename E, int kG, int kNv, int kVec>
__global__ __launch_bounds__(kSplitParts * kWave) void sddmm_split_kernel(SddmmParams p)
{
    sddmm_rows_body<E, kG, kNv, kVec, false, kSplitParts>(p, rows_work(p, blockIdx.x));
}

// Many short rows of small depth (fp32, 16-byte vectors, d <= 4 kG): kR =
// 64 / kG rows per wave, one per group of kG lanes, lane gl of a group holding
// X[row][4 gl .. 4 gl + 3] in registers.  One wave per row (the kernels
// above) pays the row's dependent start -- row order, offsets, X, column
// window, staging -- once per row; with tens of thousands of rows of a few
// dozen entries (sparse attention: 32 heads x 4096 rows of ~80) that start,
// repeated round after round of resident waves, is most of the time.  Here a
// wave takes kR rows at once and walks them together: chunk c of a group's
// row is its entries c kG ... c kG + kG - 1, one column index per lane
// (read one chunk ahead); step t of the chunk gathers entry t's Y row (kG
// lanes x 16 bytes, its offset taken from lane t by ds_bpermute), takes the
// lane's 4-element dot product and the group's butterfly sum, and lane t
// keeps it; after kG steps each lane writes its entry.  Steps are issued in
// double-buffered batches of kU.  Every load and store goes through a buffer
// resource, with an out-of-range offset for lanes and entries that have none
// (read as zero, store dropped), so nothing branches on lane data.  Each
// output is summed exactly as the one-row kernels sum it (V::dot over the
// lane's vector, then group_sum<kG>), so results are bit-identical to them.
//
// multirow_rows is the walk of one wave over its rows (batch entry z; the
// group of lane l takes `row` if `has`, else nothing); the kernel maps row
// slots to rows through the row order.
template <typename E, int kG>
__device__ __forceinline__ void multirow_rows(const SddmmParams &p, long long z, bool has,
                                              int row)
{
    constexpr int kC = kG;           // entries per chunk: one column index per lane
    constexpr int kU = 4;            // steps per batch of gathers
    constexpr int kBpc = kC / kU;    // batches per chunk
    static_assert(kC % kU == 0, "whole batches per chunk");
    constexpr int kVecE = 16 / (int)Elem<E>::kBytes;  // elements per 16-byte vector
    using V = GVec<E, kVecE>;
    using VT = typename V::T;
    const int lane = threadIdx.x % kWave;
    const int grp = lane / kG;
    const int gl = lane - grp * kG;
    const int p0 = p.row_offsets[row];
    const int len = has ? p.row_offsets[row + 1] - p0 : 0;

    const unsigned rowbytes = (unsigned)p.d * Elem<E>::kBytes;
    const E *xz = static_cast<const E *>(p.x) + z * p.stride_x;
    const E *yz = static_cast<const E *>(p.y) + z * p.stride_y;
    float *oz = p.out + z * p.stride_out;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<E *>(xz), 0, (int)((unsigned)p.m * rowbytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<E *>(yz), 0, (int)p.y_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int *>(p.col_indices), 0, (int)((unsigned)p.nnz * 4u), 0x00020000);
    const __amdgpu_buffer_rsrc_t ro =
        __builtin_amdgcn_make_buffer_rsrc(oz, 0, (int)((unsigned)p.nnz * 4u), 0x00020000);

    // lanes past d (d < kVecE kG) gather nothing: their offsets get the top bit
    const bool lane_ok = kVecE * gl < p.d;
    const unsigned lane_mask = lane_ok ? 0u : kOutOfRange;
    const VT xr = V::buf_load(rx, has && lane_ok ? (unsigned)row * rowbytes + 16u * gl
                                                   : kOutOfRange);

    // chunk c's Y-row offset of this lane's entry (out of range past the row)
    auto chunk_offsets = [&](int c) -> unsigned {
        const int j = c * kC + gl;
        const bool ok = j < len;
        const unsigned col =
            __builtin_amdgcn_raw_buffer_load_b32(rc, (int)(ok ? (unsigned)(p0 + j) * 4u : kOutOfRange), 0, 0);
        return col * rowbytes + (ok ? 0u : kOutOfRange);
    };
    // chunks of the wave: the most any of its rows needs (wave-uniform)
    const int nch = __builtin_amdgcn_readfirstlane(
        group_reduce<kWave>((len + kC - 1) / kC, OpMax{}));
    if (nch == 0) return;
    const int batches = nch * kBpc;

    unsigned off_c = chunk_offsets(0);  // the current chunk's offsets
    unsigned off_n = chunk_offsets(1);  // the next chunk's
    const int src0 = 4 * grp * kG;      // ds_bpermute byte address of lane 0 of the group
    auto issue = [&](int b, VT (&yy)[kU]) {
        // batch b: steps (b % kBpc) kU ... of chunk b / kBpc, whose offsets are
        // off_c, or off_n for the first batch of the next chunk
        const unsigned src = (b % kBpc == 0 && b > 0) ? off_n : off_c;
        const int t0 = (b % kBpc) * kU;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const unsigned o = (unsigned)__builtin_amdgcn_ds_bpermute(src0 + 4 * (t0 + u), (int)src);
            // (a batch past the last reads out of range: zeros, no branch)
            yy[u] = V::buf_load(ry, b < batches ? (o + 16u * gl) | lane_mask : kOutOfRange);
        }
    };
    float res = 0.f;
    auto consume = [&](int b, const VT (&yy)[kU]) {
        const int t0 = (b % kBpc) * kU;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const float sum = group_sum<kG>(V::dot(xr, yy[u], 0.f));
            res = gl == t0 + u ? sum : res;
        }
        if (b % kBpc == kBpc - 1) {
            // the chunk is done: lane gl holds its entry's sum
            const int c = b / kBpc;
            const int j = c * kC + gl;
            const unsigned oo = j < len ? (unsigned)(p0 + j) * 4u : kOutOfRange;
            float scale = p.alpha;
            if (p.mask_values) {
                const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<float *>(p.mask_values + z * p.stride_values), 0,
                    (int)((unsigned)p.nnz * 4u), 0x00020000);
                scale *= __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rm, (int)oo, 0, 0));
            }
            float r = scale * res;
            if (p.beta != 0.f)
                r = fmaf(p.beta, __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ro, (int)oo, 0, 0)), r);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(r), ro, (int)oo, 0, 0);
            off_c = off_n;
            off_n = chunk_offsets(c + 2);
        }
    };

    VT ya[kU], yb[kU];
    issue(0, ya);
    // one exit, at the end (a second exit would leave pending loads on an
    // edge into the loop header, and the compiler would then wait for every
    // load in flight at its top)
    for (int b = 0; b < batches; b += 2) {
        issue(b + 1, yb);
        keep_issued_above();
        consume(b, ya);
        issue(b + 2, ya);
        keep_issued_above();
        consume(b + 1, yb);
    }
}

template <typename E, int kG>
__global__ __launch_bounds__(kWave) void sddmm_multirow_kernel(SddmmParams p)
{
    constexpr int kR = kWave / kG;   // rows per wave
    const long long units = ((long long)p.m + kR - 1) / kR;
    const long long w = xcd_work_index(p.batch, units);
    if (w < 0) return;
    const long long z = w / units;
    const int unit = (int)(w - z * units);
    // this group's row; a slot past m takes slot 0's row as a stand-in, with
    // no entries (loads stay unconditional and in bounds)
    const int slot = unit * kR + (int)threadIdx.x / kG;
    const bool has = slot < p.m;
    const int sl = has ? slot : 0;
    const int *rsrc = p.row_indices ? p.row_indices : p.row_offsets;
    const int rv = rsrc[sl];
    multirow_rows<E, kG>(p, z, has, p.row_indices ? rv : sl);
}

// Batched scores on masks whose neighbouring rows share most of their columns
// (sparse attention's band).  A workgroup takes a panel of kRows consecutive
// rows and kWaves batch entries and forms the panel's column union once
// (panel_union.h).  Each wave then computes the dense 16 x U block
// X[panel] Y[union]^T of its batch entry in 16 x 16 tiles with
// v_mfma_f32_16x16x4f32 -- every union column's Y row is loaded once per
// panel instead of once per entry -- and stores the tile values that are mask
// entries.  The 64 lanes split d four ways: lane l holds, of X's row l % 16
// and of union column 16 T + l % 16's Y row, elements 16 v + 4 (l / 16) ... + 3
// for v = 0 ... kG / 4 - 1, so the four lanes of a row read 64 contiguous bytes
// per instruction; MFMA step 4 v + s multiplies element 16 v + 4 (l / 16) + s of
// both, and the kG steps of a tile cover all of d.  A panel whose union is too
// wide for its entry count runs the multi-row walk above on its rows instead.
// Y rows that a tile's padding columns or lanes past d would read come from an
// out-of-range buffer offset (zeros), and only mask entries are stored.  Sums
// differ in rounding from the per-entry kernels (the MFMA's accumulation
// order), within the same bound.
namespace pu = panel_union;

// Batch entries (waves) per workgroup of the union kernel.
constexpr int kUnionWaves = 4;

// kSm: the row softmax of the scaled scores (sp_sddmm_softmax): one walk over
// the tiles keeps their scores in registers, then each row's exact maximum,
// the sum of exp(s - max) and the normalised writes are taken from them, so
// the values are formed as the row kernel forms them (no running-maximum
// rescaling); panels that fall back run the row kernel's softmax body on
// their rows.
template <typename E, int kG, int kW, bool kSm>
__global__ __launch_bounds__(kW * kWave) void sddmm_union_kernel(SddmmParams p)
{
    typedef float f4 __attribute__((ext_vector_type(4)));
    constexpr int kVecE = 16 / (int)Elem<E>::kBytes;  // elements per 16-byte vector
    constexpr unsigned kEb = Elem<E>::kBytes;
    constexpr int kS = kG * kVecE / 4;  // MFMA steps per tile: elements of d per lane
    __shared__ pu::SharedT<kW> s;
    extern __shared__ unsigned s_dyn[];
    pu::Panel pp;
    if (!pu::panel_of<kW>(p.m, p.batch, p.row_offsets, pp)) return;
    if (pp.pn == 0) return;  // the whole workgroup: nothing to compute
    const int nu = pu::build<kW>(p.row_offsets, p.col_indices, p.k, pp, s, s_dyn);
    // (uniform in the wave; the buffer resources below depend on it)
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int z = pp.hg * kW + wave;
    if (z >= p.batch) return;
    const int r0 = pp.r0, nr = pp.nr, e0 = pp.e0;
    if (nu < 0) {
        if constexpr (kSm) {
            // one row at a time on this wave, through its own staging region
            SddmmParams pr = p;
            pr.row_indices = nullptr;
#pragma unroll 1
            for (int i = 0; i < nr; ++i)
                sddmm_rows_body<E, kG, 1, kVecE, true, 1, kW>(pr, z * p.m + r0 + i);
        } else {
            constexpr int kR = kWave / kG;
#pragma unroll 1
            for (int u = 0; u < pu::kRows / kR; ++u) {
                const int slot = u * kR + lane / kG;
                multirow_rows<E, kG>(p, z, slot < nr, slot < nr ? r0 + slot : r0);
            }
        }
        return;
    }
    const int ntiles = (nu + 15) / 16;

    const unsigned rowbytes = (unsigned)p.d * kEb;
    const E *xz = static_cast<const E *>(p.x) + z * p.stride_x;
    const E *yz = static_cast<const E *>(p.y) + z * p.stride_y;
    float *oz = p.out + z * p.stride_out;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<E *>(xz), 0, (int)((unsigned)p.m * rowbytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<E *>(yz), 0, (int)p.y_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t ro =
        __builtin_amdgcn_make_buffer_rsrc(oz, 0, (int)((unsigned)p.nnz * 4u), 0x00020000);
    const int jl = lane % 16;   // the lane's row of X, column of the tile
    const int q = lane / 16;    // which 16-byte piece of each 64-byte block of a row
    // byte offsets of the lane's vectors within a row (out of range past d):
    // vector v holds elements 4 kVecE v + kVecE q ... + kVecE - 1
    unsigned voff[kS / kVecE];
#pragma unroll
    for (int v = 0; v < kS / kVecE; ++v) {
        const int e = 4 * kVecE * v + kVecE * q;
        voff[v] = e < p.d ? (unsigned)e * kEb : kOutOfRange;
    }
    float xa[kS];
    {
        const unsigned base = jl < nr ? (unsigned)(r0 + jl) * rowbytes : kOutOfRange;
#pragma unroll
        for (int v = 0; v < kS / kVecE; ++v)
            load_widen<E, kVecE>(rx, base + voff[v] | (base & kOutOfRange), &xa[kVecE * v]);
    }
    auto load_tile = [&](int T, float (&yb)[kS]) {
        const int u = 16 * T + jl;
        const unsigned base =
            u < nu ? (unsigned)s.ucol[min(u, pu::kMaxCols - 1)] * rowbytes : kOutOfRange;
#pragma unroll
        for (int v = 0; v < kS / kVecE; ++v)
            load_widen<E, kVecE>(ry, base + voff[v] | (base & kOutOfRange), &yb[kVecE * v]);
    };
    const float alpha = p.alpha, beta = p.beta;
    const float *mvz = p.mask_values ? p.mask_values + z * p.stride_values : nullptr;
    auto tile_acc = [&](const float (&yb)[kS]) {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < kS; ++t)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[t], yb[t], acc, 0, 0, 0);
        return acc;  // lane l: rows 4 (l / 16) .. + 3 of tile column l % 16
    };
    auto tile_out = [&](int T, const float (&yb)[kS]) {
        const f4 acc = tile_acc(yb);
        const int u = 16 * T + jl;
        const int uc = min(u, pu::kMaxCols - 1);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const unsigned idx = u < nu ? s.emap[(4 * q + r) * pu::kEmapStride + uc] : 0u;
            const unsigned oo = idx ? (unsigned)(e0 + (int)idx - 1) * 4u : kOutOfRange;
            float scale = alpha;
            if (mvz) {
                const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<float *>(mvz), 0, (int)((unsigned)p.nnz * 4u), 0x00020000);
                scale *= __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rm, (int)oo, 0, 0));
            }
            float res = scale * acc[r];
            if (beta != 0.f)
                res = fmaf(beta, __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ro, (int)oo, 0, 0)),
                           res);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(res), ro, (int)oo, 0, 0);
        }
    };
    // each tile loaded just before use: fewer registers, and the other
    // resident waves hide the loads (7 % faster than a tile prefetched)
    auto walk = [&](auto visit) {
        for (int T = 0; T < ntiles; ++T) {
            float yt[kS];
            load_tile(T, yt);
            visit(T, yt);
        }
    };
    if constexpr (!kSm) {
        walk(tile_out);
    } else {
        // one walk: every tile's scaled scores stay in registers (at most
        // kMaxCols / 16 tiles of 4 values a lane), so Y is read once; then
        // each row's maximum, the exps and their sum (per tile over the row's
        // 16-lane group, then tile by tile), and the normalised writes.
        static_assert(pu::kMaxCols == 16 * 16, "score registers cover 16 tiles");
        constexpr int kTiles = pu::kMaxCols / 16;
        float sv[kTiles][4];
        unsigned long long has = 0ull;  // bit 4 T + r: the lane's entry of tile T, row r
        // per row (the lanes of a 16-lane group hold the same four rows)
        float rmax[4], rsum[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            rmax[r] = -INFINITY;
            rsum[r] = 0.f;
        }
#pragma unroll
        for (int T = 0; T < kTiles; ++T) {
            if (T < ntiles) {
                float yt[kS];
                load_tile(T, yt);
                const f4 acc = tile_acc(yt);
                const int u = 16 * T + jl;
                const int uc = min(u, pu::kMaxCols - 1);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const unsigned idx = u < nu ? s.emap[(4 * q + r) * pu::kEmapStride + uc] : 0u;
                    has |= idx ? 1ull << (4 * T + r) : 0ull;
                    sv[T][r] = idx ? alpha * acc[r] : -INFINITY;
                    rmax[r] = fmaxf(rmax[r], sv[T][r]);  // the lane's maximum so far
                }
            }
        }
        // the row's maximum (exact in any order)
#pragma unroll
        for (int r = 0; r < 4; ++r) rmax[r] = group_reduce<16>(rmax[r], OpMax{});
        // sv becomes exp(s - max) (0 where no entry)
#pragma unroll
        for (int T = 0; T < kTiles; ++T) {
            if (T < ntiles) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool e = (has >> (4 * T + r)) & 1ull;
                    sv[T][r] = e ? expf(sv[T][r] - rmax[r]) : 0.f;
                    rsum[r] += group_sum<16>(sv[T][r]);
                }
            }
        }
        float rinv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) rinv[r] = 1.f / rsum[r];
#pragma unroll
        for (int T = 0; T < kTiles; ++T) {
            if (T < ntiles) {
                const int u = 16 * T + jl;
                const int uc = min(u, pu::kMaxCols - 1);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const unsigned idx = u < nu ? s.emap[(4 * q + r) * pu::kEmapStride + uc] : 0u;
                    const unsigned oo = idx ? (unsigned)(e0 + (int)idx - 1) * 4u : kOutOfRange;
                    const float e = sv[T][r] * rinv[r];
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(e), ro, (int)oo, 0, 0);
                }
            }
        }
    }
}

// Y stored d x k (the operand not transposed): Yop(c, l) = Y[l][c].  One wave
// per row slot as above, but lanes are dealt to entries, 64 at a time: for each
// l the wave gathers Y[l][c] of its 64 columns -- all within row l of Y, whose
// columns ascend with the lanes -- and multiplies by X[i][l], which every lane
// shares (a wave-uniform, scalar load).  Each lane sums its entry's d products
// in order with FMA; kU gathers are issued before their FMAs.  Idle lanes of a
// row's last pass gather column 0 (in bounds) and store nothing.
template <typename E, bool kBuf>
__global__ __launch_bounds__(kWave) void sddmm_cols_kernel(SddmmParams p)
{
    using V1 = GVec<E, 1>;
    constexpr unsigned kEb = Elem<E>::kBytes;
    constexpr int kU = 16;
    const long long w = xcd_work_index(p.batch, p.m);
    if (w < 0) return;
    const long long z = w / p.m;
    const int slot = (int)(w - z * p.m);
    const int lane = threadIdx.x;
    const int row = p.row_indices ? p.row_indices[slot] : slot;
    const int p0 = p.row_offsets[row];
    const int p1 = p.row_offsets[row + 1];
    const E *__restrict__ xr =
        static_cast<const E *>(p.x) + z * p.stride_x + (size_t)row * (size_t)p.d;
    const E *__restrict__ yz = static_cast<const E *>(p.y) + z * p.stride_y;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<E *>(yz), 0, (int)p.y_bytes, 0x00020000);
    const unsigned row_bytes = (unsigned)p.k * kEb;

    for (int base = p0; base < p1; base += kWave) {
        const int q = base + lane;
        const bool live = q < p1;
        const int c = live ? p.col_indices[q] : 0;
        float acc = 0.f;
        int l = 0;
        for (; l + kU <= p.d; l += kU) {
            float yv[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                if constexpr (kBuf)
                    V1::to_f32(V1::buf_load(rsrc, (unsigned)(l + u) * row_bytes +
                                                      (unsigned)c * kEb),
                               &yv[u]);
                else
                    yv[u] = Elem<E>::f32(yz[(size_t)(l + u) * (size_t)p.k + (size_t)c]);
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) acc = fmaf(Elem<E>::f32(xr[l + u]), yv[u], acc);
        }
        for (; l < p.d; ++l)
            acc = fmaf(Elem<E>::f32(xr[l]),
                       Elem<E>::f32(yz[(size_t)l * (size_t)p.k + (size_t)c]), acc);
        if (live) store_entry(p, z, q, acc);
    }
}

// Y stored d x k without a workspace, for sparse masks: the columns of Y a
// panel of rows touches are staged through LDS, transposed.
// A workgroup of four waves owns a panel of kRows consecutive row slots (in
// the given row order) and one of q.splits contiguous ranges of Y's columns;
// wave w owns the panel's rows w, w + 4, ...  The panel's X rows are copied
// into LDS once.  Each row keeps a cursor to its next pending CSR entry.  The
// range is walked in chunks: a chunk starts at the smallest pending column of
// the panel and ends before the (q.kc + 1)-th distinct column the panel's
// pending entries touch, so one chunk can span many columns when few of them
// are touched.  Per chunk:
//  scan     each wave loads 64-entry windows of column indices for all its
//           rows at once (kRounds windows per row, kept in registers) and
//           sets one bit per touched column in a bitmap of the next kDkSpan
//           columns;
//  cut      a block prefix over the bitmap's words ranks the touched columns;
//           the chunk ends at the column of rank q.kc, at the bitmap's end, or
//           where a row's loaded windows end, whichever comes first;
//  stage    the chunk's touched columns of Y are gathered (consecutive threads
//           take consecutive columns) into LDS rows, one per rank;
//  table    each wave writes, per row, the LDS row of each of its entries in
//           the chunk;
//  compute  each wave takes its rows' entries in the chunk one after another,
//           64 to a pass: each entry gets one lane, which sums its d products
//           in l order with FMA (X and Y rows read from LDS), so rows with few
//           entries in a chunk leave no lane idle.
// Staged rows have a pitch of an odd number of 16-byte units (16 lanes
// reading 16 bytes from 16 different rows hit distinct banks when the rows
// are consecutive) and are zero-padded to whole vectors (padding adds
// 0 * 0, which leaves a sum unchanged).  Only the columns a panel touches are
// read from Y, once per panel and column range.
// Global loads are unconditional and from valid addresses: surplus items
// repeat the last item, and values are chosen only after loading.  (A load
// under a branch makes the compiler wait for every load in flight where the
// branches join, which would serialise the loads.)
constexpr int kDkSpan = 8192;   // columns covered by a chunk's bitmap (one word per thread)
constexpr int kDkYBatch = 16;   // staged Y vectors per thread in flight
constexpr int kDkXItems = 8;    // staged X vectors per thread in flight

// Panel heights and windows per row per chunk, by 16-byte vectors per row.
__host__ __device__ constexpr int dk_rows(int dv) { return dv <= 64 ? 32 : dv <= 128 ? 16 : 8; }
__host__ __device__ constexpr int dk_rounds(int dv) { return dv <= 32 ? 2 : 1; }

// X rows of a panel into LDS: thread -> vector tid % 2^xsh of rows
// tid / 2^xsh + u * (kThreads >> xsh) (2^xsh >= dv; kDkXItems * (kThreads >>
// xsh) covers the panel's rows), zero beyond d.  Loaded into registers by
// load(), written to LDS by store(), so that a caller can issue other loads
// in between (a write waits for its load, and loads complete in order).
template <int kThreads, bool kVec>
struct DkStageX {
    float4 xb[kDkXItems];
    int xv, xr0, xstep;

    template <class RowOf>
    __device__ __forceinline__ void load(const SddmmParams &p, const float *xz, int nrows, int xsh,
                                         RowOf row_of)
    {
        const int tid = threadIdx.x;
        const int dv = (p.d + 3) / 4;
        xv = min(tid & ((1 << xsh) - 1), dv - 1);
        xr0 = tid >> xsh;
        xstep = kThreads >> xsh;
        int xrow[kDkXItems];
#pragma unroll
        for (int u = 0; u < kDkXItems; ++u) xrow[u] = row_of(min(xr0 + u * xstep, nrows - 1));
        __builtin_amdgcn_sched_barrier(0);
        const int e = 4 * xv;
#pragma unroll
        for (int u = 0; u < kDkXItems; ++u) {
            const float *src = xz + (size_t)xrow[u] * (size_t)p.d + e;
            if constexpr (kVec) {  // d % 4 == 0
                xb[u] = *reinterpret_cast<const float4 *>(src);
            } else {
                const int last = p.d - 1 - e;  // >= 0
                xb[u] = make_float4(src[0], src[min(1, last)], src[min(2, last)], src[min(3, last)]);
            }
        }
    }

    __device__ __forceinline__ void store(const SddmmParams &p, int nrows, unsigned x_pitch,
                                          unsigned char *lds)
    {
        const int e = 4 * xv;
#pragma unroll
        for (int u = 0; u < kDkXItems; ++u) {
            const int r = min(xr0 + u * xstep, nrows - 1);
            float4 v = xb[u];
            if constexpr (!kVec) {
                if (e + 1 >= p.d) v.y = 0.f;
                if (e + 2 >= p.d) v.z = 0.f;
                if (e + 3 >= p.d) v.w = 0.f;
            }
            *reinterpret_cast<float4 *>(lds + (unsigned)r * x_pitch + (unsigned)xv * 16u) = v;
        }
    }
};

template <int kThreads, bool kVec, class RowOf>
__device__ __forceinline__ void dk_stage_x(const SddmmParams &p, const float *xz, int nrows,
                                           int xsh, unsigned x_pitch, unsigned char *lds,
                                           RowOf row_of)
{
    DkStageX<kThreads, kVec> sx;
    sx.load(p, xz, nrows, xsh, row_of);
    sx.store(p, nrows, x_pitch, lds);
}

template <int kRows, int kRounds, bool kVec>
__global__ __launch_bounds__(4 * kWave) void sddmm_dk_panel_kernel(SddmmParams p, DkPanelParams q)
{
    constexpr int kWaves = 4;
    constexpr int kThreads = kWaves * kWave;
    constexpr int kRpw = kRows / kWaves;  // rows per wave
    constexpr int kTab = kRounds * kWave; // table entries per row
    constexpr int kWords = kDkSpan / 32;
    static_assert(kWords == kThreads, "one bitmap word per thread");
    extern __shared__ __align__(16) unsigned char lds[];

    const long long units = (long long)q.panels * q.splits;
    const long long w = xcd_work_index(p.batch, units);
    if (w < 0) return;
    const long long z = w / units;
    const int rem = (int)(w - z * units);
    const int panel = rem / q.splits;
    const int split = rem - panel * q.splits;
    const int slot0 = panel * kRows;
    const int nrows = min(kRows, p.m - slot0);
    const int cb = (int)((long long)p.k * split / q.splits);
    const int ce = (int)((long long)p.k * (split + 1) / q.splits);
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int dv = (p.d + 3) / 4;  // 16-byte vectors per staged row

    unsigned *s_tab = reinterpret_cast<unsigned *>(lds + q.off_tab) + wave * kRpw * kTab;
    unsigned *s_bits = reinterpret_cast<unsigned *>(lds + q.off_bits);  // two bitmaps
    unsigned *s_rank = reinterpret_cast<unsigned *>(lds + q.off_rank);  // touched columns below each word
    int *s_col = reinterpret_cast<int *>(lds + q.off_col);              // column of each rank
    int *s_misc = reinterpret_cast<int *>(lds + q.off_misc);
    int *s_wmin = s_misc;       // [4] smallest pending column past the chunk, per wave
    int *s_wlim = s_misc + 4;   // [4] end of the loaded windows, per wave
    int *s_wsum = s_misc + 8;   // [4] touched columns per wave's words
    int *s_cut = s_misc + 12;   // [1] column of rank q.kc

    const float *__restrict__ xz = static_cast<const float *>(p.x) + z * p.stride_x;
    const float *__restrict__ yz = static_cast<const float *>(p.y) + z * p.stride_y;
    const int *__restrict__ ci = p.col_indices;
    // row id of panel row r, read from a valid stand-in array when there is
    // no row order (row_offsets has m + 1 entries)
    const int *rsrc = p.row_indices ? p.row_indices : p.row_offsets;
    auto row_of = [&](int r) {
        const int v = rsrc[slot0 + r];
        return p.row_indices ? v : slot0 + r;
    };
    // column index of entry at, or INT_MAX when ok is false (entry 0 exists:
    // nnz > 0 here)
    auto col_at = [&](bool ok, int at) {
        const int c = ci[ok ? at : 0];
        return ok ? c : INT_MAX;
    };

    // This wave's rows: lane i < kRpw holds row wave + 4 i's cursor, end and
    // (per chunk) entry count.
    const int my_r = wave + kWaves * lane;
    const bool my_ok = lane < kRpw && my_r < nrows;
    const int my_row = row_of(my_ok ? my_r : 0);
    __builtin_amdgcn_sched_barrier(0);
    int my_cur = p.row_offsets[my_row];
    int my_end = p.row_offsets[my_row + 1];
    __builtin_amdgcn_sched_barrier(0);
    DkStageX<kThreads, kVec> sx;
    sx.load(p, xz, nrows, q.x_shift, row_of);
    __builtin_amdgcn_sched_barrier(0);
    if (!my_ok) my_cur = my_end = 0;
    int my_n = 0;
    s_bits[tid] = 0u;
    s_bits[kWords + tid] = 0u;
    unsigned live_rows = 0;  // bit i: row wave + 4 i exists
#pragma unroll
    for (int i = 0; i < kRpw; ++i)
        if (wave + kWaves * i < nrows) live_rows |= 1u << i;
    // Cursors to each row's first entry in the range; wm = the smallest
    // pending column of the wave's rows (INT_MAX: none).
    int wm = INT_MAX;
    {
        unsigned act = live_rows;
        while (act != 0u) {
            int col[kRpw];
#pragma unroll
            for (int i = 0; i < kRpw; ++i) {
                const int base = __builtin_amdgcn_readlane(my_cur, i);
                const int end = __builtin_amdgcn_readlane(my_end, i);
                col[i] = col_at((act >> i & 1u) && lane < end - base, base + lane);
            }
#pragma unroll
            for (int i = 0; i < kRpw; ++i) {
                if (!(act >> i & 1u)) continue;
                const int cnt = (int)__popcll(__builtin_amdgcn_ballot_w64(col[i] < cb));
                if (lane == i) my_cur += cnt;
                if (cnt < kWave) {
                    wm = min(wm, __builtin_amdgcn_readlane(col[i], cnt));
                    act &= ~(1u << i);
                }
            }
        }
    }
    // X into LDS after the rows' first column loads are issued (a write
    // waits for its load, and loads complete in order)
    sx.store(p, nrows, q.x_pitch, lds);
    if (lane == 0) s_wmin[wave] = wm;
    __syncthreads();
    int chunk0 = min(min(s_wmin[0], s_wmin[1]), min(s_wmin[2], s_wmin[3]));

    // epilogue operands, read from a valid stand-in array when absent
    const float *__restrict__ vz = p.mask_values ? p.mask_values + z * p.stride_values : nullptr;
    float *__restrict__ oz = p.out + z * p.stride_out;
    const float *vsrc = vz ? vz : reinterpret_cast<const float *>(ci);
    const float *psrc = p.beta != 0.f ? oz : reinterpret_cast<const float *>(ci);

    for (int chunk = 0; chunk0 < ce; ++chunk) {
        unsigned *bits = s_bits + (chunk & 1) * kWords;
        const int limw = (int)min((long long)chunk0 + kDkSpan, (long long)ce);
        // ---- scan: col[i][t] = column of row i's entry 64 t + lane from its
        // cursor (INT_MAX past the row); rows whose kRounds windows all lie
        // below limw bound the chunk at their next entry's column (wl).
        int col[kRpw][kRounds];
        unsigned loaded = 0;  // bit i * kRounds + t: window t of row i was loaded
        int wl = limw;
        {
            unsigned act = live_rows;
#pragma unroll
            for (int t = 0; t < kRounds; ++t) {
#pragma unroll
                for (int i = 0; i < kRpw; ++i) {
                    const int base = __builtin_amdgcn_readlane(my_cur, i) + kWave * t;
                    const int end = __builtin_amdgcn_readlane(my_end, i);
                    col[i][t] = col_at((act >> i & 1u) && lane < end - base, base + lane);
                }
#pragma unroll
                for (int i = 0; i < kRpw; ++i) {
                    if (!(act >> i & 1u)) continue;
                    loaded |= 1u << (i * kRounds + t);
                    const int c = col[i][t];
                    const bool in = c < limw;
                    const int cnt = (int)__popcll(__builtin_amdgcn_ballot_w64(in));
                    // (columns ascend within a row; the range check only keeps
                    // LDS accesses in bounds for input that breaks that)
                    const unsigned rel = (unsigned)(c - chunk0);
                    if (in && rel < (unsigned)kDkSpan) atomicOr(&bits[rel >> 5], 1u << (rel & 31u));
                    if (cnt < kWave) act &= ~(1u << i);
                }
            }
#pragma unroll
            for (int i = 0; i < kRpw; ++i) {
                if (!(act >> i & 1u)) continue;
                const int at = __builtin_amdgcn_readlane(my_cur, i) + kTab;
                const int c = col_at(at < __builtin_amdgcn_readlane(my_end, i), at);
                wl = min(wl, c);
            }
        }
        if (lane == 0) s_wlim[wave] = wl;
        __syncthreads();
        // ---- cut: rank the touched columns below lim0; end the chunk at the
        // column of rank q.kc when there are more
        const int lim0 = min(min(s_wlim[0], s_wlim[1]), min(s_wlim[2], s_wlim[3]));
        const unsigned word = bits[tid];
        const int wbase = tid * 32;  // first column of this word, relative to chunk0
        auto below = [](int nbits) {
            return nbits >= 32 ? 0xffffffffu : nbits <= 0 ? 0u : (1u << nbits) - 1u;
        };
        const unsigned word0 = word & below(lim0 - chunk0 - wbase);
        const int cnt = __popc(word0);
        const int incl = wave_inclusive_sum(cnt);
        if (lane == kWave - 1) s_wsum[wave] = incl;
        __syncthreads();
        int excl = incl - cnt, total = 0;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            const int sv = s_wsum[v];
            if (v < wave) excl += sv;
            total += sv;
        }
        s_rank[tid] = (unsigned)excl;
        if (total > q.kc && excl <= q.kc && q.kc < excl + cnt) {
            // this word holds rank q.kc: its column ends the chunk
            unsigned wb = word0;
            for (int j = q.kc - excl; j > 0; --j) wb &= wb - 1u;
            *s_cut = chunk0 + wbase + (int)__builtin_ctz(wb);
        }
        __syncthreads();
        const int lim = total > q.kc ? *s_cut : lim0;
        const int ns = min(total, q.kc);
        {
            unsigned wb = word0 & below(lim - chunk0 - wbase);
            for (int j = excl; wb != 0u; ++j) {
                s_col[j] = chunk0 + wbase + (int)__builtin_ctz(wb);
                wb &= wb - 1u;
            }
        }
        // the other bitmap is free (last read before this chunk's first barrier)
        s_bits[((chunk + 1) & 1) * kWords + tid] = 0u;
        __syncthreads();
        // ---- stage the touched columns of Y in rank order: item i -> rank
        // i % ns, vector i / ns (i / ns as a multiply by ceil(2^25 / ns) and a
        // shift, exact for i < 2^16 and ns <= 256); surplus items repeat the
        // last one
        {
            const int nitems = ns * dv;
            const unsigned long long magic = ((1u << 25) + (unsigned)ns - 1u) / (unsigned)ns;
            for (int i0 = 0; i0 < nitems; i0 += kDkYBatch * kThreads) {
                float4 yb[kDkYBatch];
                int sl[kDkYBatch], vv[kDkYBatch];
#pragma unroll
                for (int u = 0; u < kDkYBatch; ++u) {
                    const int i = min(i0 + u * kThreads + tid, nitems - 1);
                    vv[u] = (int)(((unsigned long long)(unsigned)i * magic) >> 25);
                    sl[u] = i - vv[u] * ns;
                }
#pragma unroll
                for (int u = 0; u < kDkYBatch; ++u) {
                    const size_t c = (size_t)s_col[sl[u]];
                    const int l = 4 * vv[u];
                    const float *src = yz + (size_t)l * (size_t)p.k + c;
                    if constexpr (kVec) {  // d % 4 == 0: all four rows exist
                        yb[u] = make_float4(src[0], src[(size_t)p.k], src[2 * (size_t)p.k],
                                            src[3 * (size_t)p.k]);
                    } else {
                        const int last = p.d - 1 - l;  // >= 0
                        yb[u] = make_float4(src[0], src[(size_t)min(1, last) * (size_t)p.k],
                                            src[(size_t)min(2, last) * (size_t)p.k],
                                            src[(size_t)min(3, last) * (size_t)p.k]);
                    }
                }
#pragma unroll
                for (int u = 0; u < kDkYBatch; ++u) {
                    float4 v = yb[u];
                    if constexpr (!kVec) {
                        const int l = 4 * vv[u];
                        if (l + 1 >= p.d) v.y = 0.f;
                        if (l + 2 >= p.d) v.z = 0.f;
                        if (l + 3 >= p.d) v.w = 0.f;
                    }
                    *reinterpret_cast<float4 *>(lds + q.off_y + (unsigned)sl[u] * q.y_pitch +
                                                (unsigned)vv[u] * 16u) = v;
                }
            }
        }
        // ---- table: per row, the entries in the chunk (a prefix of its
        // loaded windows), the LDS row of each, and the next pending column
        wm = INT_MAX;
#pragma unroll
        for (int i = 0; i < kRpw; ++i) {
            int n = 0;
#pragma unroll
            for (int t = 0; t < kRounds; ++t)
                if (loaded >> (i * kRounds + t) & 1u)
                    n += (int)__popcll(__builtin_amdgcn_ballot_w64(col[i][t] < lim));
            if (lane == i) my_n = n;
            // the entry after the chunk: in the loaded windows, unless all of
            // them were taken (then it is the one that bounded the chunk)
            int next = INT_MAX;
#pragma unroll
            for (int t = 0; t < kRounds; ++t)
                if (n >> 6 == t && (loaded >> (i * kRounds + t) & 1u))
                    next = __builtin_amdgcn_readlane(col[i][t], n & 63);
            if (n == kTab) {
                const int at = __builtin_amdgcn_readlane(my_cur, i) + kTab;
                next = col_at(at < __builtin_amdgcn_readlane(my_end, i), at);
            }
            if (live_rows >> i & 1u) wm = min(wm, next);
#pragma unroll
            for (int t = 0; t < kRounds; ++t) {
                if (kWave * t < n && kWave * t + lane < n) {
                    const unsigned rel = (unsigned)(col[i][t] - chunk0);
                    unsigned off = q.off_y;
                    if (rel < (unsigned)(lim - chunk0)) {
                        const unsigned wd = rel >> 5, b = rel & 31u;
                        off += (s_rank[wd] + (unsigned)__popc(bits[wd] & ((1u << b) - 1u))) * q.y_pitch;
                    }
                    s_tab[i * kTab + kWave * t + lane] = off;
                }
            }
        }
        if (lane == 0) s_wmin[wave] = wm;
        __syncthreads();
        const int next0 = min(min(s_wmin[0], s_wmin[1]), min(s_wmin[2], s_wmin[3]));
        // ---- compute: the wave's entries in the chunk, rows after one
        // another, 64 to a pass, one lane each
        int pre[kRpw], cur[kRpw], n[kRpw];
        int total_w = 0;
#pragma unroll
        for (int i = 0; i < kRpw; ++i) {
            n[i] = __builtin_amdgcn_readlane(my_n, i);
            cur[i] = __builtin_amdgcn_readlane(my_cur, i);
            pre[i] = total_w;
            total_w += n[i];
        }
        for (int t0 = 0; t0 < total_w; t0 += kWave) {
            const int e = t0 + lane;
            int ri = 0, j = 0, at = 0;
#pragma unroll
            for (int i = 0; i < kRpw; ++i) {
                if (e >= pre[i] && e < pre[i] + n[i]) {
                    ri = i;
                    j = e - pre[i];
                    at = cur[i] + j;
                }
            }
            const bool ok = e < total_w;
            const float v = vsrc[at];  // at = 0 for idle lanes: a valid entry
            const float prior = psrc[at];
            const unsigned off = s_tab[ri * kTab + j];
            if (ok) {
                const unsigned char *yr = lds + off;
                const unsigned char *xr = lds + (unsigned)(wave + kWaves * ri) * q.x_pitch;
                float acc = 0.f;
#pragma unroll 4
                for (int u = 0; u < dv; ++u) {
                    const float4 xv = *reinterpret_cast<const float4 *>(xr + u * 16);
                    const float4 yv = *reinterpret_cast<const float4 *>(yr + u * 16);
                    acc = fmaf(xv.x, yv.x, acc);
                    acc = fmaf(xv.y, yv.y, acc);
                    acc = fmaf(xv.z, yv.z, acc);
                    acc = fmaf(xv.w, yv.w, acc);
                }
                float r = p.alpha * (vz ? v : 1.f) * acc;
                if (p.beta != 0.f) r = fmaf(p.beta, prior, r);
                oz[at] = r;
            }
        }
        my_cur += my_n;
        chunk0 = next0;
    }
}

// Y stored d x k without a workspace, for masks that touch most columns of a
// tile: a workgroup of kWaves waves owns a panel of kRows consecutive rows and
// one tile of at most kDkTileCols consecutive columns [c0, c1) of Y, which it
// stages whole.  X is read once per tile and Y once per panel, so the largest
// tiles LDS holds read the least: 64 x 64 (eight waves, one workgroup per CU)
// for d <= 256.  Panels are runs of consecutive rows whatever the row order
// (the order only schedules work).
// All global reads are issued before the workgroup's one barrier, in two
// dependent levels: the tile of Y (16-byte reads along Y's rows, each lane
// writing its 4 columns into 4 transposed LDS rows), the rows' CSR bounds and
// the panel's X rows; then per row a 64-entry window of column indices from
// the row's start.  A row's first entry at or past c0 is found in that window
// (or, for longer rows, by a 64-way search and a window read from there); its
// entries in the tile (at most 64) are listed per wave, rows after one
// another.  Each listed entry gets 16 lanes, 4 entries a step: lane gl sums
// vectors gl, gl + 16, ... of the entry's X and Y rows in order with FMA (16
// lanes read 256 contiguous bytes of one LDS row, so no bank conflicts,
// whatever the columns), and group_sum adds the 16 partial sums.
constexpr int kDkTileCols = 64;
constexpr int kDkTileYItems = 4096;  // Y vectors per batch: d <= 256 at 16 column quads is one

template <int kRows, int kWaves, int kNv, bool kVec>
__global__ __launch_bounds__(kWaves * kWave) void sddmm_dk_tile_kernel(SddmmParams p, DkPanelParams q)
{
    constexpr int kThreads = kWaves * kWave;
    constexpr int kRpw = kRows / kWaves;
    extern __shared__ __align__(16) unsigned char lds[];

    const long long units = (long long)q.panels * q.splits;  // splits = tiles per panel
    const long long w = xcd_work_index(p.batch, units);
    if (w < 0) return;
    const long long z = w / units;
    const int rem = (int)(w - z * units);
    const int panel = rem / q.splits;
    const int tile = rem - panel * q.splits;
    const int slot0 = panel * kRows;
    const int nrows = min(kRows, p.m - slot0);
    const int c0 = tile * q.kc;
    const int c1 = min(c0 + q.kc, p.k);
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int dv = (p.d + 3) / 4;
    const int cq = (c1 - c0 + 3) / 4;      // column quads in the tile (<= 16)

    const float *__restrict__ xz = static_cast<const float *>(p.x) + z * p.stride_x;
    const float *__restrict__ yz = static_cast<const float *>(p.y) + z * p.stride_y;
    const int *__restrict__ ci = p.col_indices;
    // Panels are runs of consecutive rows whatever the row order: the order
    // only schedules work (results do not depend on it), and tiles whose
    // columns are mostly touched need no balancing, so the row ids cost no
    // read.
    auto row_of = [&](int r) { return slot0 + r; };

    // Every load below is unconditional and from a valid address: surplus
    // items repeat the last item (loading and storing the same value again),
    // and no value is chosen between a load and a constant.  (A load under a
    // branch, or one the compiler turns into a branch, makes it wait for every
    // load in flight where the branches join, which would serialise the
    // levels.)
    // this wave's rows (lane i < kRpw: row wave + 4 i)
    const int my_r = wave + kWaves * lane;
    const bool my_ok = lane < kRpw && my_r < nrows;
    const int my_row = row_of(my_ok ? my_r : 0);
    // ---- level 1a: the tile of Y: item i -> element row l = i / cq, column
    // quad i % cq; i / cq as (i * ceil(2^20 / cq)) >> 20, exact for
    // i < 2^14 and cq <= 16 (the error stays below 1/64 < 1/cq)
    const int ny = p.d * cq;  // items
    const unsigned long long cq_magic = ((1u << 20) + (unsigned)cq - 1u) / (unsigned)cq;
    auto y_item = [&](int i, int &l, int &qd) {
        i = min(i, ny - 1);
        l = (int)(((unsigned long long)(unsigned)i * cq_magic) >> 20);
        qd = i - l * cq;
    };
    auto load_y = [&](int i) {
        int l, qd;
        y_item(i, l, qd);
        const float *src = yz + (size_t)l * (size_t)p.k + (c0 + 4 * qd);
        float4 v;
        if constexpr (kVec) {  // k % 4 == 0, so the quad lies inside the row
            v = *reinterpret_cast<const float4 *>(src);
        } else {
            const int last = c1 - 1 - (c0 + 4 * qd);  // >= 0
            v.x = src[0];
            v.y = src[min(1, last)];
            v.z = src[min(2, last)];
            v.w = src[min(3, last)];
        }
        return v;
    };
    auto store_y = [&](int i, const float4 &v) {
        int l, qd;
        y_item(i, l, qd);
        float *dst = reinterpret_cast<float *>(lds + q.off_y + (unsigned)(4 * qd) * q.y_pitch) + l;
        const unsigned pf = q.y_pitch / 4u;
        dst[0] = v.x;
        dst[pf] = v.y;
        dst[2 * pf] = v.z;
        dst[3 * pf] = v.w;
    };
    static_assert(kDkTileYItems % kThreads == 0, "whole Y batches per thread");
    constexpr int kYB = kDkTileYItems / kThreads;  // Y vectors per thread per batch
    float4 yb[kYB];
#pragma unroll
    for (int u = 0; u < kYB; ++u) yb[u] = load_y(u * kThreads + tid);
    __builtin_amdgcn_sched_barrier(0);
    // ---- level 1b: this wave's CSR bounds, then the panel's X rows
    int my_start = p.row_offsets[my_row];
    int my_end = p.row_offsets[my_row + 1];
    __builtin_amdgcn_sched_barrier(0);
    DkStageX<kThreads, kVec> sx;
    sx.load(p, xz, nrows, q.x_shift, row_of);
    __builtin_amdgcn_sched_barrier(0);
    if (!my_ok) my_start = my_end = 0;
    // ---- level 2: per row, the 64-entry window of column indices from its
    // start (issued before X is written to LDS, which waits for X's loads)
    int win[kRpw];
#pragma unroll
    for (int i = 0; i < kRpw; ++i) {
        const int s = __builtin_amdgcn_readlane(my_start, i);
        const int e = __builtin_amdgcn_readlane(my_end, i);
        const bool in = lane < e - s;
        const int c = ci[in ? s + lane : 0];  // nnz > 0 here, so entry 0 exists
        win[i] = in ? c : INT_MAX;
    }
    __builtin_amdgcn_sched_barrier(0);
    sx.store(p, nrows, q.x_pitch, lds);
    // ---- stage Y (more batches when d * cq > 4096) and its zero rows
    // l in [d, 4 dv) (X's padding is zero, but 0 * NaN is not)
#pragma unroll
    for (int u = 0; u < kYB; ++u) store_y(u * kThreads + tid, yb[u]);
    for (int i0 = kYB * kThreads; i0 < ny; i0 += kYB * kThreads) {
#pragma unroll
        for (int u = 0; u < kYB; ++u) yb[u] = load_y(i0 + u * kThreads + tid);
#pragma unroll
        for (int u = 0; u < kYB; ++u) store_y(i0 + u * kThreads + tid, yb[u]);
    }
    // zero rows l in [d, 64 kNv) of the staged columns, and the same elements
    // of the staged X rows (the 16-lane groups read whole groups of vectors)
    constexpr int kPad = 64 * kNv;  // staged elements per row
    for (int i = tid; i < (kPad - p.d) * (4 * cq + kRows); i += kThreads) {
        const int c = i / (kPad - p.d), l = p.d + (i - c * (kPad - p.d));
        float *row = c < 4 * cq
                         ? reinterpret_cast<float *>(lds + q.off_y + (unsigned)c * q.y_pitch)
                         : reinterpret_cast<float *>(lds + (unsigned)(c - 4 * cq) * q.x_pitch);
        row[l] = 0.f;
    }
    // ---- each row's entries in the tile: base (first entry >= c0), count,
    // and per lane j < count entry j's column
    int base[kRpw], cnt[kRpw], colt[kRpw];
#pragma unroll
    for (int i = 0; i < kRpw; ++i) {
        const int s = __builtin_amdgcn_readlane(my_start, i);
        const int e = __builtin_amdgcn_readlane(my_end, i);
        const int below = (int)__popcll(__builtin_amdgcn_ballot_w64(win[i] < c0));
        const bool past = __builtin_amdgcn_ballot_w64(win[i] >= c1) != 0ull;  // INT_MAX past the end
        if (below < kWave && past) {
            // (cross-lane reads with every lane active: a lane reads another's
            // register only while that lane is active)
            const int src = min(lane + below, kWave - 1);
            base[i] = s + below;
            colt[i] = __shfl(win[i], src);
            if (lane + below >= kWave) colt[i] = INT_MAX;
            cnt[i] = (int)__popcll(__builtin_amdgcn_ballot_w64(win[i] >= c0 && win[i] < c1));
        } else {
            // the tile's entries reach past the window: find the first entry
            // >= c0 (64-way search beyond the window when all of it is below)
            // and read a window from there
            int b = s + below;
            if (below == kWave) {
                int lo = s + kWave, hi = e;
                while (hi - lo > kWave) {
                    const int step = (hi - lo + kWave - 1) / kWave;
                    const int at = lo + lane * step;
                    const int c = at < hi ? ci[at] : INT_MAX;
                    const int nb = (int)__popcll(__builtin_amdgcn_ballot_w64(c < c0));
                    const int nlo = nb == 0 ? lo : lo + (nb - 1) * step + 1;
                    hi = min(hi, lo + nb * step);
                    lo = nlo;
                }
                const int c = lane < hi - lo ? ci[lo + lane] : INT_MAX;
                b = lo + (int)__popcll(__builtin_amdgcn_ballot_w64(c < c0));
            }
            base[i] = b;
            const bool in = lane < e - b;
            const int cr = ci[in ? b + lane : 0];
            const int c = in ? cr : INT_MAX;
            colt[i] = c < c1 ? c : INT_MAX;
            cnt[i] = (int)__popcll(__builtin_amdgcn_ballot_w64(c < c1));
        }
    }
    // epilogue operands, read from a valid stand-in array when absent
    const float *__restrict__ vz = p.mask_values ? p.mask_values + z * p.stride_values : nullptr;
    float *__restrict__ oz = p.out + z * p.stride_out;
    const float *vsrc = vz ? vz : reinterpret_cast<const float *>(ci);
    const float *psrc = p.beta != 0.f ? oz : reinterpret_cast<const float *>(ci);
    // ---- the wave's entries in the tile, rows after one another: list entry
    // e = pre[i] + j is row i's j-th, coded (row << 6) | (column - c0)
    unsigned short *s_list =
        reinterpret_cast<unsigned short *>(lds + q.off_tab) + wave * (kRpw * kWave);
    int pre[kRpw];
    int total = 0;
#pragma unroll
    for (int i = 0; i < kRpw; ++i) {
        pre[i] = total;
        total += cnt[i];
        if (lane < cnt[i]) {
            // (columns ascend within a row; the range check only keeps LDS
            // reads in bounds for input that breaks that)
            const unsigned rel = (unsigned)(colt[i] - c0);
            s_list[pre[i] + lane] = (unsigned short)((i << 6) | (rel < (unsigned)(c1 - c0) ? rel : 0u));
        }
    }
    // ---- compute: 64 list entries per pass, 16 lanes per entry (4 entries a
    // step): lane gl of a group sums vectors gl, gl + 16, ... of the X and Y
    // rows in order with FMA (16 lanes read 256 contiguous bytes of one row:
    // no bank conflicts), group_sum adds the 16 partial sums, and lane
    // (g, gl) keeps the sum of step gl, entry t0 + 4 gl + g, which it writes.
    constexpr int kG = 16, kNg = kWave / kG;
    const int g = lane / kG;
    const int gl = lane - g * kG;
    // the position of list entry e, and its epilogue operands
    auto position = [&](int e) {
        int at = 0;
#pragma unroll
        for (int i = 0; i < kRpw; ++i)
            if (e >= pre[i] && e < pre[i] + cnt[i]) at = base[i] + (e - pre[i]);
        return at;
    };
    // the first pass's operands are read before the barrier, which waits
    // only for LDS: their latency overlaps it and the first steps
    int at = position(gl * kNg + g);
    float v = vsrc[at];
    float prior = psrc[at];
    __syncthreads();
    for (int t0 = 0; t0 < total; t0 += kWave) {
        const int live = min(kWave, total - t0);
        const int eo = t0 + gl * kNg + g;  // the entry this lane writes
        if (t0 > 0) {
            at = position(eo);
            v = vsrc[at];
            prior = psrc[at];
        }
        const int steps = (live + kNg - 1) / kNg;
        float kept = 0.f;
        // two steps at a time (one for kNv > 4, for registers), so that their
        // LDS reads overlap
        constexpr int kH = kNv <= 4 ? 2 : 1;
        for (int st = 0; st < steps; st += kH) {
            float4 xv[kH][kNv], yv[kH][kNv];
#pragma unroll
            for (int h = 0; h < kH; ++h) {
                const unsigned code = s_list[min(t0 + (st + h) * kNg + g, total - 1)];
                const unsigned char *xr = lds + (unsigned)(wave + kWaves * (int)(code >> 6)) * q.x_pitch;
                const unsigned char *yr = lds + q.off_y + (code & 63u) * q.y_pitch;
#pragma unroll
                for (int u = 0; u < kNv; ++u) {
                    xv[h][u] = *reinterpret_cast<const float4 *>(xr + (u * kG + gl) * 16);
                    yv[h][u] = *reinterpret_cast<const float4 *>(yr + (u * kG + gl) * 16);
                }
            }
#pragma unroll
            for (int h = 0; h < kH; ++h) {
                float acc = 0.f;
#pragma unroll
                for (int u = 0; u < kNv; ++u) {
                    acc = fmaf(xv[h][u].x, yv[h][u].x, acc);
                    acc = fmaf(xv[h][u].y, yv[h][u].y, acc);
                    acc = fmaf(xv[h][u].z, yv[h][u].z, acc);
                    acc = fmaf(xv[h][u].w, yv[h][u].w, acc);
                }
                const float sum = group_sum<kG>(acc);
                if (gl == st + h) kept = sum;  // (a step past the last holds no entry this lane writes)
            }
        }
        if (eo < total) {
            float r = p.alpha * (vz ? v : 1.f) * kept;
            if (p.beta != 0.f) r = fmaf(p.beta, prior, r);
            oz[at] = r;
        }
    }
}

// out_z = in_z^T for a rows x cols matrix in_z (row-major, z = blockIdx.z):
// 32 x 32 tiles through LDS (one padding column, so the transposed reads hit
// distinct banks), 256 threads reading 4 rows each.  (c_base, r_base) is the
// first tile's corner, so that grids too large for one launch can be split.
template <typename E>
__global__ __launch_bounds__(256) void transpose_kernel(const E *__restrict__ in, E *__restrict__ out,
                                                        int rows, int cols, int r_base, int c_base,
                                                        long long stride_in, long long stride_out)
{
    constexpr int kT = 32;
    __shared__ E tile[kT][kT + 1];
    const E *iz = in + blockIdx.z * stride_in;
    E *oz = out + blockIdx.z * stride_out;
    const int c0 = c_base + (int)blockIdx.x * kT, r0 = r_base + (int)blockIdx.y * kT;
    const int tx = threadIdx.x % kT, ty = threadIdx.x / kT;  // ty in [0, 8)
#pragma unroll
    for (int i = 0; i < kT; i += 8) {
        const int r = r0 + ty + i, c = c0 + tx;
        if (r < rows && c < cols) tile[ty + i][tx] = iz[(size_t)r * cols + c];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kT; i += 8) {
        const int c = c0 + ty + i, r = r0 + tx;  // out row c, column r
        if (c < cols && r < rows) oz[(size_t)c * rows + r] = tile[tx][ty + i];
    }
}

template <typename E>
hipError_t launch_transpose(const void *in, void *out, int rows, int cols, long long stride_in,
                            long long stride_out, int batch, hipStream_t s)
{
    // Tiles per launch in each dimension: x, y and z stay within the grid limits.
    constexpr long long kMaxX = 1LL << 20, kMaxYZ = 65535;
    const long long tx = (cols + 31) / 32, ty = (rows + 31) / 32;
    for (long long z0 = 0; z0 < batch; z0 += kMaxYZ)
        for (long long y0 = 0; y0 < ty; y0 += kMaxYZ)
            for (long long x0 = 0; x0 < tx; x0 += kMaxX) {
                const dim3 grid((unsigned)std::min(kMaxX, tx - x0),
                                (unsigned)std::min(kMaxYZ, ty - y0),
                                (unsigned)std::min(kMaxYZ, (long long)batch - z0));
                hipLaunchKernelGGL((transpose_kernel<E>), grid, dim3(256), 0, s,
                                   static_cast<const E *>(in) + z0 * stride_in,
                                   static_cast<E *>(out) + z0 * stride_out, rows, cols,
                                   (int)(y0 * 32), (int)(x0 * 32), stride_in, stride_out);
                const hipError_t e = hipGetLastError();
                if (e != hipSuccess) return e;
            }
    return hipSuccess;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *dst, long long count,
                                                        long long stride)
{
    float *dz = dst + (long long)blockIdx.y * stride;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < count;
         i += (long long)gridDim.x * 256)
        dz[i] = 0.f;
}

template <typename E, int kG, int kNv, int kVec, bool kSm>
hipError_t launch_t(const SddmmParams &p, bool split, hipStream_t s)
{
    dim3 grid((unsigned)rows_grid(p));
    if constexpr (!kSm) {
        if (split) {
            hipLaunchKernelGGL((sddmm_split_kernel<E, kG, kNv, kVec>), grid,
                               dim3(kSplitParts * kWave), 0, s, p);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((sddmm_kernel<E, kG, kNv, kVec, kSm>), grid, dim3(kWave), 0, s, p);
    return hipGetLastError();
}

template <typename E>
hipError_t launch_multirow_e(int g, const SddmmParams &p, hipStream_t s)
{
    const long long units = ((long long)p.m + kWave / g - 1) / (kWave / g);
    const dim3 grid((unsigned)xcd_grid(p.batch, units));
    if (g == 8)
        hipLaunchKernelGGL((sddmm_multirow_kernel<E, 8>), grid, dim3(kWave), 0, s, p);
    else
        hipLaunchKernelGGL((sddmm_multirow_kernel<E, 16>), grid, dim3(kWave), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_multirow(Dtype dtype, int g, const SddmmParams &p, hipStream_t s)
{
    switch (dtype) {
    case Dtype::f16: return launch_multirow_e<_Float16>(g, p, s);
    case Dtype::bf16: return launch_multirow_e<bf16>(g, p, s);
    default: return launch_multirow_e<float>(g, p, s);
    }
}

template <typename E, bool kSm>
hipError_t launch_union_e(int g, const SddmmParams &p, hipStream_t s)
{
    constexpr int kW = kUnionWaves;
    const dim3 grid((unsigned)pu::grid<kW>(p.m, p.batch));
    const size_t lds = pu::dynamic_lds(p.k);
    if (g == 8)
        hipLaunchKernelGGL((sddmm_union_kernel<E, 8, kW, kSm>), grid, dim3(kW * kWave), lds, s, p);
    else
        hipLaunchKernelGGL((sddmm_union_kernel<E, 16, kW, kSm>), grid, dim3(kW * kWave), lds, s,
                           p);
    return hipGetLastError();
}

hipError_t launch_union(Dtype dtype, int g, bool softmax, const SddmmParams &p, hipStream_t s)
{
    switch (dtype) {
    case Dtype::f16:
        return softmax ? launch_union_e<_Float16, true>(g, p, s)
                       : launch_union_e<_Float16, false>(g, p, s);
    case Dtype::bf16:
        return softmax ? launch_union_e<bf16, true>(g, p, s) : launch_union_e<bf16, false>(g, p, s);
    default:
        return softmax ? launch_union_e<float, true>(g, p, s)
                       : launch_union_e<float, false>(g, p, s);
    }
}

template <typename E, int kG, int kVec, bool kSm>
hipError_t launch_nv(int nv, const SddmmParams &p, bool split, hipStream_t s)
{
    switch (nv) {
    case 1: return launch_t<E, kG, 1, kVec, kSm>(p, split, s);
    case 2: return launch_t<E, kG, 2, kVec, kSm>(p, split, s);
    case 4: return launch_t<E, kG, 4, kVec, kSm>(p, split, s);
    case 8: return launch_t<E, kG, 8, kVec, kSm>(p, split, s);
    default: return launch_t<E, kG, 0, kVec, kSm>(p, split, s);
    }
}

template <typename E, int kVec, bool kSm>
hipError_t launch_g(int g, int nv, const SddmmParams &p, bool split, hipStream_t s)
{
    switch (g) {
    case 4: return launch_nv<E, 4, kVec, kSm>(nv, p, split, s);
    case 8: return launch_nv<E, 8, kVec, kSm>(nv, p, split, s);
    default: return launch_nv<E, 16, kVec, kSm>(nv, p, split, s);
    }
}

// Element type E: 16-byte vectors of kVec16 elements, or single elements;
// scores written as they are, or row-softmaxed.
template <typename E, int kVec16>
hipError_t launch_typed(bool vec, bool softmax, bool split, int g, int nv,
                        const SddmmParams &p, hipStream_t s)
{
    if (softmax)
        return vec ? launch_g<E, kVec16, true>(g, nv, p, false, s)
                   : launch_g<E, 1, true>(g, nv, p, false, s);
    return vec ? launch_g<E, kVec16, false>(g, nv, p, split, s)
               : launch_g<E, 1, false>(g, nv, p, split, s);
}

template <typename E>
hipError_t launch_cols(bool buf, const SddmmParams &p, hipStream_t s)
{
    const dim3 grid((unsigned)xcd_grid(p.batch, p.m));
    if (buf)
        hipLaunchKernelGGL((sddmm_cols_kernel<E, true>), grid, dim3(kWave), 0, s, p);
    else
        hipLaunchKernelGGL((sddmm_cols_kernel<E, false>), grid, dim3(kWave), 0, s, p);
    return hipGetLastError();
}

inline bool aligned16(const void *ptr)
{
    return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0;
}

// waves: the kernel's workgroup size in waves (its launch bound)
template <class Kernel>
hipError_t launch_dk_fn(Kernel fn, int waves, const SddmmParams &p, const DkPanelParams &q,
                        hipStream_t s)
{
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)q.lds);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)xcd_grid(p.batch, (long long)q.panels * q.splits));
    hipLaunchKernelGGL(fn, grid, dim3(waves * kWave), q.lds, s, p, q);
    return hipGetLastError();
}

template <bool kVec>
hipError_t launch_dk_v(bool tile, const SddmmParams &p, const DkPanelParams &q, hipStream_t s)
{
    if (tile) {
        switch (q.nv) {
        case 1: return launch_dk_fn(sddmm_dk_tile_kernel<64, 8, 1, kVec>, 8, p, q, s);
        case 2: return launch_dk_fn(sddmm_dk_tile_kernel<64, 8, 2, kVec>, 8, p, q, s);
        case 4: return launch_dk_fn(sddmm_dk_tile_kernel<64, 8, 4, kVec>, 8, p, q, s);
        case 8: return launch_dk_fn(sddmm_dk_tile_kernel<16, 4, 8, kVec>, 4, p, q, s);
        default: return launch_dk_fn(sddmm_dk_tile_kernel<8, 4, 16, kVec>, 4, p, q, s);
        }
    }
    switch (q.rows * 4 + q.rounds) {
    case 32 * 4 + 2: return launch_dk_fn(sddmm_dk_panel_kernel<32, 2, kVec>, 4, p, q, s);
    case 32 * 4 + 1: return launch_dk_fn(sddmm_dk_panel_kernel<32, 1, kVec>, 4, p, q, s);
    case 16 * 4 + 1: return launch_dk_fn(sddmm_dk_panel_kernel<16, 1, kVec>, 4, p, q, s);
    default: return launch_dk_fn(sddmm_dk_panel_kernel<8, 1, kVec>, 4, p, q, s);
    }
}

hipError_t launch_dk(bool tile, const SddmmParams &p, const DkPanelParams &q, bool vec,
                     hipStream_t s)
{
    return vec ? launch_dk_v<true>(tile, p, q, s) : launch_dk_v<false>(tile, p, q, s);
}

// LDS per workgroup of the d x k panel kernel: two workgroups per CU.
constexpr unsigned kDkLdsBudget = 76u * 1024u;
constexpr int kDkTargetGroups = 512;  // workgroups wanted before splitting Y's columns
constexpr double kDkTileDensity = 0.05;  // mean mask density from which the tile kernel runs
constexpr unsigned kDkTileLdsBudget = 150u * 1024u;  // 64-row tiles: one workgroup per CU

// The shape of the d x k kernels for fp32 operands, or false when they do not
// apply (d beyond 1024, or LDS cannot hold a useful chunk).  Masks of mean
// density 1/20 or more (few columns of a 32-row tile untouched) take the tile
// kernel, one tile per workgroup; sparser ones the panel kernel.
bool plan_dk_panel(const SddmmArgs &a, SddmmPlan *plan)
{
    if (a.dtype != Dtype::f32 || a.d <= 0 || a.k <= 0 || a.softmax) return false;
    const int dv = (a.d + 3) / 4;  // 16-byte vectors per staged row
    if (dv > 256) return false;
    DkPanelParams &q = plan->dk;
    q.rows = dk_rows(dv);
    q.rounds = dk_rounds(dv);
    q.x_pitch = q.y_pitch = 16u * ((unsigned)dv | 1u);  // an odd number of 16-byte units
    q.x_shift = 0;
    while ((1 << q.x_shift) < dv) ++q.x_shift;  // X's vectors per row, to a power of 2
    q.panels = (a.m + q.rows - 1) / q.rows;
    const unsigned xbytes = (unsigned)q.rows * q.x_pitch;
    const bool xvec = a.d % 4 == 0 && aligned16(a.x) && a.stride_x % 4 == 0;
    const double density = (double)a.nnz / ((double)a.m * (double)a.k);
    if (density >= kDkTileDensity) {
        // 64 x 64 tiles with eight waves when LDS holds them (d <= 256), else
        // the panel kernel's heights with four waves and the widest tile
        // that leaves room for two workgroups per CU
        // 16 lanes per entry read kNv vectors each: rows padded to 16 kNv
        // vectors (and one more, so that a pitch is an odd number of 16 bytes)
        q.nv = dv <= 16 ? 1 : dv <= 32 ? 2 : dv <= 64 ? 4 : dv <= 128 ? 8 : 16;
        q.rows = q.nv <= 4 ? 64 : q.nv == 8 ? 16 : 8;
        q.x_pitch = q.y_pitch = 16u * (16u * (unsigned)q.nv + 1u);
        const unsigned xb = (unsigned)q.rows * q.x_pitch;
        const unsigned list = (unsigned)q.rows * kWave * 2u;
        const unsigned budget = q.rows == 64 ? kDkTileLdsBudget : kDkLdsBudget;
        int kc = xb + list < budget
                     ? (int)std::min<unsigned>(kDkTileCols, (budget - xb - list) / q.y_pitch) & ~3
                     : 0;
        q.panels = (a.m + q.rows - 1) / q.rows;
        if (kc >= 8) {
            q.kc = kc;
            q.splits = (a.k + kc - 1) / kc;
            if (xcd_grid(a.batch, (long long)q.panels * q.splits) <= 0x7fffffffLL) {
                q.off_y = xb;
                q.off_tab = xb + (unsigned)kc * q.y_pitch;  // per-wave entry lists
                q.lds = q.off_tab + (unsigned)q.rows * kWave * 2u;
                // 16-byte reads of X and Y rows
                plan->vec = xvec && a.k % 4 == 0 && aligned16(a.y) && a.stride_y % 4 == 0;
                plan->kind = SddmmPlan::kDkTile;
                return true;
            }
        }
    }
    q.rows = dk_rows(dv);
    q.x_pitch = q.y_pitch = 16u * ((unsigned)dv | 1u);
    q.panels = (a.m + q.rows - 1) / q.rows;
    const unsigned tab = (unsigned)q.rows * (unsigned)q.rounds * kWave * 4u;
    const unsigned fixed = xbytes + tab + 2u * 1024u + 1024u + 1024u + 64u;
    if (fixed >= kDkLdsBudget) return false;
    q.kc = (int)std::min<unsigned>(256u, (kDkLdsBudget - fixed) / q.y_pitch);
    if (q.kc < 8) return false;
    const long long units = (long long)a.batch * q.panels;
    const long long want = (kDkTargetGroups + units - 1) / units;
    const long long most = std::max<long long>(1, a.k / (2LL * q.kc));
    q.splits = (int)std::max<long long>(1, std::min(want, most));
    if (xcd_grid(a.batch, (long long)q.panels * q.splits) > 0x7fffffffLL) return false;
    q.off_y = xbytes;
    q.off_tab = q.off_y + (unsigned)q.kc * q.y_pitch;
    q.off_bits = q.off_tab + tab;
    q.off_rank = q.off_bits + 2u * 1024u;
    q.off_col = q.off_rank + 1024u;
    q.off_misc = q.off_col + 1024u;
    q.lds = q.off_misc + 64u;
    plan->vec = xvec;
    plan->kind = SddmmPlan::kDkPanel;
    return true;
}

}  // namespace

hipError_t launch_fill_zero(float *dst, long long count, hipStream_t stream)
{
    if (count <= 0) return hipSuccess;
    const long long blocks = std::min<long long>((count + 255) / 256, 65536);
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks, 1), dim3(256), 0,
                       stream, dst, count, 0LL);
    return hipGetLastError();
}

// Lanes per entry kG: the smallest of 4/8/16 covering the row's vectors (16
// beyond).  Vectors per lane kNv rounded up to 1/2/4/8; wider rows take the
// kNv == 0 loop.  d == 0 with no mask values and beta == 0 zero-fills every
// batch's outputs; otherwise the kernels run with empty dot products.
hipError_t plan_sddmm(const SddmmArgs &a, SddmmPlan *plan)
{
    plan->kind = SddmmPlan::kNothing;
    plan->dtype = a.dtype;
    plan->softmax = false;
    plan->split = false;
    plan->multirow = false;
    plan->panel_union = false;
    plan->t_src = nullptr;
    plan->t_src_stride = 0;
    plan->t_batch = 0;
    if (a.m == 0 || a.nnz == 0) return hipSuccess;
    if (xcd_grid(a.batch, a.m) > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    // A row's 64-entry windows spread over a workgroup of waves (outputs are
    // bit-identical: an entry needs no combine step): on request, and by
    // default for one batch entry whose rows average 16 entries or more.  A
    // row of one window leaves the other waves nothing to do (they exit at
    // once), so uniform rows lose little while the longest rows of a
    // heavy-tailed structure no longer set the launch's duration (the card's
    // I4).  Batched problems keep one wave per row slot: their many row slots
    // already fill the GPU.  The softmax needs whole rows.
    const bool auto_split = a.batch == 1 && (long long)a.nnz >= 16LL * a.m;
    plan->split = !a.softmax && (a.parts > 1 || auto_split);
    SddmmParams &p = plan->p;
    p.m = a.m;
    p.batch = a.batch;
    p.d = a.d;
    p.k = a.k;
    p.nnz = a.nnz;
    p.row_indices = a.row_indices;
    p.row_offsets = a.row_offsets;
    p.col_indices = a.col_indices;
    p.mask_values = a.mask_values;
    p.x = a.x;
    p.y = a.y;
    p.alpha = a.alpha;
    p.beta = a.beta;
    p.out = a.out;
    p.stride_values = a.stride_values;
    p.stride_x = a.stride_x;
    p.stride_y = a.stride_y;
    p.stride_out = a.stride_out;
    const int eb = a.dtype == Dtype::f32 ? 4 : 2;  // bytes per element of X and Y
    const int vlen = 16 / eb;                        // elements per 16-byte vector
    // Buffer offsets into Y must stay below 2^31 (padding offsets lie beyond).
    const bool buf = (long long)a.k * (long long)a.d * eb <= (1LL << 31);
    p.y_bytes = buf ? (unsigned)((long long)a.k * a.d * eb) : 0u;
    plan->buf = buf;
    if (a.y_layout == 1 && a.workspace == nullptr) {
        if (!plan_dk_panel(a, plan)) plan->kind = SddmmPlan::kCols;
        return hipSuccess;
    }
    if (a.y_layout == 1) {
        // Y^T (k x d per batch entry, or one shared copy) into the workspace,
        // then the k x d kernels on it.
        plan->t_src = a.y;
        plan->t_src_stride = a.stride_y;
        plan->t_batch = a.stride_y == 0 ? 1 : a.batch;
        p.y = a.workspace;
        p.stride_y = a.stride_y == 0 ? 0 : (long long)a.k * a.d;
    }
    plan->softmax = a.softmax;
    if (a.d == 0 && a.mask_values == nullptr && a.beta == 0.f && !a.softmax) {
        plan->kind = SddmmPlan::kFill;
        return hipSuccess;
    }
    const bool vec = (a.d % vlen == 0) && aligned16(a.x) && aligned16(p.y) &&
                     (a.stride_x % vlen == 0) && (p.stride_y % vlen == 0);
    // Register-resident X and buffer gathers need valid offsets below Y's size
    // and padding offsets (>= 2^31) beyond it.
    const int kvec = vec ? vlen : 1;
    const int dv = (a.d + kvec - 1) / kvec;
    const int g = dv <= 4 ? 4 : dv <= 8 ? 8 : 16;
    const int need = (dv + g - 1) / g;
    int nv = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : 0;
    if (!buf) nv = 0;
    plan->kind = SddmmPlan::kRows;
    plan->vec = vec;
    plan->g = g;
    plan->nv = nv;
    // Rows of one 16-byte vector per lane with 8 or 16 lanes per entry (fp32 d
    // from 20 to 64; 16-bit d from 40 to 128) not split over waves: several
    // rows per wave (sddmm_multirow_kernel).  Its buffer resources need X, Y
    // and the outputs of one batch entry under 2 GiB.
    const int rpw = kWave / g;
    const bool multirow_shape =
        vec && !plan->split && nv == 1 && (g == 8 || g == 16) && buf &&
        (long long)a.nnz * 4 < (1LL << 31) && (long long)a.m * a.d * eb < (1LL << 31);
    plan->multirow = multirow_shape && !a.softmax &&
                     xcd_grid(a.batch, ((long long)a.m + rpw - 1) / rpw) <= 0x7fffffffLL;
    // Batched problems of that shape on up to 65,536 columns, scores alone or
    // with their row softmax: the panel-union kernel, which falls back panel by
    // panel (to the multi-row walk, or to the row kernel's softmax body) where
    // columns are not shared.  One batch entry would leave three of its four
    // waves idle.
    plan->panel_union = multirow_shape && a.batch >= 2 && a.k <= pu::kMaxK &&
                        pu::grid<kUnionWaves>(a.m, a.batch) <= 0x7fffffffLL;
    return hipSuccess;
}

hipError_t run_sddmm(const SddmmPlan &plan, hipStream_t stream)
{
    const SddmmParams &p = plan.p;
    if (plan.t_src != nullptr && p.d > 0 && p.k > 0) {
        const long long stride_out = (long long)p.k * p.d;
        const hipError_t e =
            plan.dtype == Dtype::f32
                ? launch_transpose<float>(plan.t_src, const_cast<void *>(p.y), p.d, p.k,
                                          plan.t_src_stride, stride_out, plan.t_batch, stream)
                : launch_transpose<unsigned short>(plan.t_src, const_cast<void *>(p.y), p.d,
                                                   p.k, plan.t_src_stride, stride_out,
                                                   plan.t_batch, stream);
        if (e != hipSuccess) return e;
    }
    switch (plan.kind) {
    case SddmmPlan::kNothing:
        return hipSuccess;
    case SddmmPlan::kFill: {
        const long long blocks = std::min<long long>((p.nnz + 255) / 256, 65536);
        for (long long z0 = 0; z0 < p.batch; z0 += 65535) {  // batch entries on grid y
            const long long nz = std::min<long long>(65535, p.batch - z0);
            hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks, (unsigned)nz), dim3(256),
                               0, stream, p.out + z0 * p.stride_out, (long long)p.nnz,
                               p.stride_out);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    case SddmmPlan::kDkPanel:
        return launch_dk(false, p, plan.dk, plan.vec, stream);
    case SddmmPlan::kDkTile:
        return launch_dk(true, p, plan.dk, plan.vec, stream);
    case SddmmPlan::kCols:
        switch (plan.dtype) {
        case Dtype::f16: return launch_cols<_Float16>(plan.buf, p, stream);
        case Dtype::bf16: return launch_cols<bf16>(plan.buf, p, stream);
        default: return launch_cols<float>(plan.buf, p, stream);
        }
    default:
        break;
    }
    if (plan.panel_union) return launch_union(plan.dtype, plan.g, plan.softmax, p, stream);
    if (plan.multirow) return launch_multirow(plan.dtype, plan.g, p, stream);
    const bool sm = plan.softmax, sp = plan.split;
    switch (plan.dtype) {
    case Dtype::f16:
        return launch_typed<_Float16, 8>(plan.vec, sm, sp, plan.g, plan.nv, p, stream);
    case Dtype::bf16: return launch_typed<bf16, 8>(plan.vec, sm, sp, plan.g, plan.nv, p, stream);
    default: return launch_typed<float, 4>(plan.vec, sm, sp, plan.g, plan.nv, p, stream);
    }
}

const char *sddmm_kernel_name(const SddmmArgs &a)
{
    SddmmPlan plan;
    if (plan_sddmm(a, &plan) != hipSuccess) return "unsupported";
    switch (plan.kind) {
    case SddmmPlan::kNothing: return "none";
    case SddmmPlan::kFill: return "fill";
    case SddmmPlan::kCols: return "columns";
    case SddmmPlan::kDkPanel: return "dk_panel";
    case SddmmPlan::kDkTile: return "dk_tile";
    case SddmmPlan::kRows:
        return plan.panel_union ? "panel_union"
               : plan.multirow  ? "multirow"
               : plan.split     ? "split"
                                : "rows";
    }
    return "unknown";
}

hipError_t launch_sddmm(const SddmmArgs &a, hipStream_t stream)
{
    SddmmPlan plan;
    const hipError_t e = plan_sddmm(a, &plan);
    return e != hipSuccess ? e : run_sddmm(plan, stream);
}

}  // namespace spk
