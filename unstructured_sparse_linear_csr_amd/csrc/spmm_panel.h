// CSR SpMM with B staged in LDS and shared by a panel of rows ("Sparse GPU
// Kernels for Deep Learning", summary card, "Summary": SpMM on plain CSR with
// 1-D tiling and vector memory access on misaligned sparse rows).
//
// Why.  The wide kernel (spmm_wide.h) gathers one B row segment from L2 per
// entry: each FMA consumes 4 freshly gathered bytes, and the chip's L2 row
// gather runs at 20-26 TB/s, which caps that kernel near 10-13 TFLOP/s.  LDS
// reads run about five times faster (16-byte reads of 256-byte rows: ~110
// TB/s), so a workgroup that copies a block of B into LDS once and lets many
// rows read it there moves the bound from the L2 gather to LDS bandwidth and
// the FMA rate.  The copy pays off when the rows sharing it touch each B row
// several times: rows per workgroup times density well above 1.
//
// Mapping.  A workgroup of kWaves waves owns a panel of kRows consecutive work
// slots (rows in row_indices order) by one column tile of kT = 4 * kVecs * kLpr
// columns.  Each wave holds kRounds rounds of kRpw = 64 / kLpr rows; a group of
// kLpr lanes serves one row and a lane owns kVecs vectors of 4 output columns
// of it, in registers for the whole launch (C is written once; no atomics, no
// split of a row's sum).  A lane thus pays one address computation per entry
// for 4 * kVecs FMAs.  K is walked in chunks of kKc rows of B: chunk c's block
// B[c*kKc .. c*kKc + kKc)[tile columns] sits in LDS while the next chunk's
// block is loaded into registers; with two buffers it is written to the other
// one when the chunk is done (one workgroup barrier per chunk), with one
// buffer after every wave has left the chunk (two barriers).
//
// Entries.  Within a chunk, a row's entries with columns in the chunk are
// contiguous (columns ascend within a row).  Each row keeps a cursor: a window
// of kEpl * kLpr entries from the cursor (aligned down to a multiple of 4; the
// misaligned prefix masked) is staged in LDS as (LDS byte offset of the B row
// within the chunk block, value) pairs, entries outside [cursor, row end) or
// beyond the chunk become padding that reads a zero row with value 0, and the
// cursor moves past the chunk's entries.  The first window of each row's next
// chunk is loaded into registers as soon as its cursor is known, so its
// latency overlaps the rest of the chunk.
//
// Order of summation: every entry of a row in CSR order, sequentially, one FMA
// each (padding adds 0 * 0) -- the wide kernel's order, so results are
// bit-identical to it and independent of the row order.
#pragma once

#include <type_traits>

#include "sp_device.h"
#include "sp_types.h"
#include "spmm_wide.h"

namespace spk {
namespace spmm_detail {

// f(integral_constant<int, I>) for I = kFirst ... kEnd - 1, in order.
template <int kFirst, int kEnd, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (kFirst < kEnd) {
        f(std::integral_constant<int, kFirst>{});
        static_for<kFirst + 1, kEnd>(f);
    }
}

struct PanelParams {
    int k;       // rows of B
    int chunks;  // ceil(k / kKc)
    int panels;  // ceil(m / kRows)
    int tiles;   // ceil(n / kT)
};

// kLpr lanes per row, each owning kVecs vectors of 4 columns: vector v of
// lane l covers tile columns (v * kLpr + l) * 4 ... + 3, so one 16-byte LDS
// read per vector covers kLpr * 16 contiguous bytes of a B row per group.
template <int kLpr, int kVecs, int kWaves, int kRounds, int kEpl, int kKc, int kBufs>
struct PanelShape {
    static constexpr int kT = 4 * kVecs * kLpr;            // columns per tile
    static constexpr int kRpw = kWave / kLpr;              // rows of a wave at a time
    static constexpr int kRows = kWaves * kRpw * kRounds;  // rows per workgroup
    static constexpr int kThreads = kWaves * kWave;
    static constexpr int kKcRows = kKc;                    // B rows per chunk
    static constexpr int kWin = kEpl * kLpr;               // staged entries per row per window
    static constexpr int kPitch = kWin + kU + 4;           // see spmm_wide_body
    static constexpr int kStageBytes = kWaves * kRpw * kPitch * 4;  // one field
    static constexpr int kVecPerRow = kT / 4;              // float4s per B row of the tile
    static constexpr int kBlockVecs = kKc * kVecPerRow;    // float4s per chunk block
    static constexpr int kNb = kBlockVecs / kThreads;      // per thread
    static_assert(kBlockVecs % kThreads == 0, "whole chunk blocks per thread");
    static_assert(kEpl % 4 == 0 && kWin % kU == 0, "whole segments and batches");
    static_assert(kBufs == 1 || kBufs == 2, "one or two block buffers");
    // LDS: staged offsets, staged values, the zero row, then the B buffers
    static constexpr int kZeroOffset = 2 * kStageBytes;
    static constexpr int kBufOffset = kZeroOffset + kT * 4;
    static constexpr int kBufBytes = kKc * kT * 4;
    static constexpr size_t lds_bytes(int chunks)
    {
        return (size_t)kBufOffset + (size_t)(chunks > 1 ? kBufs : 1) * kBufBytes;
    }
};

// acc += the products of the staged slots [0, wend) (rounded up to whole
// batches of 4; slots from `win` on are padding) with their B vectors in LDS
// (lane_b + staged offset + v * kVecStride for vector v).  Four rotating sets
// of staged pairs and two of B vectors: at step s the pairs of batch s + 2 are
// read, the B vectors of batch s + 1 fetched, and batch s is summed, entries in
// slot order.
template <int kVecs, int kVecStride>
__device__ __forceinline__ void panel_batches(const int *g_off, const float *g_val,
                                              const unsigned char *lane_b, int wend, int win,
                                              float *acc)
{
    constexpr int kB = 4;
    int4 o[4];
    float4 v[4];
    float4 b[2][kB][kVecs];
    auto read = [&](int slot, int4 &oo, float4 &vv) {
        slot = min(slot, win);
        oo = *reinterpret_cast<const int4 *>(g_off + slot);
        vv = *reinterpret_cast<const float4 *>(g_val + slot);
    };
    auto fetch1 = [&](int off, float4 (&bb)[kVecs]) {
        const unsigned char *src = lane_b + off;
#pragma unroll
        for (int x = 0; x < kVecs; ++x)
            bb[x] = *reinterpret_cast<const float4 *>(src + x * kVecStride);
    };
    auto fetch = [&](const int4 &oo, float4 (&bb)[kB][kVecs]) {
        fetch1(oo.x, bb[0]);
        fetch1(oo.y, bb[1]);
        fetch1(oo.z, bb[2]);
        fetch1(oo.w, bb[3]);
    };
    auto sum = [&](const float4 &vv, const float4 (&bb)[kB][kVecs]) {
        const float a[kB] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int u = 0; u < kB; ++u)
#pragma unroll
            for (int x = 0; x < kVecs; ++x) GVec<float, 4>::fma(a[u], bb[u][x], acc + 4 * x);
    };
    read(0, o[0], v[0]);
    read(kB, o[1], v[1]);
    fetch(o[0], b[0]);
    for (int j = 0;; j += 4 * kB) {
        // steps j, j + kB, j + 2 kB, j + 3 kB (buffer sets 0 .. 3)
        read(j + 2 * kB, o[2], v[2]);
        fetch(o[1], b[1]);
        keep_issued_above();
        sum(v[0], b[0]);
        if (j + kB >= wend) break;
        read(j + 3 * kB, o[3], v[3]);
        fetch(o[2], b[0]);
        keep_issued_above();
        sum(v[1], b[1]);
        if (j + 2 * kB >= wend) break;
        read(j + 4 * kB, o[0], v[0]);
        fetch(o[3], b[1]);
        keep_issued_above();
        sum(v[2], b[0]);
        if (j + 3 * kB >= wend) break;
        read(j + 5 * kB, o[1], v[1]);
        fetch(o[0], b[0]);
        keep_issued_above();
        sum(v[3], b[1]);
        if (j + 4 * kB >= wend) break;
    }
}

template <int kLpr, int kVecs, int kWaves, int kRounds, int kEpl, int kKc, int kBufs>
__device__ __forceinline__ void spmm_panel_body(const SpmmParams &p, const PanelParams &q,
                                                long long w)
{
    using S = PanelShape<kLpr, kVecs, kWaves, kRounds, kEpl, kKc, kBufs>;
    constexpr int kT = S::kT, kRpw = S::kRpw, kWin = S::kWin, kPitch = S::kPitch;
    constexpr int kSeg = kEpl / 4;
    constexpr int kAcc = 4 * kVecs;
    extern __shared__ __align__(16) unsigned char smem[];

    if (w < 0) return;  // padding slot of the XCD order (uniform for the workgroup)
    const int tile = (int)(w / q.panels);
    const int panel = (int)(w - (long long)tile * q.panels);
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int grp = kRpw == 1 ? 0 : lane / kLpr;
    const int gl = kRpw == 1 ? lane : lane - grp * kLpr;

    int *g_off = reinterpret_cast<int *>(smem) + (wave * kRpw + grp) * kPitch;
    float *g_val = reinterpret_cast<float *>(smem + S::kStageBytes) + (wave * kRpw + grp) * kPitch;
    float *s_zero = reinterpret_cast<float *>(smem + S::kZeroOffset);
    unsigned char *s_buf = smem + S::kBufOffset;

    const float *__restrict__ vals = static_cast<const float *>(p.values);
    const float *__restrict__ bm = static_cast<const float *>(p.b);

    for (int i = tid; i < kT; i += S::kThreads) s_zero[i] = 0.f;

    // This lane group's rows, one per round.
    int row[kRounds], cur[kRounds], end[kRounds];
    float acc[kRounds][kAcc];
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
        const int slot = panel * S::kRows + (r * kWaves + wave) * kRpw + grp;
        const bool has = slot < p.m;
        row[r] = has ? (p.row_indices ? p.row_indices[slot] : slot) : -1;
        cur[r] = has ? p.row_offsets[row[r]] : 0;
        end[r] = has ? p.row_offsets[row[r] + 1] : 0;
#pragma unroll
        for (int t = 0; t < kAcc; ++t) acc[r][t] = 0.f;
    }

    // ---- B chunk blocks: thread tid moves float4 j*kThreads + tid of a block
    float4 breg[S::kNb];
    auto load_block = [&](int c) {
        const int k0 = c * kKc;
#pragma unroll
        for (int j = 0; j < S::kNb; ++j) {
            const int e = j * S::kThreads + tid;
            const int kk = e / S::kVecPerRow;
            const int gcol = tile * kT + (e - kk * S::kVecPerRow) * 4;
            breg[j] = (k0 + kk < q.k && gcol < p.n)
                          ? *reinterpret_cast<const float4 *>(bm + (size_t)(k0 + kk) * p.n + gcol)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto store_block = [&](int c) {
        float *buf = reinterpret_cast<float *>(s_buf + (kBufs == 2 ? (c & 1) : 0) * S::kBufBytes);
#pragma unroll
        for (int j = 0; j < S::kNb; ++j)
            *reinterpret_cast<float4 *>(buf + (j * S::kThreads + tid) * 4) = breg[j];
    };

    // ---- CSR windows: kSeg 16-byte segments of columns and values per lane,
    // starting at the cursor rounded down to a multiple of 4
    int4 wc[kRounds][kSeg];
    float4 wv[kRounds][kSeg];
    int wbase[kRounds];
    auto load_window = [&](int r, int base) {
        wbase[r] = base;
#pragma unroll
        for (int sg = 0; sg < kSeg; ++sg) {
            const int e = base + (sg * kLpr + gl) * 4;
            int4 c4 = make_int4(0, 0, 0, 0);
            float4 v4 = make_float4(0.f, 0.f, 0.f, 0.f);
            if (e < end[r]) {
                if (e + 4 <= p.nnz) {
                    c4 = *reinterpret_cast<const int4 *>(p.col_indices + e);
                    v4 = *reinterpret_cast<const float4 *>(vals + e);
                } else {
                    int cc[4] = {0, 0, 0, 0};
                    float vv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (e + t < p.nnz) {
                            cc[t] = p.col_indices[e + t];
                            vv[t] = vals[e + t];
                        }
                    c4 = make_int4(cc[0], cc[1], cc[2], cc[3]);
                    v4 = make_float4(vv[0], vv[1], vv[2], vv[3]);
                }
            }
            wc[r][sg] = c4;
            wv[r][sg] = v4;
        }
    };

    load_block(0);
    store_block(0);
    if (q.chunks > 1) load_block(1);
#pragma unroll
    for (int r = 0; r < kRounds; ++r) load_window(r, cur[r] & ~3);
    __syncthreads();

    for (int c = 0; c < q.chunks; ++c) {
        const int k0 = c * kKc;
        const int kend = min(k0 + kKc, q.k);
        // LDS byte address of this lane's first vector in the chunk's block,
        // and the offset from the block to the zero row (padding slots)
        const unsigned char *blk = s_buf + (kBufs == 2 ? (c & 1) : 0) * S::kBufBytes;
        const unsigned char *lane_b = blk + gl * 16;
        const int zoff = (int)(reinterpret_cast<const unsigned char *>(s_zero) - blk);
        // one pass per round, unrolled at compile time (each round's state
        // stays in its own registers)
        static_for<0, kRounds>([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            for (;;) {
                // ---- stage the window held in registers: an entry is in if
                // it lies in [cursor, row end) and its column in the chunk
                const int base = wbase[r];
                const unsigned span = (unsigned)(end[r] - cur[r]);
                int taken = 0;
#pragma unroll
                for (int sg = 0; sg < kSeg; ++sg) {
                    const int slot0 = (sg * kLpr + gl) * 4;
                    const int e = base + slot0;
                    const int cc[4] = {wc[r][sg].x, wc[r][sg].y, wc[r][sg].z, wc[r][sg].w};
                    const float vv[4] = {wv[r][sg].x, wv[r][sg].y, wv[r][sg].z, wv[r][sg].w};
                    int off[4];
                    float val[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const bool in = (unsigned)(e + t - cur[r]) < span &&
                                        (unsigned)(cc[t] - k0) < (unsigned)(kend - k0);
                        off[t] = in ? (cc[t] - k0) * (kT * 4) : zoff;
                        val[t] = in ? vv[t] : 0.f;
                        taken += in;
                    }
                    *reinterpret_cast<int4 *>(g_off + slot0) = make_int4(off[0], off[1], off[2], off[3]);
                    *reinterpret_cast<float4 *>(g_val + slot0) =
                        make_float4(val[0], val[1], val[2], val[3]);
                }
                for (int j = gl; j < kU; j += kLpr) {
                    g_off[kWin + j] = zoff;
                    g_val[kWin + j] = 0.f;
                }
                taken = group_reduce<kLpr>(taken, OpAdd{});
                const int ncur = cur[r] + taken;
                // The window ended inside the chunk with the row going on: the
                // next entries may belong to the chunk too.
                const bool more = ncur == base + kWin && ncur < end[r];
                const int my_end = ncur - base;
                cur[r] = ncur;
                // Next window: the rest of this chunk, else this round's first
                // window of the next chunk (its data arrives during the rest of
                // the chunk).
                load_window(r, more ? ncur : (ncur & ~3));
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

                // ---- accumulate (the bound is wave-uniform, so the pipelined
                // steps are straight-line code)
                const int wend = __builtin_amdgcn_readfirstlane(
                    strided_wave_reduce<kLpr>(my_end, OpMax{}));
                if (wend > 0)
                    panel_batches<kVecs, kLpr * 16>(g_off, g_val, lane_b, wend, kWin, acc[r]);
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                if (!__any(more)) break;  // wave-uniform
            }
        });
        if (c + 1 < q.chunks) {
            if constexpr (kBufs == 2) {
                // Block c + 1 goes to the buffer chunk c - 1 used; every wave
                // left chunk c - 1 at the previous barrier.
                store_block(c + 1);
                if (c + 2 < q.chunks) load_block(c + 2);
                __syncthreads();
            } else {
                __syncthreads();  // every wave is done with block c
                store_block(c + 1);
                if (c + 2 < q.chunks) load_block(c + 2);
                __syncthreads();
            }
        }
    }

#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
        if (row[r] < 0) continue;
        float *crow = p.c + (size_t)row[r] * (size_t)p.n;
#pragma unroll
        for (int x = 0; x < kVecs; ++x) {
            const int col = tile * kT + (x * kLpr + gl) * 4;
            if (col < p.n) GVec<float, 4>::store(crow + col, acc[r] + 4 * x);  // n % 4 == 0
        }
    }
}

}  // namespace spmm_detail
}  // namespace spk
