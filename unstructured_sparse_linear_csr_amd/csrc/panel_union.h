// The column union of a panel of consecutive CSR rows, shared by the kernels
// that compute such a panel as dense MFMA tiles (batched SDDMM in sddmm.hip,
// batched SpMM in spmm.hip).
//
// A workgroup of kWaves waves takes a panel of kRows consecutive rows and
// kWaves batch entries, one per wave.  The structure is shared by the batch
// entries, so the union is formed once for all of them, in LDS:
//  - a bitmap of the k columns (`ds_or`);
//  - a popcount prefix over its words: each set bit's rank is its column's
//    slot in the union;
//  - the union's columns in slot order;
//  - for every (panel row, slot) the entry it holds, as 1 + entry - e0
//    (0 = none).
// A panel whose union is wide against its entry count (more than kMaxCols
// columns, or tiles holding more than kReuse slots per entry) would spend more
// on products no entry needs than a per-entry gather costs: build() then
// stops after the count and returns -1, and the caller runs its per-entry
// path on the panel.
#pragma once

#include "sp_device.h"

namespace spk {
namespace panel_union {

constexpr int kRows = 16;          // rows per panel: the MFMA tile's height
constexpr int kWaves = 4;          // batch entries per workgroup, one per wave (default)
constexpr int kThreads = kWaves * kWave;
constexpr int kMaxCols = 256;      // distinct columns per panel on the tile path
constexpr int kMaxK = 65536;       // columns the LDS bitmap covers
constexpr int kReuse = 6;          // tile slots per entry the tile path accepts
constexpr int kCache = 8;          // column indices a thread keeps between the passes
// entry map rows padded by two slots, so that the four rows one read
// instruction of the tile loops touches fall in different banks
constexpr int kEmapStride = kMaxCols + 2;

template <int kW = kWaves> struct SharedT {
    __align__(16) unsigned short emap[kRows * kEmapStride];
    int ucol[kMaxCols];
    int wsum[kW];
};
using Shared = SharedT<>;

// Dynamic LDS: the bitmap and each word's rank.
inline size_t dynamic_lds(int k) { return 2 * sizeof(unsigned) * (size_t)((k + 31) / 32); }

// Workgroups of a launch over m rows and `batch` entries, kW per workgroup.
template <int kW = kWaves> inline long long grid(int m, int batch)
{
    return xcd_grid(((long long)batch + kW - 1) / kW, ((long long)m + kRows - 1) / kRows);
}

struct Panel {
    int hg;  // group of kW batch entries
    int r0;  // first row
    int nr;  // rows (kRows but for the last panel)
    int e0;  // first entry
    int pn;  // entries
};

// This workgroup's panel; false for a padding slot of the launch.
template <int kW = kWaves>
__device__ __forceinline__ bool panel_of(int m, int batch, const int *row_offsets, Panel &pp)
{
    const int panels = (m + kRows - 1) / kRows;
    const int groups = (batch + kW - 1) / kW;
    const long long w = xcd_work_index(groups, panels);
    if (w < 0) return false;
    pp.hg = (int)(w / panels);
    pp.r0 = (int)(w - (long long)pp.hg * panels) * kRows;
    pp.nr = min(kRows, m - pp.r0);
    pp.e0 = row_offsets[pp.r0];
    pp.pn = row_offsets[pp.r0 + pp.nr] - pp.e0;
    return true;
}

// Sets column c's bit (c < k) with one atomic per run of lanes that set bits
// of the same word.  A panel row's entries sit on consecutive lanes of a
// 16-lane DPP row in column order, so equal words form runs; the bits of a run
// are ORed into its first lane (the row mirrored, a shift-right scan, mirrored
// back), which alone issues the ds_or: the row's lanes no longer all hit the
// same LDS word.  Every lane of the wave must be active.
__device__ __forceinline__ void mark_column(unsigned c, unsigned k, unsigned *s_bits)
{
    const bool ok = c < k;
    const unsigned wd = ok ? (c >> 5) + 1u : 0u;   // word + 1 (0: nothing to set)
    unsigned bits = ok ? 1u << (c & 31) : 0u;
    // mirrored: lane i holds lane 15 - i's word and bits
    const unsigned mw = dpp_read<kDppRowMirror>(wd);
    unsigned mb = dpp_read<kDppRowMirror>(bits);
    // (row_shr reads lane i - s, and 0 at the row's start: no word matches 0)
    {
        const unsigned w1 = dpp_read<kDppRowShr1>(mw), b1 = dpp_read<kDppRowShr1>(mb);
        mb |= w1 == mw ? b1 : 0u;
        const unsigned w2 = dpp_read<kDppRowShr2>(mw), b2 = dpp_read<kDppRowShr2>(mb);
        mb |= w2 == mw ? b2 : 0u;
        const unsigned w4 = dpp_read<kDppRowShr4>(mw), b4 = dpp_read<kDppRowShr4>(mb);
        mb |= w4 == mw ? b4 : 0u;
        const unsigned w8 = dpp_read<kDppRowShr8>(mw), b8 = dpp_read<kDppRowShr8>(mb);
        mb |= w8 == mw ? b8 : 0u;
    }
    // back: lane i holds the OR of its run from lane i on
    bits = dpp_read<kDppRowMirror>(mb);
    const bool first = dpp_read<kDppRowShr1>(wd) != wd;
    if (ok && first) atomicOr(&s_bits[wd - 1u], bits);
}

// Forms the panel's union (pp.pn > 0; every thread of the workgroup calls
// it).  Returns the union's size with s.ucol and s.emap filled, or -1 for a
// panel that takes the per-entry path (no barrier follows that return, and
// every thread takes it).  Column indices past k, which a valid CSR never
// has, are left out.
template <int kW = kWaves>
__device__ __forceinline__ int build(const int *row_offsets, const int *col_indices, int k,
                                     const Panel &pp, SharedT<kW> &s, unsigned *s_dyn)
{
    constexpr int kT = kW * kWave;       // threads of the workgroup
    constexpr int kTpr = kT / kRows;     // threads per panel row
    // more entries than kRows rows of kMaxCols: some row alone is wider than
    // the tile path takes
    if (pp.pn > kRows * kMaxCols) return -1;
    const int nw = (k + 31) >> 5;
    unsigned *s_bits = s_dyn;
    unsigned *s_rank = s_dyn + nw;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;

    // kTpr threads per panel row; each keeps its first kCache column indices
    const int mr = tid / kTpr, mq = tid % kTpr;
    const int rb = row_offsets[pp.r0 + min(mr, pp.nr)];
    const int re = row_offsets[pp.r0 + min(mr + 1, pp.nr)];
    unsigned cc[kCache];
#pragma unroll
    for (int t = 0; t < kCache; ++t) {
        const int j = rb + mq + kTpr * t;
        cc[t] = j < re ? (unsigned)col_indices[j] : ~0u;
    }
    for (int i = tid; i < nw; i += kT) s_bits[i] = 0u;
    for (int i = tid; i < kRows * kEmapStride / 2; i += kT)
        reinterpret_cast<unsigned *>(s.emap)[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kCache; ++t) mark_column(cc[t], (unsigned)k, s_bits);
    for (int j = rb + mq + kTpr * kCache; j < re; j += kTpr) {
        const unsigned c = (unsigned)col_indices[j];
        if (c < (unsigned)k) atomicOr(&s_bits[c >> 5], 1u << (c & 31));
    }
    __syncthreads();
    // rank of each word's first bit: this thread's words, then the block's
    const int wpt = (nw + kT - 1) / kT;
    const int w0 = tid * wpt;
    int cnt = 0;
    for (int j = 0; j < wpt; ++j) cnt += w0 + j < nw ? __popc(s_bits[w0 + j]) : 0;
    const int incl = wave_inclusive_sum(cnt);
    if (lane == kWave - 1) s.wsum[wave] = incl;
    __syncthreads();
    int run = incl - cnt, nu = 0;
#pragma unroll
    for (int v = 0; v < kW; ++v) {
        run += v < wave ? s.wsum[v] : 0;
        nu += s.wsum[v];
    }
    const int ntiles = (nu + 15) / 16;
    if (nu > kMaxCols || pp.pn >= 65535 || 256 * ntiles > kReuse * pp.pn) return -1;
    // the union's columns in rank order
    for (int j = 0; j < wpt; ++j) {
        const int wi = w0 + j;
        if (wi < nw) {
            unsigned bits = s_bits[wi];
            s_rank[wi] = run;
            while (bits) {
                s.ucol[run++] = wi * 32 + __builtin_ctz(bits);
                bits &= bits - 1u;
            }
        }
    }
    __syncthreads();
    auto slot_of = [&](unsigned c) {
        return s_rank[c >> 5] + __popc(s_bits[c >> 5] & ((1u << (c & 31)) - 1u));
    };
#pragma unroll
    for (int t = 0; t < kCache; ++t)
        if (cc[t] < (unsigned)k)
            s.emap[mr * kEmapStride + slot_of(cc[t])] =
                (unsigned short)(rb + mq + kTpr * t - pp.e0 + 1);
    for (int j = rb + mq + kTpr * kCache; j < re; j += kTpr) {
        const unsigned c = (unsigned)col_indices[j];
        if (c < (unsigned)k)
            s.emap[mr * kEmapStride + slot_of(c)] = (unsigned short)(j - pp.e0 + 1);
    }
    __syncthreads();
    return nu;
}

}  // namespace panel_union
}  // namespace spk
