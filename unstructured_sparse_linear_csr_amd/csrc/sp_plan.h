// Variant selection, separated from the launch, for the operations whose
// bodies can share a launch (SpMM on wide B, SDDMM with Y stored k x d).
#pragma once

#include "sp_launch.h"
#include "sddmm_rows.h"
#include "spmm_panel.h"
#include "spmm_wide.h"

namespace spk {

struct SpmmPlan {
    enum Kind { kWide, kNarrow, kLds, kBalanced, kSplit, kPanel, kUnion } kind;
    spmm_detail::SpmmParams p;
    spmm_detail::PanelParams q;  // panel kernel
    int panel = 0;               // panel kernel: 0 many tiles (64-row panels), 1 few (32)
    Dtype dtype;
    bool vec, vec_csr, buf;
    int lpr;     // wide: lanes per row
    int e;       // narrow and LDS kernels: lanes per entry slot
    int blocks;  // LDS kernel: workgroups
    int lds_kvec = 0;  // LDS kernel: B elements per LDS vector (8: 16-bit B kept 16-bit)
};

// Y stored d x k without a workspace (sddmm.hip): panels of `rows` row slots,
// each over `splits` contiguous ranges of Y's columns, staging up to `kc`
// touched columns at a time; byte offsets of the dynamic LDS regions.
struct DkPanelParams {
    int rows, kc, splits, panels;
    int rounds;  // panel kernel: 64-entry windows per row per chunk
    int nv;      // tile kernel: vectors per lane of a 16-lane group
    int x_shift;  // log2 of X's vectors per row rounded up to a power of 2
    unsigned x_pitch, y_pitch;  // LDS bytes per staged X row / Y column
    unsigned off_y, off_tab, off_bits, off_rank, off_col, off_misc;
    unsigned lds;
};

struct SddmmPlan {
    enum Kind { kNothing, kFill, kCols, kRows, kDkPanel, kDkTile } kind;
    sddmm_detail::SddmmParams p;
    Dtype dtype;
    bool vec, buf;
    bool softmax;  // rows kernel: row softmax of the scores before they are written
    bool split;    // rows kernel: a workgroup of waves per row, sharing its windows
    bool multirow; // rows kernel: several rows per wave (small depth, many short rows)
    bool panel_union;  // multi-row problems, batched: shared-column panels as MFMA tiles
    int g, nv;     // rows kernel: lanes per entry, vectors per lane (0: generic loop)
    // Y stored d x k with a workspace: transpose it into p.y first
    const void *t_src;        // NULL: no transpose
    long long t_src_stride;   // elements between batch entries of the d x k source
    int t_batch;              // source operands to transpose (1 when shared)
    DkPanelParams dk;         // kDkPanel, kDkTile (splits = column tiles per panel)
};

// hipErrorInvalidConfiguration when the grid would exceed the launch limits.
hipError_t plan_spmm(const SpmmArgs &a, SpmmPlan *plan);
hipError_t run_spmm(const SpmmPlan &plan, hipStream_t stream);
hipError_t plan_sddmm(const SddmmArgs &a, SddmmPlan *plan);
hipError_t run_sddmm(const SddmmPlan &plan, hipStream_t stream);

}  // namespace spk
