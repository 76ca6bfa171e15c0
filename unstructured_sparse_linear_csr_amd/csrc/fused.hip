// An SpMM and an SDDMM in one launch.  On problems of the sizes the card
// targets ("Sparse GPU Kernels for Deep Learning", summary card, "Summary":
// SpMM and SDDMM for DL workloads), each kernel alone leaves the chip
// two-thirds idle -- a few thousand one-wave workgroups, each a short chain
// of dependent loads -- and pays its own launch.  Here the grid is the two
// grids end to end: workgroups [0, gridDim.x - spmm_blocks) run the SDDMM row
// body on SDDMM work unit b, the remaining spmm_blocks run the wide SpMM body
// on SpMM work unit b - (gridDim.x - spmm_blocks), so both sets of waves are
// resident together and their latencies overlap.  Each body is the same code
// the separate launches run, so results are bit-identical to them.
//
// Fused variants exist for the fp32 vector paths (16-byte aligned operands,
// B and Y under 2 GiB); any other pair is launched as two kernels.
#include "sp_device.h"
#include "sp_launch.h"
#include "sp_plan.h"

namespace spk {

namespace {

using spmm_detail::SpmmParams;
using sddmm_detail::SddmmParams;

template <int kLpr, int kG, int kNv>
__global__ __launch_bounds__(kWave) void spmm_sddmm_kernel(SpmmParams a, SddmmParams b,
                                                           long long spmm_blocks)
{
    // The SDDMM's workgroups first, then the SpMM's: measured 1-2 % faster on the
    // Transformer-FFN pair than the other order (interleaving the two, which
    // puts each problem on half the XCDs, was slower still)
    const long long blk = blockIdx.x;
    const long long sddmm_blocks = (long long)gridDim.x - spmm_blocks;
    if (blk < sddmm_blocks)
        sddmm_detail::sddmm_rows_body<float, kG, kNv, 4>(b, sddmm_detail::rows_work(b, blk));
    else
        spmm_detail::spmm_wide_body<float, kLpr, 4, true, true>(
            a, spmm_detail::wide_work(a, blk - sddmm_blocks));
}

template <int kLpr, int kG, int kNv>
hipError_t launch_fused_t(const SpmmParams &a, const SddmmParams &b, hipStream_t s)
{
    const long long na = spmm_detail::wide_grid(a);
    const long long nb = sddmm_detail::rows_grid(b);
    hipLaunchKernelGGL((spmm_sddmm_kernel<kLpr, kG, kNv>), dim3((unsigned)(na + nb)),
                       dim3(kWave), 0, s, a, b, na);
    return hipGetLastError();
}

template <int kLpr, int kG>
hipError_t launch_fused_nv(int nv, const SpmmParams &a, const SddmmParams &b, hipStream_t s)
{
    switch (nv) {
    case 1: return launch_fused_t<kLpr, kG, 1>(a, b, s);
    case 2: return launch_fused_t<kLpr, kG, 2>(a, b, s);
    default: return launch_fused_t<kLpr, kG, 4>(a, b, s);
    }
}

template <int kLpr>
hipError_t launch_fused_g(int g, int nv, const SpmmParams &a, const SddmmParams &b,
                          hipStream_t s)
{
    switch (g) {
    case 4: return launch_fused_nv<kLpr, 4>(nv, a, b, s);
    case 8: return launch_fused_nv<kLpr, 8>(nv, a, b, s);
    default: return launch_fused_nv<kLpr, 16>(nv, a, b, s);
    }
}

bool fusable(const SpmmPlan &x, const SddmmPlan &y)
{
    return x.kind == SpmmPlan::kWide && x.dtype == Dtype::f32 && x.vec && x.vec_csr && x.buf &&
           y.kind == SddmmPlan::kRows && y.dtype == Dtype::f32 && y.vec && y.buf && !y.softmax &&
           (y.nv == 1 || y.nv == 2 || y.nv == 4) &&
           spmm_detail::wide_grid(x.p) + sddmm_detail::rows_grid(y.p) <= 0x7fffffffLL;
}

}  // namespace

hipError_t launch_spmm_sddmm(const SpmmArgs &x, const SddmmArgs &y, hipStream_t stream)
{
    SpmmPlan px;
    SddmmPlan py;
    // The pair's SpMM sums every row in entry order (the wide kernel's body).
    SpmmArgs xs = x;
    xs.auto_balance = false;
    hipError_t e = plan_spmm(xs, &px);
    if (e != hipSuccess) return e;
    e = plan_sddmm(y, &py);
    if (e != hipSuccess) return e;
    if (!fusable(px, py)) {
        e = run_spmm(px, stream);
        return e != hipSuccess ? e : run_sddmm(py, stream);
    }
    switch (px.lpr) {
    case 8: return launch_fused_g<8>(py.g, py.nv, px.p, py.p, stream);
    case 16: return launch_fused_g<16>(py.g, py.nv, px.p, py.p, stream);
    case 32: return launch_fused_g<32>(py.g, py.nv, px.p, py.p, stream);
    default: return launch_fused_g<64>(py.g, py.nv, px.p, py.p, stream);
    }
}

}  // namespace spk
