"""GPU parity of the SDDMM kernel that walks several short rows per wave.

It takes fp32 problems whose depth d is a multiple of 4 from 20 to 64 (8 or 16
lanes per entry, one 16-byte vector of the X row per lane) when row slots are
not split over waves (SDDMM, "Sparse GPU Kernels for Deep Learning", Section
5).  Batched problems on at most 65,536 columns take the panel-union kernel
(its own tests), so the batched cases here use K = 65,600 columns.  Each output is summed exactly as the one-row
kernels sum it, so the default entry points' results must equal, bit for bit,
those of sp_sddmm_balanced (one batch entry, a row's windows split over a
workgroup of waves, which never takes this kernel), and both must meet the
stated tolerance against the oracle: |gpu - oracle| <= 1e-5 * sum |x y| per
entry, plus |beta prior| where a prior is accumulated.
"""
import numpy as np
import pytest
import torch

import oracle
from unstructured_sparse_linear_csr_amd import binding as sp
from unstructured_sparse_linear_csr_amd import inputs

from gpu_util import DevCsr, check_close, csr_of_row_lists, dev, host, note

pytestmark = pytest.mark.gpu

# beyond the panel-union kernel's 65,536 columns
WIDE_K = 65600
# row lengths around the chunk (8 or 16 entries) and batch (4 entries) sizes
MIXED = [0, 1, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 0, 2]


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sp.lib()
    yield
    torch.cuda.synchronize()


def swizzle(a: DevCsr):
    ri = torch.empty(a.m, dtype=torch.int32, device="cuda")
    sp.sp_row_swizzle(a.m, a.d_ro, ri)
    return ri


def mixed_csr(seed, m, k, lengths=MIXED):
    lens = np.resize(np.asarray(lengths, np.int32), m)
    return csr_of_row_lists(inputs.random_row_lists(seed, m, k, lens))


def balanced(a: DevCsr, x, y, ri=None):
    """Scores of one batch entry through the split kernel (never multi-row)."""
    out = torch.full((a.nnz,), float("nan"), dtype=torch.float32, device="cuda")
    sp.sp_sddmm_balanced(a.m, a.k, x.shape[1], a.nnz, ri, a.d_ro, a.d_ci, dev(x), dev(y), out)
    return host(out)


def batched(a: DevCsr, xs, ys, alpha, ri=None, shared_x=False, shared_y=False):
    """sp_sddmm_batched over len(xs) entries; returns (outputs, kernel name)."""
    d = xs[0].shape[1]
    nb = len(xs)
    x = dev(xs[0] if shared_x else np.stack(xs))
    y = dev(ys[0] if shared_y else np.stack(ys))
    sx = 0 if shared_x else a.m * d
    sy = 0 if shared_y else a.k * d
    out = torch.full((nb, a.nnz), float("nan"), dtype=torch.float32, device="cuda")
    name = sp.sp_sddmm_kernel_name(a.m, a.k, d, a.nnz, x, y, nb, sx, sy, a.nnz)
    sp.sp_sddmm_batched(a.m, a.k, d, a.nnz, ri, a.d_ro, a.d_ci, x, y, alpha, out, nb, sx, sy,
                        a.nnz)
    return host(out), name


def check_entry(a: DevCsr, got, x, y, alpha, ri, what):
    """Bit-equal to the split kernel (scaled by a power of two) and within the
    tolerance of the oracle."""
    ref = balanced(a, x, y, ri) * np.float32(alpha)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (
        f"{what}: {int((got != ref).sum())} of {got.size} outputs differ from the one-row sums")
    s, s_abs = oracle.sddmm(a.m, a.k, x.shape[1], a.ro, a.ci, x, y)
    check_close(got, alpha * s, abs(alpha) * s_abs, what)


@pytest.mark.parametrize("d", [20, 24, 28, 32, 36, 44, 48, 60, 64])
def test_depths_and_lengths(d):
    """Every depth the kernel takes (8 lanes per entry up to d = 32, 16 above),
    lanes past d idle, rows of 0 to 100 entries, m not a multiple of the rows
    per wave, three batch entries with their own X and Y."""
    a = mixed_csr(d, 301, WIDE_K)
    xs = [inputs.random_dense(100 * d + z, a.m, d) for z in range(3)]
    ys = [inputs.random_dense(200 * d + z, a.k, d) for z in range(3)]
    note(f"multirow sddmm d={d} m={a.m} nnz={a.nnz}")
    got, name = batched(a, xs, ys, 1.0)
    assert name == "multirow"
    for z in range(3):
        check_entry(a, got[z], xs[z], ys[z], 1.0, None, f"d={d} entry {z}")


@pytest.mark.parametrize("shared", ["x", "y"])
def test_shared_operand(shared):
    """One X (or one Y) shared by every batch entry (stride 0)."""
    d = 64
    a = mixed_csr(7, 123, WIDE_K)
    xs = [inputs.random_dense(10 + z, a.m, d) for z in range(3)]
    ys = [inputs.random_dense(20 + z, a.k, d) for z in range(3)]
    if shared == "x":
        xs = [xs[0]] * 3
    else:
        ys = [ys[0]] * 3
    note(f"multirow sddmm shared {shared}")
    got, name = batched(a, xs, ys, 2.0, shared_x=shared == "x", shared_y=shared == "y")
    assert name == "multirow"
    for z in range(3):
        check_entry(a, got[z], xs[z], ys[z], 2.0, None, f"shared {shared} entry {z}")


@pytest.mark.parametrize("m,lengths", [
    (1, [5]),                        # one row, one partial wave
    (9, [3] * 9),                    # 8 rows per wave at d = 32: a second wave of one row
    (17, [0] * 16 + [37]),           # every row empty but the last
    (40, [0, 2000] + [3] * 38),      # one long row among short ones in the same wave
    (66, [1] * 66),                  # nnz not a multiple of 4
])
@pytest.mark.parametrize("d", [32, 64])
def test_ragged(m, lengths, d):
    a = mixed_csr(m + d, m, WIDE_K, lengths)
    x = inputs.random_dense(1 + m, m, d)
    y = inputs.random_dense(2 + m, a.k, d)
    note(f"multirow sddmm ragged m={m} d={d} nnz={a.nnz}")
    got, name = batched(a, [x, x], [y, y], 1.0, shared_x=True, shared_y=True)
    assert name == "multirow"
    for z in range(2):
        check_entry(a, got[z], x, y, 1.0, None, f"ragged m={m} d={d} entry {z}")


@pytest.mark.parametrize("beta", [0.0, 0.75])
def test_general_epilogue(beta):
    """sp_sddmm_general through this kernel: element-wise mask values, alpha,
    and beta times a prior (a NaN prior with beta = 0, never read)."""
    d = 48
    # rows of 9 entries on average: one batch entry below the split's threshold
    a = mixed_csr(31, 257, 640, [0, 1, 3, 5, 8, 9, 15, 17, 30, 2])
    x = inputs.random_dense(41, a.m, d)
    y = inputs.random_dense(42, a.k, d)
    mv = inputs.random_dense(43, a.nnz)
    prior = inputs.random_dense(44, a.nnz) if beta else np.full(a.nnz, np.nan, np.float32)
    dx, dy, dmv = dev(x), dev(y), dev(mv)
    out = dev(prior)
    name = sp.sp_sddmm_kernel_name(a.m, a.k, d, a.nnz, dx, dy, mask_values=dmv, beta=beta)
    assert name == "multirow"
    note(f"multirow sddmm general beta={beta}")
    sp.sp_sddmm_general(a.m, a.k, d, a.nnz, swizzle(a), a.d_ro, a.d_ci, dmv, dx, dy, sp.SP_Y_KD,
                        0.5, beta, out)
    ref, scale = oracle.sddmm_general(a.m, a.k, d, a.ro, a.ci, x, y, sp.SP_Y_KD, mv, 0.5,
                                      beta, prior if beta else None)
    check_close(host(out), ref, scale, f"general beta={beta}")


def test_not_taken_outside_its_shapes():
    """d = 16 (4 lanes per entry), d = 68 (two vectors per lane), one batch
    entry of long rows (split over waves) and bf16 operands of d = 32 (4 lanes
    per entry) keep the other kernels."""
    a = mixed_csr(5, 64, 300, [40])
    for d, nb in ((16, 2), (68, 2), (64, 1)):
        x = torch.zeros(nb, a.m, d, device="cuda")
        y = torch.zeros(nb, a.k, d, device="cuda")
        name = sp.sp_sddmm_kernel_name(a.m, a.k, d, a.nnz, x, y, nb, a.m * d, a.k * d, a.nnz)
        assert name == ("split" if nb == 1 else "rows"), (d, nb, name)
    # one batch entry of short rows: this kernel
    s = mixed_csr(6, 64, 300, [3])
    x = torch.zeros(s.m, 64, device="cuda")
    y = torch.zeros(s.k, 64, device="cuda")
    assert sp.sp_sddmm_kernel_name(s.m, s.k, 64, s.nnz, x, y) == "multirow"
    xb = torch.zeros(2, a.m, 32, device="cuda", dtype=torch.bfloat16)
    yb = torch.zeros(2, a.k, 32, device="cuda", dtype=torch.bfloat16)
    assert sp.sp_sddmm_kernel_name(a.m, a.k, 32, a.nnz, xb, yb, 2, a.m * 32, a.k * 32,
                                   a.nnz) == "rows"


def to16(x32, kind):
    """(device tensor of the 16-bit rounding of x32, its exact fp32 values)."""
    tdt, code = {"f16": (torch.float16, oracle.F16), "bf16": (torch.bfloat16, oracle.BF16)}[kind]
    t = torch.from_numpy(np.ascontiguousarray(x32)).to(tdt)
    vals = oracle.decode16(code, t.view(torch.int16).numpy().view(np.uint16))
    return t.cuda(), vals.astype(np.float32).reshape(x32.shape)


@pytest.mark.parametrize("kind,d", [("f16", 64), ("bf16", 64), ("bf16", 40), ("f16", 128)])
def test_16bit(kind, d):
    """16-bit X and Y (8 elements per 16-byte vector: 8 lanes per entry up to
    d = 64, 16 up to 128), three batch entries: bit-equal to the one-row
    kernel's sums (one batch entry of rows averaging 16+ entries takes the
    split kernel) and within the bound of the oracle on the decoded values."""
    a = mixed_csr(d + 7, 301, WIDE_K)
    x16, x = to16(np.stack([inputs.random_dense(300 * d + z, a.m, d) for z in range(3)]), kind)
    y16, y = to16(np.stack([inputs.random_dense(400 * d + z, a.k, d) for z in range(3)]), kind)
    out = torch.full((3, a.nnz), float("nan"), device="cuda")
    name = sp.sp_sddmm_kernel_name(a.m, a.k, d, a.nnz, x16, y16, 3, a.m * d, a.k * d, a.nnz)
    assert name == "multirow"
    note(f"multirow sddmm {kind} d={d}")
    sp.sp_sddmm_ex(a.m, a.k, d, a.nnz, None, a.d_ro, a.d_ci, x16, y16, 0.5, out, 3, a.m * d,
                   a.k * d, a.nnz)
    got = host(out)
    for z in range(3):
        one = torch.full((a.nnz,), float("nan"), device="cuda")
        assert sp.sp_sddmm_kernel_name(a.m, a.k, d, a.nnz, x16[z], y16[z]) == "split"
        sp.sp_sddmm_ex(a.m, a.k, d, a.nnz, None, a.d_ro, a.d_ci, x16[z], y16[z], 0.5, one)
        ref = host(one)
        assert np.array_equal(got[z].view(np.uint32), ref.view(np.uint32)), f"{kind} entry {z}"
        s, s_abs = oracle.sddmm(a.m, a.k, d, a.ro, a.ci, x[z], y[z])
        check_close(got[z], 0.5 * s, 0.5 * s_abs, f"{kind} d={d} entry {z}")
