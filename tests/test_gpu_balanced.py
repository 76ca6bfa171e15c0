"""GPU parity of sp_spmm_balanced (workgroups of 4 waves sharing 4 rows'
entries evenly) against the oracle, within the fp32 tolerance; deterministic
for a given row order; narrow B falls back to sp_spmm's kernels (bit-equal)."""
import numpy as np
import pytest
import torch

import oracle
from unstructured_sparse_linear_csr_amd import binding as sp
from unstructured_sparse_linear_csr_amd import inputs

from gpu_util import DevCsr, check_close, csr_of_row_lists, dev, host, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sp.lib()
    yield
    torch.cuda.synchronize()


def swizzle(a):
    ri = torch.empty(a.m, dtype=torch.int32, device="cuda")
    sp.sp_row_swizzle(a.m, a.d_ro, ri)
    return ri


def run_balanced(a, b_np, ri=None, b_dev=None):
    n = b_np.shape[1] if b_np is not None else b_dev.shape[1]
    c = torch.full((a.m, n), float("nan"), device="cuda")
    sp.sp_spmm_balanced(a.m, a.k, n, a.nnz, ri, a.d_vals, a.d_ro, a.d_ci,
                        dev(b_np) if b_dev is None else b_dev, c)
    return host(c)


@pytest.mark.parametrize("swz", [True, False])
def test_imbalance_workload(swz):
    w = inputs.imbalance()
    a = csr_of_row_lists(w["a"])
    ri = swizzle(a) if swz else None
    note(f"spmm_balanced lognormal rows swizzle={swz}")
    c1 = run_balanced(a, w["b"], ri)
    c2 = run_balanced(a, w["b"], ri)
    assert np.array_equal(c1.view(np.int32), c2.view(np.int32))
    ref, s = oracle.spmm(a.m, a.k, w["n"], a.ro, a.ci, a.vals, w["b"])
    check_close(c1, ref, s, f"balanced imbalance swizzle={swz}")


def test_transformer_ffn():
    w = inputs.transformer_ffn()
    a = csr_of_row_lists(w["a"])
    note("spmm_balanced ffn")
    c = run_balanced(a, w["b"], swizzle(a))
    ref, s = oracle.spmm(a.m, a.k, w["n"], a.ro, a.ci, a.vals, w["b"])
    check_close(c, ref, s, "balanced ffn")


@pytest.mark.parametrize("m,n", [(1, 256), (3, 132), (1023, 256), (1026, 258), (517, 600),
                                 (130, 1024)])
def test_shapes_and_long_rows(m, n):
    """m around multiples of 4 (empty serpentine slots), widths with partial
    lane tiles and several column tiles, the scalar path (n % 4 != 0), one row
    of 5,000 entries among short and empty rows."""
    k = 9000
    rng = np.random.default_rng(900 + m + n)
    lengths = rng.integers(0, 40, m).astype(np.int32)
    lengths[::7] = 0
    lengths[m // 2] = 5000
    rl = inputs.random_row_lists(901 + m, m, k, lengths)
    a = csr_of_row_lists(rl)
    b = inputs.random_dense(902 + n, k, n)
    note(f"spmm_balanced m={m} n={n}")
    c = run_balanced(a, b, swizzle(a))
    ref, s = oracle.spmm(m, k, n, a.ro, a.ci, a.vals, b)
    check_close(c, ref, s, f"balanced m={m} n={n}")
    assert np.all(c[lengths == 0] == 0.0)


def test_unaligned_operands():
    w = inputs.transformer_ffn()
    a = csr_of_row_lists(w["a"])
    m, k, n = a.m, a.k, w["n"]
    bb = torch.zeros(k * n + 1, device="cuda")
    bb[1:] = dev(w["b"].reshape(-1))
    vv = torch.zeros(a.nnz + 1, device="cuda")
    vv[1:] = a.d_vals
    cc = torch.full((m * n + 1,), float("nan"), device="cuda")
    note("spmm_balanced unaligned B, values, C")
    sp.sp_spmm_balanced(m, k, n, a.nnz, swizzle(a), vv[1:], a.d_ro, a.d_ci, bb[1:], cc[1:])
    ref, s = oracle.spmm(m, k, n, a.ro, a.ci, a.vals, w["b"])
    check_close(host(cc[1:]).reshape(m, n), ref, s, "balanced unaligned")


@pytest.mark.parametrize("n", [4, 64, 128])
def test_narrow_falls_back(n):
    w = inputs.imbalance()
    a = csr_of_row_lists(w["a"])
    b = dev(inputs.random_dense(910 + n, a.k, n))
    ri = swizzle(a)
    c1 = torch.empty(a.m, n, device="cuda")
    c2 = torch.empty(a.m, n, device="cuda")
    note(f"spmm_balanced narrow n={n}")
    sp.sp_spmm_balanced(a.m, a.k, n, a.nnz, ri, a.d_vals, a.d_ro, a.d_ci, b, c1)
    sp.sp_spmm(a.m, a.k, n, a.nnz, ri, a.d_vals, a.d_ro, a.d_ci, b, c2)
    assert torch.equal(c1, c2)


def test_b_beyond_2gib():
    """B of (2^22 + 3) x 136 fp32 (2.3 GB): the 64-bit gather path."""
    k, n, m = (1 << 22) + 3, 136, 64
    rng = np.random.default_rng(920)
    cols = [np.unique(rng.integers(0, k, int(c))) for c in rng.integers(0, 300, m)]
    cols[5] = np.unique(np.append(cols[5], k - 1))
    lengths = np.array([len(c) for c in cols], np.int32)
    ro = oracle.csr_offsets_from_lengths(lengths)
    ci = np.concatenate(cols).astype(np.int32)
    used = np.unique(ci)
    remap = np.searchsorted(used, ci).astype(np.int32)
    vals = inputs.random_dense(921, ci.size)
    b_small = inputs.random_dense(922, used.size, n)
    a = DevCsr(m, k, ro, ci, vals)
    note("spmm_balanced B 2.3 GB")
    b_big = torch.zeros((k, n), device="cuda")
    b_big[torch.from_numpy(used).long().cuda()] = dev(b_small)
    c = run_balanced(a, None, swizzle(a), b_dev=b_big)
    del b_big
    torch.cuda.empty_cache()
    ref, s = oracle.spmm(m, used.size, n, ro, remap, vals, b_small)
    check_close(c, ref, s, "balanced 2.3 GB B")


# ------------------------------------------------------------ sp_sddmm_balanced
# Each row's windows of 64 entries are dealt to 4 waves; every entry's
# arithmetic is that of sp_sddmm, so the outputs must be bit-identical to it
# (and within the fp32 tolerance of the oracle).

def run_sddmm_pair(a, x_np, y_np, ri=None):
    d = x_np.shape[1]
    x, y = dev(x_np), dev(y_np)
    o1 = torch.full((a.nnz,), float("nan"), device="cuda")
    o2 = torch.full((a.nnz,), float("nan"), device="cuda")
    sp.sp_sddmm(a.m, a.k, d, a.nnz, ri, a.d_ro, a.d_ci, x, y, o1)
    sp.sp_sddmm_balanced(a.m, a.k, d, a.nnz, ri, a.d_ro, a.d_ci, x, y, o2)
    return host(o1), host(o2)


@pytest.mark.parametrize("swz", [True, False])
def test_sddmm_balanced_imbalance_workload(swz):
    w = inputs.imbalance()
    a = csr_of_row_lists(w["a"])
    ri = swizzle(a) if swz else None
    note(f"sddmm_balanced lognormal rows swizzle={swz}")
    plain, bal = run_sddmm_pair(a, w["x"], w["y"], ri=ri)
    assert np.array_equal(plain.view(np.int32), bal.view(np.int32))
    ref, s = oracle.sddmm(a.m, a.k, w["d"], a.ro, a.ci, w["x"], w["y"])
    check_close(bal, ref, s, f"sddmm balanced imbalance swizzle={swz}")


def test_sddmm_balanced_transformer_ffn():
    w = inputs.transformer_ffn()
    a = csr_of_row_lists(w["a"])
    note("sddmm_balanced ffn")
    plain, bal = run_sddmm_pair(a, w["x"], w["y"], ri=swizzle(a))
    assert np.array_equal(plain.view(np.int32), bal.view(np.int32))
    ref, s = oracle.sddmm(a.m, a.k, w["d"], a.ro, a.ci, w["x"], w["y"])
    check_close(bal, ref, s, "sddmm balanced ffn")


@pytest.mark.parametrize("d", [1, 3, 8, 64, 256, 600])
def test_sddmm_balanced_row_lengths(d):
    # rows around every window boundary up to 5 windows (wave 0 of a row then
    # takes windows 0 and 4), a 47-window row, and empty rows
    k = 4000
    lengths = np.array([0, 1, 63, 64, 65, 127, 128, 129, 255, 256, 257, 320, 0, 3000, 5, 0] * 3,
                       dtype=np.int32)
    m = lengths.size
    a = csr_of_row_lists(inputs.random_row_lists(930 + d, m, k, lengths))
    x = inputs.random_dense(931 + d, m, d)
    y = inputs.random_dense(932 + d, k, d)
    note(f"sddmm_balanced row lengths d={d} nnz={a.nnz}")
    plain, bal = run_sddmm_pair(a, x, y, ri=swizzle(a))
    assert np.array_equal(plain.view(np.int32), bal.view(np.int32))
    ref, s = oracle.sddmm(m, k, d, a.ro, a.ci, x, y)
    check_close(bal, ref, s, f"sddmm balanced lengths d={d}")
