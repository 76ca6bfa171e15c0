"""GPU parity of the SpMM that stages B in LDS per row panel (spmm_panel.h).

The panel kernel is chosen for fp32 problems of one batch entry with 16-byte
aligned operands, n of at least one 128-column tile, enough (panel, tile)
workgroups to give each of the GPU's 256 CUs one, and rows per panel times
density at least 4.  It has two shapes: 64-row panels with B in chunks of 128
rows in two LDS buffers (many column tiles), and 32-row panels with chunks of
224 rows in one buffer and 128-entry windows (one or two tiles).  It sums every row in CSR order with one FMA per entry, as the wide
kernel does, so its outputs must be bit-identical to the wide kernel's; a
2-entry batch (which never takes the panel kernel) with both entries equal
gives the wide kernel's result for comparison.  Every output is also checked
against the oracle within |gpu - oracle| <= 1e-5 * sum|a*b|.
"""
import numpy as np
import pytest
import torch

import oracle
from unstructured_sparse_linear_csr_amd import binding as sp
from unstructured_sparse_linear_csr_amd import inputs

from gpu_util import DevCsr, check_close, dev, host, note

pytestmark = pytest.mark.gpu

MANY_KC, FEW_KC = 128, 224    # B rows per chunk of the two shapes
UNION_MAX_K = 65536           # rows of B up to which batches may take the panel-union kernel


def swizzle(a):
    ri = torch.empty(a.m, dtype=torch.int32, device="cuda")
    sp.sp_row_swizzle(a.m, a.d_ro, ri)
    return ri


def panel_and_wide(a, b_np, ri=None):
    """(sp_spmm's result, the 2-entry batch's result, the kernel that batch
    took) for A B; sp_spmm must take the panel kernel.  The batch takes the
    wide kernel, or for few rows of 256+ entries the split kernel (which sums
    a row in four parts, so it is not bit-comparable)."""
    n = b_np.shape[1]
    b = dev(b_np)
    c = torch.full((a.m, n), float("nan"), device="cuda")
    assert sp.sp_spmm_kernel_name(a.m, a.k, n, a.nnz, a.d_vals, a.d_ci, b, c) == "panel"
    # Batches of 64, 128 or 256 columns on at most 65,536 rows of B take the
    # panel-union kernel; the reference batch gets B with zero rows appended
    # past 65,536 (the structure is unchanged), which keeps it on the wide kernel.
    kk, b_ref = a.k, b
    if n in (64, 128, 256):
        kk = UNION_MAX_K + 64
        b_ref = dev(np.concatenate([b_np, np.zeros((kk - a.k, n), np.float32)]))
    c2 = torch.full((2, a.m, n), float("nan"), device="cuda")
    other = sp.sp_spmm_kernel_name(a.m, kk, n, a.nnz, a.d_vals, a.d_ci, b_ref, c2, 2, 0, 0,
                                   a.m * n)
    assert other in ("wide", "split")
    sp.sp_spmm(a.m, a.k, n, a.nnz, ri, a.d_vals, a.d_ro, a.d_ci, b, c)
    sp.sp_spmm_batched(a.m, kk, n, a.nnz, ri, a.d_vals, a.d_ro, a.d_ci, b_ref, c2, 2, 0, 0,
                       a.m * n)
    c2 = host(c2)
    assert np.array_equal(c2[0].view(np.int32), c2[1].view(np.int32))
    return host(c), c2[0], other


def check(a, b_np, what, ri=None):
    c, ref2, other = panel_and_wide(a, b_np, ri)
    if other == "wide":
        assert np.array_equal(c.view(np.int32), ref2.view(np.int32)), f"{what}: not bit-equal to wide"
    ref, s = oracle.spmm(a.m, a.k, b_np.shape[1], a.ro, a.ci, a.vals, b_np)
    return check_close(c, ref, s, what)


def of_row_lists(rl):
    return DevCsr(rl.m, rl.k, oracle.csr_offsets_from_lengths(rl.lengths), rl.cols, rl.values)


def csr(seed, m, k, lengths):
    return of_row_lists(inputs.random_row_lists(seed, m, k, np.asarray(lengths, np.int32)))


def lengths_for(seed, m, k, density_lo, density_hi):
    lo = max(1, int(k * density_lo))
    hi = max(lo + 1, int(k * density_hi) + 1)
    return np.random.default_rng(seed).integers(lo, min(hi, k + 1), m)


# ---------------------------------------------------------------- workloads

def test_resnet_1x1_whole():
    w = inputs.resnet_1x1()
    a = of_row_lists(w["a"])
    note("spmm panel resnet 1024x256x6272")
    check(a, w["b"], "panel resnet", ri=swizzle(a))


@pytest.mark.parametrize("sparsity", [0.5, 0.7, 0.8])
def test_lstm_whole(sparsity):
    w = inputs.lstm(sparsity)
    a = of_row_lists(w["a"])
    note(f"spmm panel lstm s={sparsity}")
    check(a, w["b"], f"panel lstm {sparsity}", ri=swizzle(a))


# ---------------------------------------------------------------- edges, 64-row panels
# n = 1024 (8 tiles) and m >= 2048 rows give 256 workgroups

@pytest.mark.parametrize("k", [1, 5, MANY_KC - 1, MANY_KC, MANY_KC + 1, 2 * MANY_KC + 3, 7 * MANY_KC])
def test_many_chunk_counts(k):
    m, n = 2048, 1024
    lengths = lengths_for(k, m, k, 0.125, 0.25)
    lengths[::17] = 0
    a = csr(100 + k, m, k, lengths)
    b = inputs.random_dense(101 + k, k, n)
    note(f"spmm panel (64-row) chunks k={k} nnz={a.nnz}")
    check(a, b, f"panel many k={k}")


@pytest.mark.parametrize("n", [1028, 1088, 1152, 1212, 1280, 1400])
def test_many_tile_widths(n):
    # ragged last tiles (n % 128 != 0, n % 4 == 0; a lane's two column vectors
    # lie 64 columns apart, so a ragged tile can end in either)
    m, k = 2048, 300
    a = csr(200 + n, m, k, lengths_for(n, m, k, 0.1, 0.3))
    b = inputs.random_dense(201 + n, k, n)
    note(f"spmm panel (64-row) width n={n}")
    check(a, b, f"panel many n={n}", ri=swizzle(a))


@pytest.mark.parametrize("extra", [1, 31, 63])
def test_many_partial_panels(extra):
    m, k, n = 2048 + extra, 300, 1024
    lengths = lengths_for(extra, m, k, 0.1, 0.3)
    lengths[0] = 3
    a = csr(300 + extra, m, k, lengths)
    b = inputs.random_dense(301 + extra, k, n)
    note(f"spmm panel (64-row) m={m}")
    check(a, b, f"panel many m={m}", ri=swizzle(a))


def _long_range_rows(seed, m, kc, win):
    # rows with more than a window of entries inside one chunk, rows whose
    # entries all fall in one chunk, and short rows
    k = 3 * kc
    rng = np.random.default_rng(seed)
    rows = []
    for i in range(m):
        if i % 3 == 0:
            cols = np.sort(rng.choice(kc, win + win // 2, replace=False)) + kc   # chunk 1 only
        elif i % 3 == 1:
            cols = np.sort(rng.choice(k, 3 * (win + 3), replace=False))           # > win per chunk
        else:
            cols = np.sort(rng.choice(k, 9, replace=False))
        rows.append(cols)
    lengths = np.array([r.size for r in rows], np.int32)
    ci = np.concatenate(rows).astype(np.int32)
    return DevCsr(m, k, oracle.csr_offsets_from_lengths(lengths), ci,
                  inputs.random_dense(seed + 1, ci.size)), k


def test_many_rows_beyond_one_window_per_chunk():
    a, k = _long_range_rows(7, 2048, MANY_KC, 64)
    b = inputs.random_dense(9, k, 1024)
    note(f"spmm panel (64-row) long chunk ranges nnz={a.nnz}")
    check(a, b, "panel many long ranges", ri=swizzle(a))


def test_nan_outside_touched_rows_of_b():
    # padding slots read a zero row with value 0, so B values that no entry
    # touches (NaN in every odd row of B here) never enter a sum
    m, k, n = 2048, 600, 1024
    rl = inputs.random_row_lists(14, m, k // 2, lengths_for(13, m, k // 2, 0.1, 0.3))
    rl.cols = (2 * rl.cols).astype(np.int32)
    rl.k = k
    b = inputs.random_dense(15, k, n)
    b[1::2] = np.nan
    a = of_row_lists(rl)
    note("spmm panel NaN in untouched B rows")
    check(a, b, "panel untouched NaN rows", ri=swizzle(a))


# ---------------------------------------------------------------- edges, 32-row panels
# n of one or two tiles and m >= 8192 (4096 for two tiles) rows

@pytest.mark.parametrize("k", [100, FEW_KC, FEW_KC + 1, 2 * FEW_KC + 1, 700])
def test_few_chunk_counts(k):
    m, n = 8192, 128
    lengths = lengths_for(k, m, k, 0.125, 0.25)
    lengths[::13] = 0
    a = csr(400 + k, m, k, lengths)
    b = inputs.random_dense(401 + k, k, n)
    note(f"spmm panel (32-row) chunks k={k} nnz={a.nnz}")
    check(a, b, f"panel few k={k}", ri=swizzle(a))


@pytest.mark.parametrize("n", [132, 192, 252])
def test_few_tile_widths(n):
    m, k = 4096, 500
    a = csr(500 + n, m, k, lengths_for(n, m, k, 0.15, 0.3))
    b = inputs.random_dense(501 + n, k, n)
    note(f"spmm panel (32-row) width n={n}")
    check(a, b, f"panel few n={n}", ri=swizzle(a))


@pytest.mark.parametrize("extra", [1, 17])
def test_few_partial_panels(extra):
    m, k, n = 8192 + extra, 400, 128
    lengths = lengths_for(extra + 7, m, k, 0.15, 0.3)
    lengths[-1] = 2
    a = csr(600 + extra, m, k, lengths)
    b = inputs.random_dense(601 + extra, k, n)
    note(f"spmm panel (32-row) m={m}")
    check(a, b, f"panel few m={m}")


def test_few_rows_beyond_one_window_per_chunk():
    a, k = _long_range_rows(17, 8192, FEW_KC, 128)
    b = inputs.random_dense(19, k, 128)
    note(f"spmm panel (32-row) long chunk ranges nnz={a.nnz}")
    check(a, b, "panel few long ranges", ri=swizzle(a))


def test_one_entry_rows_exact():
    # one entry per row: one rounding of an exact product, so bit-exact (k = 8
    # columns keeps the density high enough for the panel kernel)
    m, n, k8 = 8192, 128, 8
    ci = (np.arange(m) * 5 % k8).astype(np.int32)
    vals = inputs.random_dense(11, m)
    a = DevCsr(m, k8, np.arange(m + 1), ci, vals)
    b = inputs.random_dense(12, k8, n)
    note("spmm panel one-entry rows k=8")
    c, wide0, other = panel_and_wide(a, b)
    want = (vals.astype(np.float64)[:, None] * b.astype(np.float64)[ci]).astype(np.float32)
    assert np.array_equal(c, want)
    assert other == "wide" and np.array_equal(c.view(np.int32), wide0.view(np.int32))


def test_empty_rows():
    m, k, n = 8192, 64, 128
    lengths = np.zeros(m, np.int32)
    lengths[::3] = 64           # full rows between empty ones
    a = csr(16, m, k, lengths)
    b = inputs.random_dense(17, k, n)
    note("spmm panel full and empty rows")
    c, wide0, other = panel_and_wide(a, b)
    assert np.all(c[lengths == 0] == 0)
    assert other == "wide" and np.array_equal(c.view(np.int32), wide0.view(np.int32))


def test_small_problems_take_other_kernels():
    # too few workgroups for the panel kernel: the Transformer-FFN SpMM
    w = inputs.transformer_ffn()
    a = of_row_lists(w["a"])
    b = dev(w["b"])
    c = torch.empty(a.m, w["n"], device="cuda")
    assert sp.sp_spmm_kernel_name(a.m, a.k, w["n"], a.nnz, a.d_vals, a.d_ci, b, c) == "wide"
