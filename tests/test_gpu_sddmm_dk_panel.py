"""GPU parity of the general SDDMM with Y stored d x k and no workspace.

For fp32 operands and d up to 1024, the call stages Y through LDS,
transposed: masks of mean density 1/20 or more by tiles of up to 64
consecutive columns (one per workgroup, staged whole), where each entry gets
16 lanes whose partial sums meet in a DPP tree; sparser masks by the columns
each panel of rows touches (chunks of up to 256 distinct columns), where
each entry gets one lane, which sums its d products in l order with FMA.
Every output is checked against the oracle within
|gpu - oracle| <= 1e-5 * (|alpha v| sum|x y| + |beta prior|), and so is the
same call with a workspace (Y transposed there first).  With small-integer
operands every partial sum is exact in fp32, so the outputs must equal the
oracle's bit for bit.
Cases: the Transformer-FFN (tiles) and sparse-attention (panels) shapes,
depths on both sides of the vector width and of the panel heights at both
densities, rows with more than 64 entries in a chunk, rows of thousands of
entries (the tiles' 64-way search for a row's first entry in the tile),
rows that skip long stretches of columns, panels cut short by m, empty rows,
batches with shared and per-entry Y, NaN in columns no entry touches, and
the depth beyond which the element-gather kernel takes over.
"""
import numpy as np
import pytest
import torch

import oracle
from unstructured_sparse_linear_csr_amd import binding as sp
from unstructured_sparse_linear_csr_amd import inputs

from gpu_util import DevCsr, check_close, csr_of_row_lists, dev, host, note

pytestmark = pytest.mark.gpu

DK = sp.SP_Y_DK


def swizzle(a: DevCsr):
    ri = torch.empty(a.m, dtype=torch.int32, device="cuda")
    sp.sp_row_swizzle(a.m, a.d_ro, ri)
    return ri


def dk_both(a: DevCsr, x, y_dk, mv=None, alpha=1.0, beta=0.0, prior=None, ri=None,
            batch=1, stride_values=0, stride_x=0, stride_y=0, stride_out=0):
    """(no workspace, with workspace) results of the same d x k call."""
    k = a.k
    d = x.shape[-1]
    outs = []
    for use_ws in (False, True):
        if prior is not None:
            out = dev(prior.astype(np.float32))
        else:
            out = torch.full((batch, a.nnz) if batch > 1 else (a.nnz,), float("nan"),
                             device="cuda")
        ws = None
        if use_ws:
            ws = torch.empty(max(1, sp.sp_sddmm_general_workspace(k, d, batch, stride_y)),
                             dtype=torch.uint8, device="cuda")
        sp.sp_sddmm_general(a.m, k, d, a.nnz, ri, a.d_ro, a.d_ci,
                            None if mv is None else dev(mv), dev(x), dev(y_dk), DK, alpha,
                            beta, out, batch, stride_values, stride_x, stride_y, stride_out,
                            workspace=ws)
        outs.append(host(out))
    return outs[0], outs[1]


def check(a, x, y_dk, what, mv=None, alpha=1.0, beta=0.0, prior=None, ri=None):
    got, with_ws = dk_both(a, x, y_dk, mv, alpha, beta, prior, ri)
    ref, s = oracle.sddmm_general(a.m, a.k, x.shape[1], a.ro, a.ci, x, y_dk, DK, mv, alpha,
                                  beta, prior)
    check_close(got, ref, s, what)
    check_close(with_ws, ref, s, what + " (workspace)")
    return got


def small_ints(seed, *shape):
    return np.random.default_rng(seed).integers(-3, 4, shape).astype(np.float32)


def check_exact(a, x, y_dk, what, ri=None):
    """Integer operands: exact sums, so bit-equal to the oracle rounded to fp32."""
    got, _ = dk_both(a, x, y_dk, ri=ri)
    ref, _ = oracle.sddmm_general(a.m, a.k, x.shape[1], a.ro, a.ci, x, y_dk, DK)
    assert np.array_equal(got, ref.astype(np.float32)), what


def random_csr(seed, m, k, lo, hi):
    lengths = np.random.default_rng(seed).integers(lo, hi, m).astype(np.int32)
    rl = inputs.random_row_lists(seed + 1, m, k, lengths)
    return DevCsr(m, k, oracle.csr_offsets_from_lengths(lengths), rl.cols,
                  inputs.random_dense(seed + 2, int(lengths.sum())))


# ---------------------------------------------------------------- workloads

def test_transformer_ffn_whole():
    w = inputs.transformer_ffn()
    a = csr_of_row_lists(w["a"])
    y_dk = np.ascontiguousarray(w["y"].T)
    prior = inputs.random_dense(71, a.nnz)
    ri = swizzle(a)
    note("sddmm dk panel ffn 2048x512 d=256")
    check(a, w["x"], y_dk, "dk ffn plain")
    check(a, w["x"], y_dk, "dk ffn general", a.vals, -1.25, 2.0, prior, ri)


def test_attention_heads_whole():
    w = inputs.sparse_attention()
    ro, ci, _ = oracle.csr_from_dense(w["mask"])
    seq, hd, heads = w["seq"], w["head_dim"], 3
    a = DevCsr(seq, seq, ro, ci)
    q, kk = w["q"][:heads], w["k"][:heads]
    kt = np.ascontiguousarray(np.transpose(kk, (0, 2, 1)))
    note("sddmm dk panel attention 3 heads")
    got, with_ws = dk_both(a, q, kt, None, 0.125, 0.0, None, swizzle(a), heads, 0, seq * hd,
                           seq * hd, a.nnz)
    for z in range(heads):
        ref, s = oracle.sddmm_general(seq, seq, hd, ro, ci, q[z], kt[z], DK, None, 0.125)
        check_close(got[z], ref, s, f"dk attention head {z}")
        check_close(with_ws[z], ref, s, f"dk attention head {z} (workspace)")


def test_attention_exact_small_ints():
    w = inputs.sparse_attention()
    ro, ci, _ = oracle.csr_from_dense(w["mask"])
    seq, hd = w["seq"], w["head_dim"]
    a = DevCsr(seq, seq, ro, ci)
    note("sddmm dk panel attention integer operands")
    check_exact(a, small_ints(1, seq, hd), small_ints(2, hd, seq), "dk attention exact",
                swizzle(a))


def test_transformer_ffn_exact_small_ints():
    w = inputs.transformer_ffn()
    a = csr_of_row_lists(w["a"])
    note("sddmm dk panel ffn integer operands")
    check_exact(a, small_ints(3, a.m, w["d"]), small_ints(4, w["d"], a.k), "dk ffn exact")


# ---------------------------------------------------------------- depths

@pytest.mark.parametrize("dense", [True, False], ids=["tiles", "panels"])
@pytest.mark.parametrize("d", [1, 3, 4, 8, 12, 17, 32, 64, 68, 69, 100, 128, 256, 260, 261,
                               300, 512, 516, 517, 700, 1000])
def test_depths(d, dense):
    # d % 4 != 0: X loaded element-wise and staged rows zero-padded; panel
    # heights from 32 to 8 rows as d grows; mean density 11 % (tiles) or 1.4 %
    m, k = 300, 700
    a = random_csr(600 + d, m, k, 0, 160 if dense else 20)
    x = inputs.random_dense(610 + d, m, d)
    y_dk = inputs.random_dense(620 + d, d, k)
    mv = inputs.random_dense(630 + d, a.nnz)
    note(f"sddmm dk depth d={d} dense={dense}")
    check(a, x, y_dk, f"dk d={d} dense={dense}", mv, 0.75, ri=swizzle(a))
    check_exact(a, small_ints(650 + d, m, d), small_ints(660 + d, d, k),
                f"dk d={d} dense={dense} exact")


@pytest.mark.parametrize("d", [1025, 2000])
def test_depths_beyond_panel(d):
    # beyond d = 1024 the element-gather kernel runs
    m, k = 70, 150
    a = random_csr(640 + d, m, k, 0, 60)
    x = inputs.random_dense(641 + d, m, d)
    y_dk = inputs.random_dense(642 + d, d, k)
    note(f"sddmm dk beyond panel d={d}")
    got, _ = dk_both(a, x, y_dk, None, 1.5)
    ref, s = oracle.sddmm_general(m, k, d, a.ro, a.ci, x, y_dk, DK, None, 1.5)
    check_close(got, ref, s, f"dk d={d} gather")


# ---------------------------------------------------------------- structure edges

def test_rows_denser_than_a_window_per_chunk():
    # panels (density 1.5 %): half the rows hold 200 consecutive columns, so
    # more than 64 entries of a row fall in one chunk (d = 64 stages up to 178
    # distinct columns per chunk)
    m, k, d = 256, 10000, 64
    rows = []
    rng = np.random.default_rng(650)
    for i in range(m):
        start = int(rng.integers(0, k - 200))
        rows.append(np.arange(start, start + 200) if i % 2 == 0
                    else np.sort(rng.choice(k, 90, replace=False)))
    lengths = np.array([len(r) for r in rows], np.int32)
    ci = np.concatenate(rows).astype(np.int32)
    a = DevCsr(m, k, oracle.csr_offsets_from_lengths(lengths), ci)
    x = inputs.random_dense(651, m, d)
    y_dk = inputs.random_dense(652, d, k)
    note("sddmm dk panel dense chunk ranges")
    check(a, x, y_dk, "dk dense ranges", ri=swizzle(a))


def test_rows_of_thousands_of_entries():
    # panels (density 2 %), d = 4 stages 256 columns per chunk: rows with more
    # than two 64-entry windows in a chunk end it at their next entry's column
    m, k, d = 128, 200000, 4
    a = random_csr(655, m, k, 3000, 5000)
    x = inputs.random_dense(656, m, d)
    y_dk = inputs.random_dense(657, d, k)
    note(f"sddmm dk panel long rows nnz={a.nnz}")
    check(a, x, y_dk, "dk long rows", ri=swizzle(a))
    check_exact(a, small_ints(658, m, d), small_ints(659, d, k), "dk long rows exact")


@pytest.mark.parametrize("d", [16, 64, 256])
def test_tiles_of_long_dense_rows(d):
    # tiles (density 60 %): rows of ~2500 entries, so a tile's first entry lies
    # beyond the first 64-entry window (64-way search), and the last, ragged
    # tile
    m, k = 96, 4100
    a = random_csr(700 + d, m, k, 2000, 2900)
    x = inputs.random_dense(701 + d, m, d)
    y_dk = inputs.random_dense(702 + d, d, k)
    prior = inputs.random_dense(703 + d, a.nnz)
    note(f"sddmm dk tiles long dense rows d={d} nnz={a.nnz}")
    check(a, x, y_dk, f"dk tiles long rows d={d}", a.vals, 0.5, 2.0, prior, ri=swizzle(a))
    check_exact(a, small_ints(704 + d, m, d), small_ints(705 + d, d, k),
                f"dk tiles long rows d={d} exact")


def test_sparse_far_apart_columns():
    # two entries per row, thousands of columns apart: chunks start at the
    # smallest pending column and skip the stretches no row touches
    m, k, d = 512, 1 << 20, 32
    rng = np.random.default_rng(660)
    rows = [np.sort(rng.choice(k, 2, replace=False)) for _ in range(m)]
    ci = np.concatenate(rows).astype(np.int32)
    a = DevCsr(m, k, oracle.csr_offsets_from_lengths(np.full(m, 2, np.int32)), ci)
    x = inputs.random_dense(661, m, d)
    y_dk = inputs.random_dense(662, d, k)
    note("sddmm dk panel far-apart columns k=2^20")
    check(a, x, y_dk, "dk far apart")


@pytest.mark.parametrize("dense", [True, False], ids=["tiles", "panels"])
@pytest.mark.parametrize("m", [1, 31, 33, 63, 65, 129])
def test_partial_panels_and_empty_rows(m, dense):
    k, d = 4000, 64
    a = random_csr(670 + m, m, k, 0, 800 if dense else 80)
    x = inputs.random_dense(671 + m, m, d)
    y_dk = inputs.random_dense(672 + m, d, k)
    note(f"sddmm dk m={m} dense={dense}")
    check(a, x, y_dk, f"dk m={m} dense={dense}", None, -2.0)


def test_all_rows_empty_but_one():
    m, k, d = 200, 300, 16
    lengths = np.zeros(m, np.int32)
    lengths[137] = 250
    rl = inputs.random_row_lists(680, m, k, lengths)
    a = DevCsr(m, k, oracle.csr_offsets_from_lengths(lengths), rl.cols)
    x = inputs.random_dense(681, m, d)
    y_dk = inputs.random_dense(682, d, k)
    note("sddmm dk panel one non-empty row")
    check(a, x, y_dk, "dk one row")


def test_column_splits_of_long_rows():
    # panels (density 3 %) with one panel's worth of rows and a wide k: the
    # columns are split over several workgroups per panel, and every row
    # spans every split
    m, k, d = 32, 100000, 256
    a = random_csr(690, m, k, 2000, 4000)
    x = inputs.random_dense(691, m, d)
    y_dk = inputs.random_dense(692, d, k)
    prior = inputs.random_dense(693, a.nnz)
    note(f"sddmm dk panel column splits nnz={a.nnz}")
    check(a, x, y_dk, "dk splits", a.vals, 0.5, -1.0, prior)


@pytest.mark.parametrize("dense", [True, False], ids=["tiles", "panels"])
def test_nan_in_untouched_columns(dense):
    # NaN in every odd column of Y, which no entry touches: tiles stage them
    # but no entry reads them; panels never read them
    m, k, d = 400, 6000, 48
    lens = np.random.default_rng(701).integers(0, 600 if dense else 60, m).astype(np.int32)
    rl = inputs.random_row_lists(700, m, k // 2, lens)
    ci = (2 * rl.cols).astype(np.int32)
    a = DevCsr(m, k, oracle.csr_offsets_from_lengths(rl.lengths), ci)
    x = inputs.random_dense(702, m, d)
    y_dk = inputs.random_dense(703, d, k)
    y_dk[:, 1::2] = np.nan
    note(f"sddmm dk NaN in untouched columns dense={dense}")
    got = check(a, x, y_dk, f"dk NaN untouched dense={dense}")
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("dense", [True, False], ids=["tiles", "panels"])
@pytest.mark.parametrize("shared_y", [True, False])
def test_batched(shared_y, dense):
    m, k, d, batch = 150, 5000, 64, 3
    a = random_csr(710, m, k, 0, 1000 if dense else 100)
    xs = inputs.random_dense(711, batch, m, d)
    ys = inputs.random_dense(712, d, k) if shared_y else inputs.random_dense(712, batch, d, k)
    mvs = inputs.random_dense(713, batch, a.nnz)
    priors = inputs.random_dense(714, batch, a.nnz)
    sy = 0 if shared_y else k * d
    note(f"sddmm dk batched shared_y={shared_y} dense={dense}")
    got, with_ws = dk_both(a, xs, ys, mvs, -0.5, 1.5, priors, None, batch, a.nnz, m * d, sy,
                           a.nnz)
    for z in range(batch):
        yz = ys if shared_y else ys[z]
        ref, s = oracle.sddmm_general(m, k, d, a.ro, a.ci, xs[z], yz, DK, mvs[z], -0.5, 1.5,
                                      priors[z])
        check_close(got[z], ref, s, f"dk batched z={z} dense={dense}")
        check_close(with_ws[z], ref, s, f"dk batched z={z} dense={dense} (workspace)")
