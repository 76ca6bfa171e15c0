"""GPU parity: the HIP path (through the C ABI) against the CPU oracle,
element by element on the same seeded inputs.

Integer work (CSR structure, row swizzle order) must be bit-identical; fp32
outputs must satisfy |gpu - oracle| <= 1e-5 * sum|a*b| per element, with exact
equality where the arithmetic fixes it (identity and permutation products,
one-entry rows, d = 1).  Every workload runs at full size in the launch
configuration the bench times (swizzled row order, default variants), every
element checked.
"""
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


def run_spmm(a: DevCsr, b_np, row_indices=None):
    k, n = b_np.shape
    b = dev(b_np)
    c = torch.full((a.m, n), float("nan"), dtype=torch.float32, device="cuda")
    sp.sp_spmm(a.m, a.k, n, a.nnz, row_indices, a.d_vals, a.d_ro, a.d_ci, b, c)
    return host(c)


def run_sddmm(a: DevCsr, x_np, y_np, alpha=1.0, row_indices=None):
    m, d = x_np.shape
    out = torch.full((a.nnz,), float("nan"), dtype=torch.float32, device="cuda")
    if alpha == 1.0:
        sp.sp_sddmm(a.m, a.k, d, a.nnz, row_indices, a.d_ro, a.d_ci, dev(x_np), dev(y_np), out)
    else:
        sp.sp_sddmm_batched(a.m, a.k, d, a.nnz, row_indices, a.d_ro, a.d_ci, dev(x_np),
                            dev(y_np), alpha, out, 1, 0, 0, 0)
    return host(out)


def swizzle(a: DevCsr):
    ri = torch.empty(a.m, dtype=torch.int32, device="cuda")
    sp.sp_row_swizzle(a.m, a.d_ro, ri)
    return ri


# ------------------------------------------------------------------ CSR build

def test_offsets_from_lengths_bit_exact():
    cases = {
        "transformer_ffn": inputs.transformer_ffn()["a"].lengths,
        "multi_tile_100003": np.random.default_rng(1).integers(0, 300, 100003).astype(np.int32),
        "single_row": np.array([7], np.int32),
        "all_empty": np.zeros(5000, np.int32),
        "m0": np.zeros(0, np.int32),
        # either side of a 2,048-element scan tile
        "tile_edge_2047": np.random.default_rng(3).integers(0, 600, 2047).astype(np.int32),
        "tile_edge_2049": np.random.default_rng(4).integers(0, 600, 2049).astype(np.int32),
        "tiles_6144": np.random.default_rng(5).integers(0, 600, 6144).astype(np.int32),
    }
    for name, lengths in cases.items():
        note(f"offsets_from_lengths {name} m={lengths.shape[0]}")
        m = lengths.shape[0]
        ro = torch.full((m + 1,), -7, dtype=torch.int32, device="cuda")
        sp.sp_csr_offsets_from_lengths(m, dev(lengths) if m else None, ro)
        assert np.array_equal(host(ro), oracle.csr_offsets_from_lengths(lengths)), name


def _csr_from_dense_gpu(mask, dense_values=None):
    m, k = mask.shape
    a = sp.csr_from_dense(dev(mask), None if dense_values is None else dev(dense_values))
    torch.cuda.synchronize()
    return (host(a.row_offsets), host(a.col_indices),
            None if a.values is None else host(a.values))


def test_csr_from_dense_tiny_bit_exact():
    w = inputs.tiny()
    note("csr_from_dense tiny 256x256")
    ro, ci, v = _csr_from_dense_gpu(w["mask"], w["dense_values"])
    ro_o, ci_o, v_o = oracle.csr_from_dense(w["mask"], w["dense_values"])
    assert np.array_equal(ro, ro_o) and np.array_equal(ci, ci_o)
    assert np.array_equal(v.view(np.int32), v_o.view(np.int32))


def test_csr_from_dense_attention_mask_bit_exact():
    mask = inputs.attention_mask(4096)
    note("csr_from_dense attention mask 4096x4096")
    ro, ci, v = _csr_from_dense_gpu(mask)
    ro_o, ci_o, _ = oracle.csr_from_dense(mask)
    assert v is None
    assert int(ro[-1]) == 325664
    assert np.array_equal(ro, ro_o) and np.array_equal(ci, ci_o)


@pytest.mark.parametrize("m,k,p", [(1, 1, 1.0), (3, 70, 0.5), (65, 129, 0.3),
                                   (200, 1000, 0.02), (7, 5, 0.0)])
def test_csr_from_dense_shapes(m, k, p):
    rng = np.random.default_rng(m * 1000 + k)
    mask = (rng.random((m, k)) < p).astype(np.uint8)
    mask[mask > 0] = rng.integers(1, 256, int(mask.sum()))  # any nonzero byte marks an entry
    vals = rng.standard_normal((m, k)).astype(np.float32)
    vals[0, 0] = 0.0  # an explicit zero value at a set position stays an entry
    note(f"csr_from_dense m={m} k={k} p={p}")
    ro, ci, v = _csr_from_dense_gpu(mask, vals)
    ro_o, ci_o, v_o = oracle.csr_from_dense(mask, vals)
    assert np.array_equal(ro, ro_o) and np.array_equal(ci, ci_o)
    assert np.array_equal(v.view(np.int32), v_o.view(np.int32))


# ------------------------------------------------------------------ swizzle

def _swizzle_cases():
    rng = np.random.default_rng(2)
    return {
        "transformer_ffn": inputs.transformer_ffn()["a"].lengths,
        "imbalance_lognormal": inputs.imbalance()["a"].lengths,
        "lstm_0.9": inputs.lstm(0.9)["a"].lengths,
        "ties_5000": rng.integers(0, 4, 5000).astype(np.int32),
        "tiles_9001": rng.integers(0, 50, 9001).astype(np.int32),
        "one": np.array([3], np.int32),
        "all_equal": np.full(300, 2, np.int32),
        "zeros": np.zeros(17, np.int32),
        # the scan tile edge, and either side of the switch from 32 to 16
        # lanes per row in the rank sort
        "tile_edge_2049": rng.integers(0, 600, 2049).astype(np.int32),
        "few_rows_4096": rng.integers(0, 40, 4096).astype(np.int32),
        "few_rows_4097": rng.integers(0, 40, 4097).astype(np.int32),
    }


@pytest.mark.parametrize("name", list(_swizzle_cases()))
def test_row_swizzle_bit_exact(name):
    lengths = _swizzle_cases()[name]
    ro = oracle.csr_offsets_from_lengths(lengths)
    note(f"row_swizzle {name} m={lengths.shape[0]}")
    a = DevCsr(lengths.shape[0], 1, ro, np.zeros(int(ro[-1]), np.int32))
    got = host(swizzle(a))
    assert np.array_equal(got, oracle.row_swizzle(ro)), name


@pytest.mark.parametrize("name", list(_swizzle_cases()))
def test_build_from_lengths_bit_exact(name):
    lengths = _swizzle_cases()[name]
    m = lengths.shape[0]
    note(f"build_from_lengths {name} m={m}")
    ro = torch.full((m + 1,), -7, dtype=torch.int32, device="cuda")
    ri = torch.full((m,), -7, dtype=torch.int32, device="cuda")
    sp.sp_csr_build_from_lengths(m, dev(lengths), ro, ri)
    ro_o = oracle.csr_offsets_from_lengths(lengths)
    assert np.array_equal(host(ro), ro_o), name
    assert np.array_equal(host(ri), oracle.row_swizzle(ro_o)), name


# Many rows: the workspace form (radix sort above 16,384 rows).  Keys k - length
# take 1 pass for k < 256, 2 up to k < 65,536, 3 beyond; the rows include
# ties, empty rows and rows of length k (key 0).
def _swizzle_ws_cases():
    rng = np.random.default_rng(12)
    lstm = inputs.lstm(0.9)["a"].lengths
    return {
        "limit_16384_k40": (rng.integers(0, 41, 16384).astype(np.int32), 40),
        "just_above_16385_k40": (rng.integers(0, 41, 16385).astype(np.int32), 40),
        "one_pass_k255": (rng.integers(0, 256, 40000).astype(np.int32), 255),
        "two_passes_k256": (rng.integers(0, 257, 40000).astype(np.int32), 256),
        "lstm_rows_x8_65536": (np.tile(lstm, 8), 2048),
        "ties_65536_k9": (rng.integers(0, 10, 65536).astype(np.int32), 9),
        "three_passes_k70000": (rng.integers(0, 70001, 50000).astype(np.int32), 70000),
        "all_empty_30000_k0": (np.zeros(30000, np.int32), 0),
        "rows_1100000_k8192": (rng.integers(0, 1639, 1100000).astype(np.int32), 8192),
    }


@pytest.mark.parametrize("name", list(_swizzle_ws_cases()))
def test_row_swizzle_ws_bit_exact(name):
    lengths, k = _swizzle_ws_cases()[name]
    m = lengths.shape[0]
    ro = oracle.csr_offsets_from_lengths(lengths)
    note(f"row_swizzle_ws {name} m={m} k={k}")
    ws_bytes = sp.sp_row_swizzle_workspace(m)
    assert (ws_bytes == 0) == (m <= 16384)
    ws = torch.full((max(ws_bytes, 1),), 0xAB, dtype=torch.uint8, device="cuda")
    ri = torch.full((m,), -7, dtype=torch.int32, device="cuda")
    sp.sp_row_swizzle_ws(m, k, dev(ro), ri, ws if ws_bytes else None)
    assert np.array_equal(host(ri), oracle.row_swizzle(ro)), name


def test_row_swizzle_ws_matches_rank_sort_65536():
    # both device methods at m = 65,536 give the one order
    lengths = np.tile(inputs.lstm(0.9)["a"].lengths, 8)
    m = lengths.shape[0]
    ro = dev(oracle.csr_offsets_from_lengths(lengths))
    note("row_swizzle rank vs radix m=65536")
    ri_rank = torch.empty(m, dtype=torch.int32, device="cuda")
    sp.sp_row_swizzle(m, ro, ri_rank)
    ws = torch.empty(sp.sp_row_swizzle_workspace(m), dtype=torch.uint8, device="cuda")
    ri_radix = torch.empty(m, dtype=torch.int32, device="cuda")
    sp.sp_row_swizzle_ws(m, 2048, ro, ri_radix, ws)
    assert np.array_equal(host(ri_rank), host(ri_radix))


# ------------------------------------------------------------------ SpMM, workloads

def test_spmm_tiny():
    w = inputs.tiny()
    ro, ci, v = oracle.csr_from_dense(w["mask"], w["dense_values"])
    a = DevCsr(256, 256, ro, ci, v)
    note("spmm tiny 256x256x64")
    c = run_spmm(a, w["b"])
    ref, s = oracle.spmm(256, 256, 64, ro, ci, v, w["b"])
    check_close(c, ref, s, "spmm tiny")


@pytest.fixture(scope="module")
def ffn():
    w = inputs.transformer_ffn()
    a = csr_of_row_lists(w["a"])
    return w, a


def test_spmm_transformer_ffn_swizzled(ffn):
    w, a = ffn
    note("spmm transformer_ffn 2048x512x256 swizzled")
    c = run_spmm(a, w["b"], row_indices=swizzle(a))
    ref, s = oracle.spmm(a.m, a.k, w["n"], a.ro, a.ci, a.vals, w["b"])
    check_close(c, ref, s, "spmm transformer_ffn")


def test_sddmm_transformer_ffn_swizzled(ffn):
    w, a = ffn
    note("sddmm transformer_ffn 2048x512 d=256 swizzled")
    out = run_sddmm(a, w["x"], w["y"], row_indices=swizzle(a))
    ref, s = oracle.sddmm(a.m, a.k, w["d"], a.ro, a.ci, w["x"], w["y"])
    check_close(out, ref, s, "sddmm transformer_ffn")


def test_spmm_resnet_1x1():
    w = inputs.resnet_1x1()
    a = csr_of_row_lists(w["a"])
    note("spmm resnet 1024x256x6272 swizzled")
    c = run_spmm(a, w["b"], row_indices=swizzle(a))
    ref, s = oracle.spmm(a.m, a.k, w["n"], a.ro, a.ci, a.vals, w["b"])
    check_close(c, ref, s, "spmm resnet")


@pytest.mark.parametrize("sparsity", inputs.LSTM_SPARSITIES)
def test_spmm_lstm_whole(sparsity):
    # every element of every sweep point (the oracle takes about 3 s at 50 %)
    w = inputs.lstm(sparsity)
    a = csr_of_row_lists(w["a"])
    note(f"spmm lstm 8192x2048x128 s={sparsity} swizzled")
    c = run_spmm(a, w["b"], row_indices=swizzle(a))
    ref, s = oracle.spmm(a.m, a.k, w["n"], a.ro, a.ci, a.vals, w["b"])
    check_close(c, ref, s, f"spmm lstm {sparsity}")


def test_spmm_imbalance_swizzle_on_and_off():
    # In the natural order every row is summed in entry order; in the swizzled
    # order sp_spmm runs the balanced kernel, whose skewed groups of four rows
    # split their entries over four waves: both meet the tolerance, and the
    # swizzled call is sp_spmm_balanced's, bit for bit, run to run.
    w = inputs.imbalance()
    a = csr_of_row_lists(w["a"])
    ri = swizzle(a)
    note("spmm imbalance lognormal cov0.5, swizzle on/off")
    c_off = run_spmm(a, w["b"])
    c_on = run_spmm(a, w["b"], row_indices=ri)
    ref, s = oracle.spmm(a.m, a.k, w["n"], a.ro, a.ci, a.vals, w["b"])
    check_close(c_off, ref, s, "spmm imbalance natural")
    check_close(c_on, ref, s, "spmm imbalance swizzled")
    assert np.array_equal(c_on.view(np.int32), run_spmm(a, w["b"], row_indices=ri).view(np.int32))
    b = dev(w["b"])
    c = torch.empty(a.m, w["n"], device="cuda")
    assert sp.sp_spmm_kernel_name(a.m, a.k, w["n"], a.nnz, a.d_vals, a.d_ci, b, c,
                                  row_indices=ri) == "balanced"
    sp.sp_spmm_balanced(a.m, a.k, w["n"], a.nnz, ri, a.d_vals, a.d_ro, a.d_ci, b, c)
    assert np.array_equal(c_on.view(np.int32), host(c).view(np.int32))


def test_spmm_uniform_rows_swizzle_on_and_off_bit_equal():
    # Rows of similar length: the balanced kernel's groups run one row per
    # wave, summed as the wide kernel sums them in any order.
    w = inputs.transformer_ffn()
    a = csr_of_row_lists(w["a"])
    note("spmm transformer_ffn swizzle on/off")
    c_off = run_spmm(a, w["b"])
    c_on = run_spmm(a, w["b"], row_indices=swizzle(a))
    assert np.array_equal(c_on.view(np.int32), c_off.view(np.int32))


# ------------------------------------------------------------------ SpMM, exact cases

def test_spmm_identity_and_permutation_bit_exact():
    k, n = 300, 132
    b = inputs.random_dense(4, k, n)
    ident = DevCsr(k, k, np.arange(k + 1), np.arange(k), np.ones(k, np.float32))
    note("spmm identity")
    assert np.array_equal(run_spmm(ident, b).view(np.int32), b.view(np.int32))
    perm = np.random.default_rng(5).permutation(k).astype(np.int32)
    p = DevCsr(k, k, np.arange(k + 1), perm, np.ones(k, np.float32))
    note("spmm permutation")
    assert np.array_equal(run_spmm(p, b, row_indices=swizzle(p)).view(np.int32),
                          b[perm].view(np.int32))


def test_spmm_one_entry_rows_bit_exact():
    m, k, n = 1000, 777, 68
    rl = inputs.random_row_lists(6, m, k, np.ones(m, np.int32))
    a = csr_of_row_lists(rl)
    b = inputs.random_dense(7, k, n)
    note("spmm one-entry rows")
    c = run_spmm(a, b)
    ref, _ = oracle.spmm(m, k, n, a.ro, a.ci, a.vals, b)
    assert np.array_equal(c.view(np.int32), ref.astype(np.float32).view(np.int32))


def test_spmm_narrow_exact_cases():
    # n = 8 and n = 4 take the lanes-over-entries kernel: identity and
    # one-entry rows stay exact through its shuffle tree (it adds zeros).
    for n in (4, 8, 16):
        k = 300
        b = inputs.random_dense(50 + n, k, n)
        ident = DevCsr(k, k, np.arange(k + 1), np.arange(k), np.ones(k, np.float32))
        note(f"spmm narrow identity n={n}")
        assert np.array_equal(run_spmm(ident, b).view(np.int32), b.view(np.int32))
        rl = inputs.random_row_lists(60 + n, 500, k, np.ones(500, np.int32))
        a = csr_of_row_lists(rl)
        note(f"spmm narrow one-entry rows n={n}")
        c = run_spmm(a, b)
        ref, _ = oracle.spmm(500, k, n, a.ro, a.ci, a.vals, b)
        assert np.array_equal(c.view(np.int32), ref.astype(np.float32).view(np.int32))


def test_spmm_hbm_stream_whole():
    # The streaming workload (CSR ~430 MB, n = 8) in the bench's launch
    # configuration, every element checked (the oracle takes about 2 s).
    w = inputs.hbm_stream()
    a = csr_of_row_lists(w["a"])
    note("spmm hbm_stream 65536x8192x8 swizzled")
    c = run_spmm(a, w["b"], row_indices=swizzle(a))
    ref, s = oracle.spmm(a.m, a.k, w["n"], a.ro, a.ci, a.vals, w["b"])
    check_close(c, ref, s, "spmm hbm_stream")


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 16])
def test_spmm_lds_resident_b(n):
    # Narrow B that fits in LDS with >= (CUs * k * n) entries: the streaming
    # kernel with B copied into LDS once per workgroup.
    m, k = 8192, 256
    lengths = np.random.default_rng(80 + n).integers(100, 220, m).astype(np.int32)
    lengths[::97] = 0                                   # some empty rows
    # nnz = 3 (mod 4) with a non-empty last row: the final 16-byte segment of
    # the CSR arrays extends past nnz
    lengths[-1] += (3 - int(lengths.sum()) % 4) % 4
    assert int(lengths.sum()) % 4 == 3 and lengths[-1] > 0
    a = csr_of_row_lists(inputs.random_row_lists(81 + n, m, k, lengths))
    b = inputs.random_dense(82 + n, k, n)
    note(f"spmm lds-resident B n={n} nnz={a.nnz}")
    ri = swizzle(a)
    cd = torch.empty(m, n, device="cuda")
    assert sp.sp_spmm_kernel_name(m, k, n, a.nnz, a.d_vals, a.d_ci, dev(b), cd,
                                  row_indices=ri) == "lds"
    c = run_spmm(a, b, row_indices=ri)
    ref, s = oracle.spmm(m, k, n, a.ro, a.ci, a.vals, b)
    check_close(c, ref, s, f"spmm lds n={n}")
    # one-entry rows through the same kernel are exact
    rl = inputs.random_row_lists(83 + n, 1100000, k, np.ones(1100000, np.int32))
    a1 = csr_of_row_lists(rl)
    note(f"spmm lds-resident B one-entry rows n={n}")
    c1 = run_spmm(a1, b)
    ref1, _ = oracle.spmm(1100000, k, n, a1.ro, a1.ci, a1.vals, b)
    assert np.array_equal(c1.view(np.int32), ref1.astype(np.float32).view(np.int32))


@pytest.mark.parametrize("k,n,m", [(8192, 8, 16384), (8192, 12, 10000), (8192, 16, 8000),
                                   (3000, 12, 12000), (16384, 3, 16384), (5000, 8, 10000)])
def test_spmm_lds_column_slices(k, n, m):
    # Narrow B too large for LDS whole, with enough entries per CU: the
    # streaming kernel over column slices of B (2-4 slices, one uneven: 8 + 4
    # columns; the scalar path's 2 + 1), every entry checked.
    lengths = np.random.default_rng(84 + n + k).integers(250, 360, m).astype(np.int32)
    lengths[::89] = 0
    lengths[-1] += (3 - int(lengths.sum()) % 4) % 4   # last CSR segment past nnz
    assert int(lengths.sum()) % 4 == 3 and lengths[-1] > 0
    a = csr_of_row_lists(inputs.random_row_lists(85 + n + k, m, k, lengths))
    b = inputs.random_dense(86 + n + k, k, n)
    note(f"spmm lds column slices k={k} n={n} m={m} nnz={a.nnz}")
    ri = swizzle(a)
    cd = torch.empty(m, n, device="cuda")
    assert sp.sp_spmm_kernel_name(m, k, n, a.nnz, a.d_vals, a.d_ci, dev(b), cd,
                                  row_indices=ri) == "lds"
    c = run_spmm(a, b, row_indices=ri)
    ref, s = oracle.spmm(m, k, n, a.ro, a.ci, a.vals, b)
    check_close(c, ref, s, f"spmm lds slices k={k} n={n}")
    assert np.all(c[lengths == 0] == 0)


def test_spmm_hbm_stream_n4_whole():
    w = inputs.hbm_stream(n=4)
    a = csr_of_row_lists(w["a"])
    note("spmm hbm_stream 65536x8192x4 (B in LDS)")
    c = run_spmm(a, w["b"])
    ref, s = oracle.spmm(a.m, a.k, w["n"], a.ro, a.ci, a.vals, w["b"])
    check_close(c, ref, s, "spmm hbm_stream n=4")


# ------------------------------------------------------------------ SpMM, edges

WIDTHS = [1, 2, 3, 4, 5, 8, 12, 16, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256,
          257, 260, 1000]


@pytest.mark.parametrize("n", WIDTHS)
def test_spmm_widths(n):
    m, k = 131, 97
    rng = np.random.default_rng(n)
    lengths = rng.integers(0, 40, m).astype(np.int32)  # includes empty rows
    a = csr_of_row_lists(inputs.random_row_lists(8 + n, m, k, lengths))
    b = inputs.random_dense(9 + n, k, n)
    note(f"spmm width n={n}")
    c = run_spmm(a, b, row_indices=swizzle(a))
    ref, s = oracle.spmm(m, k, n, a.ro, a.ci, a.vals, b)
    check_close(c, ref, s, f"spmm n={n}")
    assert np.all(c[lengths == 0] == 0)


def test_spmm_misaligned_rows_and_pointers():
    # Row lengths 0..9 cycling: row starts fall on every offset mod 4.  Then
    # the same product through CSR, B and C arrays that start 4 bytes past
    # an aligned address (the scalar-load variants).
    m, k, n = 400, 150, 64
    lengths = (np.arange(m) % 10).astype(np.int32)
    rl = inputs.random_row_lists(10, m, k, lengths)
    ro = oracle.csr_offsets_from_lengths(lengths)
    b_np = inputs.random_dense(11, k, n)
    ref, s = oracle.spmm(m, k, n, ro, rl.cols, rl.values, b_np)
    a = DevCsr(m, k, ro, rl.cols, rl.values)
    note("spmm misaligned row starts, aligned arrays")
    c_al = run_spmm(a, b_np)
    check_close(c_al, ref, s, "spmm misaligned rows")
    note("spmm misaligned row starts, unaligned arrays")
    nnz = rl.nnz
    ci_buf = torch.zeros(nnz + 1, dtype=torch.int32, device="cuda")
    v_buf = torch.zeros(nnz + 1, dtype=torch.float32, device="cuda")
    b_buf = torch.zeros(k * n + 1, dtype=torch.float32, device="cuda")
    c_buf = torch.zeros(m * n + 1, dtype=torch.float32, device="cuda")
    ci_buf[1:] = dev(rl.cols)
    v_buf[1:] = dev(rl.values)
    b_buf[1:] = dev(b_np.reshape(-1))
    sp.sp_spmm(m, k, n, nnz, None, v_buf[1:], a.d_ro, ci_buf[1:], b_buf[1:], c_buf[1:])
    c_un = host(c_buf[1:]).reshape(m, n)
    check_close(c_un, ref, s, "spmm unaligned")
    assert np.array_equal(c_un.view(np.int32), c_al.view(np.int32))


def test_spmm_empty_structures():
    m, k, n = 50, 40, 36
    b = inputs.random_dense(12, k, n)
    a = DevCsr(m, k, np.zeros(m + 1, np.int32), np.zeros(0, np.int32),
               np.zeros(0, np.float32))
    note("spmm nnz=0")
    c = run_spmm(a, b)
    assert np.array_equal(c, np.zeros((m, n), np.float32))
    # m == 0 and n == 0 enqueue nothing and leave the output untouched
    c_keep = torch.full((4, 4), 3.0, device="cuda")
    sp.sp_spmm(0, k, 4, 0, None, None, dev(np.zeros(1, np.int32)), None, dev(b), c_keep)
    sp.sp_spmm(4, k, 0, 0, None, None, dev(np.zeros(5, np.int32)), None, dev(b), c_keep)
    assert np.all(host(c_keep) == 3.0)


def test_spmm_long_rows():
    m, k, n = 96, 65536, 128
    lengths = np.random.default_rng(13).integers(3000, 6000, m).astype(np.int32)
    a = csr_of_row_lists(inputs.random_row_lists(14, m, k, lengths))
    b = inputs.random_dense(15, k, n)
    note("spmm long rows k=65536")
    c = run_spmm(a, b, row_indices=swizzle(a))
    ref, s = oracle.spmm(m, k, n, a.ro, a.ci, a.vals, b)
    check_close(c, ref, s, "spmm long rows")


def test_spmm_wide_operand_64bit_offsets():
    # k * n >= 2^30 takes the 64-bit-offset variant (B is 4 GiB).  B is zero
    # except the rows A reads, which hold seeded N(0,1) data; the oracle runs
    # on A with its columns renumbered onto those rows.
    m, k, n = 64, 32768, 32772
    rng = np.random.default_rng(16)
    lengths = rng.integers(1, 20, m).astype(np.int32)
    a = csr_of_row_lists(inputs.random_row_lists(17, m, k, lengths))
    used = np.unique(a.ci)
    assert used[-1] > k // 2  # offsets beyond 2^31 bytes are exercised
    b_used = inputs.random_dense(18, used.shape[0], n)
    note("spmm 64-bit offsets, B 32768x32772")
    b = torch.zeros(k, n, dtype=torch.float32, device="cuda")
    b[dev(used.astype(np.int64))] = dev(b_used)
    c = torch.empty(m, n, dtype=torch.float32, device="cuda")
    sp.sp_spmm(m, k, n, a.nnz, None, a.d_vals, a.d_ro, a.d_ci, b, c)
    got = host(c)
    del b
    remap = np.full(k, -1, np.int64)
    remap[used] = np.arange(used.shape[0])
    ref, s = oracle.spmm(m, used.shape[0], n, a.ro, remap[a.ci].astype(np.int32),
                         a.vals, b_used)
    check_close(got, ref, s, "spmm 64-bit offsets")


def test_spmm_batched_shared_structure():
    m, k, n, batch = 120, 90, 40, 3
    lengths = np.random.default_rng(19).integers(0, 30, m).astype(np.int32)
    rl = inputs.random_row_lists(20, m, k, lengths)
    ro = oracle.csr_offsets_from_lengths(lengths)
    nnz = rl.nnz
    vals = inputs.random_dense(21, batch, nnz)
    bs = inputs.random_dense(22, batch, k, n)
    c = torch.full((batch, m, n), float("nan"), device="cuda")
    d_ro, d_ci = dev(ro), dev(rl.cols)
    note("spmm batched 3, per-batch values and B")
    sp.sp_spmm_batched(m, k, n, nnz, None, dev(vals), d_ro, d_ci, dev(bs), c, batch,
                       nnz, k * n, m * n)
    got = host(c)
    for z in range(batch):
        ref, s = oracle.spmm(m, k, n, ro, rl.cols, vals[z], bs[z])
        check_close(got[z], ref, s, f"spmm batched z={z}")
    note("spmm batched 3, shared values (stride 0)")
    sp.sp_spmm_batched(m, k, n, nnz, None, dev(vals[0]), d_ro, d_ci, dev(bs), c, batch,
                       0, k * n, m * n)
    got = host(c)
    for z in range(batch):
        ref, s = oracle.spmm(m, k, n, ro, rl.cols, vals[0], bs[z])
        check_close(got[z], ref, s, f"spmm batched shared z={z}")


def test_spmm_deterministic():
    w = inputs.transformer_ffn()
    a = csr_of_row_lists(w["a"])
    ri = swizzle(a)
    note("spmm determinism")
    c1 = run_spmm(a, w["b"], row_indices=ri)
    c2 = run_spmm(a, w["b"], row_indices=ri)
    assert np.array_equal(c1.view(np.int32), c2.view(np.int32))


# ------------------------------------------------------------------ SDDMM

def test_sddmm_tiny():
    w = inputs.tiny()
    ro, ci, _ = oracle.csr_from_dense(w["mask"])
    a = DevCsr(256, 256, ro, ci)
    note("sddmm tiny d=32")
    out = run_sddmm(a, w["x"], w["y"])
    ref, s = oracle.sddmm(256, 256, 32, ro, ci, w["x"], w["y"])
    check_close(out, ref, s, "sddmm tiny")


DEPTHS = [1, 2, 3, 4, 5, 7, 8, 16, 31, 32, 33, 48, 64, 100, 128, 256, 260, 512, 516,
          1000, 2052]


@pytest.mark.parametrize("d", DEPTHS)
def test_sddmm_depths(d):
    m, k = 77, 130
    lengths = np.random.default_rng(d).integers(0, 100, m).astype(np.int32)
    rl = inputs.random_row_lists(30 + d, m, k, lengths)
    ro = oracle.csr_offsets_from_lengths(lengths)
    a = DevCsr(m, k, ro, rl.cols)
    x = inputs.random_dense(31 + d, m, d)
    y = inputs.random_dense(32 + d, k, d)
    note(f"sddmm depth d={d}")
    out = run_sddmm(a, x, y, row_indices=swizzle(a))
    ref, s = oracle.sddmm(m, k, d, ro, rl.cols, x, y)
    check_close(out, ref, s, f"sddmm d={d}")
    if d == 1:
        assert np.array_equal(out.view(np.int32), ref.astype(np.float32).view(np.int32))


def test_sddmm_alpha_and_unaligned():
    m, k, d = 90, 60, 64
    lengths = (np.arange(m) % 13).astype(np.int32)
    rl = inputs.random_row_lists(40, m, k, lengths)
    ro = oracle.csr_offsets_from_lengths(lengths)
    a = DevCsr(m, k, ro, rl.cols)
    x = inputs.random_dense(41, m, d)
    y = inputs.random_dense(42, k, d)
    ref, s = oracle.sddmm(m, k, d, ro, rl.cols, x, y)
    note("sddmm alpha=0.125")
    out = run_sddmm(a, x, y, alpha=0.125)
    # 1/8 is a power of two: scaling the fp32 result is exact
    check_close(out, 0.125 * ref, 0.125 * s, "sddmm alpha")
    out1 = run_sddmm(a, x, y)
    assert np.array_equal(out.view(np.int32), (out1 * np.float32(0.125)).view(np.int32))
    note("sddmm unaligned x/y")
    xb = torch.zeros(m * d + 1, device="cuda")
    yb = torch.zeros(k * d + 1, device="cuda")
    xb[1:] = dev(x.reshape(-1))
    yb[1:] = dev(y.reshape(-1))
    o = torch.empty(a.nnz, device="cuda")
    sp.sp_sddmm(m, k, d, a.nnz, None, a.d_ro, a.d_ci, xb[1:], yb[1:], o)
    check_close(host(o), ref, s, "sddmm unaligned")


def test_sddmm_batched_and_d0():
    m, k, d, batch = 64, 50, 32, 4
    lengths = np.random.default_rng(43).integers(0, 50, m).astype(np.int32)
    rl = inputs.random_row_lists(44, m, k, lengths)
    ro = oracle.csr_offsets_from_lengths(lengths)
    a = DevCsr(m, k, ro, rl.cols)
    xs = inputs.random_dense(45, batch, m, d)
    ys = inputs.random_dense(46, batch, k, d)
    out = torch.full((batch, a.nnz), float("nan"), device="cuda")
    note("sddmm batched 4")
    sp.sp_sddmm_batched(m, k, d, a.nnz, None, a.d_ro, a.d_ci, dev(xs), dev(ys), 1.0,
                        out, batch, m * d, k * d, a.nnz)
    got = host(out)
    for z in range(batch):
        ref, s = oracle.sddmm(m, k, d, ro, rl.cols, xs[z], ys[z])
        check_close(got[z], ref, s, f"sddmm batched z={z}")
    note("sddmm d=0")
    sp.sp_sddmm_batched(m, k, 0, a.nnz, None, a.d_ro, a.d_ci, None, None, 1.0, out,
                        batch, 0, 0, a.nnz)
    assert np.all(host(out) == 0.0)


def test_sddmm_deterministic(ffn):
    w, a = ffn
    ri = swizzle(a)
    note("sddmm determinism, swizzle on/off")
    o1 = run_sddmm(a, w["x"], w["y"], row_indices=ri)
    o2 = run_sddmm(a, w["x"], w["y"], row_indices=ri)
    o3 = run_sddmm(a, w["x"], w["y"])
    assert np.array_equal(o1.view(np.int32), o2.view(np.int32))
    assert np.array_equal(o1.view(np.int32), o3.view(np.int32))


# ------------------------------------------------------------------ sparse attention

def test_sparse_attention_pipeline():
    w = inputs.sparse_attention()
    bh, seq, hd = w["batch"], w["seq"], w["head_dim"]
    ro, ci, _ = oracle.csr_from_dense(w["mask"])
    a = DevCsr(seq, seq, ro, ci)
    nnz = a.nnz
    assert nnz == 325664
    ri = swizzle(a)
    q, kk, v = dev(w["q"]), dev(w["k"]), dev(w["v"])
    s_dev = torch.empty(bh, nnz, device="cuda")
    note("attention sddmm batched 32 x 4096 d=64 alpha=1/8")
    sp.sp_sddmm_batched(seq, seq, hd, nnz, ri, a.d_ro, a.d_ci, q, kk, 0.125, s_dev, bh,
                        seq * hd, seq * hd, nnz)
    s_gpu = host(s_dev)
    p_host = np.empty((bh, nnz), np.float32)
    for z in range(bh):
        ref, mag = oracle.sddmm(seq, seq, hd, ro, ci, w["q"][z], w["k"][z])
        check_close(s_gpu[z], 0.125 * ref, 0.125 * mag, f"attention S head {z}")
        # Row softmax on the host, from the GPU's scores (each kernel is
        # checked on its own inputs).
        p_host[z] = oracle.softmax_rows(ro, s_gpu[z]).astype(np.float32)
    o_dev = torch.empty(bh, seq, hd, device="cuda")
    note("attention spmm batched 32 x 4096 n=64")
    sp.sp_spmm_batched(seq, seq, hd, nnz, ri, dev(p_host), a.d_ro, a.d_ci, v, o_dev, bh,
                       nnz, seq * hd, seq * hd)
    o_gpu = host(o_dev)
    for z in range(bh):
        ref, mag = oracle.spmm(seq, seq, hd, ro, ci, p_host[z], w["v"][z])
        check_close(o_gpu[z], ref, mag, f"attention O head {z}")


# ------------------------------------------------------------------ HIP graphs

def test_graph_replays_match_eager(ffn):
    # The bench replays a captured step.  Every replay, with eager work and
    # synchronisations between replays, must equal the eager result bit for bit.
    w, a = ffn
    m, k, n, d = a.m, a.k, w["n"], w["d"]
    lengths = dev(w["a"].lengths)
    b, x, y = dev(w["b"]), dev(w["x"]), dev(w["y"])
    ro = torch.empty(m + 1, dtype=torch.int32, device="cuda")
    ri = torch.empty(m, dtype=torch.int32, device="cuda")
    c = torch.empty(m, n, device="cuda")
    out = torch.empty(a.nnz, device="cuda")

    def step():
        sp.sp_csr_offsets_from_lengths(m, lengths, ro)
        sp.sp_row_swizzle(m, ro, ri)
        sp.sp_spmm(m, k, n, a.nnz, ri, a.d_vals, ro, a.d_ci, b, c)
        sp.sp_sddmm(m, k, d, a.nnz, ri, ro, a.d_ci, x, y, out)

    note("graph: eager reference step")
    step()
    ref = [host(t).copy() for t in (ro, ri, c, out)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        for t in (ro, ri, c, out):
            t.fill_(-1)          # eager work between replays
        torch.cuda.synchronize()
        note(f"graph replay {r}")
        g.replay()
        got = [host(t) for t in (ro, ri, c, out)]
        for want, have, name in zip(ref, got, ("row_offsets", "row_indices", "c", "out")):
            assert np.array_equal(want.view(np.int32), have.view(np.int32)), (r, name)


# ------------------------------------------------------------------ row softmax

def _softmax_bound(ro, s, p_ref):
    """Per-element bound of the fp32 softmax: relative (|s - max| + 8) * 2^-23
    (rounding of s - max amplified by exp, expf itself, the row sum and the
    division), in units of the exact result, plus an absolute 2^-126 (below
    fp32's smallest normal a value has no relative precision)."""
    b = np.zeros_like(p_ref)
    for i in range(ro.shape[0] - 1):
        seg = slice(ro[i], ro[i + 1])
        if ro[i + 1] > ro[i]:
            x = s[seg].astype(np.float64) - float(s[seg].max())
            b[seg] = p_ref[seg] * (np.abs(x) + 8.0) * 2.0 ** -23 + 2.0 ** -126
    return b


def _check_softmax(got, ro, s, what):
    ref = oracle.softmax_rows(ro, s)
    bound = _softmax_bound(ro, s, ref)
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(np.isfinite(got)), what
    assert np.all(err <= bound), f"{what}: worst {np.max(err / np.maximum(bound, 1e-300)):.3g}"


@pytest.mark.parametrize("case", ["short", "long", "mixed_empty", "held_edge"])
def test_row_softmax(case):
    rng = np.random.default_rng({"short": 90, "long": 91, "mixed_empty": 92,
                                 "held_edge": 94}[case])
    if case == "short":
        lengths = rng.integers(1, 80, 700)
    elif case == "long":
        lengths = rng.integers(250, 900, 60)          # beyond the register-held path
    elif case == "held_edge":
        # rows either side of the 128 entries a 16-lane group holds in
        # registers, one per lane group and mixed within waves; m = 4q + 3
        lengths = np.tile(np.array([127, 128, 129, 1, 16, 17, 300], np.int32), 41)[:287]
    else:
        lengths = rng.integers(0, 400, 500)
        lengths[::7] = 0
    lengths = lengths.astype(np.int32)
    m = lengths.shape[0]
    ro = oracle.csr_offsets_from_lengths(lengths)
    nnz = int(ro[-1])
    s = (inputs.random_dense(93, nnz) * np.float32(4.0)).astype(np.float32)
    d_ro = dev(ro)
    ri = torch.empty(m, dtype=torch.int32, device="cuda")
    sp.sp_row_swizzle(m, d_ro, ri)
    out = torch.full((nnz,), float("nan"), device="cuda")
    note(f"row softmax {case} m={m} nnz={nnz}")
    sp.sp_csr_row_softmax(m, nnz, ri, d_ro, dev(s), out)
    _check_softmax(host(out), ro, s, f"softmax {case}")
    note(f"row softmax {case} in place")
    buf = dev(s)
    sp.sp_csr_row_softmax(m, nnz, None, d_ro, buf, buf)
    _check_softmax(host(buf), ro, s, f"softmax {case} in place")


def test_row_softmax_batched_attention_mask():
    mask = inputs.attention_mask(4096)
    ro, ci, _ = oracle.csr_from_dense(mask)
    nnz = int(ro[-1])
    batch = 4
    s = (inputs.random_dense(94, batch, nnz) * np.float32(3.0)).astype(np.float32)
    out = torch.empty(batch, nnz, device="cuda")
    note("row softmax batched attention mask")
    sp.sp_csr_row_softmax(4096, nnz, None, dev(ro), dev(s), out, batch, nnz, nnz)
    got = host(out)
    for z in range(batch):
        _check_softmax(got[z], ro, s[z], f"softmax attention z={z}")


def test_sparse_attention_all_device():
    # SDDMM (scale 1/8) -> row softmax -> SpMM, every step on the device,
    # against the oracle pipeline in double with the propagated bound: S within
    # e_S = 1e-5 sum|q k| / 8; softmax maps that to a relative P error of at most
    # 2 max_row(e_S) plus its own rounding; O inherits sum_j P_j |V_j| times those
    # relative errors, plus the SpMM's 1e-5.
    w = inputs.sparse_attention()
    heads = [0, 7, 31]
    seq, hd, bh = w["seq"], w["head_dim"], w["batch"]
    ro, ci, _ = oracle.csr_from_dense(w["mask"])
    a = DevCsr(seq, seq, ro, ci)
    nnz = a.nnz
    ri = swizzle(a)
    q, kk, v = dev(w["q"]), dev(w["k"]), dev(w["v"])
    s_dev = torch.empty(bh, nnz, device="cuda")
    o_dev = torch.empty(bh, seq, hd, device="cuda")
    note("attention all-device: sddmm, softmax, spmm")
    sp.sp_sddmm_batched(seq, seq, hd, nnz, ri, a.d_ro, a.d_ci, q, kk, 0.125, s_dev, bh,
                        seq * hd, seq * hd, nnz)
    sp.sp_csr_row_softmax(seq, nnz, ri, a.d_ro, s_dev, s_dev, bh, nnz, nnz)
    sp.sp_spmm_batched(seq, seq, hd, nnz, ri, s_dev, a.d_ro, a.d_ci, v, o_dev, bh, nnz,
                       seq * hd, seq * hd)
    o_gpu = host(o_dev)
    rows = np.repeat(np.arange(seq), np.diff(ro))
    for z in heads:
        s_ref, s_abs = oracle.sddmm(seq, seq, hd, ro, ci, w["q"][z], w["k"][z])
        s_ref, e_s = 0.125 * s_ref, 0.125 * 1e-5 * s_abs
        p_ref = oracle.softmax_rows(ro, s_ref.astype(np.float32))
        # row maxima of e_S and of the softmax rounding term
        e_row = np.zeros(seq)
        np.maximum.at(e_row, rows, e_s)
        smax = np.full(seq, -np.inf)
        np.maximum.at(smax, rows, s_ref)
        x_row = np.zeros(seq)
        np.maximum.at(x_row, rows, np.abs(s_ref - smax[rows]))
        rel = 2.0 * e_row + (x_row + 8.0) * 2.0 ** -23 + 1e-5
        o_ref, _ = oracle.spmm(seq, seq, hd, ro, ci, p_ref, w["v"][z])
        pv, _ = oracle.spmm(seq, seq, hd, ro, ci, p_ref, np.abs(w["v"][z]))
        err = np.abs(o_gpu[z].astype(np.float64) - o_ref)
        assert np.all(err <= rel[:, None] * pv * 1.01), f"attention head {z}"
