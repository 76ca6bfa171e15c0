"""Pins of the CPU oracle against facts outside the oracle itself.

Each test checks an oracle routine against something its own code does not
produce: a hand-worked example (tests/golden), brute force over a dense
densified matrix in pure Python, an exhaustive search over permutations, a
library routine on a special case (numpy BLAS, scipy softmax), a closed form
or an invariant.  Shapes are non-square throughout so that a transposed
operand or a swapped index fails.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from unstructured_sparse_linear_csr_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _densify(m, k, ro, ci, vals):
    """Scatter CSR entries into a dense m x k float64 array (entries unique)."""
    dense = np.zeros((m, k), np.float64)
    present = np.zeros((m, k), bool)
    for i in range(m):
        for p in range(ro[i], ro[i + 1]):
            assert not present[i, ci[p]], "duplicate entry"
            present[i, ci[p]] = True
            dense[i, ci[p]] = vals[p]
    return dense, present


def _tiny_case(seed, m, k, p_keep):
    rng = np.random.default_rng(seed)
    mask = (rng.random((m, k)) < p_keep).astype(np.uint8)
    dv = rng.standard_normal((m, k)).astype(np.float32)
    return mask, dv


# ---------------------------------------------------------------- CSR build

def test_csr_from_dense_hand_example():
    g = _golden("csr_hand.json")
    ro, ci, v = oracle.csr_from_dense(np.array(g["mask"], np.uint8),
                                      np.array(g["dense_values"], np.float32))
    assert ro.tolist() == g["row_offsets"]
    assert ci.tolist() == g["col_indices"]
    assert v.tolist() == g["values"]


@pytest.mark.parametrize("seed,m,k,p", [(1, 7, 5, 0.4), (2, 5, 9, 0.7),
                                        (3, 1, 1, 1.0), (4, 6, 3, 0.0),
                                        (5, 33, 17, 0.2)])
def test_csr_from_dense_round_trip(seed, m, k, p):
    mask, dv = _tiny_case(seed, m, k, p)
    ro, ci, v = oracle.csr_from_dense(mask, dv)
    assert ro.shape == (m + 1,)
    assert int(ro[m]) == int(mask.sum()) == oracle.mask_nnz(mask)
    assert oracle.csr_check(m, k, ro, ci) == 0
    dense, present = _densify(m, k, ro, ci, v)
    assert np.array_equal(present, mask.astype(bool))
    assert np.array_equal(dense[present], dv.astype(np.float64)[present])


def test_csr_offsets_from_lengths_hand_and_cross_check():
    g = _golden("swizzle_hand.json")
    lengths = np.diff(np.array(g["row_offsets"], np.int32)).astype(np.int32)
    assert oracle.csr_offsets_from_lengths(lengths).tolist() == g["row_offsets"]
    # Cross-check against the dense-mask builder: a mask holding each row's
    # listed columns must give the same offsets.
    a = inputs.random_row_lists(7, 40, 23, np.arange(40) % 24)
    mask = np.zeros((40, 23), np.uint8)
    ro_lists = oracle.csr_offsets_from_lengths(a.lengths)
    for i in range(40):
        mask[i, a.cols[ro_lists[i]:ro_lists[i + 1]]] = 1
    ro_mask, ci_mask, _ = oracle.csr_from_dense(mask)
    assert np.array_equal(ro_mask, ro_lists)
    assert np.array_equal(ci_mask, a.cols)


def test_csr_offsets_empty():
    assert oracle.csr_offsets_from_lengths(np.zeros(0, np.int32)).tolist() == [0]
    assert oracle.csr_offsets_from_lengths(np.zeros(3, np.int32)).tolist() == [0] * 4


def test_attention_mask_count_closed_form():
    # Band: row i keeps min(i+1, 64) keys -> 2080 + (4096-64)*64 = 260128.
    # Strided keys outside the band: row i >= 64 keeps j = 0, 128, ..., <= i-64,
    # i.e. floor((i-64)/128)+1 of them; summed over t = i-64 in [0, 4031]:
    # 4032 + 128*(0+...+30) + 31*64 = 4032 + 59520 + 1984 = 65536.
    closed_form = (64 * 65 // 2 + (4096 - 64) * 64) + (4032 + 128 * 465 + 31 * 64)
    assert closed_form == 325664
    mask = inputs.attention_mask(4096)
    assert oracle.mask_nnz(mask) == closed_form


def test_csr_check_detects_each_fault():
    ro = np.array([0, 2, 2, 5], np.int32)
    ci = np.array([0, 2, 0, 1, 3], np.int32)
    assert oracle.csr_check(3, 4, ro, ci) == 0
    assert oracle.csr_check(3, 4, np.array([1, 2, 2, 5], np.int32), ci) == 1
    assert oracle.csr_check(3, 4, np.array([0, 2, 1, 5], np.int32), ci) == 2
    assert oracle.csr_check(3, 4, ro, ci[:4]) == 3
    assert oracle.csr_check(3, 3, ro, ci) == 4
    assert oracle.csr_check(3, 4, ro, np.array([0, 2, 0, 3, 1], np.int32)) == 5
    assert oracle.csr_check(3, 4, ro, np.array([0, 0, 0, 1, 3], np.int32)) == 5
    assert oracle.csr_check(3, 4, ro[:3], ci) == -1


# ---------------------------------------------------------------- swizzle

def test_swizzle_hand_example():
    g = _golden("swizzle_hand.json")
    out = oracle.row_swizzle(np.array(g["row_offsets"], np.int32))
    assert out.tolist() == g["row_indices"]


@pytest.mark.parametrize("seed", range(12))
def test_swizzle_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    m = int(rng.integers(0, 8))
    lengths = rng.integers(0, 4, size=m).astype(np.int32)  # many ties
    ro = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    valid = []
    for perm in itertools.permutations(range(m)):
        ok = all(lengths[perm[r]] > lengths[perm[r + 1]]
                 or (lengths[perm[r]] == lengths[perm[r + 1]]
                     and perm[r] < perm[r + 1])
                 for r in range(m - 1))
        if ok:
            valid.append(list(perm))
    assert len(valid) == 1
    assert oracle.row_swizzle(ro).tolist() == valid[0]


def test_swizzle_properties_at_scale():
    w = inputs.imbalance()
    ro = oracle.csr_offsets_from_lengths(w["a"].lengths)
    order = oracle.row_swizzle(ro)
    lengths = np.diff(ro)
    assert sorted(order.tolist()) == list(range(w["m"]))
    ls = lengths[order]
    assert np.all(ls[:-1] >= ls[1:])
    ties = ls[:-1] == ls[1:]
    assert np.all(order[:-1][ties] < order[1:][ties])


# ---------------------------------------------------------------- SpMM

def test_spmm_hand_example():
    g = _golden("spmm_hand.json")
    c, a = oracle.spmm(g["m"], g["k"], g["n"], g["row_offsets"],
                       g["col_indices"], g["values"], np.array(g["b"], np.float32))
    assert c.tolist() == g["c"]
    assert a.tolist() == g["abs_sum"]


def _brute_force_spmm(dense_a, b):
    """Pure-Python dense product summing k ascending, all terms included."""
    m, k = dense_a.shape
    n = b.shape[1]
    c = [[0.0] * n for _ in range(m)]
    s = [[0.0] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            acc = 0.0
            mag = 0.0
            for kk in range(k):
                t = float(dense_a[i, kk]) * float(b[kk, j])
                acc += t
                mag += abs(t)
            c[i][j] = acc
            s[i][j] = mag
    return np.array(c), np.array(s)


@pytest.mark.parametrize("seed,m,k,n,p", [(11, 6, 9, 5, 0.3), (12, 9, 4, 7, 0.8),
                                          (13, 3, 3, 1, 1.0), (14, 5, 8, 3, 0.0),
                                          (15, 17, 13, 11, 0.25)])
def test_spmm_brute_force_bit_identical(seed, m, k, n, p):
    # Both sum the same exact double products in ascending column order; the
    # zero terms of the dense sum leave the accumulator unchanged.
    mask, dv = _tiny_case(seed, m, k, p)
    ro, ci, v = oracle.csr_from_dense(mask, dv)
    b = np.random.default_rng(seed + 1000).standard_normal((k, n)).astype(np.float32)
    dense, _ = _densify(m, k, ro, ci, v)
    c_ref, s_ref = _brute_force_spmm(dense, b)
    c, s = oracle.spmm(m, k, n, ro, ci, v, b)
    assert np.array_equal(c, c_ref)
    assert np.array_equal(s, s_ref)


def test_spmm_dense_limit_matches_blas():
    # 0 % sparsity: the CSR product equals the dense GEMM up to double rounding.
    rng = np.random.default_rng(21)
    m, k, n = 37, 29, 19
    mask = np.ones((m, k), np.uint8)
    dv = rng.standard_normal((m, k)).astype(np.float32)
    b = rng.standard_normal((k, n)).astype(np.float32)
    ro, ci, v = oracle.csr_from_dense(mask, dv)
    c, s = oracle.spmm(m, k, n, ro, ci, v, b)
    ref = dv.astype(np.float64) @ b.astype(np.float64)
    assert np.all(np.abs(c - ref) <= 1e-13 * s)
    assert np.allclose(s, np.abs(dv.astype(np.float64)) @ np.abs(b.astype(np.float64)),
                       rtol=1e-13, atol=0)


def test_spmm_identity_permutation_and_power_of_two_scaling():
    rng = np.random.default_rng(22)
    k, n = 12, 7
    b = rng.standard_normal((k, n)).astype(np.float32)
    # identity
    ro = np.arange(k + 1, dtype=np.int32)
    ci = np.arange(k, dtype=np.int32)
    c, _ = oracle.spmm(k, k, n, ro, ci, np.ones(k, np.float32), b)
    assert np.array_equal(c, b.astype(np.float64))
    # permutation (rows of C are rows of B in permuted order), 5 x 12 selection
    perm = rng.permutation(k)[:5].astype(np.int32)
    c, _ = oracle.spmm(5, k, n, np.arange(6, dtype=np.int32), perm,
                       np.ones(5, np.float32), b)
    assert np.array_equal(c, b[perm].astype(np.float64))
    # diagonal of powers of two
    scale = np.float32(2.0) ** rng.integers(-6, 7, size=k).astype(np.float32)
    c, _ = oracle.spmm(k, k, n, ro, ci, scale, b)
    assert np.array_equal(c, (scale[:, None] * b).astype(np.float64))


def test_spmm_columns_are_independent_spmv():
    # n = 1 is SpMV; column j of A B must equal A (B[:, j]) exactly.
    a = inputs.random_row_lists(31, 23, 41, (np.arange(23) * 7) % 42)
    ro = oracle.csr_offsets_from_lengths(a.lengths)
    b = inputs.random_dense(32, 41, 6)
    c, s = oracle.spmm(23, 41, 6, ro, a.cols, a.values, b)
    for j in range(6):
        cj, sj = oracle.spmm(23, 41, 1, ro, a.cols, a.values,
                             np.ascontiguousarray(b[:, j:j + 1]))
        assert np.array_equal(cj[:, 0], c[:, j])
        assert np.array_equal(sj[:, 0], s[:, j])
    # homogeneity under an exact scaling of B
    c2, s2 = oracle.spmm(23, 41, 6, ro, a.cols, a.values, b * np.float32(4.0))
    assert np.array_equal(c2, 4.0 * c) and np.array_equal(s2, 4.0 * s)


def test_spmm_rows_matches_full():
    a = inputs.random_row_lists(41, 50, 30, np.arange(50) % 31)
    ro = oracle.csr_offsets_from_lengths(a.lengths)
    b = inputs.random_dense(42, 30, 9)
    c, s = oracle.spmm(50, 30, 9, ro, a.cols, a.values, b)
    rows = np.array([49, 0, 7, 7, 30], np.int32)
    cr, sr = oracle.spmm_rows(rows, 9, ro, a.cols, a.values, b)
    assert np.array_equal(cr, c[rows]) and np.array_equal(sr, s[rows])


def test_spmm_empty_rows_and_empty_matrix():
    ro = np.zeros(4, np.int32)
    c, s = oracle.spmm(3, 5, 2, ro, np.zeros(0, np.int32), np.zeros(0, np.float32),
                       np.ones((5, 2), np.float32))
    assert np.array_equal(c, np.zeros((3, 2))) and np.array_equal(s, np.zeros((3, 2)))
    c, s = oracle.spmm(0, 5, 2, np.zeros(1, np.int32), np.zeros(0, np.int32),
                       np.zeros(0, np.float32), np.ones((5, 2), np.float32))
    assert c.shape == (0, 2)


# ---------------------------------------------------------------- SDDMM

def test_sddmm_hand_example():
    g = _golden("sddmm_hand.json")
    out, a = oracle.sddmm(g["m"], g["k"], g["d"], g["row_offsets"],
                          g["col_indices"], np.array(g["x"], np.float32),
                          np.array(g["y"], np.float32))
    assert out.tolist() == g["out"]
    assert a.tolist() == g["abs_sum"]


@pytest.mark.parametrize("seed,m,k,d,p", [(51, 5, 7, 3, 0.5), (52, 8, 3, 9, 0.9),
                                          (53, 4, 6, 1, 0.6), (54, 13, 11, 16, 0.3)])
def test_sddmm_brute_force_bit_identical(seed, m, k, d, p):
    mask, _ = _tiny_case(seed, m, k, p)
    ro, ci, _ = oracle.csr_from_dense(mask)
    rng = np.random.default_rng(seed + 2000)
    x = rng.standard_normal((m, d)).astype(np.float32)
    y = rng.standard_normal((k, d)).astype(np.float32)
    # Full X Y^T in pure Python (l ascending), then read at the mask.
    full = [[sum(float(x[i, l]) * float(y[j, l]) for l in range(d))
             for j in range(k)] for i in range(m)]
    mag = [[sum(abs(float(x[i, l]) * float(y[j, l])) for l in range(d))
            for j in range(k)] for i in range(m)]
    out, a = oracle.sddmm(m, k, d, ro, ci, x, y)
    want = [full[i][ci[q]] for i in range(m) for q in range(ro[i], ro[i + 1])]
    want_mag = [mag[i][ci[q]] for i in range(m) for q in range(ro[i], ro[i + 1])]
    assert out.tolist() == want
    assert a.tolist() == want_mag


def test_sddmm_all_ones_mask_is_full_product():
    rng = np.random.default_rng(55)
    m, k, d = 21, 17, 33
    x = rng.standard_normal((m, d)).astype(np.float32)
    y = rng.standard_normal((k, d)).astype(np.float32)
    ro, ci, _ = oracle.csr_from_dense(np.ones((m, k), np.uint8))
    out, a = oracle.sddmm(m, k, d, ro, ci, x, y)
    ref = (x.astype(np.float64) @ y.astype(np.float64).T).reshape(-1)
    assert np.all(np.abs(out - ref) <= 1e-13 * a)


def test_sddmm_d1_is_exact_product():
    rng = np.random.default_rng(56)
    x = rng.standard_normal((6, 1)).astype(np.float32)
    y = rng.standard_normal((4, 1)).astype(np.float32)
    mask = (rng.random((6, 4)) < 0.6).astype(np.uint8)
    ro, ci, _ = oracle.csr_from_dense(mask)
    out, _ = oracle.sddmm(6, 4, 1, ro, ci, x, y)
    rows = np.repeat(np.arange(6), np.diff(ro))
    assert np.array_equal(out, x[rows, 0].astype(np.float64) * y[ci, 0].astype(np.float64))
    # and in fp32 the single product rounds to the fp32 product
    assert np.array_equal(out.astype(np.float32), x[rows, 0] * y[ci, 0])


def test_sddmm_ignores_mask_values():
    # I3: no element-wise scaling; the routine takes no values at all, and an
    # all-ones-valued mask and a random-valued mask give the same result.
    g = _golden("sddmm_hand.json")
    out, _ = oracle.sddmm(g["m"], g["k"], g["d"], g["row_offsets"],
                          g["col_indices"], np.array(g["x"], np.float32),
                          np.array(g["y"], np.float32))
    assert out.tolist() == g["out"]


# ---------------------------------------------------------------- softmax

def test_softmax_hand_example():
    g = _golden("softmax_hand.json")
    p = oracle.softmax_rows(g["row_offsets"], np.array(g["s"], np.float32))
    assert np.allclose(p, g["p"], rtol=0, atol=1e-15)


def test_softmax_matches_scipy_and_sums_to_one():
    from scipy.special import softmax
    a = inputs.random_row_lists(61, 30, 50, np.arange(30) % 9 + 1)
    ro = oracle.csr_offsets_from_lengths(a.lengths)
    s = (inputs.random_dense(62, a.nnz) * 5).astype(np.float32)
    p = oracle.softmax_rows(ro, s)
    for i in range(30):
        seg = slice(ro[i], ro[i + 1])
        ref = softmax(s[seg].astype(np.float64))
        assert np.allclose(p[seg], ref, rtol=1e-14, atol=0)
        assert math.isclose(p[seg].sum(), 1.0, rel_tol=0, abs_tol=1e-14)


def test_softmax_shift_invariance_and_uniform_rows():
    ro = np.array([0, 4, 7], np.int32)
    s = np.array([1.5, -2.0, 0.25, 3.0, 7.0, 7.0, 7.0], np.float32)
    p = oracle.softmax_rows(ro, s)
    p_shift = oracle.softmax_rows(ro, s + np.float32(64.0))
    assert np.allclose(p, p_shift, rtol=1e-14, atol=0)
    assert np.allclose(p[4:], 1.0 / 3.0, rtol=0, atol=1e-16)


# ---------------------------------------------------------------- general SDDMM

def test_sddmm_general_hand_example():
    g = _golden("sddmm_general_hand.json")
    for case in g["cases"]:
        y = np.array(case["y"], np.float32)
        out, a = oracle.sddmm_general(
            g["m"], g["k"], g["d"], g["row_offsets"], g["col_indices"],
            np.array(g["x"], np.float32), y, case["y_layout"],
            None if case["mask_values"] is None else np.array(case["mask_values"], np.float32),
            case["alpha"], case["beta"],
            None if case["out_in"] is None else np.array(case["out_in"], np.float32))
        assert out.tolist() == case["out"], case["name"]
        assert a.tolist() == case["abs_sum"], case["name"]


@pytest.mark.parametrize("seed,m,k,d", [(111, 5, 7, 3), (112, 9, 4, 6), (113, 3, 8, 1)])
def test_sddmm_general_brute_force(seed, m, k, d):
    rng = np.random.default_rng(seed)
    mask = (rng.random((m, k)) < 0.6).astype(np.uint8)
    ro, ci, mv = oracle.csr_from_dense(mask, rng.standard_normal((m, k)).astype(np.float32))
    x = rng.standard_normal((m, d)).astype(np.float32)
    y_kd = rng.standard_normal((k, d)).astype(np.float32)
    prior = rng.standard_normal(int(ro[-1])).astype(np.float32)
    alpha, beta = -1.5, 0.25
    want = []
    for i in range(m):
        for q in range(ro[i], ro[i + 1]):
            dot = 0.0
            for l in range(d):
                dot += float(x[i, l]) * float(y_kd[ci[q], l])
            want.append(alpha * float(mv[q]) * dot + beta * float(prior[q]))
    out0, _ = oracle.sddmm_general(m, k, d, ro, ci, x, y_kd, 0, mv, alpha, beta, prior)
    # the d x k layout of the same operand gives the same sums in the same order
    out1, _ = oracle.sddmm_general(m, k, d, ro, ci, x, np.ascontiguousarray(y_kd.T), 1, mv,
                                   alpha, beta, prior)
    assert out0.tolist() == want
    assert out1.tolist() == want


def test_sddmm_general_reduces_to_specialised_form():
    w = inputs.tiny()
    ro, ci, _ = oracle.csr_from_dense(w["mask"])
    spec, spec_abs = oracle.sddmm(256, 256, 32, ro, ci, w["x"], w["y"])
    gen, gen_abs = oracle.sddmm_general(256, 256, 32, ro, ci, w["x"], w["y"])
    assert np.array_equal(spec, gen) and np.array_equal(spec_abs, gen_abs)
    # alpha = 0: only the accumulated prior remains, scaled exactly
    prior = inputs.random_dense(5, int(ro[-1]))
    only, _ = oracle.sddmm_general(256, 256, 32, ro, ci, w["x"], w["y"], 0, None, 0.0, 2.0,
                                   prior)
    assert np.array_equal(only, 2.0 * prior.astype(np.float64))


# ---------------------------------------------------------------- transpose

def test_csr_transpose_hand_example():
    g = _golden("transpose_hand.json")
    t_ro, t_ci, t_v, t_perm = oracle.csr_transpose(g["m"], g["k"], g["row_offsets"],
                                                   g["col_indices"], g["values"])
    assert t_ro.tolist() == g["t_row_offsets"]
    assert t_ci.tolist() == g["t_col_indices"]
    assert t_v.tolist() == g["t_values"]
    assert t_perm.tolist() == g["t_perm"]


@pytest.mark.parametrize("seed,m,k,p", [(201, 7, 5, 0.4), (202, 5, 9, 0.7), (203, 1, 1, 1.0),
                                        (204, 6, 3, 0.0), (205, 33, 17, 0.2), (206, 4, 40, 0.5)])
def test_csr_transpose_is_dense_transpose(seed, m, k, p):
    mask, dv = _tiny_case(seed, m, k, p)
    ro, ci, v = oracle.csr_from_dense(mask, dv)
    t_ro, t_ci, t_v, t_perm = oracle.csr_transpose(m, k, ro, ci, v)
    # the CSR of the transposed dense matrix, built independently
    ro_ref, ci_ref, v_ref = oracle.csr_from_dense(mask.T.copy(), dv.T.copy())
    assert np.array_equal(t_ro, ro_ref)
    assert np.array_equal(t_ci, ci_ref)
    assert np.array_equal(t_v, v_ref)
    assert oracle.csr_check(k, m, t_ro, t_ci) == 0
    # the permutation names the source entry of every transposed entry
    assert sorted(t_perm.tolist()) == list(range(int(ro[-1])))
    assert np.array_equal(v[t_perm], t_v)
    assert np.array_equal(ci[t_perm], np.repeat(np.arange(k), np.diff(t_ro)))
    # transposing twice gives A back
    r2, c2, v2, _ = oracle.csr_transpose(k, m, t_ro, t_ci, t_v)
    assert np.array_equal(r2, ro) and np.array_equal(c2, ci) and np.array_equal(v2, v)


@pytest.mark.parametrize("seed,m,k,n,p", [(211, 6, 9, 5, 0.3), (212, 9, 4, 7, 0.8),
                                          (213, 3, 3, 1, 1.0), (214, 5, 8, 3, 0.0),
                                          (215, 17, 13, 11, 0.25)])
def test_spmm_transposed_brute_force(seed, m, k, n, p):
    mask, dv = _tiny_case(seed, m, k, p)
    ro, ci, v = oracle.csr_from_dense(mask, dv)
    dy = np.random.default_rng(seed + 1000).standard_normal((m, n)).astype(np.float32)
    dense_a, _ = _densify(m, k, ro, ci, v)
    # pure-Python dense A^T dY, rows of A ascending
    want = [[0.0] * n for _ in range(k)]
    for j in range(k):
        for l in range(n):
            acc = 0.0
            for i in range(m):
                acc += float(dense_a[i, j]) * float(dy[i, l])
            want[j][l] = acc
    dx, a = oracle.spmm_transposed(m, k, n, ro, ci, v, dy)
    assert dx.tolist() == want
    assert np.allclose(a, np.abs(dense_a).T @ np.abs(dy.astype(np.float64)), rtol=1e-12)
    # and it is the plain SpMM of the transposed CSR, term for term
    t_ro, t_ci, t_v, _ = oracle.csr_transpose(m, k, ro, ci, v)
    c2, a2 = oracle.spmm(k, m, n, t_ro, t_ci, t_v, dy)
    assert np.array_equal(c2, dx) and np.array_equal(a2, a)


# ---------------------------------------------------------------- 16-bit formats

def test_decode16_hand_values():
    g = _golden("float16_hand.json")
    for kind, key in ((oracle.F16, "binary16"), (oracle.BF16, "bfloat16")):
        for hexbits, value in g[key]:
            got = oracle.decode16(kind, np.array([int(hexbits, 16)], np.uint16))[0]
            if value == "nan":
                assert math.isnan(got), (key, hexbits)
            else:
                assert got == float(value), (key, hexbits, got)


def test_decode16_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    # binary16 against numpy's own conversion
    f16 = oracle.decode16(oracle.F16, bits)
    ref = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(f16), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(f16[ok], ref[ok])
    # bfloat16 against the binary32 whose upper half it is
    b16 = oracle.decode16(oracle.BF16, bits)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns
        ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(np.isnan(b16), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(b16[ok], ref[ok])
    # every finite value is exactly an fp32 value (widening loses nothing)
    for v in (f16, b16):
        fin = np.isfinite(v)
        assert np.array_equal(v[fin].astype(np.float32).astype(np.float64), v[fin])
