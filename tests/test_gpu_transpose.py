"""GPU parity of the CSR transpose and of the backward product dX = A^T dY.

The transpose is integer and permutation work: bit-exact against the oracle's
counting sort (row offsets, column indices, values and source permutation).
dX = A^T dY runs as transpose -> row swizzle -> SpMM and meets the fp32
tolerance against the oracle's direct A^T dY (same summation order: rows of A
ascending).
"""
import numpy as np
import pytest
import torch

import oracle
from unstructured_sparse_linear_csr_amd import binding as sp
from unstructured_sparse_linear_csr_amd import inputs

from gpu_util import check_close, dev, host, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sp.lib()
    yield
    torch.cuda.synchronize()


def gpu_transpose(m, k, ro, ci, vals=None, want_perm=True, want_values=True):
    nnz = int(ci.shape[0])
    ws = torch.empty(sp.sp_csr_transpose_workspace(m, k, nnz), dtype=torch.uint8,
                     device="cuda")
    ws.fill_(0xAB)  # contents on entry must not matter
    t_ro = torch.full((k + 1,), -1, dtype=torch.int32, device="cuda")
    t_ci = torch.full((max(nnz, 1),), -1, dtype=torch.int32, device="cuda")[:nnz]
    t_v = (torch.full((max(nnz, 1),), float("nan"), device="cuda")[:nnz]
           if (want_values and vals is not None) else None)
    t_p = torch.full((max(nnz, 1),), -1, dtype=torch.int32, device="cuda")[:nnz] if want_perm else None
    d_v = dev(vals) if vals is not None else None
    sp.sp_csr_transpose(m, k, nnz, dev(ro), dev(ci) if nnz else None, d_v, t_ro,
                        t_ci if nnz else None, t_v if nnz else None, t_p if nnz else None, ws)
    return (host(t_ro), host(t_ci), None if t_v is None else host(t_v),
            None if t_p is None else host(t_p))


def check_transpose(m, k, ro, ci, vals, what):
    note(f"transpose {what} m={m} k={k} nnz={ci.shape[0]}")
    g_ro, g_ci, g_v, g_p = gpu_transpose(m, k, ro, ci, vals)
    r_ro, r_ci, r_v, r_p = oracle.csr_transpose(m, k, ro, ci, vals)
    assert np.array_equal(g_ro, r_ro), f"{what}: row offsets"
    assert np.array_equal(g_ci, r_ci), f"{what}: column indices"
    assert np.array_equal(g_p, r_p), f"{what}: permutation"
    if vals is not None:
        assert np.array_equal(g_v.view(np.int32), r_v.view(np.int32)), f"{what}: values"


def row_lists(seed, m, k, max_len):
    lengths = np.random.default_rng(seed).integers(0, max_len + 1, m).astype(np.int32)
    lengths = np.minimum(lengths, k)
    rl = inputs.random_row_lists(seed + 1, m, k, lengths)
    return oracle.csr_offsets_from_lengths(lengths), rl.cols, rl.values


def test_transpose_hand_example():
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "transpose_hand.json")))
    note("transpose hand example")
    t_ro, t_ci, t_v, t_p = gpu_transpose(g["m"], g["k"], np.array(g["row_offsets"], np.int32),
                                         np.array(g["col_indices"], np.int32),
                                         np.array(g["values"], np.float32))
    assert t_ro.tolist() == g["t_row_offsets"]
    assert t_ci.tolist() == g["t_col_indices"]
    assert t_v.tolist() == g["t_values"]
    assert t_p.tolist() == g["t_perm"]


# Columns across 0 to 4 radix passes, nnz across one tile, several tiles and a
# ragged last tile, empty rows and columns.  With k <= 16384 (and nnz <= 2^18)
# the counting method runs instead: rows longer than its 2048-entry LDS piece,
# k at its LDS limit, ranges of 1024 mostly empty rows, and k one past the
# limit (the radix method again).
CASES = [
    ("k1_no_pass", 281, 300, 1, 1),
    ("k2", 282, 500, 2, 2),
    ("k256_one_pass", 283, 700, 256, 60),
    ("k257_two_passes", 284, 700, 257, 60),
    ("k4096_ragged", 285, 333, 4096, 90),
    ("k70000_three_passes", 286, 3000, 70000, 40),
    ("tall", 287, 20000, 37, 20),
    ("count_long_rows", 288, 6, 16000, 9000),
    ("count_k16384", 289, 2500, 16384, 120),
    ("count_sparse_rows", 290, 100000, 50, 1),
    ("radix_k16385", 291, 2500, 16385, 120),
    # the radix method with each entry's row carried in its key above the two
    # column passes: 32,768 rows are the most that fit (15 bits above 16), one
    # more row takes the row-id array instead
    ("radix_row_in_key_2p15", 292, 32768, 300, 20),
    ("radix_row_id_array_2p15_plus1", 293, 32769, 300, 20),
]


@pytest.mark.parametrize("name,seed,m,k,max_len", CASES)
def test_transpose_cases(name, seed, m, k, max_len):
    ro, ci, v = row_lists(seed, m, k, max_len)
    check_transpose(m, k, ro, ci, v, name)


def test_transpose_four_passes():
    """k above 2^24: four radix passes; entries spread over the whole range and
    bunched at both ends."""
    m, k = 900, (1 << 24) + 77
    rng = np.random.default_rng(301)
    cols = [np.unique(np.concatenate([rng.integers(0, k, 30), [0, 1, k - 2, k - 1]]))
            for _ in range(m)]
    lengths = np.array([len(c) for c in cols], np.int32)
    ro = oracle.csr_offsets_from_lengths(lengths)
    ci = np.concatenate(cols).astype(np.int32)
    v = inputs.random_dense(302, ci.size)
    check_transpose(m, k, ro, ci, v, "four_passes")


def test_transpose_transformer_ffn_and_optional_outputs():
    w = inputs.transformer_ffn()
    a = w["a"]
    ro = oracle.csr_offsets_from_lengths(a.lengths)
    check_transpose(a.m, a.k, ro, a.cols, a.values, "transformer_ffn")
    note("transpose without values and without permutation")
    g_ro, g_ci, g_v, g_p = gpu_transpose(a.m, a.k, ro, a.cols, None, want_perm=False)
    r_ro, r_ci, _, _ = oracle.csr_transpose(a.m, a.k, ro, a.cols)
    assert g_v is None and g_p is None
    assert np.array_equal(g_ro, r_ro) and np.array_equal(g_ci, r_ci)


def test_transpose_empty():
    note("transpose nnz=0")
    ro = np.zeros(6, np.int32)
    g_ro, g_ci, _, _ = gpu_transpose(5, 9, ro, np.zeros(0, np.int32), None)
    assert g_ro.tolist() == [0] * 10 and g_ci.size == 0
    note("transpose m=0")
    g_ro, _, _, _ = gpu_transpose(0, 4, np.zeros(1, np.int32), np.zeros(0, np.int32), None)
    assert g_ro.tolist() == [0] * 5


def test_transpose_deterministic_and_values_gather():
    ro, ci, v = row_lists(311, 5000, 3000, 200)
    m, k = 5000, 3000
    note("transpose determinism")
    r1 = gpu_transpose(m, k, ro, ci, v)
    r2 = gpu_transpose(m, k, ro, ci, v)
    for x, y in zip(r1, r2):
        assert np.array_equal(x.view(np.int32), y.view(np.int32))
    note("sp_csr_transpose_values")
    new_v = inputs.random_dense(312, ci.size)
    t_v = torch.full((ci.size,), float("nan"), device="cuda")
    sp.sp_csr_transpose_values(ci.size, dev(r1[3]), dev(new_v), t_v)
    _, _, want, _ = oracle.csr_transpose(m, k, ro, ci, new_v)
    assert np.array_equal(host(t_v).view(np.int32), want.view(np.int32))


def test_transpose_streaming_size():
    """The 65536 x 8192 matrix of the streaming workload (53.7 M entries,
    two radix passes over 13 107 tiles)."""
    w = inputs.hbm_stream(n=4)
    a = w["a"]
    ro = oracle.csr_offsets_from_lengths(a.lengths)
    note(f"transpose hbm_stream nnz={a.nnz}")
    g_ro, g_ci, _, g_p = gpu_transpose(a.m, a.k, ro, a.cols, None, want_values=False)
    r_ro, r_ci, _, r_p = oracle.csr_transpose(a.m, a.k, ro, a.cols)
    assert np.array_equal(g_ro, r_ro)
    assert np.array_equal(g_ci, r_ci)
    assert np.array_equal(g_p, r_p)


def backward(m, k, n, ro, ci, v, dy):
    """dX = A^T dY through the library: transpose, swizzle, SpMM."""
    g_ro, g_ci, g_v, _ = gpu_transpose(m, k, ro, ci, v, want_perm=False)
    d_ro = dev(g_ro)
    ri = torch.empty(k, dtype=torch.int32, device="cuda")
    sp.sp_row_swizzle(k, d_ro, ri)
    dx = torch.full((k, n), float("nan"), device="cuda")
    sp.sp_spmm(k, m, n, ci.size, ri, dev(g_v), d_ro, dev(g_ci), dev(dy), dx)
    return host(dx)


def test_backward_transformer_ffn():
    w = inputs.transformer_ffn()
    a = w["a"]
    ro = oracle.csr_offsets_from_lengths(a.lengths)
    dy = inputs.random_dense(321, a.m, w["n"])
    note("backward dX = A^T dY transformer_ffn 512x256")
    dx = backward(a.m, a.k, w["n"], ro, a.cols, a.values, dy)
    ref, s = oracle.spmm_transposed(a.m, a.k, w["n"], ro, a.cols, a.values, dy)
    check_close(dx, ref, s, "backward ffn")


@pytest.mark.parametrize("sparsity", [0.5, 0.9, 0.98])
def test_backward_lstm(sparsity):
    w = inputs.lstm(sparsity)
    a = w["a"]
    ro = oracle.csr_offsets_from_lengths(a.lengths)
    dy = inputs.random_dense(330, a.m, w["n"])
    note(f"backward dX = A^T dY lstm s={sparsity}")
    dx = backward(a.m, a.k, w["n"], ro, a.cols, a.values, dy)
    ref, s = oracle.spmm_transposed(a.m, a.k, w["n"], ro, a.cols, a.values, dy)
    check_close(dx, ref, s, f"backward lstm {sparsity}")


def test_backward_tiny_and_narrow():
    w = inputs.tiny()
    ro, ci, v = oracle.csr_from_dense(w["mask"], inputs.random_dense(340, 256, 256))
    for n in (1, 3, 64):
        dy = inputs.random_dense(341 + n, 256, n)
        note(f"backward tiny n={n}")
        dx = backward(256, 256, n, ro, ci, v, dy)
        ref, s = oracle.spmm_transposed(256, 256, n, ro, ci, v, dy)
        check_close(dx, ref, s, f"backward tiny n={n}")
