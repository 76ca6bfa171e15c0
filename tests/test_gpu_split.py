"""GPU parity of sp_spmm on few, long rows, where each row's entries are cut
into four parts taken by the four waves of a workgroup and the partial sums
are added in part order: against the oracle within the fp32 tolerance,
deterministic, over lane layouts (8-64 lanes per row, several column tiles,
the scalar path), ragged and empty rows, batches, and 16-bit operands."""
import numpy as np
import pytest
import torch

import oracle
from unstructured_sparse_linear_csr_amd import binding as sp
from unstructured_sparse_linear_csr_amd import inputs

from gpu_util import DevCsr, check_close, dev, host, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sp.lib()
    yield
    torch.cuda.synchronize()


def long_rows(seed, m, k):
    """Rows of 300-3000 entries, with empty rows and rows of 1-3 entries."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(300, 3000, m).astype(np.int32)
    lengths[::11] = 0
    lengths[1::13] = rng.integers(1, 4, lengths[1::13].size)
    rl = inputs.random_row_lists(seed + 1, m, k, np.minimum(lengths, k))
    return DevCsr(m, k, oracle.csr_offsets_from_lengths(rl.lengths), rl.cols, rl.values)


def swizzle(a):
    ri = torch.empty(a.m, dtype=torch.int32, device="cuda")
    sp.sp_row_swizzle(a.m, a.d_ro, ri)
    return ri


@pytest.mark.parametrize("n", [32, 64, 128, 256, 42, 1000])
def test_long_rows_widths(n):
    """8/16/32/64 lanes per row, several column tiles (n = 1000), and the
    scalar path (n = 42)."""
    m, k = 96, 4096
    a = long_rows(1200 + n, m, k)
    assert a.nnz >= 256 * m
    b = inputs.random_dense(1210 + n, k, n)
    note(f"spmm long rows m={m} n={n} nnz={a.nnz}")
    c = torch.full((m, n), float("nan"), device="cuda")
    sp.sp_spmm(m, k, n, a.nnz, swizzle(a), a.d_vals, a.d_ro, a.d_ci, dev(b), c)
    got = host(c)
    ref, s = oracle.spmm(m, k, n, a.ro, a.ci, a.vals, b)
    check_close(got, ref, s, f"long rows n={n}")
    assert np.all(got[np.diff(a.ro) == 0] == 0)
    c2 = torch.full((m, n), float("nan"), device="cuda")
    sp.sp_spmm(m, k, n, a.nnz, swizzle(a), a.d_vals, a.d_ro, a.d_ci, dev(b), c2)
    assert np.array_equal(got.view(np.int32), host(c2).view(np.int32))


def test_long_rows_batched():
    m, k, n, batch = 40, 3000, 128, 3
    a = long_rows(1220, m, k)
    vals = inputs.random_dense(1221, batch, a.nnz)
    bs = inputs.random_dense(1222, batch, k, n)
    c = torch.full((batch, m, n), float("nan"), device="cuda")
    note(f"spmm long rows batched batch={batch}")
    sp.sp_spmm_batched(m, k, n, a.nnz, None, dev(vals), a.d_ro, a.d_ci, dev(bs), c, batch,
                       a.nnz, k * n, m * n)
    got = host(c)
    for z in range(batch):
        ref, s = oracle.spmm(m, k, n, a.ro, a.ci, vals[z], bs[z])
        check_close(got[z], ref, s, f"long rows batched z={z}")


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_long_rows_16bit(kind):
    tdt, code = {"f16": (torch.float16, oracle.F16), "bf16": (torch.bfloat16, oracle.BF16)}[kind]
    m, k, n = 64, 4096, 256
    a = long_rows(1230, m, k)

    def to16(x):
        t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(tdt)
        return t.cuda(), oracle.decode16(code, t.view(torch.int16).numpy().view(np.uint16))

    d_v, v = to16(a.vals)
    d_b, b = to16(inputs.random_dense(1231, k, n))
    c = torch.full((m, n), float("nan"), device="cuda")
    note(f"spmm_ex long rows {kind}")
    sp.sp_spmm_ex(m, k, n, a.nnz, swizzle(a), d_v, a.d_ro, a.d_ci, d_b, c)
    ref, s = oracle.spmm(m, k, n, a.ro, a.ci, v, b)
    check_close(host(c), ref, s, f"long rows {kind}")
