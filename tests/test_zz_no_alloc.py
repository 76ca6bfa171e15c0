"""The allocation-free row swizzle (sp_row_swizzle_noalloc) through the C ABI,
against the workspace form it mirrors (sp_row_swizzle_ws, same order bit for
bit) and the oracle, on consecutive calls that share the library's per-GPU
scratch array: a large structure, then a smaller one (the second must not see
the first's leftovers), then one small enough for the rank sort."""
import numpy as np
import pytest
import torch

import oracle
from unstructured_sparse_linear_csr_amd import binding as sp

from gpu_util import host, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sp.lib()
    yield
    torch.cuda.synchronize()


def _devi(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to("cuda")


def _orders(m, k, seed, longest):
    # row lengths in [0, longest] (longest <= k), with every length up to
    # `longest` likely present; nnz stays below 2^31
    lengths = np.random.default_rng(seed).integers(0, longest + 1, m).astype(np.int32)
    assert int(lengths.sum()) < 2 ** 31
    ro_h = oracle.csr_offsets_from_lengths(lengths)
    ro = _devi(ro_h)
    ws_bytes = sp.sp_row_swizzle_workspace(m)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None
    ri_ws = torch.full((m,), -1, dtype=torch.int32, device="cuda")
    sp.sp_row_swizzle_ws(m, k, ro, ri_ws, ws)
    ri_na = torch.full((m,), -2, dtype=torch.int32, device="cuda")
    sp.sp_row_swizzle_noalloc(m, k, ro, ri_na)
    return host(ri_ws), host(ri_na), oracle.row_swizzle(ro_h)


def test_noalloc_matches_workspace_form_on_consecutive_calls():
    # 1.1 M rows (two radix passes), then 70,000 rows with k = 70,000 (three
    # passes, smaller), then 9,000 rows (the rank sort, no scratch)
    for m, k, longest, seed in ((1_100_000, 8192, 1900, 51), (70_000, 70_000, 30_000, 52),
                                (9_000, 100, 100, 53)):
        note(f"row_swizzle_noalloc m={m} k={k}")
        ws, na, ref = _orders(m, k, seed, longest)
        assert np.array_equal(na, ws), (m, k)
        assert np.array_equal(na, ref), (m, k)


def test_noalloc_at_its_row_limit_and_beyond():
    top = sp.SP_ROW_SWIZZLE_NOALLOC_MAX_ROWS
    note(f"row_swizzle_noalloc m={top}")
    ws, na, ref = _orders(top, 1000, 54, 1000)
    assert np.array_equal(na, ws) and np.array_equal(na, ref)
    ro = torch.zeros(top + 2, dtype=torch.int32, device="cuda")
    ri = torch.empty(top + 1, dtype=torch.int32, device="cuda")
    with pytest.raises(sp.SpError) as err:
        sp.sp_row_swizzle_noalloc(top + 1, 1000, ro, ri)
    assert err.value.status == sp.SP_ERROR_INVALID_VALUE
