"""GPU parity of the panel-union SpMM (batched; fp32, or 16-bit values and B
widened to fp32; n = 64, 128 or 256; at most 65,536 rows of B).

A workgroup takes 16 consecutive rows and four batch entries, forms the union
of the rows' columns once, and computes each entry's C[panel] = A[panel,
union] B[union] as MFMA tiles; a panel whose union is too wide for its entry
count, or whose union rows of B hold a value that is not finite, runs the wide
kernel's accumulation instead (SpMM, "Sparse GPU Kernels for Deep Learning",
Section 5; the attention output P V of Section 7.3).  Tile sums round
differently from the per-entry kernels, so the bar is the stated tolerance
against the oracle, |gpu - oracle| <= 1e-5 * sum |a b| per element; panels
that fall back must equal the wide kernel bit for bit (the same structure with
B given 65,600 rows, which the union kernel never takes).
"""
import numpy as np
import pytest
import torch

import oracle
from unstructured_sparse_linear_csr_amd import binding as sp
from unstructured_sparse_linear_csr_amd import inputs

from gpu_util import DevCsr, check_close, dev, host, note

pytestmark = pytest.mark.gpu

WIDE_K = 65600   # beyond the union kernel's 65,536 rows of B


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sp.lib()
    yield
    torch.cuda.synchronize()


def from_lists(m, k, lists):
    ro = np.zeros(m + 1, np.int64)
    ro[1:] = np.cumsum([len(c) for c in lists])
    ci = (np.concatenate([np.asarray(c, np.int32) for c in lists]) if ro[-1]
          else np.zeros(0, np.int32))
    return DevCsr(m, k, ro.astype(np.int32), ci)


def band_lists(m, k, band, stride):
    """Row i: columns max(0, i - band + 1) .. i and every stride-th column below
    the band (the sparse-attention mask's shape, for any size)."""
    out = []
    for i in range(m):
        cols = set(range(max(0, i - band + 1), min(i + 1, k)))
        cols.update(range(0, min(max(0, i - band + 1), k), stride))
        out.append(sorted(cols))
    return out


def random_lists(seed, n, k, length):
    rng = np.random.default_rng(seed)
    return [sorted(rng.choice(k, size=min(length, k), replace=False).tolist())
            for _ in range(n)]


def run(a: DevCsr, vals, bs, n, shared_values=False, shared_b=False, k=None):
    """sp_spmm_batched over len(bs) entries (C NaN-filled first); returns
    (C, kernel name)."""
    k = a.k if k is None else k
    nb = len(bs)
    v = dev(vals[0] if shared_values else np.stack(vals))
    b = dev(bs[0] if shared_b else np.stack(bs))
    sv = 0 if shared_values else a.nnz
    sb = 0 if shared_b else k * n
    c = torch.full((nb, a.m, n), float("nan"), dtype=torch.float32, device="cuda")
    name = sp.sp_spmm_kernel_name(a.m, k, n, a.nnz, v, a.d_ci, b, c, nb, sv, sb, a.m * n)
    sp.sp_spmm_batched(a.m, k, n, a.nnz, None, v, a.d_ro, a.d_ci, b, c, nb, sv, sb, a.m * n)
    return host(c), name


def check_oracle(a: DevCsr, got, vals, b, what):
    ref, absum = oracle.spmm(a.m, b.shape[0], b.shape[1], a.ro, a.ci, vals, b)
    check_close(got, ref, absum, what)


def test_attention_heads():
    """P V of six attention heads: seq 4096, head dim 64, the 64-token band plus
    every 128th column; P positive (softmax-like), V N(0, 1)."""
    w = inputs.sparse_attention(batch=1, heads=6)
    ro, ci, _ = oracle.csr_from_dense(w["mask"])
    a = DevCsr(w["seq"], w["seq"], ro, ci)
    vals = [np.abs(inputs.random_dense(300 + z, a.nnz)) / 80.0 for z in range(6)]
    note(f"panel-union spmm attention 6 heads nnz={a.nnz}")
    got, name = run(a, vals, list(w["v"]), 64)
    assert name == "panel_union"
    for z in range(6):
        check_oracle(a, got[z], vals[z], w["v"][z], f"head {z}")


@pytest.mark.parametrize("n", [64, 128, 256])
def test_widths(n):
    """Each width the kernel takes; 300 rows (a partial last panel), five batch
    entries (a partial last group of four)."""
    a = from_lists(300, 300, band_lists(300, 300, 24, 50))
    vals = [inputs.random_dense(10 * n + z, a.nnz) for z in range(5)]
    bs = [inputs.random_dense(20 * n + z, a.k, n) for z in range(5)]
    note(f"panel-union spmm n={n} nnz={a.nnz}")
    got, name = run(a, vals, bs, n)
    assert name == "panel_union"
    for z in range(5):
        check_oracle(a, got[z], vals[z], bs[z], f"n={n} entry {z}")


def test_mixed_tile_and_fallback_panels():
    """Rows 0..159 banded (tile path), rows 160..319 of 60 random columns out of
    4,000 (the wide kernel's accumulation), in one launch; the fallback rows
    equal the wide kernel's bit for bit."""
    k = 4000
    lists = band_lists(160, k, 32, 64) + random_lists(5, 160, k, 60)
    a = from_lists(320, k, lists)
    n = 64
    vals = [inputs.random_dense(30 + z, a.nnz) for z in range(4)]
    bs = [inputs.random_dense(40 + z, k, n) for z in range(4)]
    note("panel-union spmm mixed panels")
    got, name = run(a, vals, bs, n)
    assert name == "panel_union"
    wide_bs = [np.concatenate([b, np.zeros((WIDE_K - k, n), np.float32)]) for b in bs]
    ref, wname = run(a, vals, wide_bs, n, k=WIDE_K)
    assert wname == "wide"
    for z in range(4):
        check_oracle(a, got[z], vals[z], bs[z], f"mixed entry {z}")
        assert np.array_equal(got[z][160:].view(np.uint32), ref[z][160:].view(np.uint32)), \
            f"mixed entry {z}: fallback rows differ from the wide kernel"


def test_empty_rows_and_panels():
    """Empty rows inside tiled panels and a whole empty panel are written as
    zeros (C starts NaN-filled)."""
    lists = band_lists(80, 80, 12, 20)
    for i in list(range(16, 32)) + [3, 40, 41, 79]:
        lists[i] = []
    a = from_lists(80, 80, lists)
    n = 128
    vals = [inputs.random_dense(50 + z, a.nnz) for z in range(2)]
    bs = [inputs.random_dense(60 + z, a.k, n) for z in range(2)]
    note("panel-union spmm empty rows")
    got, name = run(a, vals, bs, n)
    assert name == "panel_union"
    for z in range(2):
        assert np.all(got[z][16:32] == 0) and np.all(got[z][[3, 40, 41, 79]] == 0)
        check_oracle(a, got[z], vals[z], bs[z], f"empty rows entry {z}")


def test_non_finite_b_rows():
    """An Inf in one row of B (column 40 of the mask, which rows 40 .. 51 use)
    must not reach the other rows of the panels that load it: 0 x Inf in a tile
    would give NaN where the sparse product is finite."""
    lists = band_lists(96, 96, 12, 1000)
    a = from_lists(96, 96, lists)
    n = 64
    vals = [np.abs(inputs.random_dense(70 + z, a.nnz)) + 0.5 for z in range(2)]
    bs = [inputs.random_dense(80 + z, a.k, n) for z in range(2)]
    bs[1][40, 5] = np.inf
    note("panel-union spmm non-finite B")
    got, name = run(a, vals, bs, n)
    assert name == "panel_union"
    check_oracle(a, got[0], vals[0], bs[0], "finite entry")
    users = [i for i in range(a.m) if 40 in lists[i]]
    others = [i for i in range(a.m) if i not in users]
    assert users == list(range(40, 52))
    assert np.all(np.isposinf(got[1][users, 5]))
    ref, absum = oracle.spmm(a.m, a.k, n, a.ro, a.ci, vals[1], bs[1])
    check_close(got[1][others], ref[others], absum[others], "rows without the Inf")
    keep = [c for c in range(n) if c != 5]
    check_close(got[1][users][:, keep], ref[users][:, keep], absum[users][:, keep],
                "other columns of the rows with the Inf")


@pytest.mark.parametrize("shared", ["values", "b"])
def test_shared_operand(shared):
    a = from_lists(100, 100, band_lists(100, 100, 20, 30))
    n = 64
    vals = [inputs.random_dense(90 + z, a.nnz) for z in range(3)]
    bs = [inputs.random_dense(95 + z, a.k, n) for z in range(3)]
    if shared == "values":
        vals = [vals[0]] * 3
    else:
        bs = [bs[0]] * 3
    note(f"panel-union spmm shared {shared}")
    got, name = run(a, vals, bs, n, shared_values=shared == "values", shared_b=shared == "b")
    assert name == "panel_union"
    for z in range(3):
        check_oracle(a, got[z], vals[z], bs[z], f"shared {shared} entry {z}")


def test_b_row_limit():
    """k = 65,536 rows of B (columns in the bitmap's last word) takes the kernel;
    65,537 does not."""
    k = 65536
    lists = [sorted({i, k - 1 - (i % 3)} | {k - 33 + j for j in range(10)}) for i in range(40)]
    a = from_lists(40, k, lists)
    n = 64
    vals = [inputs.random_dense(100 + z, a.nnz) for z in range(2)]
    bs = [inputs.random_dense(110 + z, k, n) for z in range(2)]
    note("panel-union spmm k = 65536")
    got, name = run(a, vals, bs, n)
    assert name == "panel_union"
    for z in range(2):
        check_oracle(a, got[z], vals[z], bs[z], f"k=65536 entry {z}")
    b = torch.zeros(2, k + 1, n, device="cuda")
    c = torch.zeros(2, a.m, n, device="cuda")
    v = dev(np.stack(vals))
    assert sp.sp_spmm_kernel_name(a.m, k + 1, n, a.nnz, v, a.d_ci, b, c, 2, a.nnz,
                                  (k + 1) * n, a.m * n) == "wide"


def test_not_taken_outside_its_shapes():
    a = from_lists(64, 64, band_lists(64, 64, 8, 16))
    v = dev(np.ones((2, a.nnz), np.float32))
    for n, nb in ((32, 2), (96, 2), (64, 1)):
        b = torch.zeros(nb, a.k, n, device="cuda")
        c = torch.zeros(nb, a.m, n, device="cuda")
        name = sp.sp_spmm_kernel_name(a.m, a.k, n, a.nnz, v, a.d_ci, b, c, nb,
                                      a.nnz if nb > 1 else 0, a.k * n, a.m * n)
        assert name != "panel_union", (n, nb)


def test_deterministic():
    a = from_lists(500, 500, band_lists(500, 500, 40, 60))
    n = 64
    vals = [inputs.random_dense(120 + z, a.nnz) for z in range(4)]
    bs = [inputs.random_dense(130 + z, a.k, n) for z in range(4)]
    note("panel-union spmm determinism")
    g1, _ = run(a, vals, bs, n)
    g2, _ = run(a, vals, bs, n)
    assert np.array_equal(g1.view(np.uint32), g2.view(np.uint32))


@pytest.mark.parametrize("kind,n", [("f16", 64), ("bf16", 64), ("bf16", 128)])
def test_16bit(kind, n):
    """16-bit values and B, widened to fp32 on load (C fp32): rows 0..159 banded
    (tiles), rows 160..319 of 60 random columns (the wide kernel's
    accumulation, bit-equal to the 16-bit wide kernel); the oracle takes the
    decoded values."""
    tdt, code = {"f16": (torch.float16, oracle.F16), "bf16": (torch.bfloat16, oracle.BF16)}[kind]
    k = 3000
    lists = band_lists(160, k, 32, 64) + random_lists(9, 160, k, 60)
    a = from_lists(320, k, lists)

    def to16(x32):
        t = torch.from_numpy(np.ascontiguousarray(x32)).to(tdt)
        vals = oracle.decode16(code, t.view(torch.int16).numpy().view(np.uint16))
        return t.cuda(), vals.astype(np.float32).reshape(x32.shape)

    v16, vals = to16(np.stack([inputs.random_dense(200 + z, a.nnz) for z in range(4)]))
    b16, bs = to16(np.stack([inputs.random_dense(210 + z, k, n) for z in range(4)]))
    c = torch.full((4, a.m, n), float("nan"), device="cuda")
    name = sp.sp_spmm_kernel_name(a.m, k, n, a.nnz, v16, a.d_ci, b16, c, 4, a.nnz, k * n, a.m * n)
    assert name == "panel_union"
    note(f"panel-union spmm {kind} n={n}")
    sp.sp_spmm_ex(a.m, k, n, a.nnz, None, v16, a.d_ro, a.d_ci, b16, c, 4, a.nnz, k * n, a.m * n)
    got = host(c)
    # the wide kernel's reference: B with zero rows appended past 65,536
    bw = torch.zeros(4, WIDE_K, n, dtype=tdt, device="cuda")
    bw[:, :k] = b16
    cw = torch.full((4, a.m, n), float("nan"), device="cuda")
    assert sp.sp_spmm_kernel_name(a.m, WIDE_K, n, a.nnz, v16, a.d_ci, bw, cw, 4, a.nnz,
                                  WIDE_K * n, a.m * n) == "wide"
    sp.sp_spmm_ex(a.m, WIDE_K, n, a.nnz, None, v16, a.d_ro, a.d_ci, bw, cw, 4, a.nnz,
                  WIDE_K * n, a.m * n)
    ref_w = host(cw)
    for z in range(4):
        check_oracle(a, got[z], vals[z], bs[z], f"{kind} n={n} entry {z}")
        assert np.array_equal(got[z][160:].view(np.uint32), ref_w[z][160:].view(np.uint32)), \
            f"{kind} entry {z}: fallback rows differ from the wide kernel"
