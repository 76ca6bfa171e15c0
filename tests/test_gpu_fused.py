"""GPU checks of sp_spmm_sddmm: one launch carrying an SpMM and an SDDMM must
give exactly (bit for bit) what the two separate entry points give -- the
SpMM as sp_spmm gives it in the natural row order (every row summed in entry
order) -- whether the pair is fused or falls back to two launches, and meet
the oracle's tolerance."""
import numpy as np
import pytest
import torch

import oracle
from unstructured_sparse_linear_csr_amd import binding as sp
from unstructured_sparse_linear_csr_amd import inputs

from gpu_util import check_close, csr_of_row_lists, dev, host, note

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


class Pair:
    """An SpMM problem (csr a, dense b) and an SDDMM problem (mask s, x, y)."""

    def __init__(self, a, b, s, x, y, alpha=1.0, ri_a=None, ri_s=None):
        self.a, self.s = a, s
        self.b, self.x, self.y = b, x, y
        self.alpha = alpha
        self.ri_a, self.ri_s = ri_a, ri_s
        self.n = b.shape[1]
        self.d = x.shape[1]

    def fused(self):
        c = torch.full((self.a.m, self.n), float("nan"), device="cuda")
        out = torch.full((self.s.nnz,), float("nan"), device="cuda")
        sp.sp_spmm_sddmm(self.a.m, self.a.k, self.n, self.a.nnz, self.ri_a, self.a.d_vals,
                         self.a.d_ro, self.a.d_ci, self.b, c, self.s.m, self.s.k, self.d,
                         self.s.nnz, self.ri_s, self.s.d_ro, self.s.d_ci, self.x, self.y,
                         self.alpha, out)
        return host(c), host(out)

    def separate(self):
        # the pair's SpMM sums every row in entry order: sp_spmm's result in
        # the natural row order (row order changes no sum of those kernels)
        c = torch.full((self.a.m, self.n), float("nan"), device="cuda")
        out = torch.full((self.s.nnz,), float("nan"), device="cuda")
        sp.sp_spmm(self.a.m, self.a.k, self.n, self.a.nnz, None, self.a.d_vals,
                   self.a.d_ro, self.a.d_ci, self.b, c)
        sp.sp_sddmm_batched(self.s.m, self.s.k, self.d, self.s.nnz, self.ri_s, self.s.d_ro,
                            self.s.d_ci, self.x, self.y, self.alpha, out, 1, 0, 0, 0)
        return host(c), host(out)

    def check(self, what):
        note(f"spmm_sddmm {what}")
        c1, o1 = self.fused()
        c2, o2 = self.separate()
        assert np.array_equal(c1.view(np.int32), c2.view(np.int32)), f"{what}: C differs"
        assert np.array_equal(o1.view(np.int32), o2.view(np.int32)), f"{what}: out differs"
        return c1, o1


def test_transformer_ffn_pair_and_oracle():
    w = inputs.transformer_ffn()
    a = csr_of_row_lists(w["a"])
    ri = swizzle(a)
    pair = Pair(a, dev(w["b"]), a, dev(w["x"]), dev(w["y"]), 1.0, ri, ri)
    c, out = pair.check("transformer_ffn")
    ref_c, s_c = oracle.spmm(a.m, a.k, w["n"], a.ro, a.ci, a.vals, w["b"])
    check_close(c, ref_c, s_c, "fused spmm ffn")
    ref_o, s_o = oracle.sddmm(a.m, a.k, w["d"], a.ro, a.ci, w["x"], w["y"])
    check_close(out, ref_o, s_o, "fused sddmm ffn")


def test_different_structures():
    """SpMM on the LSTM 90 % matrix, SDDMM on the attention mask (one head)."""
    wl = inputs.lstm(0.9)
    a = csr_of_row_lists(wl["a"])
    wa = inputs.sparse_attention()
    ro, ci, _ = oracle.csr_from_dense(wa["mask"])
    from gpu_util import DevCsr
    s = DevCsr(4096, 4096, ro, ci)
    pair = Pair(a, dev(wl["b"]), s, dev(wa["q"][0]), dev(wa["k"][0]), 0.125, swizzle(a),
                swizzle(s))
    pair.check("lstm spmm + attention sddmm")


@pytest.mark.parametrize("n,d", [(4, 4), (12, 32), (64, 100), (256, 512), (1000, 8)])
def test_widths_and_depths(n, d):
    """Lanes per row 8-64, every SDDMM group size; d = 100 and 512 and n = 1000
    include pairs that are not fused (scalar or generic paths)."""
    m, k = 300, 200
    lengths = np.random.default_rng(700 + n).integers(0, 60, m).astype(np.int32)
    a = csr_of_row_lists(inputs.random_row_lists(701 + n, m, k, lengths))
    pair = Pair(a, dev(inputs.random_dense(702, k, n)), a, dev(inputs.random_dense(703, m, d)),
                dev(inputs.random_dense(704, k, d)), 1.0, swizzle(a), None)
    pair.check(f"n={n} d={d}")


def test_unaligned_falls_back():
    w = inputs.transformer_ffn()
    a = csr_of_row_lists(w["a"])
    yb = torch.zeros(w["k"] * w["d"] + 1, device="cuda")
    yb[1:] = dev(w["y"].reshape(-1))
    pair = Pair(a, dev(w["b"]), a, dev(w["x"]), yb[1:], 1.0, swizzle(a), None)
    pair.check("unaligned y")


def test_one_half_empty():
    w = inputs.tiny()
    ro, ci, v = oracle.csr_from_dense(w["mask"], inputs.random_dense(710, 256, 256))
    from gpu_util import DevCsr
    a = DevCsr(256, 256, ro, ci, v)
    note("spmm_sddmm with an empty SpMM")
    out = torch.full((a.nnz,), float("nan"), device="cuda")
    sp.sp_spmm_sddmm(0, 256, 64, 0, None, None, None, None, None, None, 256, 256, 32, a.nnz,
                     None, a.d_ro, a.d_ci, dev(w["x"]), dev(w["y"]), 1.0, out)
    ref, s = oracle.sddmm(256, 256, 32, ro, ci, w["x"], w["y"])
    check_close(host(out), ref, s, "sddmm alone")
    note("spmm_sddmm with an empty SDDMM")
    c = torch.full((256, 64), float("nan"), device="cuda")
    sp.sp_spmm_sddmm(256, 256, 64, a.nnz, None, a.d_vals, a.d_ro, a.d_ci, dev(w["b"]), c,
                     0, 256, 32, 0, None, None, None, None, None, 1.0, None)
    ref, s = oracle.spmm(256, 256, 64, ro, ci, v, w["b"])
    check_close(host(c), ref, s, "spmm alone")


def test_graph_replays():
    w = inputs.transformer_ffn()
    a = csr_of_row_lists(w["a"])
    ri = swizzle(a)
    b, x, y = dev(w["b"]), dev(w["x"]), dev(w["y"])
    c = torch.empty(a.m, w["n"], device="cuda")
    out = torch.empty(a.nnz, device="cuda")
    fn = lambda: sp.sp_spmm_sddmm(a.m, a.k, w["n"], a.nnz, ri, a.d_vals, a.d_ro, a.d_ci, b, c,
                                  a.m, a.k, w["d"], a.nnz, ri, a.d_ro, a.d_ci, x, y, 1.0, out)
    note("spmm_sddmm eager then graph replays")
    fn()
    c_e, o_e = host(c).copy(), host(out).copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(3):
        c.fill_(float("nan"))
        out.fill_(float("nan"))
        g.replay()
        assert np.array_equal(host(c).view(np.int32), c_e.view(np.int32))
        assert np.array_equal(host(out).view(np.int32), o_e.view(np.int32))
