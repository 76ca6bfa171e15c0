"""GPU parity of the panel-union one-pass attention (sp_sparse_attention on
batches of fp32 heads of 32 or 64, at most 65,536 keys).

A workgroup takes 16 consecutive query rows and four batch entries, forms the
union of the rows' keys once, and walks it in 16-key tiles: scores and the
weighted sum of V on matrix cores, the online softmax in between (sparse
attention as SDDMM -> row softmax -> SpMM, "Sparse GPU Kernels for Deep
Learning", Sections 5 and 7.3).  The bar is the one-pass attention's bound
against the oracle's double pipeline (check_attention), with one
running-maximum rescaling per tile (at most 16 per panel).  Panels whose rows
share few keys, and waves that load a V value that is not finite, run the
per-row walk: those rows must equal the one-batch call (which never takes this
kernel) bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from unstructured_sparse_linear_csr_amd import binding as sp
from unstructured_sparse_linear_csr_amd import inputs

from gpu_util import DevCsr, check_attention, dev, host, note

pytestmark = pytest.mark.gpu

TILES = 16   # running-maximum rescalings per row at most (16-key tiles of a 256-key union)


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
    out = []
    for i in range(m):
        cols = set(range(max(0, i - band + 1), min(i + 1, k)))
        cols.update(range(0, min(max(0, i - band + 1), k), stride))
        out.append(sorted(cols))
    return out


def attend(a: DevCsr, qs, ks, vs, alpha, ri=None):
    """sp_sparse_attention over len(qs) heads (output NaN-filled first)."""
    nb, d = len(qs), qs[0].shape[1]
    out = torch.full((nb, a.m, d), float("nan"), device="cuda")
    sp.sp_sparse_attention(a.m, a.k, d, a.nnz, ri, a.d_ro, a.d_ci, dev(np.stack(qs)),
                           dev(np.stack(ks)), dev(np.stack(vs)), alpha, out, nb, a.m * d,
                           a.k * d, a.k * d, a.m * d)
    return host(out)


def one_head(a: DevCsr, q, k, v, alpha):
    """The same head alone: the per-row kernel."""
    out = torch.full((a.m, q.shape[1]), float("nan"), device="cuda")
    sp.sp_sparse_attention(a.m, a.k, q.shape[1], a.nnz, None, a.d_ro, a.d_ci, dev(q), dev(k),
                           dev(v), alpha, out)
    return host(out)


def test_attention_heads():
    """Four heads of the sparse-attention workload (seq 4096, head dim 64)."""
    w = inputs.sparse_attention(batch=1, heads=4)
    ro, ci, _ = oracle.csr_from_dense(w["mask"])
    a = DevCsr(w["seq"], w["seq"], ro, ci)
    ri = torch.empty(a.m, dtype=torch.int32, device="cuda")
    sp.sp_row_swizzle(a.m, a.d_ro, ri)
    note(f"panel-union attention 4 heads nnz={a.nnz}")
    got = attend(a, list(w["q"]), list(w["k"]), list(w["v"]), 0.125, ri)
    for z in range(4):
        check_attention(got[z], a.m, a.k, ro, ci, w["q"][z], w["k"][z], w["v"][z], 0.125,
                        f"head {z}", rescalings=TILES)


@pytest.mark.parametrize("d", [32, 64])
def test_depths_and_partial_groups(d):
    """Both head dimensions; 300 rows (a partial last panel), five heads (a
    partial last group of four), scores spread wide (the running maximum rises
    from tile to tile)."""
    a = from_lists(300, 300, band_lists(300, 300, 40, 50))
    qs = [inputs.random_dense(10 * d + z, a.m, d, std=2.0) for z in range(5)]
    ks = [inputs.random_dense(20 * d + z, a.k, d) for z in range(5)]
    vs = [inputs.random_dense(30 * d + z, a.k, d) for z in range(5)]
    alpha = float(np.float32(1.0 / np.sqrt(d)))
    note(f"panel-union attention d={d} nnz={a.nnz}")
    got = attend(a, qs, ks, vs, alpha)
    for z in range(5):
        check_attention(got[z], a.m, a.k, a.ro, a.ci, qs[z], ks[z], vs[z], alpha,
                        f"d={d} head {z}", rescalings=TILES)


def test_mixed_tile_and_per_row_panels():
    """Rows 0..159 banded (tiles), rows 160..319 of 60 random keys out of 4,000
    (the per-row walk, bit-equal to a one-head call), empty rows and an empty
    panel (zero rows)."""
    k, d = 4000, 64
    rng = np.random.default_rng(7)
    lists = band_lists(160, k, 32, 64)
    lists += [sorted(rng.choice(k, 60, replace=False).tolist()) for _ in range(160)]
    for i in list(range(32, 48)) + [5, 170]:
        lists[i] = []
    a = from_lists(320, k, lists)
    qs = [inputs.random_dense(40 + z, a.m, d) for z in range(4)]
    ks = [inputs.random_dense(50 + z, k, d) for z in range(4)]
    vs = [inputs.random_dense(60 + z, k, d) for z in range(4)]
    note("panel-union attention mixed panels")
    got = attend(a, qs, ks, vs, 0.125)
    for z in range(4):
        check_attention(got[z], a.m, a.k, a.ro, a.ci, qs[z], ks[z], vs[z], 0.125,
                        f"mixed head {z}", rescalings=TILES)
        ref = one_head(a, qs[z], ks[z], vs[z], 0.125)
        assert np.array_equal(got[z][160:].view(np.uint32), ref[160:].view(np.uint32)), \
            f"mixed head {z}: per-row panels differ from the one-head call"


def test_non_finite_v():
    """An Inf in V row 40 (key 40, which query rows 40 .. 51 attend to) must not
    reach the other rows of the panels that load it; those panels' rows equal
    the one-head call bit for bit."""
    d = 64
    lists = band_lists(96, 96, 12, 1000)
    a = from_lists(96, 96, lists)
    qs = [inputs.random_dense(70 + z, a.m, d) for z in range(2)]
    ks = [inputs.random_dense(80 + z, a.k, d) for z in range(2)]
    vs = [inputs.random_dense(90 + z, a.k, d) for z in range(2)]
    vs[1][40, 7] = np.inf
    note("panel-union attention non-finite V")
    got = attend(a, qs, ks, vs, 0.125)
    check_attention(got[0], a.m, a.k, a.ro, a.ci, qs[0], ks[0], vs[0], 0.125, "finite head",
                    rescalings=TILES)
    ref = one_head(a, qs[1], ks[1], vs[1], 0.125)
    users = [i for i in range(a.m) if 40 in lists[i]]
    assert users == list(range(40, 52))
    assert np.all(np.isposinf(got[1][users, 7]))
    # panels 2 and 3 (rows 32 .. 63) load key 40: the per-row walk
    assert np.array_equal(got[1][32:64].view(np.uint32), ref[32:64].view(np.uint32))
    others = [i for i in range(a.m) if not 32 <= i < 64]
    assert np.all(np.isfinite(got[1][others]))


def test_key_limit():
    """65,536 keys (keys in the bitmap's last word) take the kernel."""
    k, d = 65536, 32
    lists = [sorted({i, k - 1 - (i % 3)} | {k - 33 + j for j in range(10)}) for i in range(40)]
    a = from_lists(40, k, lists)
    qs = [inputs.random_dense(100 + z, a.m, d) for z in range(2)]
    ks = [inputs.random_dense(110 + z, k, d) for z in range(2)]
    vs = [inputs.random_dense(120 + z, k, d) for z in range(2)]
    note("panel-union attention 65536 keys")
    got = attend(a, qs, ks, vs, 0.25)
    for z in range(2):
        check_attention(got[z], a.m, a.k, a.ro, a.ci, qs[z], ks[z], vs[z], 0.25,
                        f"k=65536 head {z}", rescalings=TILES)


def test_deterministic_and_order_free():
    a = from_lists(500, 500, band_lists(500, 500, 40, 60))
    d = 64
    qs = [inputs.random_dense(130 + z, a.m, d) for z in range(4)]
    ks = [inputs.random_dense(140 + z, a.k, d) for z in range(4)]
    vs = [inputs.random_dense(150 + z, a.k, d) for z in range(4)]
    ri = torch.empty(a.m, dtype=torch.int32, device="cuda")
    sp.sp_row_swizzle(a.m, a.d_ro, ri)
    note("panel-union attention determinism")
    g1 = attend(a, qs, ks, vs, 0.125)
    g2 = attend(a, qs, ks, vs, 0.125, ri)
    assert np.array_equal(g1.view(np.uint32), g2.view(np.uint32))


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_16bit_heads(kind):
    """16-bit Q, K and V (d = 64), widened to fp32 on load: rows 0..159 banded
    (tiles), rows 160..319 of 60 random keys (the per-row walk, bit-equal to a
    one-head call), four heads; the oracle takes the decoded values."""
    tdt, code = {"f16": (torch.float16, oracle.F16), "bf16": (torch.bfloat16, oracle.BF16)}[kind]
    k, d = 2000, 64
    rng = np.random.default_rng(11)
    lists = band_lists(160, k, 32, 64)
    lists += [sorted(rng.choice(k, 60, replace=False).tolist()) for _ in range(160)]
    a = from_lists(320, k, lists)

    def to16(x32):
        t = torch.from_numpy(np.ascontiguousarray(x32)).to(tdt)
        vals = oracle.decode16(code, t.view(torch.int16).numpy().view(np.uint16))
        return t, vals.astype(np.float32).reshape(x32.shape)

    q16, q = to16(np.stack([inputs.random_dense(160 + z, a.m, d) for z in range(4)]))
    k16, kk = to16(np.stack([inputs.random_dense(170 + z, k, d) for z in range(4)]))
    v16, v = to16(np.stack([inputs.random_dense(180 + z, k, d) for z in range(4)]))
    out = torch.full((4, a.m, d), float("nan"), device="cuda")
    note(f"panel-union attention {kind}")
    sp.sp_sparse_attention(a.m, k, d, a.nnz, None, a.d_ro, a.d_ci, q16.cuda(), k16.cuda(),
                           v16.cuda(), 0.125, out, 4, a.m * d, k * d, k * d, a.m * d)
    got = host(out)
    for z in range(4):
        check_attention(got[z], a.m, k, a.ro, a.ci, q[z], kk[z], v[z], 0.125,
                        f"{kind} head {z}", rescalings=TILES)
        one = torch.full((a.m, d), float("nan"), device="cuda")
        sp.sp_sparse_attention(a.m, k, d, a.nnz, None, a.d_ro, a.d_ci, q16[z].cuda(),
                               k16[z].cuda(), v16[z].cuda(), 0.125, one)
        ref = host(one)
        assert np.array_equal(got[z][160:].view(np.uint32), ref[160:].view(np.uint32)), \
            f"{kind} head {z}: per-row panels differ from the one-head call"
