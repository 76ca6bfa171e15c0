"""GPU parity of the panel-union SDDMM (batched fp32 scores, d a multiple of 4
from 20 to 64, at most 65,536 columns).

A workgroup takes 16 consecutive rows and four batch entries, forms the union
of the rows' columns once, and computes each entry's 16 x U block of X Y^T as
MFMA tiles, storing the mask entries; a panel whose union is too wide for its
entry count runs the multi-row walk instead.  The scores are SDDMM as used for
sparse attention ("Sparse GPU Kernels for Deep Learning", Sections 5 and 7.3).
Tile sums round differently from the per-entry kernels, so the bar is the
stated tolerance against the oracle, |gpu - oracle| <= 1e-5 * sum |x y| per
entry (plus |beta prior| where a prior is accumulated); panels that fall back
must equal sp_sddmm_balanced bit for bit (the multi-row walk sums as the
one-row kernels do).
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


def swizzle(a: DevCsr):
    ri = torch.empty(a.m, dtype=torch.int32, device="cuda")
    sp.sp_row_swizzle(a.m, a.d_ro, ri)
    return ri


def band_csr(m, k, band, stride):
    """Row i: columns max(0, i - band + 1) .. i, and every stride-th column
    below the band (the sparse-attention mask's shape, for any size)."""
    lists = []
    for i in range(m):
        cols = set(range(max(0, i - band + 1), min(i + 1, k)))
        cols.update(range(0, min(max(0, i - band + 1), k), stride))
        lists.append(sorted(cols))
    return from_lists(m, k, lists)


def from_lists(m, k, lists):
    ro = np.zeros(m + 1, np.int64)
    ro[1:] = np.cumsum([len(c) for c in lists])
    ci = np.concatenate([np.asarray(c, np.int32) for c in lists]) if ro[-1] else \
        np.zeros(0, np.int32)
    return DevCsr(m, k, ro.astype(np.int32), ci)


def random_lists(seed, n, k, length):
    rng = np.random.default_rng(seed)
    return [sorted(rng.choice(k, size=min(length, k), replace=False).tolist()) for _ in range(n)]


def run_batched(a: DevCsr, xs, ys, alpha, ri=None, shared_x=False, shared_y=False):
    d = xs[0].shape[1]
    nb = len(xs)
    x = dev(xs[0] if shared_x else np.stack(xs))
    y = dev(ys[0] if shared_y else np.stack(ys))
    sx = 0 if shared_x else a.m * d
    sy = 0 if shared_y else a.k * d
    out = torch.full((nb, a.nnz), float("nan"), dtype=torch.float32, device="cuda")
    name = sp.sp_sddmm_kernel_name(a.m, a.k, d, a.nnz, x, y, nb, sx, sy, a.nnz)
    sp.sp_sddmm_batched(a.m, a.k, d, a.nnz, ri, a.d_ro, a.d_ci, x, y, alpha, out, nb, sx, sy,
                        a.nnz)
    return host(out), name


def check_oracle(a: DevCsr, got, x, y, alpha, what):
    s, s_abs = oracle.sddmm(a.m, a.k, x.shape[1], a.ro, a.ci, x, y)
    check_close(got, alpha * s, abs(alpha) * s_abs, what)


def balanced(a: DevCsr, x, y):
    out = torch.full((a.nnz,), float("nan"), dtype=torch.float32, device="cuda")
    sp.sp_sddmm_balanced(a.m, a.k, x.shape[1], a.nnz, None, a.d_ro, a.d_ci, dev(x), dev(y), out)
    return host(out)


def test_attention_heads():
    """Six heads of the sparse-attention scores (seq 4096, head dim 64, 64-token
    band plus every 128th column), swizzled rows, alpha = 1/8."""
    w = inputs.sparse_attention(batch=1, heads=6)
    ro, ci, _ = oracle.csr_from_dense(w["mask"])
    a = DevCsr(w["seq"], w["seq"], ro, ci)
    note(f"panel-union sddmm attention 6 heads nnz={a.nnz}")
    got, name = run_batched(a, list(w["q"]), list(w["k"]), 0.125, swizzle(a))
    assert name == "panel_union"
    for z in range(6):
        check_oracle(a, got[z], w["q"][z], w["k"][z], 0.125, f"head {z}")


@pytest.mark.parametrize("d", [20, 24, 28, 32, 36, 44, 48, 60, 64])
def test_depths(d):
    """Every depth the kernel takes; 300 rows (a partial last panel), five batch
    entries (a partial last group of four)."""
    a = band_csr(300, 300, 24, 50)
    xs = [inputs.random_dense(10 * d + z, a.m, d) for z in range(5)]
    ys = [inputs.random_dense(20 * d + z, a.k, d) for z in range(5)]
    note(f"panel-union sddmm d={d} nnz={a.nnz}")
    got, name = run_batched(a, xs, ys, 1.0)
    assert name == "panel_union"
    for z in range(5):
        check_oracle(a, got[z], xs[z], ys[z], 1.0, f"d={d} entry {z}")


def test_mixed_tile_and_fallback_panels():
    """Rows 0..159 banded (tile path), rows 160..319 of 60 random columns out of
    4,000 (unions far beyond 256 columns: the multi-row walk), in one launch.
    The fallback panels equal the one-row sums bit for bit."""
    k = 4000
    band = band_csr(160, k, 32, 64)
    lists = [band.ci[band.ro[i]:band.ro[i + 1]].tolist() for i in range(160)]
    lists += random_lists(5, 160, k, 60)
    a = from_lists(320, k, lists)
    d = 64
    xs = [inputs.random_dense(30 + z, a.m, d) for z in range(4)]
    ys = [inputs.random_dense(40 + z, a.k, d) for z in range(4)]
    note("panel-union sddmm mixed panels")
    got, name = run_batched(a, xs, ys, 1.0)
    assert name == "panel_union"
    tail = slice(int(a.ro[160]), a.nnz)
    for z in range(4):
        check_oracle(a, got[z], xs[z], ys[z], 1.0, f"mixed entry {z}")
        ref = balanced(a, xs[z], ys[z])
        assert np.array_equal(got[z][tail].view(np.uint32), ref[tail].view(np.uint32)), \
            f"mixed entry {z}: fallback panels differ from the one-row sums"


@pytest.mark.parametrize("ncols", [255, 256, 257])
def test_union_width_limit(ncols):
    """16 rows sharing the same ncols columns: up to 256 distinct columns the
    panel is tiled, beyond it the panel falls back."""
    k = 3000
    cols = sorted(np.random.default_rng(ncols).choice(k, ncols, replace=False).tolist())
    a = from_lists(16, k, [cols] * 16)
    d = 32
    xs = [inputs.random_dense(50 + z, a.m, d) for z in range(2)]
    ys = [inputs.random_dense(60 + z, a.k, d) for z in range(2)]
    note(f"panel-union sddmm union width {ncols}")
    got, name = run_batched(a, xs, ys, 0.5)
    assert name == "panel_union"
    for z in range(2):
        check_oracle(a, got[z], xs[z], ys[z], 0.5, f"width {ncols} entry {z}")
        if ncols > 256:
            ref = balanced(a, xs[z], ys[z]) * np.float32(0.5)
            assert np.array_equal(got[z].view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("k", [1000, 65536])
def test_bitmap_edges(k):
    """Columns in the bitmap's last word (k not a multiple of 32; k at the
    65,536-column limit), empty panels, rows of one entry, nnz not a multiple
    of 4."""
    lists = []
    for i in range(70):
        if 16 <= i < 32:
            lists.append([])                                  # an empty panel
        elif i % 7 == 0:
            lists.append([k - 1])                             # one entry, the last column
        else:                                                 # 20 shared columns at the end
            lists.append(sorted({i, k - 33} | {k - 1 - j for j in range(20)}))
    a = from_lists(70, k, lists)
    d = 48
    xs = [inputs.random_dense(70 + z, a.m, d) for z in range(3)]
    ys = [inputs.random_dense(80 + z, a.k, d) for z in range(3)]
    note(f"panel-union sddmm bitmap edges k={k} nnz={a.nnz}")
    got, name = run_batched(a, xs, ys, 1.0)
    assert name == "panel_union"
    for z in range(3):
        check_oracle(a, got[z], xs[z], ys[z], 1.0, f"k={k} entry {z}")


def test_beyond_bitmap_takes_multirow():
    a = from_lists(4, 65537, [[0], [65536], [], [5, 6]])
    x = torch.zeros(2, a.m, 64, device="cuda")
    y = torch.zeros(2, a.k, 64, device="cuda")
    assert sp.sp_sddmm_kernel_name(a.m, a.k, 64, a.nnz, x, y, 2, a.m * 64, a.k * 64,
                                   a.nnz) == "multirow"


@pytest.mark.parametrize("shared", ["x", "y"])
def test_shared_operand(shared):
    a = band_csr(100, 100, 20, 30)
    d = 40
    xs = [inputs.random_dense(90 + z, a.m, d) for z in range(3)]
    ys = [inputs.random_dense(95 + z, a.k, d) for z in range(3)]
    if shared == "x":
        xs = [xs[0]] * 3
    else:
        ys = [ys[0]] * 3
    note(f"panel-union sddmm shared {shared}")
    got, name = run_batched(a, xs, ys, 2.0, shared_x=shared == "x", shared_y=shared == "y")
    assert name == "panel_union"
    for z in range(3):
        check_oracle(a, got[z], xs[z], ys[z], 2.0, f"shared {shared} entry {z}")


@pytest.mark.parametrize("beta", [0.0, -1.5])
def test_general_epilogue(beta):
    """sp_sddmm_general on the tile path: mask values, alpha and beta times a
    prior (a NaN prior with beta = 0, never read), two batch entries."""
    a = band_csr(200, 200, 30, 40)
    d = 64
    nb = 2
    x = inputs.random_dense(101, nb, a.m, d)
    y = inputs.random_dense(102, nb, a.k, d)
    mv = inputs.random_dense(103, nb, a.nnz)
    prior = (inputs.random_dense(104, nb, a.nnz) if beta
             else np.full((nb, a.nnz), np.nan, np.float32))
    dx, dy, dmv, out = dev(x), dev(y), dev(mv), dev(prior)
    name = sp.sp_sddmm_kernel_name(a.m, a.k, d, a.nnz, dx, dy, nb, a.m * d, a.k * d, a.nnz,
                                   mask_values=dmv, stride_values=a.nnz, beta=beta)
    assert name == "panel_union"
    note(f"panel-union sddmm general beta={beta}")
    sp.sp_sddmm_general(a.m, a.k, d, a.nnz, None, a.d_ro, a.d_ci, dmv, dx, dy, sp.SP_Y_KD,
                        0.75, beta, out, nb, a.nnz, a.m * d, a.k * d, a.nnz)
    got = host(out)
    for z in range(nb):
        ref, scale = oracle.sddmm_general(a.m, a.k, d, a.ro, a.ci, x[z], y[z], sp.SP_Y_KD,
                                          mv[z], 0.75, beta, prior[z] if beta else None)
        check_close(got[z], ref, scale, f"general beta={beta} entry {z}")


def test_deterministic_and_order_free():
    """Two calls, with and without a row order, give identical bits."""
    a = band_csr(500, 500, 40, 60)
    d = 64
    xs = [inputs.random_dense(110 + z, a.m, d) for z in range(4)]
    ys = [inputs.random_dense(120 + z, a.k, d) for z in range(4)]
    note("panel-union sddmm determinism")
    g1, _ = run_batched(a, xs, ys, 1.0)
    g2, _ = run_batched(a, xs, ys, 1.0, swizzle(a))
    assert np.array_equal(g1.view(np.uint32), g2.view(np.uint32))


@pytest.mark.parametrize("kind,d", [("f16", 64), ("bf16", 64), ("bf16", 128)])
def test_16bit(kind, d):
    """16-bit X and Y widened to fp32 for the tiles: rows 0..159 banded (tiles),
    rows 160..319 of 60 random columns (the multi-row walk, bit-equal to the
    one-row kernel's sums), four batch entries; the oracle on the decoded
    values."""
    tdt, code = {"f16": (torch.float16, oracle.F16), "bf16": (torch.bfloat16, oracle.BF16)}[kind]

    def to16(x32):
        t = torch.from_numpy(np.ascontiguousarray(x32)).to(tdt)
        vals = oracle.decode16(code, t.view(torch.int16).numpy().view(np.uint16))
        return t.cuda(), vals.astype(np.float32).reshape(x32.shape)

    k = 3000
    band = band_csr(160, k, 32, 64)
    lists = [band.ci[band.ro[i]:band.ro[i + 1]].tolist() for i in range(160)]
    lists += random_lists(13, 160, k, 60)
    a = from_lists(320, k, lists)
    x16, x = to16(np.stack([inputs.random_dense(500 + z, a.m, d) for z in range(4)]))
    y16, y = to16(np.stack([inputs.random_dense(510 + z, k, d) for z in range(4)]))
    out = torch.full((4, a.nnz), float("nan"), device="cuda")
    assert sp.sp_sddmm_kernel_name(a.m, k, d, a.nnz, x16, y16, 4, a.m * d, k * d,
                                   a.nnz) == "panel_union"
    note(f"panel-union sddmm {kind} d={d}")
    sp.sp_sddmm_ex(a.m, k, d, a.nnz, None, a.d_ro, a.d_ci, x16, y16, 0.125, out, 4, a.m * d,
                   k * d, a.nnz)
    got = host(out)
    tail = slice(int(a.ro[160]), a.nnz)
    for z in range(4):
        s, s_abs = oracle.sddmm(a.m, k, d, a.ro, a.ci, x[z], y[z])
        check_close(got[z], 0.125 * s, 0.125 * s_abs, f"{kind} d={d} entry {z}")
        one = torch.full((a.nnz,), float("nan"), device="cuda")
        assert sp.sp_sddmm_kernel_name(a.m, k, d, a.nnz, x16[z], y16[z]) == "split"
        sp.sp_sddmm_ex(a.m, k, d, a.nnz, None, a.d_ro, a.d_ci, x16[z], y16[z], 0.125, one)
        ref = host(one)
        assert np.array_equal(got[z][tail].view(np.uint32), ref[tail].view(np.uint32)), \
            f"{kind} entry {z}: fallback panels differ from the one-row sums"


def test_softmax_deep_unions_and_fallback():
    """sp_sddmm_softmax through the union kernel: rows 0..159 of a 200-key band
    (unions of about 215 keys: 14 tiles, the deepest sums), rows 160..319 of 60
    random keys (the row kernel's softmax body, bit-equal to a one-head call),
    three heads; the bound of the row softmax against the oracle."""
    from gpu_util import check_scores_softmax
    k, d = 3000, 64
    lists = [list(range(i, i + 200)) for i in range(160)]   # 200 keys each, shifting by one
    lists += random_lists(17, 160, k, 60)
    a = from_lists(320, k, lists)
    xs = np.stack([inputs.random_dense(600 + z, a.m, d) for z in range(3)])
    ys = np.stack([inputs.random_dense(610 + z, k, d) for z in range(3)])
    x, y = dev(xs), dev(ys)
    out = torch.full((3, a.nnz), float("nan"), device="cuda")
    note("panel-union sddmm softmax")
    sp.sp_sddmm_softmax(a.m, k, d, a.nnz, None, a.d_ro, a.d_ci, x, y, 0.125, out, 3, a.m * d,
                        k * d, a.nnz)
    got = host(out)
    tail = slice(int(a.ro[160]), a.nnz)
    for z in range(3):
        check_scores_softmax(got[z], a.m, k, a.ro, a.ci, xs[z], ys[z], 0.125, f"head {z}")
        one = torch.full((a.nnz,), float("nan"), device="cuda")
        sp.sp_sddmm_softmax(a.m, k, d, a.nnz, None, a.d_ro, a.d_ci, dev(xs[z]), dev(ys[z]),
                            0.125, one)
        ref = host(one)
        assert np.array_equal(got[z][tail].view(np.uint32), ref[tail].view(np.uint32)), \
            f"head {z}: fallback rows differ from the row kernel's softmax"


@pytest.mark.parametrize("ncols", [1, 17, 255, 256, 257])
def test_softmax_union_width(ncols):
    """sp_sddmm_softmax on 16 rows sharing ncols columns, two heads: 2 to 16
    tiles of kept scores (256 columns fill every tile slot); one column (too
    few entries for a tile) and more than 256 take the row kernel's softmax
    body, bit-equal to a one-head call.  Against the oracle within the row
    softmax's bound."""
    from gpu_util import check_scores_softmax
    k, d = 3000, 64
    cols = sorted(np.random.default_rng(70 + ncols).choice(k, ncols, replace=False).tolist())
    a = from_lists(16, k, [cols] * 16)
    xs = np.stack([inputs.random_dense(700 + z, a.m, d) for z in range(2)])
    ys = np.stack([inputs.random_dense(710 + z, k, d) for z in range(2)])
    out = torch.full((2, a.nnz), float("nan"), device="cuda")
    note(f"panel-union sddmm softmax union width {ncols}")
    sp.sp_sddmm_softmax(a.m, k, d, a.nnz, None, a.d_ro, a.d_ci, dev(xs), dev(ys), 0.125, out, 2,
                        a.m * d, k * d, a.nnz)
    got = host(out)
    for z in range(2):
        check_scores_softmax(got[z], a.m, k, a.ro, a.ci, xs[z], ys[z], 0.125,
                             f"width {ncols} head {z}")
        if ncols == 1:
            assert np.all(got[z] == 1.0)
        if ncols == 1 or ncols > 256:
            one = torch.full((a.nnz,), float("nan"), device="cuda")
            sp.sp_sddmm_softmax(a.m, k, d, a.nnz, None, a.d_ro, a.d_ci, dev(xs[z]), dev(ys[z]),
                                0.125, one)
            assert np.array_equal(got[z].view(np.uint32), host(one).view(np.uint32))
