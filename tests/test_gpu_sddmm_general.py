"""GPU parity of the general SDDMM (sp_sddmm_general) against the oracle.

out[p] = alpha * v[p] * (X Yop)[i, col] + beta * out_prior[p], with Y stored
k x d (SP_Y_KD) or d x k (SP_Y_DK).  The tolerance is the stated one,
|gpu - oracle| <= 1e-5 * (|alpha v| sum|x y| + |beta out_prior|), per entry.
alpha and beta are fp32-representable, so both sides scale by the same numbers.
"""
import numpy as np
import pytest
import torch

import oracle
from unstructured_sparse_linear_csr_amd import binding as sp
from unstructured_sparse_linear_csr_amd import inputs

from gpu_util import DevCsr, check_close, csr_of_row_lists, dev, host, note

pytestmark = pytest.mark.gpu

KD, DK = sp.SP_Y_KD, sp.SP_Y_DK


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sp.lib()
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def ffn():
    w = inputs.transformer_ffn()
    return w, csr_of_row_lists(w["a"])


def swizzle(a: DevCsr):
    ri = torch.empty(a.m, dtype=torch.int32, device="cuda")
    sp.sp_row_swizzle(a.m, a.d_ro, ri)
    return ri


def y_in_layout(y_kd, layout):
    return y_kd if layout == KD else np.ascontiguousarray(y_kd.T)


def run_general(a: DevCsr, x, y_kd, layout, mask_values=None, alpha=1.0, beta=0.0,
                prior=None, row_indices=None):
    m, d = x.shape
    if prior is not None:
        out = dev(prior.astype(np.float32))
    else:
        out = torch.full((a.nnz,), float("nan"), dtype=torch.float32, device="cuda")
    mv = None if mask_values is None else dev(mask_values)
    sp.sp_sddmm_general(a.m, a.k, d, a.nnz, row_indices, a.d_ro, a.d_ci, mv, dev(x),
                        dev(y_in_layout(y_kd, layout)), layout, alpha, beta, out)
    return host(out)


def oracle_general(a: DevCsr, x, y_kd, layout, mask_values=None, alpha=1.0, beta=0.0,
                   prior=None):
    return oracle.sddmm_general(a.m, a.k, x.shape[1], a.ro, a.ci, x,
                                y_in_layout(y_kd, layout), layout, mask_values, alpha,
                                beta, prior)


@pytest.mark.parametrize("layout", [KD, DK])
def test_general_transformer_ffn(ffn, layout):
    """Config-2 shapes (mask 2048x512 at 90 %, d = 256), the mask's own values as
    the element-wise scale, accumulating into a prior, swizzled order."""
    w, a = ffn
    prior = inputs.random_dense(71, a.nnz)
    ri = swizzle(a)
    for alpha, beta, pr in [(0.5, 0.0, None), (-1.25, 2.0, prior), (1.0, -1.0, prior)]:
        note(f"sddmm_general ffn layout={layout} alpha={alpha} beta={beta}")
        got = run_general(a, w["x"], w["y"], layout, a.vals, alpha, beta, pr, ri)
        ref, s = oracle_general(a, w["x"], w["y"], layout, a.vals, alpha, beta, pr)
        check_close(got, ref, s, f"general ffn layout={layout} a={alpha} b={beta}")


DEPTHS_DK = [0, 1, 2, 3, 15, 16, 17, 31, 33, 64, 100, 256, 300]


@pytest.mark.parametrize("d", DEPTHS_DK)
def test_general_dk_depths(d):
    """Y stored d x k over depths around the 16-wide unroll, rows longer than
    one 64-entry pass, and empty rows."""
    m, k = 83, 211
    lengths = np.random.default_rng(500 + d).integers(0, 150, m).astype(np.int32)
    lengths[::7] = 0
    rl = inputs.random_row_lists(501 + d, m, k, lengths)
    a = DevCsr(m, k, oracle.csr_offsets_from_lengths(lengths), rl.cols)
    x = inputs.random_dense(502 + d, m, d)
    y = inputs.random_dense(503 + d, k, d)
    mv = inputs.random_dense(504 + d, a.nnz)
    note(f"sddmm_general d x k depth d={d}")
    got = run_general(a, x, y, DK, mv, 0.75, row_indices=swizzle(a))
    ref, s = oracle_general(a, x, y, DK, mv, 0.75)
    check_close(got, ref, s, f"general dk d={d}")
    if d == 1:
        # one product, no scaling: exact
        got1 = run_general(a, x, y, DK)
        ref1, _ = oracle_general(a, x, y, DK)
        assert np.array_equal(got1.view(np.int32), ref1.astype(np.float32).view(np.int32))


@pytest.mark.parametrize("layout", [KD, DK])
def test_general_reduces_to_specialised(ffn, layout):
    """With no mask values and beta = 0 the k x d call is the specialised kernel
    (bit-equal); the d x k call sums in another order and meets the tolerance
    against the same oracle."""
    w, a = ffn
    note(f"sddmm_general vs sp_sddmm layout={layout}")
    spec = torch.empty(a.nnz, device="cuda")
    sp.sp_sddmm(a.m, a.k, w["d"], a.nnz, None, a.d_ro, a.d_ci, dev(w["x"]), dev(w["y"]), spec)
    got = run_general(a, w["x"], w["y"], layout)
    if layout == KD:
        assert np.array_equal(got.view(np.int32), host(spec).view(np.int32))
    ref, s = oracle.sddmm(a.m, a.k, w["d"], a.ro, a.ci, w["x"], w["y"])
    check_close(got, ref, s, f"general plain layout={layout}")


def test_general_beta_zero_never_reads_out():
    m, k, d = 40, 70, 12
    lengths = np.random.default_rng(510).integers(1, 40, m).astype(np.int32)
    rl = inputs.random_row_lists(511, m, k, lengths)
    a = DevCsr(m, k, oracle.csr_offsets_from_lengths(lengths), rl.cols)
    x = inputs.random_dense(512, m, d)
    y = inputs.random_dense(513, k, d)
    for layout in (KD, DK):
        note(f"sddmm_general beta=0 over NaN out layout={layout}")
        nan_prior = np.full(a.nnz, np.nan, np.float32)
        got = run_general(a, x, y, layout, None, 2.0, 0.0, nan_prior)
        ref, s = oracle_general(a, x, y, layout, None, 2.0)
        check_close(got, ref, s, f"beta0 layout={layout}")


def test_general_d0_and_alpha0():
    m, k = 30, 25
    lengths = np.random.default_rng(520).integers(0, 20, m).astype(np.int32)
    rl = inputs.random_row_lists(521, m, k, lengths)
    a = DevCsr(m, k, oracle.csr_offsets_from_lengths(lengths), rl.cols)
    prior = inputs.random_dense(522, a.nnz)
    mv = inputs.random_dense(523, a.nnz)
    for layout in (KD, DK):
        note(f"sddmm_general d=0 beta=0.5 layout={layout}")
        out = dev(prior)
        sp.sp_sddmm_general(m, k, 0, a.nnz, None, a.d_ro, a.d_ci, dev(mv), None, None,
                            layout, 1.0, 0.5, out)
        assert np.array_equal(host(out), prior * np.float32(0.5))
        note(f"sddmm_general alpha=0 layout={layout}")
        x = inputs.random_dense(524, m, 8)
        y = inputs.random_dense(525, k, 8)
        got = run_general(a, x, y, layout, mv, 0.0, 0.25, prior)
        assert np.array_equal(got, prior * np.float32(0.25))


@pytest.mark.parametrize("layout", [KD, DK])
def test_general_batched(layout):
    """Per-batch X, Y, outputs and priors; mask values shared (stride 0) and
    per batch."""
    m, k, d, batch = 61, 47, 20, 3
    lengths = np.random.default_rng(530).integers(0, 47, m).astype(np.int32)
    rl = inputs.random_row_lists(531, m, k, lengths)
    a = DevCsr(m, k, oracle.csr_offsets_from_lengths(lengths), rl.cols)
    xs = inputs.random_dense(532, batch, m, d)
    ys = inputs.random_dense(533, batch, k, d)
    priors = inputs.random_dense(534, batch, a.nnz)
    mvs = inputs.random_dense(535, batch, a.nnz)
    yl = np.stack([y_in_layout(ys[z], layout) for z in range(batch)])
    for shared in (True, False):
        note(f"sddmm_general batched layout={layout} shared_values={shared}")
        out = dev(priors)
        mv = dev(mvs[0]) if shared else dev(mvs)
        sp.sp_sddmm_general(m, k, d, a.nnz, None, a.d_ro, a.d_ci, mv, dev(xs), dev(yl),
                            layout, -0.5, 1.5, out, batch, 0 if shared else a.nnz, m * d,
                            k * d, a.nnz)
        got = host(out)
        for z in range(batch):
            ref, s = oracle_general(a, xs[z], ys[z], layout, mvs[0] if shared else mvs[z],
                                    -0.5, 1.5, priors[z])
            check_close(got[z], ref, s, f"batched layout={layout} z={z}")


def test_general_attention_dk():
    """Sparse-attention scores with K given d x k (its natural transpose-free
    form): S = (Q K^T)/8 at the band+stride mask, 4 of the 32 heads."""
    w = inputs.sparse_attention()
    ro, ci, _ = oracle.csr_from_dense(w["mask"])
    seq, hd, heads = w["seq"], w["head_dim"], 4
    a = DevCsr(seq, seq, ro, ci)
    q, kk = w["q"][:heads], w["k"][:heads]
    kt = np.ascontiguousarray(np.transpose(kk, (0, 2, 1)))
    out = torch.full((heads, a.nnz), float("nan"), device="cuda")
    note("sddmm_general attention d x k, 4 heads")
    sp.sp_sddmm_general(seq, seq, hd, a.nnz, swizzle(a), a.d_ro, a.d_ci, None, dev(q),
                        dev(kt), DK, 0.125, 0.0, out, heads, 0, seq * hd, seq * hd, a.nnz)
    got = host(out)
    for z in range(heads):
        ref, s = oracle.sddmm_general(seq, seq, hd, ro, ci, q[z], kt[z], DK, None, 0.125)
        check_close(got[z], ref, s, f"attention dk head {z}")


@pytest.mark.parametrize("layout", [KD, DK])
def test_general_y_beyond_2gib(layout):
    """Y of 2^23+3 x 65 fp32 (2.2 GB): element offsets beyond buffer reach, so
    both layouts take their 64-bit addressing paths.  Only the columns the mask
    touches hold data; the oracle sees them renumbered densely."""
    k, d, m = (1 << 23) + 3, 65, 48
    rng = np.random.default_rng(540)
    cols = [np.unique(rng.integers(0, k, int(n))) for n in rng.integers(0, 90, m)]
    cols[0] = np.unique(np.append(cols[0], k - 1))  # reach the last column
    lengths = np.array([len(c) for c in cols], np.int32)
    ro = oracle.csr_offsets_from_lengths(lengths)
    ci = np.concatenate(cols).astype(np.int32)
    used = np.unique(ci)
    remap = np.searchsorted(used, ci).astype(np.int32)
    x = inputs.random_dense(541, m, d)
    y_small = inputs.random_dense(542, used.size, d)
    mv = inputs.random_dense(543, ci.size)
    note(f"sddmm_general Y 2.2 GB layout={layout}")
    if layout == KD:
        y_big = torch.zeros((k, d), device="cuda")
        y_big[torch.from_numpy(used).long().cuda()] = dev(y_small)
    else:
        y_big = torch.zeros((d, k), device="cuda")
        y_big[:, torch.from_numpy(used).long().cuda()] = dev(np.ascontiguousarray(y_small.T))
    a = DevCsr(m, k, ro, ci)
    out = torch.full((a.nnz,), float("nan"), device="cuda")
    sp.sp_sddmm_general(m, k, d, a.nnz, None, a.d_ro, a.d_ci, dev(mv), dev(x), y_big,
                        layout, 1.0, 0.0, out)
    got = host(out)
    del y_big
    torch.cuda.empty_cache()
    ref, s = oracle.sddmm_general(m, used.size, d, ro, remap, x, y_in_layout(y_small, layout),
                                  layout, mv)
    check_close(got, ref, s, f"2.2 GB Y layout={layout}")


def test_general_deterministic(ffn):
    w, a = ffn
    ri = swizzle(a)
    for layout in (KD, DK):
        note(f"sddmm_general determinism layout={layout}")
        o1 = run_general(a, w["x"], w["y"], layout, a.vals, 0.5, row_indices=ri)
        o2 = run_general(a, w["x"], w["y"], layout, a.vals, 0.5, row_indices=ri)
        o3 = run_general(a, w["x"], w["y"], layout, a.vals, 0.5)
        assert np.array_equal(o1.view(np.int32), o2.view(np.int32))
        assert np.array_equal(o1.view(np.int32), o3.view(np.int32))
