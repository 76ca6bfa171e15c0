"""GPU parity of sp_sddmm_softmax: the row softmax of alpha * (X Y^T) at a CSR
mask in one pass, against the oracle's double-precision SDDMM and softmax.

Bound per entry (relative to the exact softmax p of the exact scores s):
  2 e_row            the GPU scores' error (|ds| <= e_S = 1e-5 |alpha| sum|x y|,
                     e_row its row maximum) moves a softmax value by a factor
                     within exp(+-2 e_row);
  2 |s|_row 2^-24    the oracle's softmax reads the scores rounded to fp32;
  (x_row + 8) 2^-23  the fp32 softmax itself: exp of s - max rounded to fp32,
                     expf, the row sum and the division (x = |s - max|);
plus an absolute 2^-126: fp32 holds no value below its smallest normal with
relative precision (subnormals lose bits, and may be flushed to zero), so a
probability that small is only known to within it.
"""
import numpy as np
import pytest
import torch

import oracle
from unstructured_sparse_linear_csr_amd import binding as sp
from unstructured_sparse_linear_csr_amd import inputs

from gpu_util import DevCsr, dev, host, note, check_attention, check_scores_softmax

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


def test_attention_heads():
    w = inputs.sparse_attention()
    ro, ci, _ = oracle.csr_from_dense(w["mask"])
    seq, hd = w["seq"], w["head_dim"]
    a = DevCsr(seq, seq, ro, ci)
    heads = [0, 13, 31]
    out = torch.full((len(heads), a.nnz), float("nan"), device="cuda")
    q = dev(np.stack([w["q"][z] for z in heads]))
    kk = dev(np.stack([w["k"][z] for z in heads]))
    note("sddmm_softmax attention 3 heads, batched")
    sp.sp_sddmm_softmax(seq, seq, hd, a.nnz, swizzle(a), a.d_ro, a.d_ci, q, kk, 0.125, out,
                        len(heads), seq * hd, seq * hd, a.nnz)
    got = host(out)
    for i, z in enumerate(heads):
        check_scores_softmax(got[i], seq, seq, ro, ci, w["q"][z], w["k"][z], 0.125,
                             f"attention head {z}")


@pytest.mark.parametrize("case", ["short", "long", "mixed_empty"])
def test_row_lengths(case):
    """Rows within the four register-held windows (<= 256 entries), rows far
    beyond them (their later windows parked in the output), empty rows."""
    rng = np.random.default_rng({"short": 800, "long": 801, "mixed_empty": 802}[case])
    k = 1500
    if case == "short":
        lengths = rng.integers(1, 80, 500)
    elif case == "long":
        lengths = rng.integers(250, 1200, 60)
    else:
        lengths = rng.integers(0, 700, 300)
        lengths[::5] = 0
    lengths = lengths.astype(np.int32)
    m = lengths.size
    rl = inputs.random_row_lists(803, m, k, lengths)
    ro = oracle.csr_offsets_from_lengths(lengths)
    a = DevCsr(m, k, ro, rl.cols)
    x = inputs.random_dense(804, m, 32)
    y = inputs.random_dense(805, k, 32)
    out = torch.full((max(a.nnz, 1),), float("nan"), device="cuda")[:a.nnz]
    note(f"sddmm_softmax rows {case} m={m} nnz={a.nnz}")
    sp.sp_sddmm_softmax(m, k, 32, a.nnz, swizzle(a), a.d_ro, a.d_ci, dev(x), dev(y), 0.5, out)
    check_scores_softmax(host(out), m, k, ro, rl.cols, x, y, 0.5, f"rows {case}")


@pytest.mark.parametrize("d", [0, 1, 7, 64, 100, 600])
def test_depths_and_order(d):
    """Every row kernel variant (d = 0 gives uniform rows); results do not
    depend on the row order."""
    m, k = 150, 90
    lengths = np.random.default_rng(810 + d).integers(0, 90, m).astype(np.int32)
    rl = inputs.random_row_lists(811 + d, m, k, lengths)
    ro = oracle.csr_offsets_from_lengths(lengths)
    a = DevCsr(m, k, ro, rl.cols)
    x = inputs.random_dense(812 + d, m, d)
    y = inputs.random_dense(813 + d, k, d)
    o1 = torch.full((a.nnz,), float("nan"), device="cuda")
    o2 = torch.full((a.nnz,), float("nan"), device="cuda")
    note(f"sddmm_softmax d={d}")
    sp.sp_sddmm_softmax(m, k, d, a.nnz, swizzle(a), a.d_ro, a.d_ci, dev(x), dev(y), 1.0, o1)
    sp.sp_sddmm_softmax(m, k, d, a.nnz, None, a.d_ro, a.d_ci, dev(x), dev(y), 1.0, o2)
    g1, g2 = host(o1), host(o2)
    assert np.array_equal(g1.view(np.int32), g2.view(np.int32))
    if d == 0:
        want = np.repeat(1.0 / np.maximum(lengths, 1), lengths).astype(np.float32)
        assert np.array_equal(g1, want)
    else:
        check_scores_softmax(g1, m, k, ro, rl.cols, x, y, 1.0, f"d={d}")


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_attention_16bit(kind):
    tdt, code = {"f16": (torch.float16, oracle.F16), "bf16": (torch.bfloat16, oracle.BF16)}[kind]
    w = inputs.sparse_attention()
    ro, ci, _ = oracle.csr_from_dense(w["mask"])
    seq, hd = w["seq"], w["head_dim"]
    a = DevCsr(seq, seq, ro, ci)
    q16 = torch.from_numpy(w["q"][5]).to(tdt)
    k16 = torch.from_numpy(w["k"][5]).to(tdt)
    q = oracle.decode16(code, q16.view(torch.int16).numpy().view(np.uint16)).astype(np.float32)
    kk = oracle.decode16(code, k16.view(torch.int16).numpy().view(np.uint16)).astype(np.float32)
    out = torch.full((a.nnz,), float("nan"), device="cuda")
    note(f"sddmm_softmax attention {kind}")
    sp.sp_sddmm_softmax(seq, seq, hd, a.nnz, swizzle(a), a.d_ro, a.d_ci, q16.cuda(), k16.cuda(),
                        0.125, out)
    check_scores_softmax(host(out), seq, seq, ro, ci, q, kk, 0.125, f"attention {kind}")


def test_all_device_attention_fused_scores():
    """softmax(Q K^T / 8) V with the scores and softmax in one pass, then the
    SpMM; within the propagated bound of the oracle's double pipeline."""
    w = inputs.sparse_attention()
    ro, ci, _ = oracle.csr_from_dense(w["mask"])
    seq, hd = w["seq"], w["head_dim"]
    a = DevCsr(seq, seq, ro, ci)
    z = 21
    ri = swizzle(a)
    p_dev = torch.empty(a.nnz, device="cuda")
    o_dev = torch.empty(seq, hd, device="cuda")
    note("attention: sddmm_softmax then spmm")
    sp.sp_sddmm_softmax(seq, seq, hd, a.nnz, ri, a.d_ro, a.d_ci, dev(w["q"][z]), dev(w["k"][z]),
                        0.125, p_dev)
    sp.sp_spmm(seq, seq, hd, a.nnz, ri, p_dev, a.d_ro, a.d_ci, dev(w["v"][z]), o_dev)
    o_gpu = host(o_dev)
    s, s_abs = oracle.sddmm(seq, seq, hd, ro, ci, w["q"][z], w["k"][z])
    s, e_s = 0.125 * s, 0.125 * 1e-5 * s_abs
    p_ref = oracle.softmax_rows(ro, s.astype(np.float32))
    rows = np.repeat(np.arange(seq), np.diff(ro))
    e_row = np.zeros(seq)
    np.maximum.at(e_row, rows, e_s)
    smax = np.full(seq, -np.inf)
    np.maximum.at(smax, rows, s)
    x_row = np.zeros(seq)
    np.maximum.at(x_row, rows, np.abs(s - smax[rows]))
    a_row = np.zeros(seq)
    np.maximum.at(a_row, rows, np.abs(s))
    rel = 2.0 * e_row + 2.0 * a_row * 2.0 ** -24 + (x_row + 8.0) * 2.0 ** -23 + 1e-5
    o_ref, _ = oracle.spmm(seq, seq, hd, ro, ci, p_ref, w["v"][z])
    pv, _ = oracle.spmm(seq, seq, hd, ro, ci, p_ref, np.abs(w["v"][z]))
    err = np.abs(o_gpu.astype(np.float64) - o_ref)
    assert np.all(err <= rel[:, None] * pv * 1.01 + 2.0 ** -126)


# ---------------------------------------------------------------- one-pass attention

def test_sparse_attention_heads():
    w = inputs.sparse_attention()
    ro, ci, _ = oracle.csr_from_dense(w["mask"])
    seq, hd = w["seq"], w["head_dim"]
    a = DevCsr(seq, seq, ro, ci)
    heads = [3, 30]
    q = dev(np.stack([w["q"][z] for z in heads]))
    kk = dev(np.stack([w["k"][z] for z in heads]))
    v = dev(np.stack([w["v"][z] for z in heads]))
    out = torch.full((len(heads), seq, hd), float("nan"), device="cuda")
    note("sparse_attention 2 heads batched")
    sp.sp_sparse_attention(seq, seq, hd, a.nnz, swizzle(a), a.d_ro, a.d_ci, q, kk, v, 0.125,
                           out, len(heads), seq * hd, seq * hd, seq * hd, seq * hd)
    got = host(out)
    # a batch of fp32 heads of 64 takes the panel-union kernel: one running-
    # maximum rescaling per 16-key tile, at most 16 tiles per panel
    for i, z in enumerate(heads):
        check_attention(got[i], seq, seq, ro, ci, w["q"][z], w["k"][z], w["v"][z], 0.125,
                        f"attention head {z}", rescalings=16)


@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_sparse_attention_dims_and_lengths(d):
    """Every head dimension; rows of 1 to 700 entries (several windows, the
    running maximum rising from window to window), empty rows; the result does
    not depend on the row order."""
    rng = np.random.default_rng(820 + d)
    m, k = 240, 900
    lengths = rng.integers(0, 700, m).astype(np.int32)
    lengths[::9] = 0
    lengths[1::9] = 1
    rl = inputs.random_row_lists(821 + d, m, k, lengths)
    ro = oracle.csr_offsets_from_lengths(lengths)
    a = DevCsr(m, k, ro, rl.cols)
    q = inputs.random_dense(822 + d, m, d)
    kk = inputs.random_dense(823 + d, k, d)
    v = inputs.random_dense(824 + d, k, d)
    alpha = float(np.float32(1.0 / np.sqrt(d)))
    o1 = torch.full((m, d), float("nan"), device="cuda")
    o2 = torch.full((m, d), float("nan"), device="cuda")
    note(f"sparse_attention d={d}")
    sp.sp_sparse_attention(m, k, d, a.nnz, swizzle(a), a.d_ro, a.d_ci, dev(q), dev(kk), dev(v),
                           alpha, o1)
    sp.sp_sparse_attention(m, k, d, a.nnz, None, a.d_ro, a.d_ci, dev(q), dev(kk), dev(v),
                           alpha, o2)
    g1 = host(o1)
    assert np.array_equal(g1.view(np.int32), host(o2).view(np.int32))
    check_attention(g1, m, k, ro, rl.cols, q, kk, v, alpha, f"d={d}")


@pytest.mark.parametrize("kind,d", [("f16", 64), ("f16", 128), ("bf16", 64), ("bf16", 512)])
def test_sparse_attention_16bit(kind, d):
    tdt, code = {"f16": (torch.float16, oracle.F16), "bf16": (torch.bfloat16, oracle.BF16)}[kind]
    m, k = 300, 500
    lengths = np.random.default_rng(830 + d).integers(0, 300, m).astype(np.int32)
    rl = inputs.random_row_lists(831 + d, m, k, lengths)
    ro = oracle.csr_offsets_from_lengths(lengths)
    a = DevCsr(m, k, ro, rl.cols)

    def to16(a32):
        t = torch.from_numpy(a32).to(tdt)
        vals = oracle.decode16(code, t.view(torch.int16).numpy().view(np.uint16))
        return t.cuda(), vals.astype(np.float32)

    q16, q = to16(inputs.random_dense(832 + d, m, d))
    k16, kk = to16(inputs.random_dense(833 + d, k, d))
    v16, v = to16(inputs.random_dense(834 + d, k, d))
    out = torch.full((m, d), float("nan"), device="cuda")
    note(f"sparse_attention {kind} d={d}")
    sp.sp_sparse_attention(m, k, d, a.nnz, swizzle(a), a.d_ro, a.d_ci, q16, k16, v16, 0.0625,
                           out)
    check_attention(host(out), m, k, ro, rl.cols, q, kk, v, 0.0625, f"{kind} d={d}")


def test_sparse_attention_unsupported_shape():
    w = inputs.tiny()
    ro, ci, _ = oracle.csr_from_dense(w["mask"])
    a = DevCsr(256, 256, ro, ci)
    x = dev(inputs.random_dense(840, 256, 48))
    out = torch.empty(256, 48, device="cuda")
    note("sparse_attention d=48 rejected")
    with pytest.raises(sp.SpError) as err:
        sp.sp_sparse_attention(256, 256, 48, a.nnz, None, a.d_ro, a.d_ci, x, x, x, 1.0, out)
    assert err.value.status == sp.SP_ERROR_NOT_SUPPORTED
