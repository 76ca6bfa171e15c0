"""GPU parity of the mixed-precision entry points (sp_spmm_ex, sp_sddmm_ex).

Seeded fp32 draws are rounded once to binary16 / bfloat16 (torch's CPU
conversion, input preparation shared by both sides); the GPU gets those bits,
the oracle gets their values decoded by its own binary16/bfloat16 decoder.
Every 16-bit value is exactly an fp32 value and a product of two is exact in
fp32, so the stated fp32 tolerance applies unchanged:
|gpu - oracle| <= 1e-5 * sum|a*b| per output element.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
from unstructured_sparse_linear_csr_amd import binding as sp
from unstructured_sparse_linear_csr_amd import inputs

from gpu_util import check_close, host, note

pytestmark = pytest.mark.gpu

KINDS = {"f16": (torch.float16, oracle.F16), "bf16": (torch.bfloat16, oracle.BF16)}


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sp.lib()
    yield
    torch.cuda.synchronize()


def to16(a32, kind):
    """(device tensor of the 16-bit type, fp32 values of those bits per the oracle)."""
    tdt, code = KINDS[kind]
    t = torch.from_numpy(np.ascontiguousarray(a32, np.float32)).to(tdt)
    bits = t.view(torch.int16).numpy().view(np.uint16)
    vals = oracle.decode16(code, bits)
    assert np.all(np.isfinite(vals))
    return t.to("cuda"), vals.astype(np.float32)


def devi(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to("cuda")


def swizzle(m, d_ro):
    ri = torch.empty(m, dtype=torch.int32, device="cuda")
    sp.sp_row_swizzle(m, d_ro, ri)
    return ri


def spmm16(kind, m, k, n, ro, ci, vals32, b32, swz=True, c_offset=0):
    """sp_spmm_ex on 16-bit copies of the values and B; C starts c_offset
    floats into its allocation (c_offset = 1: only 4-byte aligned)."""
    d_v, v = to16(vals32, kind)
    d_b, b = to16(b32, kind)
    d_ro = devi(ro)
    c_buf = torch.full((m * n + c_offset,), float("nan"), device="cuda")
    c = c_buf[c_offset:].view(m, n)
    sp.sp_spmm_ex(m, k, n, ci.size, swizzle(m, d_ro) if swz else None, d_v, d_ro,
                  devi(ci), d_b, c)
    return host(c), v, b


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_spmm_transformer_ffn(kind):
    w = inputs.transformer_ffn()
    a = w["a"]
    ro = oracle.csr_offsets_from_lengths(a.lengths)
    note(f"spmm_ex {kind} transformer_ffn")
    c, v, b = spmm16(kind, a.m, a.k, w["n"], ro, a.cols, a.values, w["b"])
    ref, s = oracle.spmm(a.m, a.k, w["n"], ro, a.cols, v, b)
    check_close(c, ref, s, f"spmm {kind} ffn")


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_sddmm_transformer_ffn(kind):
    w = inputs.transformer_ffn()
    a = w["a"]
    ro = oracle.csr_offsets_from_lengths(a.lengths)
    d_x, x = to16(w["x"], kind)
    d_y, y = to16(w["y"], kind)
    d_ro = devi(ro)
    out = torch.full((a.nnz,), float("nan"), device="cuda")
    note(f"sddmm_ex {kind} transformer_ffn")
    sp.sp_sddmm_ex(a.m, a.k, w["d"], a.nnz, swizzle(a.m, d_ro), d_ro, devi(a.cols), d_x, d_y,
                   1.0, out)
    ref, s = oracle.sddmm(a.m, a.k, w["d"], ro, a.cols, x, y)
    check_close(host(out), ref, s, f"sddmm {kind} ffn")


WIDTHS = [1, 3, 8, 16, 24, 40, 64, 100, 256, 264, 520]


@pytest.mark.parametrize("n", WIDTHS)
@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_spmm_widths(kind, n):
    m, k = 97, 150
    lengths = np.random.default_rng(600 + n).integers(0, 70, m).astype(np.int32)
    rl = inputs.random_row_lists(601 + n, m, k, lengths)
    ro = oracle.csr_offsets_from_lengths(lengths)
    b32 = inputs.random_dense(602 + n, k, n)
    note(f"spmm_ex {kind} n={n}")
    c, v, b = spmm16(kind, m, k, n, ro, rl.cols, rl.values, b32)
    ref, s = oracle.spmm(m, k, n, ro, rl.cols, v, b)
    check_close(c, ref, s, f"spmm {kind} n={n}")


DEPTHS = [1, 7, 8, 16, 24, 64, 100, 128, 256, 520, 1032, 2056]


@pytest.mark.parametrize("d", DEPTHS)
@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_sddmm_depths(kind, d):
    m, k = 77, 130
    lengths = np.random.default_rng(610 + d).integers(0, 100, m).astype(np.int32)
    rl = inputs.random_row_lists(611 + d, m, k, lengths)
    ro = oracle.csr_offsets_from_lengths(lengths)
    d_x, x = to16(inputs.random_dense(612 + d, m, d), kind)
    d_y, y = to16(inputs.random_dense(613 + d, k, d), kind)
    d_ro = devi(ro)
    out = torch.full((rl.cols.size,), float("nan"), device="cuda")
    note(f"sddmm_ex {kind} d={d}")
    sp.sp_sddmm_ex(m, k, d, rl.cols.size, swizzle(m, d_ro), d_ro, devi(rl.cols), d_x, d_y,
                   0.5, out)
    ref, s = oracle.sddmm(m, k, d, ro, rl.cols, x, y)
    check_close(host(out), 0.5 * ref, 0.5 * s, f"sddmm {kind} d={d}")
    if d == 1:
        # one exact product, scaled by a power of two
        assert np.array_equal(host(out), (0.5 * ref).astype(np.float32))


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_spmm_identity_and_unaligned(kind):
    """A = I: C is B widened to fp32, bit for bit.  Then the same product with
    B, values and C one element off 16-byte alignment (the scalar path)."""
    k = n = 264
    ro = np.arange(k + 1, dtype=np.int32)
    ci = np.arange(k, dtype=np.int32)
    b32 = inputs.random_dense(620, k, n)
    note(f"spmm_ex {kind} identity")
    c, v, b = spmm16(kind, k, k, n, ro, ci, np.ones(k, np.float32), b32)
    assert np.array_equal(c.view(np.int32), b.view(np.int32))
    note(f"spmm_ex {kind} unaligned")
    tdt, _ = KINDS[kind]
    d_b, b = to16(b32, kind)
    d_v, v = to16(inputs.random_dense(621, k), kind)
    bb = torch.zeros(k * n + 1, dtype=tdt, device="cuda")
    bb[1:] = d_b.reshape(-1)
    vv = torch.zeros(k + 1, dtype=tdt, device="cuda")
    vv[1:] = d_v
    cc = torch.full((k * n + 1,), float("nan"), device="cuda")
    sp.sp_spmm_ex(k, k, n, k, None, vv[1:], devi(ro), devi(ci), bb[1:], cc[1:])
    ref, s = oracle.spmm(k, k, n, ro, ci, v, b)
    check_close(host(cc[1:]).reshape(k, n), ref, s, f"spmm {kind} unaligned")


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_lstm_whole(kind):
    w = inputs.lstm(0.9)
    a = w["a"]
    ro = oracle.csr_offsets_from_lengths(a.lengths)
    note(f"spmm_ex {kind} lstm 90%")
    c, v, b = spmm16(kind, a.m, a.k, w["n"], ro, a.cols, a.values, w["b"])
    ref, s = oracle.spmm(a.m, a.k, w["n"], ro, a.cols, v, b)
    check_close(c, ref, s, f"spmm {kind} lstm")


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_attention_batched(kind):
    """Scores and weighted sum of 4 heads in 16-bit operands, batched."""
    w = inputs.sparse_attention()
    ro, ci, _ = oracle.csr_from_dense(w["mask"])
    seq, hd, heads = w["seq"], w["head_dim"], 4
    nnz = ci.size
    d_q, q = to16(w["q"][:heads], kind)
    d_k, kk = to16(w["k"][:heads], kind)
    d_ro, d_ci = devi(ro), devi(ci)
    ri = swizzle(seq, d_ro)
    s_out = torch.full((heads, nnz), float("nan"), device="cuda")
    note(f"sddmm_ex {kind} attention 4 heads")
    sp.sp_sddmm_ex(seq, seq, hd, nnz, ri, d_ro, d_ci, d_q, d_k, 0.125, s_out, heads,
                   seq * hd, seq * hd, nnz)
    got = host(s_out)
    for z in range(heads):
        ref, s = oracle.sddmm(seq, seq, hd, ro, ci, q[z], kk[z])
        check_close(got[z], 0.125 * ref, 0.125 * s, f"attention scores {kind} head {z}")
    # P V with P rounded to the 16-bit type
    p32 = np.random.default_rng(640).random((heads, nnz)).astype(np.float32) / 80
    d_p, p = to16(p32, kind)
    d_vv, vv = to16(w["v"][:heads], kind)
    o = torch.full((heads, seq, hd), float("nan"), device="cuda")
    note(f"spmm_ex {kind} attention 4 heads")
    sp.sp_spmm_ex(seq, seq, hd, nnz, ri, d_p, d_ro, d_ci, d_vv, o, heads, nnz, seq * hd,
                  seq * hd)
    got = host(o)
    for z in range(heads):
        ref, s = oracle.spmm(seq, seq, hd, ro, ci, p[z], vv[z])
        check_close(got[z], ref, s, f"attention output {kind} head {z}")


def test_f32_dtype_is_the_fp32_path():
    w = inputs.transformer_ffn()
    a = w["a"]
    ro = oracle.csr_offsets_from_lengths(a.lengths)
    d_ro, d_ci = devi(ro), devi(a.cols)
    v = torch.from_numpy(a.values).cuda()
    b = torch.from_numpy(w["b"]).cuda()
    ri = swizzle(a.m, d_ro)
    c1 = torch.empty(a.m, w["n"], device="cuda")
    c2 = torch.empty(a.m, w["n"], device="cuda")
    note("spmm_ex f32 vs sp_spmm")
    sp.sp_spmm(a.m, a.k, w["n"], a.nnz, ri, v, d_ro, d_ci, b, c1)
    sp.sp_spmm_ex(a.m, a.k, w["n"], a.nnz, ri, v, d_ro, d_ci, b, c2)
    assert torch.equal(c1, c2)


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_spmm_b_beyond_2gib(kind):
    """B of (2^21 + 5) x 520 16-bit elements (2.2 GB): byte offsets beyond
    buffer reach, so the 64-bit path runs.  Only the rows the matrix touches
    hold data; the oracle sees them renumbered densely."""
    k, n, m = (1 << 21) + 5, 520, 40
    tdt, _ = KINDS[kind]
    rng = np.random.default_rng(650)
    cols = [np.unique(rng.integers(0, k, int(c))) for c in rng.integers(0, 60, m)]
    cols[0] = np.unique(np.append(cols[0], k - 1))
    lengths = np.array([len(c) for c in cols], np.int32)
    ro = oracle.csr_offsets_from_lengths(lengths)
    ci = np.concatenate(cols).astype(np.int32)
    used = np.unique(ci)
    remap = np.searchsorted(used, ci).astype(np.int32)
    d_bs, b_small = to16(inputs.random_dense(651, used.size, n), kind)
    d_v, v = to16(inputs.random_dense(652, ci.size), kind)
    note(f"spmm_ex {kind} B 2.2 GB")
    b_big = torch.zeros((k, n), dtype=tdt, device="cuda")
    b_big[torch.from_numpy(used).long().cuda()] = d_bs
    c = torch.full((m, n), float("nan"), device="cuda")
    sp.sp_spmm_ex(m, k, n, ci.size, None, d_v, devi(ro), devi(ci), b_big, c)
    got = host(c)
    del b_big
    torch.cuda.empty_cache()
    ref, s = oracle.spmm(m, used.size, n, ro, remap, v, b_small)
    check_close(got, ref, s, f"spmm {kind} 2.2 GB B")


# ------------------------------------------------------ the streaming (LDS) kernel
# Narrow 16-bit B with many entries per B element takes the streaming kernel:
# B widened to fp32 in LDS, values read as 2-byte loads and widened.

@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 16, 24, 32])
@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_spmm_lds_resident_b(kind, n):
    # enough rows that every width takes the streaming kernel: it needs at
    # least (256 CUs) * k * n entries, i.e. 65,536 * n here (rows average 160)
    k = 256
    m = max(8192, (65536 * n * 5 // 4) // 160)
    lengths = np.random.default_rng(700 + n).integers(100, 220, m).astype(np.int32)
    lengths[::97] = 0                                   # some empty rows
    # nnz = 3 (mod 4) with a non-empty last row: the array's final segment
    # extends past nnz (read from its last 4 entries), and nnz is odd
    lengths[-1] += (3 - int(lengths.sum()) % 4) % 4
    assert int(lengths.sum()) % 4 == 3 and lengths[-1] > 0
    rl = inputs.random_row_lists(701 + n, m, k, lengths)
    ro = oracle.csr_offsets_from_lengths(lengths)
    b32 = inputs.random_dense(702 + n, k, n)
    note(f"spmm_ex {kind} lds-resident B n={n} nnz={rl.cols.size}")
    c, v, b = spmm16(kind, m, k, n, ro, rl.cols, rl.values, b32)
    ref, s = oracle.spmm(m, k, n, ro, rl.cols, v, b)
    check_close(c, ref, s, f"spmm {kind} lds n={n}")
    # one-entry rows through the same kernel: one exact product each (the
    # streaming kernel needs at least 256 CUs * k * n entries)
    m1 = 66000 * n + 4000
    rl1 = inputs.random_row_lists(703 + n, m1, k, np.ones(m1, np.int32))
    ro1 = oracle.csr_offsets_from_lengths(rl1.lengths)
    note(f"spmm_ex {kind} lds-resident B one-entry rows n={n}")
    c1, v1, b1 = spmm16(kind, m1, k, n, ro1, rl1.cols, rl1.values, b32, swz=False)
    want = (v1.astype(np.float64)[:, None] * b1.astype(np.float64)[rl1.cols]).astype(np.float32)
    assert np.array_equal(c1, want)


@pytest.mark.parametrize("kind", ["f16", "bf16"])
@pytest.mark.parametrize("k,n,m", [(8192, 8, 16384), (8192, 12, 10000)])
def test_spmm_lds_column_slices(kind, k, n, m):
    # B of k x n does not fit in LDS as fp32: column slices (8 + 4 columns for n = 12)
    lengths = np.random.default_rng(710 + n).integers(300, 700, m).astype(np.int32)
    rl = inputs.random_row_lists(711 + n, m, k, lengths)
    ro = oracle.csr_offsets_from_lengths(lengths)
    b32 = inputs.random_dense(712 + n, k, n)
    note(f"spmm_ex {kind} lds column slices k={k} n={n} m={m} nnz={rl.cols.size}")
    c, v, b = spmm16(kind, m, k, n, ro, rl.cols, rl.values, b32)
    ref, s = oracle.spmm(m, k, n, ro, rl.cols, v, b)
    check_close(c, ref, s, f"spmm {kind} lds slices k={k} n={n}")


@functools.lru_cache(maxsize=1)
def _hbm_stream_n4():
    return inputs.hbm_stream(n=4)   # 53.7 M entries: built once for both kinds


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_spmm_hbm_stream_n4_whole(kind):
    w = _hbm_stream_n4()
    a = w["a"]
    ro = oracle.csr_offsets_from_lengths(a.lengths)
    note(f"spmm_ex {kind} hbm_stream 65536x8192x4 (B in LDS)")
    c, v, b = spmm16(kind, w["m"], w["k"], w["n"], ro, a.cols, a.values, w["b"], swz=False)
    ref, s = oracle.spmm(w["m"], w["k"], w["n"], ro, a.cols, v, b)
    check_close(c, ref, s, f"spmm {kind} hbm_stream n=4")


@pytest.mark.parametrize("tail", [0, 1, 2, 3])
@pytest.mark.parametrize("n", [1, 4, 8, 16])
@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_spmm_lds_array_end(kind, n, tail):
    # nnz = tail (mod 4) with the last row non-empty: the array's last segment
    # holds `tail` entries (4 when 0), its other words outside the buffers'
    # ranges; with an odd nnz the value range ends 2 bytes past the array
    m, k = 8192, 256
    lengths = np.random.default_rng(730 + tail).integers(100, 220, m).astype(np.int32)
    lengths[-1] += (tail - int(lengths.sum()) % 4) % 4
    assert int(lengths.sum()) % 4 == tail and lengths[-1] > 0
    rl = inputs.random_row_lists(731 + tail, m, k, lengths)
    ro = oracle.csr_offsets_from_lengths(lengths)
    b32 = inputs.random_dense(732 + n, k, n)
    note(f"spmm_ex {kind} lds array end n={n} nnz%4={tail}")
    c, v, b = spmm16(kind, m, k, n, ro, rl.cols, rl.values, b32, swz=False)
    ref, s = oracle.spmm(m, k, n, ro, rl.cols, v, b)
    check_close(c, ref, s, f"spmm {kind} lds array end n={n} tail={tail}")


@pytest.mark.parametrize("n", [4, 12])
@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_spmm_lds_misaligned_c(kind, n):
    # 16-bit B widened to fp32 vectors of 4 in LDS stores C in vectors of 4 too:
    # a C that is only 4-byte aligned must take the element-wise form instead
    m, k = 8192, 256
    lengths = np.random.default_rng(760 + n).integers(100, 220, m).astype(np.int32)
    rl = inputs.random_row_lists(761 + n, m, k, lengths)
    ro = oracle.csr_offsets_from_lengths(lengths)
    b32 = inputs.random_dense(762 + n, k, n)
    note(f"spmm_ex {kind} lds misaligned C n={n} nnz={rl.cols.size}")
    c, v, b = spmm16(kind, m, k, n, ro, rl.cols, rl.values, b32, c_offset=1)
    ref, s = oracle.spmm(m, k, n, ro, rl.cols, v, b)
    check_close(c, ref, s, f"spmm {kind} lds misaligned C n={n}")


@pytest.mark.parametrize("kind", ["f16", "bf16"])
@pytest.mark.parametrize("k,n,m", [(8192, 16, 16000), (8192, 24, 10000), (8192, 32, 8000)])
def test_spmm_lds_16bit_b_column_slices(kind, k, n, m):
    # n % 8 == 0: B kept 16-bit in LDS, 8 columns per vector; B of k x n in 2,
    # 3 and 4 column slices of 8 (enough entries for the streaming kernel)
    lengths = np.random.default_rng(740 + n).integers(300, 900, m).astype(np.int32)
    rl = inputs.random_row_lists(741 + n, m, k, lengths)
    ro = oracle.csr_offsets_from_lengths(lengths)
    b32 = inputs.random_dense(742 + n, k, n)
    note(f"spmm_ex {kind} 16-bit B in LDS, slices k={k} n={n} m={m} nnz={rl.cols.size}")
    c, v, b = spmm16(kind, m, k, n, ro, rl.cols, rl.values, b32)
    ref, s = oracle.spmm(m, k, n, ro, rl.cols, v, b)
    check_close(c, ref, s, f"spmm {kind} 16-bit B slices k={k} n={n}")


def test_sddmm_f16_subnormal_operands():
    # fp16 subnormals (2^-20 and 3 * 2^-24, below fp16's smallest normal 2^-14)
    # must enter the products unflushed: every output is a sum of exact tiny
    # products, far above fp32's own subnormal range
    m, k, d = 64, 96, 64
    lengths = np.full(m, 40, np.int32)
    rl = inputs.random_row_lists(750, m, k, lengths)
    ro = oracle.csr_offsets_from_lengths(lengths)
    x32 = np.where(np.arange(m * d).reshape(m, d) % 2 == 0, 2.0 ** -20, 3 * 2.0 ** -24)
    x32 = (x32 * np.sign(inputs.random_dense(751, m, d))).astype(np.float32)
    y32 = inputs.random_dense(752, k, d)
    d_x, x = to16(x32, "f16")
    d_y, y = to16(y32, "f16")
    assert np.all(np.abs(x) < 2.0 ** -14)               # every X element subnormal in fp16
    d_ro = devi(ro)
    out = torch.full((rl.cols.size,), float("nan"), device="cuda")
    note("sddmm_ex f16 subnormal operands")
    sp.sp_sddmm_ex(m, k, d, rl.cols.size, None, d_ro, devi(rl.cols), d_x, d_y, 1.0, out)
    ref, s = oracle.sddmm(m, k, d, ro, rl.cols, x, y)
    check_close(host(out), ref, s, "sddmm f16 subnormal")
