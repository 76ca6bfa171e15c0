"""The C ABI without a GPU: the library loads, exports every symbol that
include/sp_csr.h declares, and rejects bad arguments on the host before any
HIP call.  No call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

import torch  # noqa: F401  (load torch's HIP runtime first, as the binding does)
from unstructured_sparse_linear_csr_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sp_csr.h")

INVALID = binding.SP_ERROR_INVALID_VALUE
OK = binding.SP_SUCCESS
NULL = ctypes.c_void_p(None)
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails
                                 # validation or returns before touching memory


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sp_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from unstructured_sparse_linear_csr_amd import build
        build.build()
    return binding.lib()


def test_every_declared_symbol_is_exported_and_bound(lib):
    declared = _declared_functions()
    assert len(declared) == 29, declared
    assert sorted(binding.SIGNATURES) == declared
    for name in declared:
        assert getattr(lib, name) is not None


def _declaration(name):
    """Parameter list of `name` in the header, as (type, name) pairs with
    whitespace normalised."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    m = re.search(r"\b" + name + r"\s*\(([^)]*)\)\s*;", text)
    assert m, name
    params = []
    for part in m.group(1).split(","):
        part = " ".join(part.replace("*", " * ").split())
        if part == "void":
            continue
        typ, _, pname = part.rpartition(" ")
        params.append((typ.replace(" *", "*"), pname))
    return params


def test_core_boundary_signatures():
    """The four calls of the core boundary keep the plain argument lists:
    the swizzle over row offsets, SpMM over CSR values/offsets/columns, SDDMM
    over the mask structure and two dense operands (no scale factor), each with
    raw device pointers and a stream, and the status strings."""
    assert _declaration("sp_row_swizzle") == [
        ("int", "m"), ("const int*", "row_offsets"), ("int*", "row_indices"),
        ("sp_stream_t", "stream")]
    assert _declaration("sp_spmm") == [
        ("int", "m"), ("int", "k"), ("int", "n"), ("int", "nnz"),
        ("const int*", "row_indices"), ("const float*", "values"),
        ("const int*", "row_offsets"), ("const int*", "col_indices"),
        ("const float*", "b"), ("float*", "c"), ("sp_stream_t", "stream")]
    assert _declaration("sp_sddmm") == [
        ("int", "m"), ("int", "k"), ("int", "d"), ("int", "nnz"),
        ("const int*", "row_indices"), ("const int*", "row_offsets"),
        ("const int*", "col_indices"), ("const float*", "x"), ("const float*", "y"),
        ("float*", "out"), ("sp_stream_t", "stream")]
    assert _declaration("sp_status_string") == [("sp_status_t", "status")]
    # the ctypes layer passes exactly those arguments
    for name in ("sp_row_swizzle", "sp_spmm", "sp_sddmm", "sp_status_string"):
        assert len(binding.SIGNATURES[name][0]) == len(_declaration(name)), name
    assert ctypes.c_float not in binding.SIGNATURES["sp_sddmm"][0]


def test_probe_library_exports():
    """The ceiling probes are a library of their own, outside the declared
    interface."""
    from unstructured_sparse_linear_csr_amd import probes
    l = probes.lib()
    for name in ("sp_probe_stream_read", "sp_probe_row_gather", "sp_probe_empty"):
        assert getattr(l, name) is not None
        assert not hasattr(binding.lib(), name) or name not in binding.SIGNATURES
    # argument checks return before any launch
    assert l.sp_probe_empty(0, NULL) != 0
    assert l.sp_probe_stream_read(NULL, 1 << 20, 4, FAKE, NULL) != 0
    assert l.sp_probe_row_gather(FAKE, 4, 4, FAKE, 512, FAKE, NULL) != 0


def test_status_strings_and_version(lib):
    for code in range(4):
        assert binding.status_string(code)
    assert binding.status_string(99) == "unknown status"
    assert binding.version() == 10000


def test_spmm_validation(lib):
    f = lib.sp_spmm_batched
    s = NULL
    # negative sizes
    assert f(-1, 4, 4, 0, NULL, NULL, FAKE, NULL, NULL, FAKE, 1, 0, 0, 0, s) == INVALID
    assert f(4, -1, 4, 0, NULL, NULL, FAKE, NULL, NULL, FAKE, 1, 0, 0, 0, s) == INVALID
    assert f(4, 4, -1, 0, NULL, NULL, FAKE, NULL, NULL, FAKE, 1, 0, 0, 0, s) == INVALID
    assert f(4, 4, 4, -1, NULL, NULL, FAKE, NULL, NULL, FAKE, 1, 0, 0, 0, s) == INVALID
    assert f(4, 4, 4, 0, NULL, NULL, FAKE, NULL, NULL, FAKE, -1, 0, 0, 0, s) == INVALID
    assert f(4, 4, 4, 0, NULL, NULL, FAKE, NULL, NULL, FAKE, 1, -4, 0, 0, s) == INVALID
    # NULL for a non-empty buffer
    assert f(4, 4, 4, 8, NULL, FAKE, NULL, FAKE, FAKE, FAKE, 1, 0, 0, 0, s) == INVALID
    assert f(4, 4, 4, 8, NULL, FAKE, FAKE, NULL, FAKE, FAKE, 1, 0, 0, 0, s) == INVALID
    assert f(4, 4, 4, 8, NULL, NULL, FAKE, FAKE, FAKE, FAKE, 1, 0, 0, 0, s) == INVALID
    assert f(4, 4, 4, 8, NULL, FAKE, FAKE, FAKE, NULL, FAKE, 1, 0, 0, 0, s) == INVALID
    assert f(4, 4, 4, 8, NULL, FAKE, FAKE, FAKE, FAKE, NULL, 1, 0, 0, 0, s) == INVALID
    # overlapping batched outputs
    assert f(4, 4, 4, 8, NULL, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 16, 15, s) == INVALID
    # empty problems succeed without launching anything
    assert f(0, 4, 4, 0, NULL, NULL, NULL, NULL, NULL, NULL, 1, 0, 0, 0, s) == OK
    assert f(4, 4, 0, 0, NULL, NULL, NULL, NULL, NULL, NULL, 1, 0, 0, 0, s) == OK
    assert f(4, 4, 4, 0, NULL, NULL, NULL, NULL, NULL, NULL, 0, 0, 0, 0, s) == OK
    assert lib.sp_spmm(0, 4, 4, 0, NULL, NULL, NULL, NULL, NULL, NULL, s) == OK
    g = lib.sp_spmm_balanced
    assert g(-1, 4, 4, 0, NULL, NULL, FAKE, NULL, NULL, FAKE, s) == INVALID
    assert g(4, 4, 4, 8, NULL, NULL, FAKE, FAKE, FAKE, FAKE, s) == INVALID
    assert g(4, 4, 4, 8, NULL, FAKE, FAKE, FAKE, FAKE, NULL, s) == INVALID
    assert g(0, 4, 4, 0, NULL, NULL, NULL, NULL, NULL, NULL, s) == OK
    assert lib.sp_spmm(-2, 4, 4, 0, NULL, NULL, NULL, NULL, NULL, NULL, s) == INVALID


def test_spmm_sddmm_validation(lib):
    f = lib.sp_spmm_sddmm
    s = NULL
    fl = ctypes.c_float(1.0)

    def call(spmm=(4, 4, 4, 8), sddmm=(4, 4, 4, 8), v=FAKE, x=FAKE, c=FAKE, out=FAKE):
        m, k, n, nnz = spmm
        sm, sk, d, snnz = sddmm
        return f(m, k, n, nnz, NULL, v, FAKE, FAKE, FAKE, c, sm, sk, d, snnz, NULL, FAKE, FAKE,
                 x, FAKE, fl, out, s)

    assert call(spmm=(-1, 4, 4, 8)) == INVALID
    assert call(sddmm=(4, 4, -1, 8)) == INVALID
    assert call(v=NULL) == INVALID
    assert call(x=NULL) == INVALID
    assert call(c=NULL) == INVALID
    assert call(out=NULL) == INVALID
    # an invalid half is reported even when the other half is empty
    assert call(spmm=(0, 4, 4, 0), x=NULL) == INVALID
    assert call(sddmm=(0, 4, 4, 0), v=NULL) == INVALID
    # both halves empty: nothing to do
    assert f(0, 4, 4, 0, NULL, NULL, NULL, NULL, NULL, NULL, 0, 4, 4, 0, NULL, NULL, NULL,
             NULL, NULL, fl, NULL, s) == OK


def test_sparse_attention_validation(lib):
    f = lib.sp_sparse_attention
    s = NULL
    fl = ctypes.c_float(0.125)

    def call(m=4, k=4, d=64, nnz=8, dtype=0, ro=FAKE, ci=FAKE, q=FAKE, kk=FAKE, v=FAKE,
             out=FAKE, batch=1, so=0):
        return f(m, k, d, nnz, NULL, ro, ci, dtype, q, kk, v, fl, out, batch, 0, 0, 0, so, s)

    assert call(dtype=3) == INVALID
    assert call(m=-1) == INVALID
    assert call(d=-1) == INVALID
    assert call(ro=NULL) == INVALID
    assert call(ci=NULL) == INVALID
    assert call(q=NULL) == INVALID
    assert call(kk=NULL) == INVALID
    assert call(v=NULL) == INVALID
    assert call(out=NULL) == INVALID
    assert call(batch=2, so=255) == INVALID
    assert call(m=0, ro=NULL, ci=NULL, q=NULL, kk=NULL, v=NULL, out=NULL) == OK
    assert call(batch=0) == OK
    # unsupported head dimension: reported before any launch
    assert call(d=48) == binding.SP_ERROR_NOT_SUPPORTED
    assert call(d=32, dtype=1) == binding.SP_ERROR_NOT_SUPPORTED


def test_mixed_precision_validation(lib):
    s = NULL
    f = lib.sp_spmm_ex
    for bad in (-1, 3, 99):
        assert f(4, 4, 4, 8, NULL, bad, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 0, 0, 0, s) == INVALID
    # dtype is checked before anything else, even for an empty problem
    assert f(0, 4, 4, 0, NULL, 7, NULL, NULL, NULL, NULL, NULL, 1, 0, 0, 0, s) == INVALID
    for dt in (0, 1, 2):
        assert f(0, 4, 4, 0, NULL, dt, NULL, NULL, NULL, NULL, NULL, 1, 0, 0, 0, s) == OK
        assert f(4, 4, 4, 8, NULL, dt, NULL, FAKE, FAKE, FAKE, FAKE, 1, 0, 0, 0, s) == INVALID
        assert f(4, 4, 4, 8, NULL, dt, FAKE, FAKE, FAKE, NULL, FAKE, 1, 0, 0, 0, s) == INVALID
    for g in (lib.sp_sddmm_ex, lib.sp_sddmm_softmax):
        fl = ctypes.c_float(1.0)
        assert g(4, 4, 4, 8, NULL, FAKE, FAKE, 5, FAKE, FAKE, fl, FAKE, 1, 0, 0, 0, s) == INVALID
        for dt in (0, 1, 2):
            assert g(0, 4, 4, 0, NULL, NULL, NULL, dt, NULL, NULL, fl, NULL, 1, 0, 0, 0, s) == OK
            assert g(4, 4, 4, 8, NULL, FAKE, FAKE, dt, NULL, FAKE, fl, FAKE, 1, 0, 0, 0,
                     s) == INVALID
            assert g(4, 4, 4, 8, NULL, NULL, FAKE, dt, FAKE, FAKE, fl, FAKE, 1, 0, 0, 0,
                     s) == INVALID
    g = lib.sp_sddmm_ex
    fl = ctypes.c_float(1.0)
    assert g(4, 4, 4, 8, NULL, FAKE, FAKE, 5, FAKE, FAKE, fl, FAKE, 1, 0, 0, 0, s) == INVALID
    for dt in (0, 1, 2):
        assert g(0, 4, 4, 0, NULL, NULL, NULL, dt, NULL, NULL, fl, NULL, 1, 0, 0, 0, s) == OK
        assert g(4, 4, 4, 8, NULL, FAKE, FAKE, dt, NULL, FAKE, fl, FAKE, 1, 0, 0, 0, s) == INVALID
        assert g(4, 4, 4, 8, NULL, FAKE, FAKE, dt, FAKE, FAKE, fl, FAKE, 2, 0, 0, 7, s) == INVALID


def test_transpose_validation(lib):
    size = ctypes.c_size_t(0)
    assert lib.sp_csr_transpose_workspace(4, 5, 10000, ctypes.byref(size)) == OK
    # five int32 arrays of nnz entries (256-byte aligned) and 256 counters per
    # 4096-entry tile plus one
    arr = (10000 * 4 + 255) // 256 * 256
    assert size.value == 5 * arr + (256 * 4 * 4 + 255) // 256 * 256
    assert lib.sp_csr_transpose_workspace(-1, 5, 10, ctypes.byref(size)) == INVALID
    assert lib.sp_csr_transpose_workspace(1, 5, 10, None) == INVALID
    f = lib.sp_csr_transpose
    s = NULL
    ws = ctypes.c_void_p(0x100000)  # 256-byte aligned, never dereferenced
    need = binding.sp_csr_transpose_workspace(4, 5, 8)

    def call(m=4, k=5, nnz=8, ro=FAKE, ci=FAKE, v=FAKE, tro=FAKE, tci=FAKE, tv=FAKE,
             tp=NULL, w=ws, wb=None):
        return f(m, k, nnz, ro, ci, v, tro, tci, tv, tp, w, need if wb is None else wb, s)

    assert call(m=-1) == INVALID
    assert call(k=-1) == INVALID
    assert call(nnz=-1) == INVALID
    assert call(k=2**31 - 1) == INVALID
    assert call(k=0) == INVALID
    assert call(ro=NULL) == INVALID
    assert call(ci=NULL) == INVALID
    assert call(tro=NULL) == INVALID
    assert call(tci=NULL) == INVALID
    assert call(v=NULL) == INVALID           # t_values asked for without values
    assert call(w=NULL) == INVALID
    assert call(wb=need - 1) == INVALID
    assert call(w=ctypes.c_void_p(0x100010)) == INVALID   # misaligned workspace
    g = lib.sp_csr_transpose_values
    assert g(-1, FAKE, FAKE, FAKE, s) == INVALID
    assert g(4, NULL, FAKE, FAKE, s) == INVALID
    assert g(4, FAKE, NULL, FAKE, s) == INVALID
    assert g(4, FAKE, FAKE, NULL, s) == INVALID
    assert g(0, NULL, NULL, NULL, s) == OK


def test_sddmm_general_validation(lib):
    f = lib.sp_sddmm_general
    s = NULL
    fl = ctypes.c_float

    def call(m=4, k=4, d=4, nnz=8, ro=FAKE, ci=FAKE, mv=NULL, x=FAKE, y=FAKE, layout=0,
             out=FAKE, batch=1, sv=0, sx=0, sy=0, so=0, ws=NULL, wb=0):
        return f(m, k, d, nnz, NULL, ro, ci, mv, x, y, layout, fl(1.0), fl(0.5), out, batch,
                 sv, sx, sy, so, ws, wb, s)

    assert call(layout=2) == INVALID
    assert call(layout=-1) == INVALID
    assert call(m=-1) == INVALID
    assert call(d=-1) == INVALID
    assert call(sv=-1) == INVALID
    assert call(ro=NULL) == INVALID
    assert call(ci=NULL) == INVALID
    assert call(x=NULL) == INVALID
    assert call(y=NULL, layout=1) == INVALID
    assert call(out=NULL) == INVALID
    assert call(batch=2, so=7) == INVALID
    # a bad layout is rejected even for an empty problem
    assert call(m=0, layout=3) == INVALID
    # empty problems succeed without launching anything
    assert call(m=0, ro=NULL, ci=NULL, x=NULL, y=NULL, out=NULL) == OK
    assert call(nnz=0, ci=NULL, out=NULL, layout=1) == OK
    assert call(batch=0) == OK
    # a workspace for the d x k layout: at least k*d*4 bytes per batch entry
    # (one copy when stride_y is 0), 256-byte aligned
    ws = ctypes.c_void_p(0x100000)
    assert call(layout=1, ws=ws, wb=63) == INVALID
    assert call(layout=1, ws=ctypes.c_void_p(0x100040), wb=1 << 20) == INVALID
    assert call(layout=1, batch=2, sx=16, sy=16, so=8, ws=ws, wb=64) == INVALID
    assert call(layout=1, batch=0, ws=ws, wb=0) == OK


def test_sddmm_general_workspace_query(lib):
    q = lib.sp_sddmm_general_workspace
    size = ctypes.c_size_t(0)
    assert q(300, 24, 1, 0, ctypes.byref(size)) == OK and size.value == 300 * 24 * 4
    assert q(300, 24, 5, 0, ctypes.byref(size)) == OK and size.value == 300 * 24 * 4
    assert q(300, 24, 5, 7200, ctypes.byref(size)) == OK and size.value == 5 * 300 * 24 * 4
    assert q(0, 24, 5, 7200, ctypes.byref(size)) == OK and size.value == 0
    assert q(-1, 24, 1, 0, ctypes.byref(size)) == INVALID
    assert q(3, 24, 1, -2, ctypes.byref(size)) == INVALID
    assert q(3, 24, 1, 0, None) == INVALID


def test_sddmm_validation(lib):
    f = lib.sp_sddmm_batched
    s = NULL
    assert f(-1, 4, 4, 0, NULL, FAKE, NULL, FAKE, FAKE, 1.0, FAKE, 1, 0, 0, 0, s) == INVALID
    assert f(4, 4, -1, 0, NULL, FAKE, NULL, FAKE, FAKE, 1.0, FAKE, 1, 0, 0, 0, s) == INVALID
    assert f(4, 4, 4, 8, NULL, NULL, FAKE, FAKE, FAKE, 1.0, FAKE, 1, 0, 0, 0, s) == INVALID
    assert f(4, 4, 4, 8, NULL, FAKE, NULL, FAKE, FAKE, 1.0, FAKE, 1, 0, 0, 0, s) == INVALID
    assert f(4, 4, 4, 8, NULL, FAKE, FAKE, NULL, FAKE, 1.0, FAKE, 1, 0, 0, 0, s) == INVALID
    assert f(4, 4, 4, 8, NULL, FAKE, FAKE, FAKE, NULL, 1.0, FAKE, 1, 0, 0, 0, s) == INVALID
    assert f(4, 4, 4, 8, NULL, FAKE, FAKE, FAKE, FAKE, 1.0, NULL, 1, 0, 0, 0, s) == INVALID
    assert f(4, 4, 4, 8, NULL, FAKE, FAKE, FAKE, FAKE, 1.0, FAKE, 2, 0, 0, 7, s) == INVALID
    assert f(4, 4, 4, 0, NULL, FAKE, NULL, FAKE, FAKE, 1.0, NULL, 1, 0, 0, 0, s) == OK
    assert f(0, 4, 4, 0, NULL, NULL, NULL, NULL, NULL, 1.0, NULL, 1, 0, 0, 0, s) == OK
    for g in (lib.sp_sddmm, lib.sp_sddmm_balanced):
        assert g(-1, 4, 4, 0, NULL, FAKE, NULL, FAKE, FAKE, FAKE, s) == INVALID
        assert g(4, 4, 4, 8, NULL, NULL, FAKE, FAKE, FAKE, FAKE, s) == INVALID
        assert g(4, 4, 4, 8, NULL, FAKE, NULL, FAKE, FAKE, FAKE, s) == INVALID
        assert g(4, 4, 4, 8, NULL, FAKE, FAKE, NULL, FAKE, FAKE, s) == INVALID
        assert g(4, 4, 4, 8, NULL, FAKE, FAKE, FAKE, NULL, FAKE, s) == INVALID
        assert g(4, 4, 4, 8, NULL, FAKE, FAKE, FAKE, FAKE, NULL, s) == INVALID
        assert g(0, 4, 4, 0, NULL, NULL, NULL, NULL, NULL, NULL, s) == OK


def test_build_and_swizzle_validation(lib):
    s = NULL
    assert lib.sp_csr_offsets_from_lengths(-1, FAKE, FAKE, s) == INVALID
    assert lib.sp_csr_offsets_from_lengths(3, NULL, FAKE, s) == INVALID
    assert lib.sp_csr_offsets_from_lengths(3, FAKE, NULL, s) == INVALID
    assert lib.sp_csr_count_dense(3, -1, FAKE, FAKE, s) == INVALID
    assert lib.sp_csr_count_dense(3, 3, NULL, FAKE, s) == INVALID
    assert lib.sp_csr_count_dense(3, 3, FAKE, NULL, s) == INVALID
    assert lib.sp_csr_fill_dense(3, 3, NULL, NULL, FAKE, FAKE, NULL, s) == INVALID
    assert lib.sp_csr_fill_dense(3, 3, FAKE, NULL, NULL, FAKE, NULL, s) == INVALID
    assert lib.sp_csr_fill_dense(-3, 3, FAKE, FAKE, FAKE, FAKE, FAKE, s) == INVALID
    assert lib.sp_csr_build_from_lengths(-1, FAKE, FAKE, FAKE, s) == INVALID
    assert lib.sp_csr_build_from_lengths(3, NULL, FAKE, FAKE, s) == INVALID
    assert lib.sp_csr_build_from_lengths(3, FAKE, NULL, FAKE, s) == INVALID
    assert lib.sp_csr_build_from_lengths(3, FAKE, FAKE, NULL, s) == INVALID
    assert lib.sp_row_swizzle(-1, FAKE, FAKE, s) == INVALID
    assert lib.sp_row_swizzle(3, NULL, FAKE, s) == INVALID
    assert lib.sp_row_swizzle(3, FAKE, NULL, s) == INVALID


def test_spmm_kernel_name(lib):
    f = lib.sp_spmm_kernel_name
    name = ctypes.c_char_p()
    al = ctypes.c_void_p(0x10000)                     # 16-byte aligned stand-ins
    assert f(8, 8, 4, 8, NULL, 0, al, al, al, al, 1, 0, 0, 0, ctypes.byref(name)) == OK
    assert name.value == b"narrow"                      # fp32, n <= 16 columns
    assert f(0, 8, 4, 8, NULL, 0, al, al, al, al, 1, 0, 0, 0, ctypes.byref(name)) == OK
    assert name.value == b"none"
    # 16-bit types never take the fp32 narrow kernel
    assert f(8, 8, 512, 8, NULL, 1, al, al, al, al, 1, 0, 0, 0, ctypes.byref(name)) == OK
    assert name.value in (b"wide", b"split")
    # a row order on wide B, one batch entry: the balanced kernel
    assert f(8, 8, 512, 8, al, 0, al, al, al, al, 1, 0, 0, 0, ctypes.byref(name)) == OK
    assert name.value == b"balanced"
    assert f(8, 8, 4, 8, NULL, 7, al, al, al, al, 1, 0, 0, 0, ctypes.byref(name)) == INVALID
    assert f(-1, 8, 4, 8, NULL, 0, al, al, al, al, 1, 0, 0, 0, ctypes.byref(name)) == INVALID
    assert f(8, 8, 4, 8, NULL, 0, al, al, al, al, 1, 0, 0, 0, None) == INVALID


def test_sddmm_kernel_name(lib):
    f = lib.sp_sddmm_kernel_name
    name = ctypes.c_char_p()
    al = ctypes.c_void_p(0x10000)                     # 16-byte aligned stand-ins
    odd = ctypes.c_void_p(0x10004)
    nm = lambda: name.value

    def call(m, k, d, nnz, dtype=0, mask=NULL, x=al, y=al, layout=0, beta=0.0, batch=1,
             sv=0, sx=0, sy=0, so=0, ws=NULL, ws_bytes=0, out=True):
        return f(m, k, d, nnz, dtype, mask, x, y, layout, beta, batch, sv, sx, sy, so, ws,
                 ws_bytes, ctypes.byref(name) if out else None)

    # sparse-attention scores: 32 heads, d = 64, ~80 entries per row
    assert call(4096, 4096, 64, 325664, batch=32, sx=4096 * 64, sy=4096 * 64,
                so=325664) == OK and nm() == b"panel_union"
    # the same beyond the panel-union kernel's 65,536 columns: several rows per wave
    assert call(4096, 65537, 64, 325664, batch=32, sx=4096 * 64, sy=65537 * 64,
                so=325664) == OK and nm() == b"multirow"
    assert call(100, 100, 20, 500) == OK and nm() == b"multirow"   # d = 20: groups of 8
    # one batch entry whose rows average 16 entries or more: split over waves
    assert call(64, 64, 64, 64 * 16) == OK and nm() == b"split"
    # d = 16 (4 lanes per entry), d = 68 (two vectors per lane), misaligned X, bf16
    # at d = 32 (4 lanes per entry): one row per wave
    assert call(100, 100, 16, 500) == OK and nm() == b"rows"
    assert call(100, 100, 68, 500) == OK and nm() == b"rows"
    assert call(100, 100, 64, 500, x=odd) == OK and nm() == b"rows"
    assert call(100, 100, 32, 500, dtype=2) == OK and nm() == b"rows"
    # bf16 at d = 64 and 128 (8 and 16 lanes per entry): several rows per wave
    assert call(100, 100, 64, 500, dtype=2) == OK and nm() == b"multirow"
    assert call(100, 100, 128, 500, dtype=1) == OK and nm() == b"multirow"
    assert call(100, 100, 0, 500) == OK and nm() == b"fill"
    assert call(100, 100, 64, 500, layout=1) == OK and nm() in (b"dk_panel", b"dk_tile",
                                                                   b"columns")
    assert call(0, 100, 64, 500) == OK and nm() == b"none"
    assert call(100, 100, 64, 500, dtype=7) == INVALID
    assert call(-1, 100, 64, 500) == INVALID
    assert call(100, 100, 64, 500, layout=2) == INVALID
    assert call(100, 100, 64, 500, out=False) == INVALID


def test_row_swizzle_noalloc_validation(lib):
    s = NULL
    f = lib.sp_row_swizzle_noalloc
    top = binding.SP_ROW_SWIZZLE_NOALLOC_MAX_ROWS
    assert f(-1, 4, FAKE, FAKE, s) == INVALID
    assert f(5, -1, FAKE, FAKE, s) == INVALID
    assert f(5, 4, NULL, FAKE, s) == INVALID
    assert f(5, 4, FAKE, NULL, s) == INVALID
    assert f(top + 1, 4, FAKE, FAKE, s) == INVALID     # beyond the scratch array
    assert f(0, 4, FAKE, NULL, s) == OK


def test_row_swizzle_ws_validation(lib):
    s = NULL
    size = ctypes.c_size_t(0)
    q = lib.sp_row_swizzle_workspace
    assert q(-1, ctypes.byref(size)) == INVALID
    assert q(5, None) == INVALID
    # no workspace up to the rank sort's row limit
    assert q(16384, ctypes.byref(size)) == OK and size.value == 0
    assert q(16385, ctypes.byref(size)) == OK
    # four arrays of m ints and the radix tile counters, 256-byte multiples
    arr = (16385 * 4 + 255) // 256 * 256
    hist = (256 * (5 + 1) * 4 + 255) // 256 * 256
    assert size.value == 4 * arr + hist
    need = size.value
    f = lib.sp_row_swizzle_ws
    big = ctypes.c_void_p(0x100000)
    assert f(-1, 4, FAKE, FAKE, NULL, 0, s) == INVALID
    assert f(5, -1, FAKE, FAKE, NULL, 0, s) == INVALID
    assert f(5, 4, NULL, FAKE, NULL, 0, s) == INVALID
    assert f(5, 4, FAKE, NULL, NULL, 0, s) == INVALID
    assert f(0, 4, FAKE, NULL, NULL, 0, s) == OK              # nothing to order
    assert f(16385, 9, FAKE, FAKE, NULL, need, s) == INVALID   # workspace missing
    assert f(16385, 9, FAKE, FAKE, big, need - 1, s) == INVALID  # too short
    assert f(16385, 9, FAKE, FAKE, ctypes.c_void_p(0x100010), need, s) == INVALID  # misaligned


def test_softmax_validation(lib):
    f = lib.sp_csr_row_softmax
    s = NULL
    assert f(-1, 4, NULL, FAKE, FAKE, FAKE, 1, 0, 0, s) == INVALID
    assert f(3, -4, NULL, FAKE, FAKE, FAKE, 1, 0, 0, s) == INVALID
    assert f(3, 4, NULL, FAKE, FAKE, FAKE, -1, 0, 0, s) == INVALID
    assert f(3, 4, NULL, NULL, FAKE, FAKE, 1, 0, 0, s) == INVALID
    assert f(3, 4, NULL, FAKE, NULL, FAKE, 1, 0, 0, s) == INVALID
    assert f(3, 4, NULL, FAKE, FAKE, NULL, 1, 0, 0, s) == INVALID
    assert f(3, 4, NULL, FAKE, FAKE, FAKE, 2, 4, 3, s) == INVALID
    assert f(0, 4, NULL, NULL, NULL, NULL, 1, 0, 0, s) == OK
    assert f(3, 0, NULL, FAKE, NULL, NULL, 1, 0, 0, s) == OK


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", "/nonexistent/libsp_csr.so")
    with pytest.raises(ImportError):
        binding.lib()


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "unstructured_sparse_linear_csr_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", text, re.M), fn
                assert "liboracle" not in text, fn
