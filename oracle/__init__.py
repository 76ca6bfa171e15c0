"""CPU oracle for the CSR SpMM / SDDMM hot path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain single-threaded C, double
accumulation); this module only compiles it with gcc, loads it with ctypes and
marshals numpy arrays.  What each routine computes, and the passage of the
summary card of "Sparse GPU Kernels for Deep Learning" (Gale et al., SC 2020)
it follows, is stated at the routine in ``oracle.c``.

Parity status: every routine is pinned by the CPU tests against brute force,
closed forms or invariants (see ``tests/test_oracle.py``); none is unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Plain build: no fast-math, no FP contraction, no vectorisation flags.
GCC_CMD = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-Wextra", "-o", _LIB, _SRC, "-lm"]


def build() -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` (always recompiles)."""
    tmp = _LIB + ".tmp"
    cmd = list(GCC_CMD)
    cmd[cmd.index(_LIB)] = tmp
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None

_I32P = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_F32P = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_F64P = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_U8P = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_U16P = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if (not os.path.exists(_LIB)
            or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(_LIB)
    c_int, c_ll, vp = ctypes.c_int, ctypes.c_longlong, ctypes.c_void_p
    lib.orc_mask_nnz.argtypes = [c_int, c_int, _U8P]
    lib.orc_mask_nnz.restype = c_ll
    lib.orc_csr_from_dense.argtypes = [c_int, c_int, _U8P, vp, _I32P, _I32P, vp]
    lib.orc_csr_from_dense.restype = None
    lib.orc_csr_offsets_from_lengths.argtypes = [c_int, _I32P, _I32P]
    lib.orc_csr_offsets_from_lengths.restype = None
    lib.orc_csr_check.argtypes = [c_int, c_int, c_ll, _I32P, _I32P]
    lib.orc_csr_check.restype = c_int
    lib.orc_row_swizzle.argtypes = [c_int, _I32P, _I32P]
    lib.orc_row_swizzle.restype = None
    lib.orc_spmm.argtypes = [c_int, c_int, c_int, _I32P, _I32P, _F32P, _F32P,
                             _F64P, _F64P]
    lib.orc_spmm.restype = None
    lib.orc_spmm_rows.argtypes = [c_int, _I32P, c_int, _I32P, _I32P, _F32P,
                                  _F32P, _F64P, _F64P]
    lib.orc_spmm_rows.restype = None
    lib.orc_sddmm.argtypes = [c_int, c_int, c_int, _I32P, _I32P, _F32P, _F32P,
                              _F64P, _F64P]
    lib.orc_sddmm.restype = None
    lib.orc_sddmm_general.argtypes = [c_int, c_int, c_int, _I32P, _I32P, vp, _F32P, _F32P,
                                      c_int, ctypes.c_double, ctypes.c_double, vp, _F64P,
                                      _F64P]
    lib.orc_sddmm_general.restype = None
    lib.orc_csr_transpose.argtypes = [c_int, c_int, _I32P, _I32P, vp, _I32P, _I32P, vp, vp]
    lib.orc_csr_transpose.restype = None
    lib.orc_spmm_transposed.argtypes = [c_int, c_int, c_int, _I32P, _I32P, _F32P, _F32P,
                                        _F64P, _F64P]
    lib.orc_spmm_transposed.restype = None
    lib.orc_decode16.argtypes = [c_int, c_ll, _U16P, _F64P]
    lib.orc_decode16.restype = None
    lib.orc_softmax_rows.argtypes = [c_int, _I32P, _F32P, _F64P]
    lib.orc_softmax_rows.restype = None
    _lib = lib
    return lib


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def mask_nnz(mask: np.ndarray) -> int:
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    m, k = mask.shape
    return int(_load().orc_mask_nnz(m, k, mask))


def csr_from_dense(mask: np.ndarray, dense_values: np.ndarray | None = None):
    """Standard CSR of a dense byte mask -> (row_offsets, col_indices, values|None)."""
    lib = _load()
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    m, k = mask.shape
    nnz = int(lib.orc_mask_nnz(m, k, mask))
    ro = np.zeros(m + 1, np.int32)
    ci = np.zeros(max(nnz, 1), np.int32)
    vals = None
    dv_ptr = None
    v_ptr = None
    if dense_values is not None:
        dense_values = _f32(dense_values)
        assert dense_values.shape == (m, k)
        vals = np.zeros(max(nnz, 1), np.float32)
        dv_ptr = dense_values.ctypes.data
        v_ptr = vals.ctypes.data
    lib.orc_csr_from_dense(m, k, mask, dv_ptr, ro, ci, v_ptr)
    return ro, ci[:nnz], (vals[:nnz] if vals is not None else None)


def csr_offsets_from_lengths(lengths: np.ndarray) -> np.ndarray:
    lengths = _i32(lengths)
    ro = np.zeros(lengths.shape[0] + 1, np.int32)
    _load().orc_csr_offsets_from_lengths(lengths.shape[0], lengths, ro)
    return ro


def csr_check(m: int, k: int, row_offsets, col_indices) -> int:
    """0 if (row_offsets, col_indices) is a valid m x k CSR structure whose nnz
    is len(col_indices); otherwise the failure code of ``orc_csr_check``
    (-1 if row_offsets has the wrong length)."""
    ro = _i32(row_offsets)
    ci = _i32(col_indices)
    if ro.shape != (m + 1,):
        return -1
    return int(_load().orc_csr_check(m, k, int(ci.shape[0]), ro, _nz(ci)))


def row_swizzle(row_offsets) -> np.ndarray:
    ro = _i32(row_offsets)
    m = ro.shape[0] - 1
    out = np.zeros(max(m, 1), np.int32)
    _load().orc_row_swizzle(m, ro, out)
    return out[:m]


def _nz(a):
    """ctypes rejects zero-size arrays' NULL data pointer poorly; pad to 1."""
    return a if a.size else np.zeros(1, a.dtype)


def spmm(m: int, k: int, n: int, row_offsets, col_indices, values, b):
    """C = A B in double, and sum |a*b| per element -> (c f64[m,n], abs f64[m,n])."""
    ro, ci, v, bb = _i32(row_offsets), _i32(col_indices), _f32(values), _f32(b)
    assert ro.shape == (m + 1,) and bb.shape == (k, n)
    c = np.zeros((m, n), np.float64)
    a = np.zeros((m, n), np.float64)
    _load().orc_spmm(m, k, n, ro, _nz(ci), _nz(v), _nz(bb.reshape(-1)),
                     _nz(c.reshape(-1)), _nz(a.reshape(-1)))
    return c, a


def spmm_rows(rows, n: int, row_offsets, col_indices, values, b):
    """Rows `rows` of C = A B -> (c f64[len(rows), n], abs f64[len(rows), n])."""
    rows = _i32(rows)
    ro, ci, v, bb = _i32(row_offsets), _i32(col_indices), _f32(values), _f32(b)
    c = np.zeros((rows.shape[0], n), np.float64)
    a = np.zeros((rows.shape[0], n), np.float64)
    _load().orc_spmm_rows(rows.shape[0], _nz(rows), n, ro, _nz(ci), _nz(v),
                          _nz(bb.reshape(-1)), _nz(c.reshape(-1)),
                          _nz(a.reshape(-1)))
    return c, a


def sddmm(m: int, k: int, d: int, row_offsets, col_indices, x, y):
    """(X Y^T) at the CSR entries, in double -> (out f64[nnz], abs f64[nnz])."""
    ro, ci, xx, yy = _i32(row_offsets), _i32(col_indices), _f32(x), _f32(y)
    assert ro.shape == (m + 1,) and xx.shape == (m, d) and yy.shape == (k, d)
    nnz = int(ro[m])
    out = np.zeros(nnz, np.float64)
    a = np.zeros(nnz, np.float64)
    _load().orc_sddmm(m, k, d, ro, _nz(ci), _nz(xx.reshape(-1)),
                      _nz(yy.reshape(-1)), _nz(out), _nz(a))
    return out, a


def sddmm_general(m: int, k: int, d: int, row_offsets, col_indices, x, y, y_layout=0,
                  mask_values=None, alpha=1.0, beta=0.0, out_in=None):
    """alpha * v_p * (X Yop)[i, col] + beta * out_in[p] in double, and the
    tolerance scale -> (out f64[nnz], abs f64[nnz]).  y_layout 0: Y is k x d;
    1: Y is d x k."""
    ro, ci, xx, yy = _i32(row_offsets), _i32(col_indices), _f32(x), _f32(y)
    assert ro.shape == (m + 1,) and xx.shape == (m, d)
    assert yy.shape == ((k, d) if y_layout == 0 else (d, k))
    nnz = int(ro[m])
    mv = None if mask_values is None else _f32(mask_values)
    oi = None if out_in is None else _f32(out_in)
    out = np.zeros(nnz, np.float64)
    a = np.zeros(nnz, np.float64)
    _load().orc_sddmm_general(m, k, d, ro, _nz(ci), None if mv is None else mv.ctypes.data,
                              _nz(xx.reshape(-1)), _nz(yy.reshape(-1)), int(y_layout),
                              float(alpha), float(beta),
                              None if oi is None else oi.ctypes.data, _nz(out), _nz(a))
    return out, a


def csr_transpose(m: int, k: int, row_offsets, col_indices, values=None):
    """CSR of A^T -> (t_row_offsets[k+1], t_col_indices, t_values|None, t_perm)."""
    ro, ci = _i32(row_offsets), _i32(col_indices)
    assert ro.shape == (m + 1,)
    nnz = int(ro[m])
    t_ro = np.zeros(k + 1, np.int32)
    t_ci = np.zeros(max(nnz, 1), np.int32)
    t_perm = np.zeros(max(nnz, 1), np.int32)
    v = None if values is None else _f32(values)
    t_v = None if values is None else np.zeros(max(nnz, 1), np.float32)
    _load().orc_csr_transpose(m, k, ro, _nz(ci), None if v is None else _nz(v).ctypes.data,
                              t_ro, t_ci, None if t_v is None else t_v.ctypes.data,
                              t_perm.ctypes.data)
    return t_ro, t_ci[:nnz], (None if t_v is None else t_v[:nnz]), t_perm[:nnz]


def spmm_transposed(m: int, k: int, n: int, row_offsets, col_indices, values, dy):
    """dX = A^T dY in double -> (dx f64[k,n], abs f64[k,n])."""
    ro, ci, v, d = _i32(row_offsets), _i32(col_indices), _f32(values), _f32(dy)
    assert ro.shape == (m + 1,) and d.shape == (m, n)
    dx = np.zeros((k, n), np.float64)
    a = np.zeros((k, n), np.float64)
    _load().orc_spmm_transposed(m, k, n, ro, _nz(ci), _nz(v), _nz(d.reshape(-1)),
                                _nz(dx.reshape(-1)), _nz(a.reshape(-1)))
    return dx, a


F16, BF16 = 1, 2


def decode16(kind: int, bits) -> np.ndarray:
    """Values (float64, same shape) of binary16 (kind 1) or bfloat16 (kind 2)
    bit patterns given as uint16."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.zeros(b.shape, np.float64)
    _load().orc_decode16(int(kind), b.size, _nz(b.reshape(-1)), _nz(out.reshape(-1)))
    return out


def softmax_rows(row_offsets, s):
    """Row softmax over each row's CSR entries, in double -> f64[nnz]."""
    ro, ss = _i32(row_offsets), _f32(s)
    m = ro.shape[0] - 1
    out = np.zeros(ss.shape[0], np.float64)
    _load().orc_softmax_rows(m, ro, _nz(ss), _nz(out))
    return out
