"""Thin ctypes binding over ``libsp_csr.so`` (declared in ``include/sp_csr.h``).

Argument marshalling only: each ``sp_*`` function here has the name and
argument order of the C entry point, takes torch tensors where the C function
takes device pointers, checks dtype/device/contiguity, passes ``data_ptr()``
and the current HIP stream, and raises ``SpError`` on a non-success status.
All computation happens in the library's HIP kernels; there is no fallback.

torch is imported before the library is loaded so that the library binds to
the HIP runtime torch already loaded (both carry the soname libamdhip64.so.7)
and torch's stream handles are meaningful to it.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsp_csr.so")

SP_SUCCESS = 0
SP_ERROR_INVALID_VALUE = 1
SP_ERROR_NOT_SUPPORTED = 2
SP_ERROR_LAUNCH_FAILED = 3
SP_Y_KD = 0  # SDDMM operand Y stored k x d
SP_Y_DK = 1  # SDDMM operand Y stored d x k
SP_DTYPE_F32 = 0
SP_DTYPE_F16 = 1
SP_DTYPE_BF16 = 2

# Every symbol include/sp_csr.h declares, with its ctypes signature.
_c_int, _c_ll, _c_float, _vp = ctypes.c_int, ctypes.c_longlong, ctypes.c_float, ctypes.c_void_p
SIGNATURES = {
    "sp_status_string": ([_c_int], ctypes.c_char_p),
    "sp_version": ([], _c_int),
    "sp_csr_offsets_from_lengths": ([_c_int, _vp, _vp, _vp], _c_int),
    "sp_csr_count_dense": ([_c_int, _c_int, _vp, _vp, _vp], _c_int),
    "sp_csr_fill_dense": ([_c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp], _c_int),
    "sp_row_swizzle": ([_c_int, _vp, _vp, _vp], _c_int),
    "sp_row_swizzle_workspace": ([_c_int, ctypes.POINTER(ctypes.c_size_t)], _c_int),
    "sp_row_swizzle_ws": ([_c_int, _c_int, _vp, _vp, _vp, ctypes.c_size_t, _vp], _c_int),
    "sp_row_swizzle_noalloc": ([_c_int, _c_int, _vp, _vp, _vp], _c_int),
    "sp_csr_build_from_lengths": ([_c_int, _vp, _vp, _vp, _vp], _c_int),
    "sp_spmm": ([_c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
                _c_int),
    "sp_spmm_batched": ([_c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp,
                         _c_int, _c_ll, _c_ll, _c_ll, _vp], _c_int),
    "sp_sddmm": ([_c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
                 _c_int),
    "sp_sddmm_balanced": ([_c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp,
                           _vp], _c_int),
    "sp_sddmm_batched": ([_c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp,
                          _c_float, _vp, _c_int, _c_ll, _c_ll, _c_ll, _vp], _c_int),
    "sp_sddmm_general": ([_c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp,
                          _c_int, _c_float, _c_float, _vp, _c_int, _c_ll, _c_ll, _c_ll,
                          _c_ll, _vp, ctypes.c_size_t, _vp], _c_int),
    "sp_sddmm_general_workspace": ([_c_int, _c_int, _c_int, _c_ll,
                                    ctypes.POINTER(ctypes.c_size_t)], _c_int),
    "sp_csr_row_softmax": ([_c_int, _c_int, _vp, _vp, _vp, _vp, _c_int, _c_ll, _c_ll, _vp],
                           _c_int),
    "sp_csr_transpose_workspace": ([_c_int, _c_int, _c_int, ctypes.POINTER(ctypes.c_size_t)],
                                   _c_int),
    "sp_csr_transpose": ([_c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                          ctypes.c_size_t, _vp], _c_int),
    "sp_csr_transpose_values": ([_c_int, _vp, _vp, _vp, _vp], _c_int),
    "sp_spmm_balanced": ([_c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
                         _c_int),
    "sp_spmm_sddmm": ([_c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp,
                       _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _c_float, _vp,
                       _vp], _c_int),
    "sp_sddmm_softmax": ([_c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _c_int, _vp, _vp,
                          _c_float, _vp, _c_int, _c_ll, _c_ll, _c_ll, _vp], _c_int),
    "sp_sparse_attention": ([_c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _c_int, _vp, _vp,
                             _vp, _c_float, _vp, _c_int, _c_ll, _c_ll, _c_ll, _c_ll, _vp],
                            _c_int),
    "sp_spmm_ex": ([_c_int, _c_int, _c_int, _c_int, _vp, _c_int, _vp, _vp, _vp, _vp, _vp,
                    _c_int, _c_ll, _c_ll, _c_ll, _vp], _c_int),
    "sp_spmm_kernel_name": ([_c_int, _c_int, _c_int, _c_int, _vp, _c_int, _vp, _vp, _vp, _vp,
                             _c_int, _c_ll, _c_ll, _c_ll,
                             ctypes.POINTER(ctypes.c_char_p)], _c_int),
    "sp_sddmm_kernel_name": ([_c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _c_int,
                              _c_float, _c_int, _c_ll, _c_ll, _c_ll, _c_ll, _vp, ctypes.c_size_t,
                              ctypes.POINTER(ctypes.c_char_p)], _c_int),
    "sp_sddmm_ex": ([_c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _c_int, _vp, _vp,
                     _c_float, _vp, _c_int, _c_ll, _c_ll, _c_ll, _vp], _c_int),
}


class SpError(RuntimeError):
    """A library call returned a non-success status."""

    def __init__(self, what: str, status: int):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library.  Raises if it has not been built: there is no
    other implementation to fall back to."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing; build it with "
                "`python -m unstructured_sparse_linear_csr_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (argtypes, restype) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = argtypes
            fn.restype = restype
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().sp_status_string(status).decode()


def version() -> int:
    return lib().sp_version()


def _check(status: int, what: str) -> None:
    if status != SP_SUCCESS:
        raise SpError(what, status)


def _stream(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t, dtype, name, allow_none=False) -> ctypes.c_void_p:
    if t is None:
        if allow_none:
            return ctypes.c_void_p(None)
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr() if t.numel() else None)


_I32, _F32, _U8 = torch.int32, torch.float32, torch.uint8


# ---------------------------------------------------------------- CSR build

def sp_csr_offsets_from_lengths(m, lengths, row_offsets, stream=None):
    _check(lib().sp_csr_offsets_from_lengths(
        m, _ptr(lengths, _I32, "lengths", True), _ptr(row_offsets, _I32, "row_offsets"),
        _stream(stream)), "sp_csr_offsets_from_lengths")


def sp_csr_count_dense(m, k, mask, row_offsets, stream=None):
    _check(lib().sp_csr_count_dense(
        m, k, _ptr(mask, _U8, "mask", True), _ptr(row_offsets, _I32, "row_offsets"),
        _stream(stream)), "sp_csr_count_dense")


def sp_csr_fill_dense(m, k, mask, dense_values, row_offsets, col_indices, values,
                      stream=None):
    _check(lib().sp_csr_fill_dense(
        m, k, _ptr(mask, _U8, "mask", True), _ptr(dense_values, _F32, "dense_values", True),
        _ptr(row_offsets, _I32, "row_offsets"), _ptr(col_indices, _I32, "col_indices", True),
        _ptr(values, _F32, "values", True), _stream(stream)), "sp_csr_fill_dense")


# ---------------------------------------------------------------- swizzle

def sp_row_swizzle(m, row_offsets, row_indices, stream=None):
    _check(lib().sp_row_swizzle(
        m, _ptr(row_offsets, _I32, "row_offsets"), _ptr(row_indices, _I32, "row_indices", True),
        _stream(stream)), "sp_row_swizzle")


def sp_row_swizzle_workspace(m) -> int:
    size = ctypes.c_size_t(0)
    _check(lib().sp_row_swizzle_workspace(m, ctypes.byref(size)), "sp_row_swizzle_workspace")
    return size.value


def sp_row_swizzle_ws(m, k, row_offsets, row_indices, workspace, stream=None):
    """workspace: a uint8 device tensor of at least sp_row_swizzle_workspace(m)
    bytes, or None when that is 0."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().sp_row_swizzle_ws(
        m, k, _ptr(row_offsets, _I32, "row_offsets"), _ptr(row_indices, _I32, "row_indices", True),
        _ptr(workspace, _U8, "workspace", True), ws_bytes, _stream(stream)), "sp_row_swizzle_ws")


SP_ROW_SWIZZLE_NOALLOC_MAX_ROWS = 2000000


def sp_row_swizzle_noalloc(m, k, row_offsets, row_indices, stream=None):
    _check(lib().sp_row_swizzle_noalloc(
        m, k, _ptr(row_offsets, _I32, "row_offsets"), _ptr(row_indices, _I32, "row_indices", True),
        _stream(stream)), "sp_row_swizzle_noalloc")


def sp_csr_build_from_lengths(m, lengths, row_offsets, row_indices, stream=None):
    _check(lib().sp_csr_build_from_lengths(
        m, _ptr(lengths, _I32, "lengths", True), _ptr(row_offsets, _I32, "row_offsets"),
        _ptr(row_indices, _I32, "row_indices", True), _stream(stream)),
        "sp_csr_build_from_lengths")


# ---------------------------------------------------------------- SpMM / SDDMM

def sp_spmm(m, k, n, nnz, row_indices, values, row_offsets, col_indices, b, c,
            stream=None):
    _check(lib().sp_spmm(
        m, k, n, nnz, _ptr(row_indices, _I32, "row_indices", True),
        _ptr(values, _F32, "values", True), _ptr(row_offsets, _I32, "row_offsets"),
        _ptr(col_indices, _I32, "col_indices", True), _ptr(b, _F32, "b", True),
        _ptr(c, _F32, "c"), _stream(stream)), "sp_spmm")


def sp_spmm_batched(m, k, n, nnz, row_indices, values, row_offsets, col_indices, b, c,
                    batch, stride_values, stride_b, stride_c, stream=None):
    _check(lib().sp_spmm_batched(
        m, k, n, nnz, _ptr(row_indices, _I32, "row_indices", True),
        _ptr(values, _F32, "values", True), _ptr(row_offsets, _I32, "row_offsets"),
        _ptr(col_indices, _I32, "col_indices", True), _ptr(b, _F32, "b", True),
        _ptr(c, _F32, "c"), batch, stride_values, stride_b, stride_c, _stream(stream)),
        "sp_spmm_batched")


def sp_sddmm(m, k, d, nnz, row_indices, row_offsets, col_indices, x, y, out, stream=None):
    _check(lib().sp_sddmm(
        m, k, d, nnz, _ptr(row_indices, _I32, "row_indices", True),
        _ptr(row_offsets, _I32, "row_offsets"), _ptr(col_indices, _I32, "col_indices", True),
        _ptr(x, _F32, "x", True), _ptr(y, _F32, "y", True),
        _ptr(out, _F32, "out", True), _stream(stream)), "sp_sddmm")


def sp_sddmm_balanced(m, k, d, nnz, row_indices, row_offsets, col_indices, x, y, out,
                      stream=None):
    _check(lib().sp_sddmm_balanced(
        m, k, d, nnz, _ptr(row_indices, _I32, "row_indices", True),
        _ptr(row_offsets, _I32, "row_offsets"), _ptr(col_indices, _I32, "col_indices", True),
        _ptr(x, _F32, "x", True), _ptr(y, _F32, "y", True),
        _ptr(out, _F32, "out", True), _stream(stream)), "sp_sddmm_balanced")


def sp_sddmm_batched(m, k, d, nnz, row_indices, row_offsets, col_indices, x, y, alpha,
                     out, batch, stride_x, stride_y, stride_out, stream=None):
    _check(lib().sp_sddmm_batched(
        m, k, d, nnz, _ptr(row_indices, _I32, "row_indices", True),
        _ptr(row_offsets, _I32, "row_offsets"), _ptr(col_indices, _I32, "col_indices", True),
        _ptr(x, _F32, "x", True), _ptr(y, _F32, "y", True), float(alpha),
        _ptr(out, _F32, "out", True), batch, stride_x, stride_y, stride_out,
        _stream(stream)), "sp_sddmm_batched")


def sp_sddmm_general(m, k, d, nnz, row_indices, row_offsets, col_indices, mask_values, x, y,
                     y_layout, alpha, beta, out, batch=1, stride_values=0, stride_x=0,
                     stride_y=0, stride_out=0, workspace=None, stream=None):
    """workspace: None, or a uint8 device tensor of at least
    sp_sddmm_general_workspace bytes (used with SP_Y_DK only)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().sp_sddmm_general(
        m, k, d, nnz, _ptr(row_indices, _I32, "row_indices", True),
        _ptr(row_offsets, _I32, "row_offsets"), _ptr(col_indices, _I32, "col_indices", True),
        _ptr(mask_values, _F32, "mask_values", True), _ptr(x, _F32, "x", True),
        _ptr(y, _F32, "y", True), int(y_layout), float(alpha), float(beta),
        _ptr(out, _F32, "out", True), batch, stride_values, stride_x, stride_y, stride_out,
        _ptr(workspace, _U8, "workspace", True), ws_bytes, _stream(stream)),
        "sp_sddmm_general")


def sp_sddmm_general_workspace(k, d, batch=1, stride_y=0) -> int:
    size = ctypes.c_size_t(0)
    _check(lib().sp_sddmm_general_workspace(k, d, batch, stride_y, ctypes.byref(size)),
           "sp_sddmm_general_workspace")
    return size.value


def sp_csr_transpose_workspace(m, k, nnz) -> int:
    size = ctypes.c_size_t(0)
    _check(lib().sp_csr_transpose_workspace(m, k, nnz, ctypes.byref(size)),
           "sp_csr_transpose_workspace")
    return size.value


def sp_csr_transpose(m, k, nnz, row_offsets, col_indices, values, t_row_offsets,
                     t_col_indices, t_values, t_perm, workspace, stream=None):
    """workspace: a uint8 device tensor of at least sp_csr_transpose_workspace bytes."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().sp_csr_transpose(
        m, k, nnz, _ptr(row_offsets, _I32, "row_offsets"),
        _ptr(col_indices, _I32, "col_indices", True), _ptr(values, _F32, "values", True),
        _ptr(t_row_offsets, _I32, "t_row_offsets"),
        _ptr(t_col_indices, _I32, "t_col_indices", True),
        _ptr(t_values, _F32, "t_values", True), _ptr(t_perm, _I32, "t_perm", True),
        _ptr(workspace, _U8, "workspace", True), ws_bytes, _stream(stream)),
        "sp_csr_transpose")


def sp_csr_transpose_values(nnz, t_perm, values, t_values, stream=None):
    _check(lib().sp_csr_transpose_values(
        nnz, _ptr(t_perm, _I32, "t_perm", True), _ptr(values, _F32, "values", True),
        _ptr(t_values, _F32, "t_values", True), _stream(stream)), "sp_csr_transpose_values")


def sp_spmm_balanced(m, k, n, nnz, row_indices, values, row_offsets, col_indices, b, c,
                     stream=None):
    _check(lib().sp_spmm_balanced(
        m, k, n, nnz, _ptr(row_indices, _I32, "row_indices", True),
        _ptr(values, _F32, "values", True), _ptr(row_offsets, _I32, "row_offsets"),
        _ptr(col_indices, _I32, "col_indices", True), _ptr(b, _F32, "b", True),
        _ptr(c, _F32, "c"), _stream(stream)), "sp_spmm_balanced")


def sp_spmm_kernel_name(m, k, n, nnz, values, col_indices, b, c, batch=1, stride_values=0,
                        stride_b=0, stride_c=0, dtype=None, row_indices=None) -> str:
    """The kernel sp_spmm_ex would run for these tensors (sizes, alignment,
    and whether a row order is given)."""
    if dtype is None:
        dtype = {torch.float32: SP_DTYPE_F32, torch.float16: SP_DTYPE_F16,
                 torch.bfloat16: SP_DTYPE_BF16}[b.dtype]
    name = ctypes.c_char_p()
    addr = lambda t: ctypes.c_void_p(t.data_ptr() if t is not None else None)
    _check(lib().sp_spmm_kernel_name(m, k, n, nnz, addr(row_indices), dtype, addr(values),
                                     addr(col_indices), addr(b), addr(c), batch, stride_values,
                                     stride_b, stride_c, ctypes.byref(name)),
           "sp_spmm_kernel_name")
    return name.value.decode()


def sp_sddmm_kernel_name(m, k, d, nnz, x, y, batch=1, stride_x=0, stride_y=0, stride_out=0,
                         mask_values=None, stride_values=0, beta=0.0, y_layout=SP_Y_KD,
                         workspace=None, dtype=None) -> str:
    """The kernel sp_sddmm_general would run for these tensors (sizes,
    alignment, mask values, beta, Y's layout and the workspace)."""
    if dtype is None:
        dtype = {torch.float32: SP_DTYPE_F32, torch.float16: SP_DTYPE_F16,
                 torch.bfloat16: SP_DTYPE_BF16}[x.dtype]
    name = ctypes.c_char_p()
    addr = lambda t: ctypes.c_void_p(t.data_ptr() if t is not None else None)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().sp_sddmm_kernel_name(m, k, d, nnz, dtype, addr(mask_values), addr(x), addr(y),
                                      y_layout, float(beta), batch, stride_values, stride_x,
                                      stride_y, stride_out, addr(workspace), ws_bytes,
                                      ctypes.byref(name)),
           "sp_sddmm_kernel_name")
    return name.value.decode()


def sp_spmm_sddmm(m, k, n, nnz, row_indices, values, row_offsets, col_indices, b, c,
                  s_m, s_k, d, s_nnz, s_row_indices, s_row_offsets, s_col_indices, x, y, alpha,
                  out, stream=None):
    """sp_spmm(...) and sp_sddmm(...) as one launch where possible."""
    _check(lib().sp_spmm_sddmm(
        m, k, n, nnz, _ptr(row_indices, _I32, "row_indices", True),
        _ptr(values, _F32, "values", True), _ptr(row_offsets, _I32, "row_offsets", True),
        _ptr(col_indices, _I32, "col_indices", True), _ptr(b, _F32, "b", True),
        _ptr(c, _F32, "c", True), s_m, s_k, d, s_nnz,
        _ptr(s_row_indices, _I32, "s_row_indices", True),
        _ptr(s_row_offsets, _I32, "s_row_offsets", True),
        _ptr(s_col_indices, _I32, "s_col_indices", True), _ptr(x, _F32, "x", True),
        _ptr(y, _F32, "y", True), float(alpha), _ptr(out, _F32, "out", True),
        _stream(stream)), "sp_spmm_sddmm")


_DTYPE_CODES = {torch.float32: SP_DTYPE_F32, torch.float16: SP_DTYPE_F16,
                torch.bfloat16: SP_DTYPE_BF16}


def _dtype_of(*tensors) -> int:
    """The one element type shared by the non-None tensors."""
    kinds = {t.dtype for t in tensors if t is not None}
    if len(kinds) != 1 or next(iter(kinds)) not in _DTYPE_CODES:
        raise ValueError(f"operands must share one of float32/float16/bfloat16, got {kinds}")
    return _DTYPE_CODES[next(iter(kinds))]


def sp_spmm_ex(m, k, n, nnz, row_indices, values, row_offsets, col_indices, b, c, batch=1,
               stride_values=0, stride_b=0, stride_c=0, stream=None):
    """SpMM with values and B in float32, float16 or bfloat16 (one type); C float32."""
    code = _dtype_of(values, b)
    dt = [k_ for k_, v in _DTYPE_CODES.items() if v == code][0]
    _check(lib().sp_spmm_ex(
        m, k, n, nnz, _ptr(row_indices, _I32, "row_indices", True), code,
        _ptr(values, dt, "values", True), _ptr(row_offsets, _I32, "row_offsets"),
        _ptr(col_indices, _I32, "col_indices", True), _ptr(b, dt, "b", True),
        _ptr(c, _F32, "c"), batch, stride_values, stride_b, stride_c, _stream(stream)),
        "sp_spmm_ex")


def sp_sddmm_ex(m, k, d, nnz, row_indices, row_offsets, col_indices, x, y, alpha, out,
                batch=1, stride_x=0, stride_y=0, stride_out=0, stream=None):
    """SDDMM with X and Y in float32, float16 or bfloat16 (one type); out float32."""
    code = _dtype_of(x, y)
    dt = [k_ for k_, v in _DTYPE_CODES.items() if v == code][0]
    _check(lib().sp_sddmm_ex(
        m, k, d, nnz, _ptr(row_indices, _I32, "row_indices", True),
        _ptr(row_offsets, _I32, "row_offsets"), _ptr(col_indices, _I32, "col_indices", True),
        code, _ptr(x, dt, "x", True), _ptr(y, dt, "y", True), float(alpha),
        _ptr(out, _F32, "out", True), batch, stride_x, stride_y, stride_out, _stream(stream)),
        "sp_sddmm_ex")


def sp_sddmm_softmax(m, k, d, nnz, row_indices, row_offsets, col_indices, x, y, alpha, out,
                     batch=1, stride_x=0, stride_y=0, stride_out=0, stream=None):
    """Row softmax of alpha * (X Y^T) at the mask, X and Y float32/float16/bfloat16."""
    code = _dtype_of(x, y)
    dt = [k_ for k_, v in _DTYPE_CODES.items() if v == code][0]
    _check(lib().sp_sddmm_softmax(
        m, k, d, nnz, _ptr(row_indices, _I32, "row_indices", True),
        _ptr(row_offsets, _I32, "row_offsets"), _ptr(col_indices, _I32, "col_indices", True),
        code, _ptr(x, dt, "x", True), _ptr(y, dt, "y", True), float(alpha),
        _ptr(out, _F32, "out", True), batch, stride_x, stride_y, stride_out, _stream(stream)),
        "sp_sddmm_softmax")


def sp_sparse_attention(m, k, d, nnz, row_indices, row_offsets, col_indices, q, kmat, v,
                        alpha, out, batch=1, stride_q=0, stride_k=0, stride_v=0, stride_out=0,
                        stream=None):
    """softmax(alpha * Q K^T at the mask) V in one pass; Q, K, V one of
    float32/float16/bfloat16, out float32."""
    code = _dtype_of(q, kmat, v)
    dt = [k_ for k_, v_ in _DTYPE_CODES.items() if v_ == code][0]
    _check(lib().sp_sparse_attention(
        m, k, d, nnz, _ptr(row_indices, _I32, "row_indices", True),
        _ptr(row_offsets, _I32, "row_offsets"), _ptr(col_indices, _I32, "col_indices", True),
        code, _ptr(q, dt, "q", True), _ptr(kmat, dt, "kmat", True), _ptr(v, dt, "v", True),
        float(alpha), _ptr(out, _F32, "out", True), batch, stride_q, stride_k, stride_v,
        stride_out, _stream(stream)), "sp_sparse_attention")


def sp_csr_row_softmax(m, nnz, row_indices, row_offsets, inp, out, batch=1, stride_in=0,
                       stride_out=0, stream=None):
    _check(lib().sp_csr_row_softmax(
        m, nnz, _ptr(row_indices, _I32, "row_indices", True),
        _ptr(row_offsets, _I32, "row_offsets"), _ptr(inp, _F32, "in", True),
        _ptr(out, _F32, "out", True), batch, stride_in, stride_out, _stream(stream)),
        "sp_csr_row_softmax")


# ---------------------------------------------------------------- conveniences

@dataclass
class CsrMatrix:
    """A CSR matrix resident on the device (int32 indices, fp32 values)."""
    m: int
    k: int
    row_offsets: torch.Tensor            # int32[m+1]
    col_indices: torch.Tensor            # int32[nnz]
    values: torch.Tensor | None          # fp32[nnz], or None for a bare mask
    row_indices: torch.Tensor | None = None  # int32[m] swizzled order, or None

    @property
    def nnz(self) -> int:
        return int(self.col_indices.numel())


def csr_from_row_lengths(lengths, col_indices, values, k, stream=None) -> CsrMatrix:
    """CSR from per-row lengths plus the rows' concatenated column lists."""
    m = int(lengths.numel())
    ro = torch.empty(m + 1, dtype=_I32, device=lengths.device)
    sp_csr_offsets_from_lengths(m, lengths, ro, stream)
    return CsrMatrix(m, k, ro, col_indices, values)


def csr_from_dense(mask, dense_values=None, stream=None) -> CsrMatrix:
    """CSR of a dense byte mask: count + prefix sum, a host read of nnz to size
    the entry arrays, then the ordered fill."""
    m, k = mask.shape
    ro = torch.empty(m + 1, dtype=_I32, device=mask.device)
    sp_csr_count_dense(m, k, mask, ro, stream)
    nnz = int(ro[m].item())
    ci = torch.empty(nnz, dtype=_I32, device=mask.device)
    vals = (torch.empty(nnz, dtype=_F32, device=mask.device)
            if dense_values is not None else None)
    sp_csr_fill_dense(m, k, mask, dense_values, ro, ci, vals, stream)
    return CsrMatrix(m, k, ro, ci, vals)


def row_swizzle(a: CsrMatrix, stream=None) -> torch.Tensor:
    ri = torch.empty(a.m, dtype=_I32, device=a.row_offsets.device)
    sp_row_swizzle(a.m, a.row_offsets, ri, stream)
    a.row_indices = ri
    return ri


def spmm(a: CsrMatrix, b: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """C = A B using a.row_indices as the row order when set."""
    k, n = b.shape
    if k != a.k:
        raise ValueError(f"B has {k} rows, A has {a.k} columns")
    c = out if out is not None else torch.empty(a.m, n, dtype=_F32, device=b.device)
    sp_spmm(a.m, a.k, n, a.nnz, a.row_indices, a.values, a.row_offsets, a.col_indices,
            b, c, stream)
    return c


def sddmm(mask: CsrMatrix, x: torch.Tensor, y: torch.Tensor, alpha: float = 1.0,
          out=None, stream=None) -> torch.Tensor:
    """alpha * (X Y^T) at mask's entries, with Y given k x d."""
    m, d = x.shape
    if m != mask.m or y.shape != (mask.k, d):
        raise ValueError("shape mismatch between mask, x and y")
    o = out if out is not None else torch.empty(mask.nnz, dtype=_F32, device=x.device)
    sp_sddmm_batched(mask.m, mask.k, d, mask.nnz, mask.row_indices, mask.row_offsets,
                     mask.col_indices, x, y, alpha, o, 1, 0, 0, 0, stream)
    return o
