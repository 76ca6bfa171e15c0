"""Measured ceilings for the roofline figures (``libsp_probes.so``).

stream_read_gbs: the HBM read bandwidth a plain kernel reaches streaming an
array of the given size with 16-byte loads (best over a few grid sizes).
row_gather_tbs: the rate at which waves gather 1 KB rows of an L2-resident
matrix at random offsets, as the SpMM and SDDMM kernels gather rows of B and
Y, without their arithmetic.  launch_floor_us: the average duration of an
empty kernel launched back to back from a HIP graph.  All timed with events on
the launch stream over graph replays.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import PROBE_LIB

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_LIB):
            raise ImportError(f"{PROBE_LIB} is not built (python -m unstructured_sparse_linear_csr_amd.build)")
        import torch  # noqa: F401  (torch's HIP runtime first, as the main binding does)
        l = ctypes.CDLL(PROBE_LIB)
        vp, ci, cll = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong
        l.sp_probe_stream_read.argtypes = [vp, cll, ci, vp, vp]
        l.sp_probe_stream_read2.argtypes = [vp, vp, cll, ci, vp, vp]
        l.sp_probe_row_gather.argtypes = [vp, ci, ci, vp, ctypes.c_uint, vp, vp]
        l.sp_probe_empty.argtypes = [ci, vp]
        for f in (l.sp_probe_stream_read, l.sp_probe_stream_read2, l.sp_probe_row_gather,
                  l.sp_probe_empty):
            f.restype = ci
        _lib = l
    return _lib


def _check(code: int, what: str) -> None:
    if code != 0:
        raise RuntimeError(f"{what} failed with hipError {code}")


def _graph_us(torch, fn, reps: int) -> float:
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    best = float("inf")
    for _ in range(3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e3 / reps)
    return best


def measure(torch, stream_bytes: int, b_bytes: int = 512 * 1024, seed: int = 0) -> dict:
    l = lib()
    dev = "cuda"
    cs = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    a = torch.zeros(stream_bytes // 16 * 16, dtype=torch.uint8, device=dev)
    best_read = 0.0
    for blocks in (2048, 8192, 16384):
        out = torch.empty(blocks * 256, device=dev)
        us = _graph_us(torch, lambda: _check(l.sp_probe_stream_read(
            ctypes.c_void_p(a.data_ptr()), a.numel(), blocks, ctypes.c_void_p(out.data_ptr()),
            cs()), "sp_probe_stream_read"), 10)
        best_read = max(best_read, a.numel() / (us * 1e-6) / 1e9)
    del a
    # the same bytes as two arrays of half the size, read side by side (a CSR's
    # column indices and values)
    half = stream_bytes // 2 // 16 * 16
    a1 = torch.zeros(half, dtype=torch.uint8, device=dev)
    a2 = torch.zeros(half, dtype=torch.uint8, device=dev)
    best_read2 = 0.0
    for blocks in (2048, 8192, 16384):
        out = torch.empty(blocks * 256, device=dev)
        us = _graph_us(torch, lambda: _check(l.sp_probe_stream_read2(
            ctypes.c_void_p(a1.data_ptr()), ctypes.c_void_p(a2.data_ptr()), half, blocks,
            ctypes.c_void_p(out.data_ptr()), cs()), "sp_probe_stream_read2"), 10)
        best_read2 = max(best_read2, 2 * half / (us * 1e-6) / 1e9)
    del a1, a2
    b = torch.ones(b_bytes // 4, device=dev)
    rng = np.random.default_rng(seed)
    gathers = {}
    for waves, per_wave in ((2048, 51), (4096, 51), (16384, 256)):
        rows = b_bytes // 1024
        offs = torch.from_numpy((rng.integers(0, rows, waves * per_wave) * 1024)
                                .astype(np.uint32)).to(dev)
        out = torch.empty(waves * 64, device=dev)
        us = _graph_us(torch, lambda: _check(l.sp_probe_row_gather(
            ctypes.c_void_p(offs.data_ptr()), waves, per_wave, ctypes.c_void_p(b.data_ptr()),
            b_bytes, ctypes.c_void_p(out.data_ptr()), cs()), "sp_probe_row_gather"), 20)
        gathers[f"{waves}x{per_wave}"] = waves * per_wave * 1024 / (us * 1e-6) / 1e12
    floor = _graph_us(torch, lambda: _check(l.sp_probe_empty(2048, cs()), "sp_probe_empty"), 200)
    return {"stream_read_gbs": best_read, "stream_read2_gbs": best_read2,
            "stream_bytes": stream_bytes,
            "row_gather_tbs": gathers, "row_gather_b_bytes": b_bytes,
            "launch_floor_us": floor,
            "note": "ceilings measured on this GPU by plain probe kernels (libsp_probes.so); "
                    "the roofline's peak stays the published 8 TB/s"}
