"""The ceiling probes the bench reports beside its roofline: they run, their
results are what their loads imply, and the rates are positive and finite."""
import ctypes
import math

import numpy as np
import pytest
import torch

from unstructured_sparse_linear_csr_amd import probes

from gpu_util import note

pytestmark = pytest.mark.gpu


def test_probe_arithmetic():
    l = probes.lib()
    cs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    note("probe stream read over 1..16 MB")
    a = torch.full((1 << 22,), 0.5, device="cuda")          # 16 MB of 0.5
    out = torch.empty(64 * 256, device="cuda")
    assert l.sp_probe_stream_read(ctypes.c_void_p(a.data_ptr()), a.numel() * 4, 64,
                                  ctypes.c_void_p(out.data_ptr()), cs) == 0
    torch.cuda.synchronize()
    assert out.sum().item() == pytest.approx(0.5 * a.numel(), rel=1e-6)
    note("probe two-array stream read over 8 + 8 MB")
    a2 = torch.full((1 << 21,), 0.25, device="cuda")        # 8 MB of 0.25
    a1 = torch.full((1 << 21,), 0.5, device="cuda")         # 8 MB of 0.5
    assert l.sp_probe_stream_read2(ctypes.c_void_p(a1.data_ptr()), ctypes.c_void_p(a2.data_ptr()),
                                   a1.numel() * 4, 64, ctypes.c_void_p(out.data_ptr()), cs) == 0
    torch.cuda.synchronize()
    assert out.sum().item() == pytest.approx(0.75 * a1.numel(), rel=1e-6)
    assert l.sp_probe_stream_read2(None, None, 16, 1, None, cs) != 0  # host-side check
    note("probe row gather of 1 KB rows")
    b = torch.ones(64 * 1024 // 4, device="cuda")           # 64 rows of 1 KB
    waves, per_wave = 96, 37
    offs = torch.from_numpy((np.random.default_rng(3).integers(0, 64, waves * per_wave) * 1024)
                            .astype(np.uint32)).cuda()
    out = torch.empty(waves * 64, device="cuda")
    assert l.sp_probe_row_gather(ctypes.c_void_p(offs.data_ptr()), waves, per_wave,
                                 ctypes.c_void_p(b.data_ptr()), b.numel() * 4,
                                 ctypes.c_void_p(out.data_ptr()), cs) == 0
    torch.cuda.synchronize()
    assert torch.all(out == 4.0 * per_wave)
    assert l.sp_probe_row_gather(None, 1, 1, None, 1024, None, cs) != 0  # host-side check


def test_probe_measure():
    note("probe measure")
    c = probes.measure(torch, stream_bytes=64 << 20)
    assert math.isfinite(c["stream_read_gbs"]) and c["stream_read_gbs"] > 0
    assert math.isfinite(c["stream_read2_gbs"]) and c["stream_read2_gbs"] > 0
    assert all(math.isfinite(v) and v > 0 for v in c["row_gather_tbs"].values())
    assert 0 < c["launch_floor_us"] < 1000
