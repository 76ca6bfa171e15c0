"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np
import torch

import oracle

# Per fp32 output element: |gpu - oracle| <= REL * sum |a_ik * b_kj| (for SDDMM,
# sum |x_il * y_jl|), the oracle summing exactly-formed products in double.
REL = 1e-5
DEV = "cuda"


def note(msg: str) -> None:
    """Name the case about to run on the GPU, flushed, so a failure that ends
    the process still says what was running."""
    sys.stdout.write(f"\n[gpu case] {msg}\n")
    sys.stdout.flush()


def dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check_close(gpu: np.ndarray, ref: np.ndarray, absum: np.ndarray, what: str) -> float:
    """Assert the stated tolerance element by element; return the worst
    |gpu - oracle| / bound over elements with a nonzero bound."""
    g = gpu.astype(np.float64).reshape(ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref)
    bound = REL * absum
    bad = err > bound
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), 0.0)
    worst = float(ratio.max()) if ratio.size else 0.0
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} elements outside "
                           f"1e-5*sum|a*b|; worst ratio {worst:.3g}")
    return worst


class DevCsr:
    """A CSR structure (and optional values) uploaded to the device, plus the
    host copies the oracle reads."""

    def __init__(self, m, k, row_offsets, col_indices, values=None):
        self.m, self.k = m, k
        self.ro = np.ascontiguousarray(row_offsets, np.int32)
        self.ci = np.ascontiguousarray(col_indices, np.int32)
        self.vals = None if values is None else np.ascontiguousarray(values, np.float32)
        self.d_ro = dev(self.ro)
        self.d_ci = dev(self.ci)
        self.d_vals = None if values is None else dev(self.vals)

    @property
    def nnz(self):
        return int(self.ci.shape[0])


def csr_of_row_lists(rl) -> DevCsr:
    return DevCsr(rl.m, rl.k, oracle.csr_offsets_from_lengths(rl.lengths), rl.cols,
                  rl.values)
