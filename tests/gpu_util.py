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


def check_attention(o_gpu, m, k, ro, ci, q, kk, v, alpha, what, rescalings=None):
    """O against the oracle's double pipeline: P's relative error (scores,
    fp32 softmax, the running-maximum rescalings, a few ulps each: one per
    window of 64 entries, or `rescalings` per row when given) times
    sum_j P_j |V_j|, plus the weighted sum's own 1e-5."""
    s, s_abs = oracle.sddmm(m, k, q.shape[1], ro, ci, q, kk)
    s, e_s = alpha * s, abs(alpha) * 1e-5 * s_abs
    p_ref = oracle.softmax_rows(ro, s.astype(np.float32))
    lengths = np.diff(ro)
    rows = np.repeat(np.arange(m), lengths)
    e_row = np.zeros(m)
    np.maximum.at(e_row, rows, e_s)
    smax = np.full(m, -np.inf)
    np.maximum.at(smax, rows, s)
    x_row = np.zeros(m)
    np.maximum.at(x_row, rows, np.abs(s - smax[rows]))
    a_row = np.zeros(m)
    np.maximum.at(a_row, rows, np.abs(s))
    windows = (lengths + 63) // 64 if rescalings is None else rescalings
    rel = (2.0 * e_row + 2.0 * a_row * 2.0 ** -24 + (x_row + 8.0) * 2.0 ** -23
           + 8.0 * windows * 2.0 ** -23 + 1e-5)
    o_ref, _ = oracle.spmm(m, k, q.shape[1], ro, ci, p_ref, v)
    pv, _ = oracle.spmm(m, k, q.shape[1], ro, ci, p_ref, np.abs(v))
    err = np.abs(o_gpu.astype(np.float64) - o_ref)
    bound = rel[:, None] * pv * 1.01 + 2.0 ** -126
    assert np.all(np.isfinite(o_gpu)), what
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} out of bound; worst "
                           f"{np.max(err / np.maximum(bound, 1e-300)):.3g}")
    assert np.all(o_gpu[lengths == 0] == 0.0), f"{what}: empty rows not zero"


def check_scores_softmax(got, m, k, ro, ci, x, y, alpha, what):
    s, s_abs = oracle.sddmm(m, k, x.shape[1], ro, ci, x, y)
    s, e_s = alpha * s, abs(alpha) * 1e-5 * s_abs
    p_ref = oracle.softmax_rows(ro, s.astype(np.float32))
    rows = np.repeat(np.arange(m), np.diff(ro))
    e_row = np.zeros(m)
    np.maximum.at(e_row, rows, e_s)
    smax = np.full(m, -np.inf)
    np.maximum.at(smax, rows, s)
    x_row = np.zeros(m)
    np.maximum.at(x_row, rows, np.abs(s - smax[rows]))
    a_row = np.zeros(m)
    np.maximum.at(a_row, rows, np.abs(s))
    rel = 2.0 * e_row + 2.0 * a_row * 2.0 ** -24 + (x_row + 8.0) * 2.0 ** -23
    bound = p_ref * rel[rows] * 1.01 + 2.0 ** -126
    g = got.astype(np.float64)
    assert np.all(np.isfinite(g)), what
    err = np.abs(g - p_ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} entries out of bound; worst "
                           f"{np.max(err / np.maximum(bound, 1e-300)):.3g}")
    # each nonempty row sums to 1 within the rounding of its entries
    sums = np.zeros(m)
    np.add.at(sums, rows, g)
    nonempty = np.diff(ro) > 0
    assert np.all(np.abs(sums[nonempty] - 1.0) <= 1e-5 + np.diff(ro)[nonempty] * 2.0 ** -22)
