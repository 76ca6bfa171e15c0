"""Seeded synthetic inputs for the CSR SpMM / SDDMM workloads.

This module holds none of the method's arithmetic.  It only draws structure
(per-row column sets or dense masks) and dense operands, with numpy's PCG64,
and reports descriptive row statistics.  The oracle tests and the HIP path's
tests and bench both take their inputs from here; nothing here imports either
side.

Stand-ins.  The pages measure on 3,012 pruned DL weight matrices and on the
SuiteSparse collection ("Key points", Dataset and Matrix properties of the
summary card of "Sparse GPU Kernels for Deep Learning"); neither is available,
so each workload below is a seeded synthetic matrix with the shape, sparsity
and row-length spread of one of the pages' DL workloads: long, uniform rows
(low row-length CoV), Transformer and ResNet-50 weights, an LSTM-sized sweep
("Key points", Break-even point) and a sparse-attention mask (I3).

RNG.  Every workload seeds ``numpy.random.SeedSequence(seed)`` and spawns one
child stream per drawn array, in the order listed in the workload's
``_streams`` call, so adding an array never changes the others.  Normal
parameters are (mean, standard deviation).  Rounded row lengths use
``numpy.rint`` (round half to even) and are clipped to [1, k].
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

DEFAULT_SEED = 0


def _streams(seed: int, names):
    kids = np.random.SeedSequence(seed).spawn(len(names))
    return {nm: np.random.Generator(np.random.PCG64(kid))
            for nm, kid in zip(names, kids)}


@dataclass
class RowLists:
    """Sparse structure as per-row sorted column lists (not yet CSR).

    ``lengths[i]`` entries belong to row i; ``cols``/``values`` hold the rows'
    entries one row after another, each row's columns strictly ascending.
    Turning this into CSR row offsets is the CSR-build step of the method.
    """
    m: int
    k: int
    lengths: np.ndarray   # int32[m]
    cols: np.ndarray      # int32[nnz]
    values: np.ndarray    # float32[nnz]

    @property
    def nnz(self) -> int:
        return int(self.cols.shape[0])


def sample_columns(rng: np.random.Generator, lengths: np.ndarray, k: int,
                   max_keys: int = 1 << 24) -> np.ndarray:
    """For each row i, ``lengths[i]`` distinct columns of [0, k) chosen
    uniformly without replacement, sorted ascending; rows concatenated.

    Each row draws k independent uniform keys; the columns whose key ranks
    below the row length are the chosen set (a uniformly random subset)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    m = lengths.shape[0]
    if m == 0 or k == 0:
        return np.zeros(0, np.int32)
    rows_per_chunk = max(1, max_keys // k)
    pieces = []
    ramp = np.arange(k, dtype=np.int32)
    for r0 in range(0, m, rows_per_chunk):
        r1 = min(m, r0 + rows_per_chunk)
        keys = rng.random((r1 - r0, k))
        order = np.argsort(keys, axis=1)
        rank = np.empty_like(order, dtype=np.int32)
        np.put_along_axis(rank, order,
                          np.broadcast_to(ramp, order.shape), axis=1)
        chosen = rank < lengths[r0:r1, None]
        pieces.append(np.nonzero(chosen)[1].astype(np.int32))
    return np.concatenate(pieces)


def normal_lengths(rng, m: int, k: int, mean: float, cov: float) -> np.ndarray:
    """round(Normal(mean, cov*mean)) clipped to [1, k]."""
    raw = rng.normal(mean, cov * mean, size=m)
    return np.clip(np.rint(raw), 1, k).astype(np.int32)


def lognormal_lengths(rng, m: int, k: int, mean: float, cov: float) -> np.ndarray:
    """round(LogNormal) with arithmetic mean `mean` and CoV `cov`, clipped to
    [1, k].  sigma_ln^2 = ln(1 + cov^2), mu_ln = ln(mean) - sigma_ln^2 / 2."""
    s2 = math.log1p(cov * cov)
    raw = rng.lognormal(math.log(mean) - s2 / 2.0, math.sqrt(s2), size=m)
    return np.clip(np.rint(raw), 1, k).astype(np.int32)


def row_lists(rng_cols, rng_vals, m: int, k: int, lengths: np.ndarray,
              value_std: float) -> RowLists:
    """Row lists with the given lengths: uniform column sets, N(0, value_std) values."""
    cols = sample_columns(rng_cols, lengths, k)
    vals = rng_vals.normal(0.0, value_std, size=cols.shape[0]).astype(np.float32)
    return RowLists(m, k, lengths.astype(np.int32), cols, vals)


def bernoulli_mask(rng, m: int, k: int, p: float) -> np.ndarray:
    """Each of the m*k positions kept independently with probability p."""
    return (rng.random((m, k)) < p).astype(np.uint8)


def normal(rng, shape, std: float = 1.0) -> np.ndarray:
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
            if std != 1.0 else rng.standard_normal(shape, dtype=np.float32))


def attention_mask(seq: int = 4096, band: int = 64, stride: int = 128) -> np.ndarray:
    """Causal local-band plus strided mask: position (i, j) is kept when j <= i
    and either i - j < band (the band, self included) or j % stride == 0."""
    i = np.arange(seq, dtype=np.int32)[:, None]
    j = np.arange(seq, dtype=np.int32)[None, :]
    keep = (j <= i) & (((i - j) < band) | ((j % stride) == 0))
    return keep.astype(np.uint8)


def row_stats(lengths: np.ndarray, k: int) -> dict:
    """Sparsity, mean row length and row-length coefficient of variation: the
    per-matrix statistics the pages profile ("Key points", Matrix properties;
    I1, I2)."""
    lengths = np.asarray(lengths, dtype=np.float64)
    m = lengths.shape[0]
    nnz = float(lengths.sum())
    mean = nnz / m if m else 0.0
    std = float(lengths.std()) if m else 0.0
    return {"m": m, "k": k, "nnz": int(nnz),
            "sparsity": 1.0 - nnz / (m * k) if m * k else 0.0,
            "mean_row_length": mean,
            "row_length_cov": std / mean if mean else 0.0}


# --------------------------------------------------------------------------
# The workloads
# --------------------------------------------------------------------------

def tiny(seed: int = DEFAULT_SEED) -> dict:
    """Tiny SpMM + SDDMM: A 256x256, each element kept with p = 0.2, values
    N(0,1); B 256x64; SDDMM on the same mask with X, Y 256x32; all N(0,1)."""
    r = _streams(seed, ["mask", "a_values", "b", "x", "y"])
    m = k = 256
    return {
        "name": "tiny_256x256_p0.2",
        "m": m, "k": k, "n": 64, "d": 32,
        "mask": bernoulli_mask(r["mask"], m, k, 0.2),
        "dense_values": normal(r["a_values"], (m, k)),
        "b": normal(r["b"], (k, 64)),
        "x": normal(r["x"], (m, 32)),
        "y": normal(r["y"], (k, 32)),
    }


def transformer_ffn(seed: int = DEFAULT_SEED, m: int = 2048, k: int = 512,
                    n: int = 256, sparsity: float = 0.9, cov: float = 0.1,
                    lognormal: bool = False) -> dict:
    """Transformer-FFN-like SpMM at 90 % sparsity: A 2048x512, row lengths
    round(N(51.2, 5.12)) in [1, 512], columns uniform without replacement,
    values N(0, 0.02); B 512x256 N(0,1).  Companion SDDMM on A's mask:
    dA = (dY X^T) at A's entries with dY 2048x256 and X 512x256, N(0,1).
    With ``lognormal=True`` the row lengths are lognormal with the same mean
    and CoV ``cov`` (the row-imbalance stress workload uses cov = 0.5)."""
    r = _streams(seed, ["lengths", "cols", "values", "b", "dy", "x"])
    mean = (1.0 - sparsity) * k
    lengths = (lognormal_lengths if lognormal else normal_lengths)(
        r["lengths"], m, k, mean, cov)
    a = row_lists(r["cols"], r["values"], m, k, lengths, 0.02)
    tag = "lognormal" if lognormal else "normal"
    return {
        "name": f"transformer_ffn_{m}x{k}x{n}_s{sparsity:g}_{tag}_cov{cov:g}",
        "m": m, "k": k, "n": n, "d": n,
        "a": a,
        "b": normal(r["b"], (k, n)),
        "x": normal(r["dy"], (m, n)),   # dY: SDDMM left operand, m x d
        "y": normal(r["x"], (k, n)),    # X: SDDMM right operand, k x d
    }


def resnet_1x1(seed: int = DEFAULT_SEED) -> dict:
    """ResNet-50-like 1x1-conv SpMM: A 1024x256 at 70 % sparsity, row lengths
    round(N(76.8, 3.84)) in [1, 256], values N(0, 0.05); B 256x6272
    (32 images x 14x14 positions as columns) N(0,1)."""
    r = _streams(seed, ["lengths", "cols", "values", "b"])
    m, k, n = 1024, 256, 6272
    lengths = normal_lengths(r["lengths"], m, k, 0.3 * k, 0.05)
    a = row_lists(r["cols"], r["values"], m, k, lengths, 0.05)
    return {"name": "resnet50_1x1_1024x256x6272_s0.7", "m": m, "k": k, "n": n,
            "a": a, "b": normal(r["b"], (k, n))}


LSTM_SPARSITIES = (0.5, 0.6, 0.7, 0.8, 0.9, 0.95, 0.98)


def lstm(sparsity: float, seed: int = DEFAULT_SEED) -> dict:
    """LSTM-sized SpMM: A 8192x2048 (4 gates x hidden 2048 by input 2048) at the
    given sparsity, row lengths round(N(mu, 0.1 mu)) in [1, 2048] with
    mu = (1 - sparsity) * 2048, values N(0, 0.02); B 2048x128 N(0,1)."""
    r = _streams(seed, ["lengths", "cols", "values", "b"])
    m, k, n = 8192, 2048, 128
    lengths = normal_lengths(r["lengths"], m, k, (1.0 - sparsity) * k, 0.1)
    a = row_lists(r["cols"], r["values"], m, k, lengths, 0.02)
    return {"name": f"lstm_8192x2048x128_s{sparsity:g}", "m": m, "k": k, "n": n,
            "sparsity": sparsity, "a": a, "b": normal(r["b"], (k, n))}


def sparse_attention(seed: int = DEFAULT_SEED, batch: int = 2, heads: int = 16,
                     seq: int = 4096, head_dim: int = 64) -> dict:
    """Sparse attention: batch 2 x 16 heads, seq 4096, head dim 64; Q, K, V
    N(0,1) as [batch*heads, seq, head_dim]; one causal 64-token-band plus
    every-128th-column mask shared by all (batch, head) pairs."""
    r = _streams(seed, ["q", "k", "v"])
    bh = batch * heads
    return {"name": f"sparse_attention_b{batch}h{heads}_s{seq}_d{head_dim}",
            "batch": bh, "seq": seq, "head_dim": head_dim,
            "mask": attention_mask(seq),
            "q": normal(r["q"], (bh, seq, head_dim)),
            "k": normal(r["k"], (bh, seq, head_dim)),
            "v": normal(r["v"], (bh, seq, head_dim))}


def imbalance(seed: int = DEFAULT_SEED) -> dict:
    """Row-imbalance stress: the Transformer-FFN SpMM shape with lognormal row
    lengths of CoV 0.5 (mean 51.2)."""
    return transformer_ffn(seed, lognormal=True, cov=0.5)


def hbm_stream(seed: int = DEFAULT_SEED, m: int = 65536, k: int = 8192,
               n: int = 8, sparsity: float = 0.9) -> dict:
    """A streaming-regime SpMM at 90 % sparsity whose CSR (about 430 MB) is far
    larger than every on-chip cache, with a narrow dense operand (n = 8, or
    n = 4 so that B fits in a CU's LDS): row lengths round(N(819.2, 81.92)),
    values N(0, 0.02), B 8192xn N(0,1)."""
    r = _streams(seed, ["lengths", "cols", "values", "b"])
    lengths = normal_lengths(r["lengths"], m, k, (1.0 - sparsity) * k, 0.1)
    a = row_lists(r["cols"], r["values"], m, k, lengths, 0.02)
    # B is drawn at its widest (8 columns) and narrowed, so every n shares A.
    b = normal(r["b"], (k, 8))[:, :n] if n <= 8 else normal(r["b"], (k, n))
    return {"name": f"hbm_stream_{m}x{k}x{n}_s{sparsity:g}", "m": m, "k": k,
            "n": n, "a": a, "b": np.ascontiguousarray(b)}


def random_row_lists(seed: int, m: int, k: int, lengths) -> RowLists:
    """Small test structure with the given row lengths, values N(0,1)."""
    r = _streams(seed, ["cols", "values"])
    lengths = np.asarray(lengths, dtype=np.int32)
    cols = sample_columns(r["cols"], lengths, k)
    vals = r["values"].standard_normal(cols.shape[0], dtype=np.float32)
    return RowLists(m, k, lengths, cols, vals)


def random_dense(seed: int, *shape, std: float = 1.0) -> np.ndarray:
    return normal(_streams(seed, ["x"])["x"], shape, std)
