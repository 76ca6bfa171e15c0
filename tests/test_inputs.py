"""The seeded generators: determinism and the statistics each workload claims."""
import math

import numpy as np

import oracle
from unstructured_sparse_linear_csr_amd import inputs


def test_determinism_per_seed():
    a = inputs.transformer_ffn(seed=3)
    b = inputs.transformer_ffn(seed=3)
    c = inputs.transformer_ffn(seed=4)
    for key in ("b", "x", "y"):
        assert np.array_equal(a[key], b[key])
    assert np.array_equal(a["a"].cols, b["a"].cols)
    assert np.array_equal(a["a"].values, b["a"].values)
    assert not np.array_equal(a["a"].lengths, c["a"].lengths)


def _check_row_lists(rl):
    ro = oracle.csr_offsets_from_lengths(rl.lengths)
    assert oracle.csr_check(rl.m, rl.k, ro, rl.cols) == 0
    assert rl.values.dtype == np.float32 and rl.values.shape == rl.cols.shape
    assert rl.lengths.min() >= 1 and rl.lengths.max() <= rl.k
    return ro


def test_tiny_bernoulli_nnz():
    w = inputs.tiny()
    nnz = oracle.mask_nnz(w["mask"])
    sigma = math.sqrt(256 * 256 * 0.2 * 0.8)
    assert abs(nnz - 13107.2) < 5 * sigma
    assert w["b"].shape == (256, 64) and w["x"].shape == (256, 32)


def test_transformer_ffn_statistics():
    w = inputs.transformer_ffn()
    _check_row_lists(w["a"])
    st = inputs.row_stats(w["a"].lengths, w["k"])
    # mean 51.2, sd 5.12 over 2048 rows: standard error of the mean 0.113
    assert abs(st["mean_row_length"] - 51.2) < 0.6
    assert abs(st["row_length_cov"] - 0.1) < 0.01
    assert abs(st["sparsity"] - 0.9) < 0.002
    assert w["x"].shape == (2048, 256) and w["y"].shape == (512, 256)
    v = w["a"].values
    assert abs(float(v.std()) - 0.02) < 0.001


def test_imbalance_lognormal_statistics():
    w = inputs.imbalance()
    _check_row_lists(w["a"])
    st = inputs.row_stats(w["a"].lengths, w["k"])
    assert abs(st["mean_row_length"] - 51.2) < 2.9   # 5 standard errors
    assert abs(st["row_length_cov"] - 0.5) < 0.08


def test_resnet_statistics():
    w = inputs.resnet_1x1()
    _check_row_lists(w["a"])
    st = inputs.row_stats(w["a"].lengths, w["k"])
    assert abs(st["sparsity"] - 0.7) < 0.002
    assert abs(st["row_length_cov"] - 0.05) < 0.01
    assert w["b"].shape == (256, 6272)


def test_lstm_statistics_at_90_percent():
    w = inputs.lstm(0.9)
    _check_row_lists(w["a"])
    st = inputs.row_stats(w["a"].lengths, w["k"])
    assert abs(st["sparsity"] - 0.9) < 0.001
    assert abs(st["row_length_cov"] - 0.1) < 0.01


def test_sample_columns_uniform_marginals():
    # Every column is equally likely: with 4000 rows choosing 5 of 10, each
    # column is chosen about 2000 times (binomial sd ~ 31.6).
    rng = np.random.default_rng(5)
    cols = inputs.sample_columns(rng, np.full(4000, 5), 10)
    counts = np.bincount(cols, minlength=10)
    assert np.all(np.abs(counts - 2000) < 5 * 31.7)


def test_attention_mask_rows():
    mask = inputs.attention_mask(4096)
    lengths = mask.sum(axis=1)
    assert lengths[0] == 1 and lengths.min() >= 1
    assert lengths[4095] == 64 + 32        # band of 64 plus j=0..3968 step 128 below it
    assert np.all(np.triu(mask, 1) == 0)   # causal
    assert np.all(np.diag(mask) == 1)      # the diagonal is always in the band
