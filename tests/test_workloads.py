"""Pins of the synthetic input generators against the figures the pages print.

kompressor BENCHMARKS.md section 4 marshals the y CDF set as 200,512 int32
entries over 64 rows (kompressor README "Getting Started": "64 cdf rows"), so
the padded stride is 3133; the y latent has 1,566,720 symbols (same output
block).  The tables must be valid 16-bit quantised CDFs (torch_ans FAQ: cdf
entries are increasing positive integers) with every frequency at least 1.
"""
import numpy as np
import pytest

import oracle
import workloads as W


def test_gaussian_8_row_lengths():
    _, lengths, offsets, _ = W.gaussian_table_set(8)
    assert lengths.tolist() == [5, 9, 17, 41, 117, 345, 1037, 3133]
    assert offsets.tolist() == [-(l - 3) // 2 for l in lengths.tolist()]


def test_gaussian_64_matches_marshalled_size():
    cdf, lengths, _, scales = W.gaussian_table_set(64)
    assert cdf.shape == (64, 3133)
    assert cdf.size == 200_512
    assert int(lengths.max()) == 3133 and int(lengths.sum()) == 27_256
    assert abs(scales[0] - 0.11) < 1e-12 and abs(scales[-1] - 256.0) < 1e-9


@pytest.mark.parametrize("maker", ["gauss8", "gauss64", "z"])
def test_tables_are_valid_quantised_cdfs(maker):
    if maker == "z":
        w = W.load("z")
        cdf, lengths = w.cdf, w.lengths
        assert cdf.shape == (192, 64) and int(lengths.max()) <= 63
    else:
        cdf, lengths, _, _ = W.gaussian_table_set(8 if maker == "gauss8" else 64)
    assert oracle.check_tables(cdf, lengths) == 0
    for r in range(cdf.shape[0]):
        row = cdf[r, : lengths[r]]
        assert row[0] == 0 and row[-1] == 65536
        assert np.all(np.diff(row) >= 1)
        assert np.all(cdf[r, lengths[r]:] == 65536)


def test_quantiser_keeps_total_and_floor():
    rng = np.random.default_rng(0)
    for _ in range(50):
        p = rng.dirichlet(np.full(rng.integers(2, 300), 0.3))
        f = W.quantise_pmf(p)
        assert f.sum() == 65536 and f.min() >= 1
        # units move only between the largest entries: the small ones keep
        # their rounded value (raised to 1)
        base = np.maximum(np.rint(p * 65536), 1).astype(np.int64)
        small = base < np.sort(base)[-3]
        assert np.array_equal(f[small], base[small])


@pytest.mark.parametrize("name,n,K", [("tiny", 16384, 8), ("z", 97920, 192),
                                      ("y1080", 1566720, 64)])
def test_workload_shapes_and_bypass_rates(name, n, K):
    w = W.load(name, cache=False)
    assert w.n == n and w.num_tables == K
    assert w.symbols.dtype == np.int32 and w.indexes.dtype == np.int32
    assert w.indexes.min() >= 0 and w.indexes.max() < K
    idx = w.indexes.astype(np.int64)
    v = w.symbols.astype(np.int64) - w.offsets[idx]
    bypass = float(((v < 0) | (v >= w.lengths[idx] - 2)).mean())
    expect = {"tiny": 0.01, "z": 0.0088, "y1080": 0.001}[name]
    assert abs(bypass - expect) < 0.2 * expect
    again = W.load(name, cache=False)
    assert np.array_equal(again.symbols, w.symbols) and np.array_equal(again.indexes, w.indexes)


def test_y1080_index_field_statistics():
    w = W.load("y1080")
    idx = w.indexes.astype(np.float64)
    assert abs(idx.mean() - 20.0) < 0.5
    assert 8.5 < idx.std() < 10.5


def test_tiny_carries_the_edge_values():
    w = W.load("tiny")
    idx = w.indexes.astype(np.int64)
    v = w.symbols.astype(np.int64) - w.offsets[idx]
    mv = w.lengths[idx] - 2
    raws = set(np.where(v < 0, -2 * v - 1, np.where(v >= mv, 2 * (v - mv), -1)).tolist())
    assert set(W.EDGE_RAWS) <= raws
