"""Pins of the oracle's table builder (quantised CDFs, discretised Gaussians).

What fixes the expected values:
* golden/quantized_cdfs.txt -- small pmf rows quantised by hand;
* the closed form of the unit-by-unit adjustment (water level), a different
  algorithm from the oracle's loop, on random rows (brute force);
* the Gaussian bin masses integrated from the density by Simpson's rule, with
  no erf/erfc routine involved, quantised by that closed form;
* the longest row of the 64-row y-latent table set, 3133 entries (kompressor
  BENCHMARKS.md, section 4: 200,512 marshalled cdf entries over 64 rows);
* invariants: every row starts at 0, ends at 65536, strictly increases, is
  symmetric about its centre outside the adjusted slots.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
from scipy.special import ndtri

import oracle
from helpers import gaussian_row_by_integration, quantize_water_level, quantized_cases

TAIL_Z = float(ndtri(1.0 - 5e-10))   # two-sided tail mass 1e-9


def log_scales(K, lo=0.11, hi=256.0):
    return np.exp(np.log(lo) + (np.log(hi) - np.log(lo)) * np.arange(K) / (K - 1))


@pytest.mark.parametrize("case", quantized_cases(), ids=lambda c: c[0])
def test_golden_quantisation(case):
    name, pmf, cdf = case
    rc, got = oracle.quantize_pmf(pmf)
    assert rc == 0
    assert got.tolist() == cdf


def test_quantisation_matches_closed_form_on_random_rows():
    rng = np.random.default_rng(11)
    for trial in range(400):
        m = int(rng.integers(2, 40))
        kind = trial % 4
        if kind == 0:      # a proper pmf
            p = rng.dirichlet(np.full(m, 0.3))
        elif kind == 1:    # mass missing: deficit
            p = rng.dirichlet(np.ones(m)) * rng.uniform(0.5, 1.0)
        elif kind == 2:    # too much mass: surplus, often over several slots
            p = np.minimum(rng.dirichlet(np.ones(m)) * rng.uniform(1.0, 3.0), 1.0)
        else:              # many equal entries and exact half-unit ties
            p = (rng.integers(0, 6, m) * 2 + 1) / 2.0 / 65536.0 * rng.integers(1, 4000)
            p = np.minimum(p, 1.0)
        rc, cdf = oracle.quantize_pmf(p)
        assert rc == 0
        f = np.diff(cdf.astype(np.int64))
        assert f.min() >= 1 and cdf[-1] == 65536
        assert np.array_equal(f, quantize_water_level(p)), (trial, p.tolist())


def test_quantisation_refuses_bad_rows():
    assert oracle.quantize_pmf(np.array([0.5, -0.1, 0.6]))[0] == oracle.E_TABLE
    assert oracle.quantize_pmf(np.array([0.5, np.nan, 0.5]))[0] == oracle.E_TABLE
    assert oracle.quantize_pmf(np.array([0.5, 1.5]))[0] == oracle.E_TABLE
    assert oracle.quantize_pmf(np.array([1.0]))[0] == oracle.E_ARG
    assert oracle.quantize_pmf(np.full(65537, 1.0 / 65537))[0] == oracle.E_ARG
    rc, cdf = oracle.quantize_pmf(np.full(65536, 1.0 / 65536))
    assert rc == 0 and np.array_equal(cdf, np.arange(65537))


def test_gaussian_lengths_and_longest_row():
    rc, cdf, lengths, offsets = oracle.gaussian_tables(log_scales(8), TAIL_Z, 3133)
    assert rc == 0
    # c = ceil(s * 6.1094...), length 2c + 3
    assert lengths.tolist() == [5, 9, 17, 41, 117, 345, 1037, 3133]
    assert offsets.tolist() == [-(n - 3) // 2 for n in lengths.tolist()]
    rc, cdf, lengths, _ = oracle.gaussian_tables(log_scales(64), TAIL_Z, 3133)
    assert rc == 0
    assert int(lengths.max()) == 3133 == 200512 // 64
    assert int(lengths.sum()) == 27256


@pytest.mark.parametrize("K,tail_z", [(8, TAIL_Z), (64, TAIL_Z), (12, 1.0), (9, 2.5)])
def test_gaussian_rows_match_integrated_masses(K, tail_z):
    scales = log_scales(K)
    stride = 2 * int(math.ceil(scales[-1] * tail_z)) + 3
    rc, cdf, lengths, offsets = oracle.gaussian_tables(scales, tail_z, stride)
    assert rc == 0
    for r, s in enumerate(scales):
        ref, off, margin = gaussian_row_by_integration(float(s), tail_z)
        assert margin > 1e-6, "a mass lies too close to a rounding tie to decide"
        n = int(lengths[r])
        assert n == len(ref) and int(offsets[r]) == off
        assert cdf[r, :n].tolist() == ref, f"row {r} (scale {s})"
        assert np.all(cdf[r, n:] == 65536)


def test_gaussian_row_invariants():
    scales = np.concatenate([log_scales(64), np.random.default_rng(5).uniform(0.05, 300.0, 64)])
    stride = 2 * int(math.ceil(300.0 * TAIL_Z)) + 3
    rc, cdf, lengths, offsets = oracle.gaussian_tables(scales, TAIL_Z, stride)
    assert rc == 0
    for r in range(scales.size):
        n = int(lengths[r])
        f = np.diff(cdf[r, :n].astype(np.int64))
        assert cdf[r, 0] == 0 and cdf[r, n - 1] == 65536 and f.min() >= 1
        assert f[-1] == 1                      # escape slot: tail mass 1e-9 -> 1 unit
        sym = f[:-1]
        c = (sym.size - 1) // 2
        assert int(offsets[r]) == -c
        # symmetric about v = 0 except where the adjustment landed (the centre)
        diff = np.flatnonzero(sym != sym[::-1])
        assert np.all(np.abs(diff - c) <= max(2, sym.size // 4)), r
        # unimodal outside the top plateau (a surplus levels the largest
        # entries, then takes single units from the lowest slots among them)
        high = np.flatnonzero(sym >= sym.max() - 1)
        assert np.array_equal(high, np.arange(high[0], high[-1] + 1)) and high[0] <= c <= high[-1]
        assert np.all(np.diff(sym[: high[0] + 1]) >= 0)
        assert np.all(np.diff(sym[high[-1]:]) <= 0)


def test_gaussian_refusals():
    row = np.zeros(16, dtype=np.int32)
    for s in (0.0, -1.0, float("nan")):
        rc, *_ = oracle.gaussian_tables(np.array([s]), TAIL_Z, 16)
        assert rc == oracle.E_TABLE
    # scale 2 needs c = 13, 29 entries
    assert oracle.gaussian_tables(np.array([2.0]), TAIL_Z, 28)[0] == oracle.E_TABLE
    assert oracle.gaussian_tables(np.array([2.0]), TAIL_Z, 29)[0] == 0
    assert oracle.gaussian_tables(np.array([2.0]), -1.0, 64)[0] == oracle.E_TABLE
    del row
