"""Pins of the oracle's latent front end (quantisation, table index, dequantisation).

What fixes the expected values:
* golden/latent_front_end.txt -- hand-derived symbols (ties to even,
  saturation, exact large values) and indexes (below, at, between and above
  the table scales, NaN);
* brute force on random inputs against the IEEE single-precision operations
  as numpy performs them, and against the first-slot search on a sorted
  table (a different formulation of the index rule than the oracle's count);
* dequantisation of every int32 boundary case.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from helpers import LATENT_TABLE, latent_cases

SYMS, IDXS = latent_cases()


@pytest.mark.parametrize("y,mean,want", SYMS)
def test_golden_symbols(y, mean, want):
    rc, sym, idx = oracle.latent_symbols([y], [mean], [1.0], LATENT_TABLE)
    assert rc == 0 and int(sym[0]) == want


@pytest.mark.parametrize("scale,want", IDXS)
def test_golden_indexes(scale, want):
    rc, sym, idx = oracle.latent_symbols([0.0], [0.0], [scale], LATENT_TABLE)
    assert rc == 0 and int(idx[0]) == want


def test_random_inputs_against_ieee_single_and_first_slot_search():
    rng = np.random.default_rng(21)
    n = 200_000
    y = (rng.standard_normal(n) * rng.choice([0.5, 4.0, 300.0], n)).astype(np.float32)
    mean = (rng.standard_normal(n) * 2).astype(np.float32)
    y[:1000] = np.round(y[:1000]) + np.float32(0.5)       # ties
    mean[:1000] = 0
    table = np.exp(np.linspace(np.log(0.11), np.log(256.0), 64)).astype(np.float32)
    scales = np.exp(rng.uniform(np.log(0.01), np.log(400.0), n)).astype(np.float32)
    scales[:64] = table                                    # exactly on the table
    rc, sym, idx = oracle.latent_symbols(y, mean, scales, table)
    assert rc == 0
    assert np.array_equal(sym, np.rint(y - mean).astype(np.int32))
    first = np.searchsorted(table[:-1], scales, side="left")   # first k with table[k] >= s
    assert np.array_equal(idx, first)


def test_unsorted_table_follows_the_count_rule():
    table = np.array([3.0, 1.0, 2.0, 0.5], np.float32)
    rc, _, idx = oracle.latent_symbols(np.zeros(4), np.zeros(4), [0.9, 1.5, 2.5, 5.0], table)
    # (K - 1) - #{k < 3 : s <= table[k]}: 0.9 -> 3 - 3 = 0; 1.5 -> 3 - 2 = 1;
    # 2.5 -> 3 - 1 = 2; 5.0 -> 3
    assert rc == 0 and idx.tolist() == [0, 1, 2, 3]


def test_dequantize():
    s = np.array([0, 1, -1, 2**31 - 1, -2**31, 16777217, 3], np.int32)
    m = np.array([0.25, -0.5, 0.5, 0.0, 0.0, 0.0, 1e-8], np.float32)
    rc, out = oracle.dequantize(s, m)
    # int32 -> float rounds to nearest even: 2^31 - 1 -> 2^31, 16777217 -> 16777216;
    # 3 + 1e-8 rounds back to 3
    assert rc == 0
    assert out.tolist() == [0.25, 0.5, -0.5, 2147483648.0, -2147483648.0, 16777216.0, 3.0]


def test_empty_and_refusals():
    assert oracle.latent_symbols([], [], [], LATENT_TABLE)[0] == 0
    assert oracle.latent_symbols([1.0], [0.0], [1.0], [])[0] == oracle.E_ARG
