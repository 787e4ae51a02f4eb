"""GPU parity of the device table builder against the oracle, entry for entry.

Gaussian rows: the log-spaced 8- and 64-row sets, seeded random scales over
0.02..500 at three tail quantiles, rows that exactly fill the stride and
rows one symbol too wide, invalid scales.  Pmf rows: seeded random pmfs with
surplus, deficit and exact half-unit ties, rows at the longest length the
stride allows, invalid rows.  Finally the device-built 8-row set codes the
tiny workload to the oracle's container.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
from scipy.special import ndtri

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TAIL_Z = float(ndtri(1.0 - 5e-10))


def log_scales(K, lo=0.11, hi=256.0):
    return np.exp(np.log(lo) + (np.log(hi) - np.log(lo)) * np.arange(K) / (K - 1))


def _gpu_gauss(scales, tail_z, stride):
    import torch
    import gpu_util as G
    t, st = G.B.gaussian_tables(torch.from_numpy(np.asarray(scales, np.float64)).to(G.DEV),
                                tail_z, stride)
    torch.cuda.synchronize()
    return (t.cdf.cpu().numpy(), t.lengths.cpu().numpy(), t.offsets.cpu().numpy(),
            st.cpu().numpy())


def _check_gauss(scales, tail_z, stride):
    import gpu_util as G
    G.say(f"[tables] gaussian K={len(scales)} z={tail_z:.4f} stride={stride}")
    cdf, lengths, offsets, st = _gpu_gauss(scales, tail_z, stride)
    rc, ocdf, olen, ooff = oracle.gaussian_tables(scales, tail_z, stride)
    assert rc == 0
    assert np.all(st == 0)
    assert np.array_equal(lengths, olen) and np.array_equal(offsets, ooff)
    bad = np.argwhere(cdf != ocdf)
    assert bad.size == 0, f"{len(bad)} entries differ, first at row {bad[0][0]} slot {bad[0][1]}"


@pytest.mark.parametrize("K", [8, 64])
def test_log_spaced_sets(K):
    _check_gauss(log_scales(K), TAIL_Z, 3133)


def test_log_spaced_set_equals_the_workload_tables():
    w = W.load("y1080")
    cdf, lengths, offsets, st = _gpu_gauss(log_scales(64), TAIL_Z, w.stride)
    assert np.all(st == 0)
    assert np.array_equal(cdf, w.cdf) and np.array_equal(lengths, w.lengths)
    assert np.array_equal(offsets, w.offsets)


@pytest.mark.parametrize("tail_z", [TAIL_Z, 3.0, 1.0])
def test_random_scales(tail_z):
    rng = np.random.default_rng(int(tail_z * 1000))
    scales = np.exp(rng.uniform(np.log(0.02), np.log(500.0), 300))
    stride = 2 * int(math.ceil(scales.max() * tail_z)) + 3
    _check_gauss(scales, tail_z, stride)


def test_rows_at_the_stride_limit_and_invalid_scales():
    import gpu_util as G
    # scale 2 needs c = ceil(12.22) = 13: 29 entries
    scales = np.array([2.0, 0.5, 0.0, -3.0, np.nan, 2.0, 1e-6, 3.0])
    stride = 29
    G.say("[tables] stride limit and invalid rows")
    cdf, lengths, offsets, st = _gpu_gauss(scales, TAIL_Z, stride)
    for r, s in enumerate(scales):
        rc, ocdf, olen, ooff = oracle.gaussian_tables(np.array([s]), TAIL_Z, stride)
        assert st[r] == rc, (r, s)
        if rc == 0:
            assert lengths[r] == olen[0] and offsets[r] == ooff[0]
            assert np.array_equal(cdf[r], ocdf[0])
        else:
            assert lengths[r] == 0
    assert st.tolist() == [0, 0, -2, -2, -2, 0, 0, -2]   # scale 3 needs 41 entries


def _random_pmfs(rng, K, S):
    rows, lengths = np.zeros((K, S)), np.zeros(K, dtype=np.int32)
    for r in range(K):
        m = int(rng.integers(2, S + 1)) if r % 5 else int(rng.integers(2, 12))
        kind = r % 4
        if kind == 0:
            p = rng.dirichlet(np.full(m, 0.2))
        elif kind == 1:
            p = rng.dirichlet(np.ones(m)) * rng.uniform(0.3, 1.0)
        elif kind == 2:
            p = np.minimum(rng.dirichlet(np.ones(m)) * rng.uniform(1.0, 1.05), 1.0)
        else:              # exact half-unit ties (j + 1/2 units), the rest on one slot
            p = (rng.integers(0, 8, m) * 2 + 1) / 131072.0
            k = int(rng.integers(0, m))
            p[k] = 0.0
            p[k] = max(0.0, 1.0 - p.sum())
        rows[r, :m] = p
        rows[r, m:] = np.nan   # never read
        lengths[r] = m
    return rows, lengths


def _gpu_quantize(rows, lengths, stride):
    import torch
    import gpu_util as G
    cdf, ln, st = G.B.quantize_pmfs(torch.from_numpy(rows).to(G.DEV),
                                    torch.from_numpy(lengths).to(G.DEV), stride)
    torch.cuda.synchronize()
    return cdf.cpu().numpy(), ln.cpu().numpy(), st.cpu().numpy()


@pytest.mark.parametrize("S", [16, 600, 4096])
def test_random_pmf_rows(S):
    import gpu_util as G
    rng = np.random.default_rng(S)
    rows, lengths = _random_pmfs(rng, 200, S)
    G.say(f"[tables] pmf rows S={S}")
    cdf, ln, st = _gpu_quantize(rows, lengths, S + 1)
    assert np.all(st == 0)
    for r in range(rows.shape[0]):
        m = int(lengths[r])
        rc, ref = oracle.quantize_pmf(rows[r, :m])
        assert rc == 0 and ln[r] == m + 1
        assert np.array_equal(cdf[r, : m + 1], ref), r
        assert np.all(cdf[r, m + 1:] == 65536)


def test_longest_pmf_rows_and_invalid_rows():
    import gpu_util as G
    S = 16383
    rng = np.random.default_rng(7)
    rows = np.zeros((8, S))
    lengths = np.full(8, S, dtype=np.int32)
    rows[0] = rng.dirichlet(np.ones(S))              # every entry rounds near 4 units
    rows[1] = rng.dirichlet(np.full(S, 0.01))         # mostly raised to 1: large surplus
    rows[2] = np.full(S, 1.0 / 65536)                 # deficit of 49153 to slot 0
    rows[3] = 5.0 / 65536                             # surplus 16379: 16379 slots to 4
    rows[4, :10] = [0.1, -1e-3, 0.2, 0.3, 0.4, 0, 0, 0, 0, 0]; lengths[4] = 10
    rows[5, :3] = [0.5, np.nan, 0.5]; lengths[5] = 3
    rows[6, :2] = [0.25, 0.75]; lengths[6] = 1
    rows[7, :3] = [0.2, 0.3, 1.5]; lengths[7] = 3
    G.say("[tables] longest and invalid pmf rows")
    cdf, ln, st = _gpu_quantize(rows, lengths, S + 1)
    assert st.tolist() == [0, 0, 0, 0, -2, -2, -2, -2]
    assert ln[4:].tolist() == [0, 0, 0, 0]
    for r in range(4):
        rc, ref = oracle.quantize_pmf(rows[r])
        assert rc == 0 and np.array_equal(cdf[r], ref), r
    # a pmf row longer than the cdf stride allows is refused
    cdf, ln, st = _gpu_quantize(rows[:1, :100].copy(), np.array([100], np.int32), 100)
    assert st.tolist() == [-2]


def test_device_built_tables_code_like_the_oracle():
    import gpu_util as G
    w = W.load("tiny")
    import torch
    tables, st = G.B.gaussian_tables(torch.from_numpy(log_scales(8)).to(G.DEV), TAIL_Z,
                                     w.stride)
    G.B.check_rows(st)
    sym, idx = G.to_dev(w.symbols), G.to_dev(w.indexes)
    rc, ocdf, olen, ooff = oracle.gaussian_tables(log_scales(8), TAIL_Z, w.stride)
    rc2, ref = oracle.encode(w.symbols, w.indexes, ocdf, olen, ooff, 64)
    assert rc == 0 and rc2 == 0
    G.say("[tables] coding with device-built tables")
    s, got, nw = G.gpu_encode(sym, idx, tables, 64)
    assert s == 0 and np.array_equal(got, ref)
    s, out = G.gpu_decode(ref, idx, tables)
    assert s == 0 and np.array_equal(out, w.symbols)
