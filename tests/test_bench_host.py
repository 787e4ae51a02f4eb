"""Host-side checks of bench.py's CPU-baseline leg on the small workload: the
oracle's container must match the one handed in as the GPU's (a container
that differs is refused), the lanes are fanned out over threads in
contiguous groups that cover every lane once, and the report carries the
fields the bench line promises."""
from __future__ import annotations

import numpy as np
import pytest

import bench
import oracle
import workloads as W


@pytest.fixture(scope="module")
def tiny_inputs():
    w = W.load("tiny")
    rc, words = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, 64)
    assert rc == 0
    scales, tail_z, stride = bench.table_set()
    rc, cdf, lengths, offsets = oracle.gaussian_tables(scales, tail_z, stride)
    assert rc == 0
    return w, words, (cdf, lengths, offsets)


def test_cpu_baseline_report(tiny_inputs):
    w, words, tables = tiny_inputs
    r = bench.cpu_baseline(w, 64, words, tables, min_seconds=0.2, max_reps=5)
    assert r["kind"] == "oracle" and r["unit"] == "Gsymbol/s"
    assert r["value"] > 0 and r["single_thread"]["value"] > 0
    assert 1 <= r["cores"] <= 16
    assert f"{r['cores']} contiguous groups" in r["sample"]


def test_cpu_baseline_refuses_a_different_container(tiny_inputs):
    w, words, tables = tiny_inputs
    other = words.copy()
    other[-1] ^= np.uint32(1)
    with pytest.raises(AssertionError, match="differs from the oracle"):
        bench.cpu_baseline(w, 64, other, tables, min_seconds=0.0, max_reps=1)


@pytest.mark.parametrize("n,lanes,groups", [(16384, 64, 8), (1566720, 4096, 16), (97920, 256, 7),
                                            (10, 3, 3), (5, 64, 16)])
def test_lane_groups_cover_every_lane_once(n, lanes, groups):
    spans = bench.lane_groups(n, lanes, groups)
    assert len(spans) == groups
    assert spans[0][0] == 0 and spans[-1][1] == n
    assert all(a[1] == b[0] for a, b in zip(spans, spans[1:]))
    assert sum(lg for _, _, lg in spans) == lanes
    # every group starts where the lane partition starts its first lane
    j = 0
    for b, _, lg in spans:
        assert b == j * n // lanes
        j += lg
