"""Pins of the oracle's split records (decode parallelism beyond the lane count).

What fixes the expected values:
* golden/worked_splits.txt -- records worked out by hand from the
  intermediate states of the derivations in worked_streams.txt;
* the container with records is the plain container, word for word;
* decoding every piece from its record and checking it ends exactly at the
  next record reproduces the input on every config, at lane counts and piece
  counts that leave pieces empty, one symbol long or ragged;
* an altered record (state bit, word count) is refused as corrupt.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from helpers import single_table, worked_cases, worked_splits


@pytest.mark.parametrize("case", worked_splits(), ids=lambda c: f"{c[0]}-P{c[1]}")
def test_golden_records(case):
    name, pieces, recs = case
    c = {k["name"]: k for k in worked_cases()}[name]
    cdf, lengths, offsets = single_table(c["row"])
    n = len(c["symbols"])
    rc, words, meta = oracle.encode_split(np.asarray(c["symbols"]), np.zeros(n), cdf, lengths,
                                          offsets, c["lanes"], pieces)
    assert rc == 0 and words.tolist() == c["words"]
    assert meta.reshape(-1, 3).tolist() == recs
    rc, out = oracle.decode_split(np.asarray(c["words"], np.uint32), np.asarray(recs, np.uint32),
                                  np.zeros(n), cdf, lengths, offsets, c["lanes"], pieces)
    assert rc == 0 and out.tolist() == c["symbols"]


@pytest.mark.parametrize("name,lanes,pieces", [
    ("tiny", 64, 2), ("tiny", 64, 8), ("tiny", 1, 16), ("tiny", 3, 64), ("tiny", 16389, 4),
    ("z", 256, 4), ("z", 97925, 2), ("y1080", 4096, 4),
])
def test_round_trip_and_plain_container(name, lanes, pieces):
    w = W.load(name)
    rc, words, meta = oracle.encode_split(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets,
                                          lanes, pieces)
    rc0, plain = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, lanes)
    assert rc == rc0 == 0 and np.array_equal(words, plain)
    rc, out = oracle.decode_split(words, meta, w.indexes, w.cdf, w.lengths, w.offsets, lanes,
                                  pieces)
    assert rc == 0 and np.array_equal(out, w.symbols)
    # records of consecutive cuts never gain unread words
    left = meta[:, :, 2].astype(np.int64)
    assert np.all(np.diff(left, axis=1) <= 0)


def test_one_piece_is_the_plain_decoder():
    w = W.load("tiny")
    rc, words, meta = oracle.encode_split(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, 64, 1)
    assert rc == 0 and meta.size == 0
    rc, out = oracle.decode_split(words, meta, w.indexes, w.cdf, w.lengths, w.offsets, 64, 1)
    assert rc == 0 and np.array_equal(out, w.symbols)


def test_altered_records_are_refused():
    w = W.load("tiny")
    L, P = 64, 4
    rc, words, meta = oracle.encode_split(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, L, P)
    assert rc == 0
    for j, s, k, delta in ((3, 0, 0, 1), (10, 1, 1, 1 << 7), (20, 2, 2, 1), (30, 1, 2, -1),
                           (40, 0, 2, 1 << 30)):
        bad = meta.copy().astype(np.int64)
        bad[j, s, k] = (bad[j, s, k] + delta) % (1 << 32)
        rc, _ = oracle.decode_split(words, bad.astype(np.uint32), w.indexes, w.cdf, w.lengths,
                                    w.offsets, L, P)
        assert rc == oracle.E_CORRUPT, (j, s, k)


def test_empty_input_and_bad_arguments():
    cdf, lengths, offsets = single_table([0, 32768, 65535, 65536])
    rc, words, meta = oracle.encode_split(np.zeros(0), np.zeros(0), cdf, lengths, offsets, 2, 4)
    assert rc == 0 and words.tolist() == [2, 2, 4, 0x80000000, 0, 0x80000000, 0]
    assert meta.reshape(-1, 3).tolist() == [[0x80000000, 0, 0]] * 6
    rc, _ = oracle.decode_split(words, meta, np.zeros(0), cdf, lengths, offsets, 2, 4)
    assert rc == 0
    assert oracle.encode_split(np.zeros(1), np.zeros(1), cdf, lengths, offsets, 1, 0)[0] == oracle.E_ARG
