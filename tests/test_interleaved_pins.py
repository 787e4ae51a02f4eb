"""Pins of the oracle's interleaved streams (one shared word cursor per stream).

What fixes the expected values:
* golden/worked_interleaved.txt -- containers worked out by hand, one of
  them showing the cross-state word order (slot before state);
* width 1 is the lane container word for word (itself pinned by the worked
  lane streams);
* round trips on every config at several stream counts and widths,
  including streams shorter than their width and empty streams;
* stream sizes: the words beyond the flushed states are within a few words
  per state of the information content of the stream's puts;
* a corrupt stream (a changed word, a missing word, a wrong count) is refused.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from helpers import single_table, worked_interleaved, WORKED_ROWS


@pytest.mark.parametrize("case", worked_interleaved(), ids=lambda c: c["name"])
def test_golden_streams(case):
    cdf, lengths, offsets = single_table(WORKED_ROWS["A"])
    n = len(case["symbols"])
    rc, words = oracle.encode_interleaved(np.asarray(case["symbols"]), np.zeros(n), cdf, lengths,
                                          offsets, case["streams"], case["width"])
    assert rc == 0 and words.tolist() == case["words"]
    rc, out = oracle.decode_interleaved(np.asarray(case["words"], np.uint32), np.zeros(n), cdf,
                                        lengths, offsets, case["streams"], case["width"])
    assert rc == 0 and out.tolist() == case["symbols"]


@pytest.mark.parametrize("name,streams", [("tiny", 64), ("tiny", 1), ("z", 256), ("z", 7)])
def test_width_one_is_the_lane_container(name, streams):
    w = W.load(name)
    rc, a = oracle.encode_interleaved(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, streams, 1)
    rc2, b = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, streams)
    assert rc == rc2 == 0 and np.array_equal(a, b)


@pytest.mark.parametrize("name,streams,width", [
    ("tiny", 1, 64), ("tiny", 4, 64), ("tiny", 255, 64), ("tiny", 300, 64), ("tiny", 64, 7),
    ("z", 4, 64), ("z", 1531, 64), ("y1080", 64, 64), ("y1080", 1024, 32),
])
def test_round_trips(name, streams, width):
    w = W.load(name)
    rc, words = oracle.encode_interleaved(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets,
                                          streams, width)
    assert rc == 0 and words[0] == streams
    rc, out = oracle.decode_interleaved(words, w.indexes, w.cdf, w.lengths, w.offsets, streams,
                                        width)
    assert rc == 0 and np.array_equal(out, w.symbols)
    # per stream: flushed states, then the payload
    ends = words[1:1 + streams].astype(np.int64)
    sizes = np.diff(np.concatenate([[0], ends]))
    assert np.all(sizes >= 2 * width)


def test_size_near_information_content():
    """Beyond its 2 W flush words, a stream holds about the information of its
    puts: each state's share is within its own flush slack (at most 2 words)."""
    w = W.load("z")
    streams, width = 8, 64
    rc, words = oracle.encode_interleaved(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets,
                                          streams, width)
    assert rc == 0
    rc, lane = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, streams * width)
    # the same states cut as lanes carry the same information; totals agree to
    # within two words per state
    assert abs(int(words.size) - int(lane.size) + streams * width - streams) <= 2 * streams * width


def test_corrupt_streams_are_refused():
    w = W.load("tiny")
    S, Wd = 4, 64
    rc, words = oracle.encode_interleaved(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, S, Wd)
    assert rc == 0
    bad = words.copy(); bad[1 + S + 2 * Wd + 5] ^= 1 << 9
    assert oracle.decode_interleaved(bad, w.indexes, w.cdf, w.lengths, w.offsets, S, Wd)[0] \
        == oracle.E_CORRUPT
    assert oracle.decode_interleaved(words[:-1], w.indexes, w.cdf, w.lengths, w.offsets, S, Wd)[0] \
        == oracle.E_CORRUPT
    assert oracle.decode_interleaved(words, w.indexes, w.cdf, w.lengths, w.offsets, S + 1, Wd)[0] \
        == oracle.E_CORRUPT
    assert oracle.decode_interleaved(words, w.indexes, w.cdf, w.lengths, w.offsets, S, Wd // 2)[0] \
        == oracle.E_CORRUPT
