"""Shared test helpers: golden-file parsing and the information content of a lane.

Nothing here encodes or decodes; the information measure below is the
textbook cost of a rANS put (log2 of the inverse probability, plus the raw
width of a bypass group), used to bound stream sizes.
"""
from __future__ import annotations

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

WORKED_ROWS = {
    "A": [0, 32768, 65535, 65536],
    "B": [0, 3, 65536],
}


def worked_cases():
    """Cases of golden/worked_streams.txt; header words are decimal, lane words hex."""
    cases = []
    with open(os.path.join(GOLDEN, "worked_streams.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line.startswith("case "):
                continue
            name, row, lanes, syms, words = [f.strip() for f in line[5:].split("|")]
            L = int(lanes)
            raw = words.split()
            cases.append(dict(
                name=name,
                row=WORKED_ROWS[row],
                lanes=L,
                symbols=[int(s) for s in syms.split()],
                words=[int(w) for w in raw[: 1 + L]] + [int(w, 16) for w in raw[1 + L:]],
            ))
    return cases


def single_table(row, offset=0):
    cdf = np.asarray([row], dtype=np.int32)
    return cdf, np.asarray([len(row)], np.int32), np.asarray([offset], np.int32)


def lane_information(symbols, indexes, cdf, lengths, offsets):
    """(bits, puts): sum of log2(2^16/f) over REG puts + 4 per bypass group put."""
    bits = 0.0
    puts = 0
    for s, r in zip(np.asarray(symbols, np.int64), np.asarray(indexes, np.int64)):
        row = cdf[r]
        mv = int(lengths[r]) - 2
        v = int(s) - int(offsets[r])
        raw = None
        if v < 0:
            raw, v = -2 * v - 1, mv
        elif v >= mv:
            raw, v = 2 * (v - mv), mv
        f = int(row[v + 1]) - int(row[v])
        bits += 16.0 - math.log2(f)
        puts += 1
        if raw is not None:
            nb = 0
            while raw >> (4 * nb):
                nb += 1
            groups = 1 + nb  # count group (nb <= 8 < 15) + raw groups
            bits += 4.0 * groups
            puts += groups
    return bits, puts


def lane_words_from_container(words, lanes):
    ends = [0] + [int(e) for e in words[1:1 + lanes]]
    body = words[1 + lanes:]
    return [np.asarray(body[ends[j]:ends[j + 1]]) for j in range(lanes)]
