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


# --------------------------------------------------------------- tables
def quantized_cases():
    """Cases of golden/quantized_cdfs.txt as (name, pmf float64 array, cdf list)."""
    def num(tok):
        if "/" in tok:
            a, b = tok.split("/")
            return float(a) / float(b)
        return float(tok)
    cases = []
    with open(os.path.join(GOLDEN, "quantized_cdfs.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line.startswith("case "):
                continue
            name, pmf, cdf = [f.strip() for f in line[5:].split("|")]
            cases.append((name, np.array([num(t) for t in pmf.split()], dtype=np.float64),
                          [int(t) for t in cdf.split()]))
    return cases


def quantize_water_level(p):
    """16-bit frequencies of a pmf row by the closed form of the unit-by-unit
    adjustment: a surplus E lowers every frequency above the level T to T,
    T the smallest level whose removal sum(max(0, f - T)) is at most E, and
    the remaining units come one each from the lowest slots at T; a deficit
    goes entirely to the first largest slot (it stays the largest)."""
    f = np.maximum(np.rint(np.asarray(p, dtype=np.float64) * 65536.0), 1).astype(np.int64)
    excess = int(f.sum()) - 65536
    if excess < 0:
        f[int(np.argmax(f))] -= excess
    elif excess > 0:
        lo, hi = 1, int(f.max())
        while lo < hi:
            mid = (lo + hi) // 2
            if int(np.maximum(f - mid, 0).sum()) <= excess:
                hi = mid
            else:
                lo = mid + 1
        T = lo
        rest = excess - int(np.maximum(f - T, 0).sum())
        top = np.flatnonzero(f >= T)
        f[top] = T
        f[top[:rest]] -= 1
    return f


def normal_mass(a, b, per_unit=2000):
    """Standard-normal mass of [a, b] by composite Simpson's rule on the
    density (independent of any erf/erfc routine)."""
    n = max(64, int(math.ceil((b - a) * per_unit)))
    n += n & 1
    x = np.linspace(a, b, n + 1)
    y = np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)
    h = (b - a) / n
    return float(h / 3.0 * (y[0] + y[-1] + 4.0 * y[1:-1:2].sum() + 2.0 * y[2:-1:2].sum()))


def gaussian_row_by_integration(scale, tail_z):
    """(cdf list, offset, smallest distance of p * 65536 to a half-integer) of
    the discretised Gaussian row, from Simpson masses of each bin and of both
    tails (the tails integrated out to 40 standard deviations)."""
    c = int(math.ceil(scale * tail_z))
    p = [normal_mass((v - 0.5) / scale, (v + 0.5) / scale) for v in range(-c, c + 1)]
    edge = (c + 0.5) / scale
    p.append(2.0 * normal_mass(edge, max(edge, 0.0) + 40.0))
    p = np.array(p)
    frac = np.abs(np.mod(p * 65536.0, 1.0) - 0.5)
    f = quantize_water_level(p)
    return [0] + np.cumsum(f).tolist(), -c, float(frac.min())


# --------------------------------------------------------------- latent front end
LATENT_TABLE = [0.5, 1.0, 2.0, 4.0]


def latent_cases():
    """(symbol cases [(y, mean, symbol)], index cases [(scale, index)]) of
    golden/latent_front_end.txt."""
    syms, idxs = [], []
    with open(os.path.join(GOLDEN, "latent_front_end.txt")) as fh:
        for line in fh:
            f = line.split("#")[0].split()
            if not f:
                continue
            if f[0] == "sym":
                syms.append((float(f[1]), float(f[2]), int(f[3])))
            elif f[0] == "idx":
                idxs.append((float(f[1]), int(f[2])))
    return syms, idxs


def worked_splits():
    """Cases of golden/worked_splits.txt as (case name, pieces, records [[lo, hi, left]])."""
    out = []
    with open(os.path.join(GOLDEN, "worked_splits.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line.startswith("split "):
                continue
            name, pieces, recs = [f.strip() for f in line[6:].split("|")]
            rows = []
            for r in recs.split(","):
                lo, hi, left = r.split()
                rows.append([int(lo, 16), int(hi, 16), int(left)])
            out.append((name, int(pieces), rows))
    return out


def worked_interleaved():
    """Cases of golden/worked_interleaved.txt (row A), as dicts."""
    out = []
    with open(os.path.join(GOLDEN, "worked_interleaved.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line.startswith("case "):
                continue
            name, streams, width, syms, words = [f.strip() for f in line[5:].split("|")]
            out.append(dict(name=name, streams=int(streams), width=int(width),
                            symbols=[int(s) for s in syms.split()],
                            words=[int(w, 16) for w in words.split()]))
    return out
