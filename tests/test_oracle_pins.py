"""Pins of the CPU oracle against facts that do not come from the oracle itself.

* hand-derived worked streams (tests/golden/worked_streams.txt);
* closed form: with every frequency 2^12 a REG put appends one base-16 digit
  above 12 zero bits, so a short lane's final state is a hex number;
* round trips decode(encode(x)) == x on every synthetic workload;
* the per-lane size bound implied by the rANS state interval;
* exhaustive brute force on tiny alphabets against the separately written
  Python model, plus injectivity of the encoder;
* lane structure: the container is the header plus each lane encoded alone,
  and one lane gives the standard single stream;
* bypass edge values and every error status.
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import pytest

import oracle
from oracle import spec_model as sm
import workloads as W
from helpers import (lane_information, lane_words_from_container, single_table,
                     worked_cases)

ROW_C = [0, 20000, 50000, 65535, 65536]   # values -1, 0, 1 (offset -1) + escape
ROW_D = [0, 1, 2, 65535, 65536]           # extreme frequencies 1, 1, 65533


# ---------------------------------------------------------------- worked streams
@pytest.mark.parametrize("case", worked_cases(), ids=lambda c: c["name"])
def test_worked_stream_encode(case):
    cdf, lengths, offsets = single_table(case["row"])
    n = len(case["symbols"])
    rc, words = oracle.encode(np.asarray(case["symbols"]), np.zeros(n), cdf, lengths, offsets,
                              case["lanes"])
    assert rc == 0
    assert words.tolist() == case["words"]


@pytest.mark.parametrize("case", worked_cases(), ids=lambda c: c["name"])
def test_worked_stream_decode(case):
    cdf, lengths, offsets = single_table(case["row"])
    n = len(case["symbols"])
    rc, out = oracle.decode(np.asarray(case["words"], dtype=np.uint32), np.zeros(n), cdf,
                            lengths, offsets, case["lanes"])
    assert rc == 0
    assert out.tolist() == case["symbols"]


@pytest.mark.parametrize("case", worked_cases(), ids=lambda c: c["name"])
def test_worked_stream_spec_model(case):
    n = len(case["symbols"])
    assert sm.encode(case["symbols"], [0] * n, [case["row"]], [0], case["lanes"]) == case["words"]


# ---------------------------------------------------------------- closed form
def test_uniform_power_of_two_rows_pack_hex_digits():
    """f = 2^12 for all 16 slots: x = 2^(31+4k) + sum v_i 16^i * 2^12 (no spill for k <= 7)."""
    row = [4096 * k for k in range(17)]          # 15 values + escape, all f = 4096
    cdf, lengths, offsets = single_table(row)
    rng = np.random.default_rng(11)
    for k in range(8):
        for _ in range(20):
            v = rng.integers(0, 15, size=k)
            rc, words = oracle.encode(v, np.zeros(k), cdf, lengths, offsets, 1)
            assert rc == 0
            x = (1 << (31 + 4 * k)) + sum(int(d) << (12 + 4 * i) for i, d in enumerate(v))
            assert words.tolist() == [1, 2, x & 0xFFFFFFFF, x >> 32]


# ---------------------------------------------------------------- round trips
@pytest.mark.parametrize("name", ["tiny", "z", "y1080"])
def test_round_trip_workloads(name):
    w = W.load(name)
    for L in w.lanes:
        rc, words = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, L)
        assert rc == 0
        rc, out = oracle.decode(words, w.indexes, w.cdf, w.lengths, w.offsets, L)
        assert rc == 0
        assert np.array_equal(out, w.symbols), (name, L)


# ---------------------------------------------------------------- size bound
def _check_size_bound(symbols, indexes, cdf, lengths, offsets, lanes):
    rc, words = oracle.encode(symbols, indexes, cdf, lengths, offsets, lanes)
    assert rc == 0
    lane_streams = lane_words_from_container(words.tolist(), lanes)
    n = len(symbols)
    for j, ls in enumerate(lane_streams):
        b, e = (j * n) // lanes, ((j + 1) * n) // lanes
        bits, puts = lane_information(symbols[b:e], indexes[b:e], cdf, lengths, offsets)
        slack = 9e-5 * puts + 1e-9 * bits
        W32 = 32 * len(ls)
        assert bits + 32 - slack < W32 <= bits + 64 + slack, (j, bits, W32)


@pytest.mark.parametrize("name,lanes", [("tiny", 64), ("tiny", 7), ("z", 256), ("z", 3)])
def test_size_bound_per_lane(name, lanes):
    w = W.load(name)
    _check_size_bound(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, lanes)


def test_size_bound_extreme_frequencies():
    cdf, lengths, offsets = single_table(ROW_D)
    rng = np.random.default_rng(5)
    sym = rng.integers(-3, 6, size=3000)
    _check_size_bound(sym, np.zeros(sym.size, np.int32), cdf, lengths, offsets, 5)


def test_dominant_symbol_is_almost_free():
    """f = 65535 costs log2(65536/65535) bits: thousands of symbols fit in the flush words."""
    row = [0, 65535, 65536]
    cdf, lengths, offsets = single_table(row)
    n = 200_000
    rc, words = oracle.encode(np.zeros(n), np.zeros(n), cdf, lengths, offsets, 1)
    assert rc == 0
    assert words.size == 1 + 1 + 2          # header + just the flushed state


# ---------------------------------------------------------------- brute force
def _tables_cd():
    cdf = np.full((2, 5), 65536, dtype=np.int32)
    cdf[0, :5] = ROW_C
    cdf[1, :5] = ROW_D
    return cdf, np.asarray([5, 5], np.int32), np.asarray([-1, 2], np.int32)


def test_exhaustive_against_spec_model_and_injective():
    cdf, lengths, offsets = _tables_cd()
    rows = [ROW_C, ROW_D]
    offs = [-1, 2]
    values = [-9, -2, -1, 0, 1, 2, 3, 4, 40]
    seen = {}
    for length in range(0, 4):
        for syms in itertools.product(values, repeat=length):
            for idxs in itertools.product([0, 1], repeat=length):
                for L in (1, 2):
                    ref = sm.encode(list(syms), list(idxs), rows, offs, L)
                    rc, words = oracle.encode(np.asarray(syms, np.int64), np.asarray(idxs),
                                              cdf, lengths, offsets, L)
                    assert rc == 0
                    assert words.tolist() == ref
                    key = (L, tuple(idxs), tuple(ref))
                    assert key not in seen, "two inputs gave the same stream"
                    seen[key] = syms
                    assert sm.decode(ref, list(idxs), rows, offs, L) == list(syms)


def test_long_random_against_spec_model():
    cdf, lengths, offsets = _tables_cd()
    rows, offs = [ROW_C, ROW_D], [-1, 2]
    rng = np.random.default_rng(7)
    for L in (1, 3, 8):
        n = 400
        syms = rng.integers(-6, 8, size=n)
        far = rng.random(n) < 0.02
        syms[far] = rng.integers(-(1 << 30), (1 << 30), size=int(far.sum()))
        idxs = rng.integers(0, 2, size=n)
        ref = sm.encode(syms.tolist(), idxs.tolist(), rows, offs, L)
        rc, words = oracle.encode(syms, idxs, cdf, lengths, offsets, L)
        assert rc == 0 and words.tolist() == ref


# ---------------------------------------------------------------- lane structure
def test_container_is_header_plus_independent_lanes():
    w = W.load("tiny")
    for L in (1, 3, 64, 255):
        rc, words = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, L)
        assert rc == 0
        expect_body, ends = [], []
        for j in range(L):
            b, e = (j * w.n) // L, ((j + 1) * w.n) // L
            rc, lane = oracle.encode_lane(w.symbols, w.indexes, b, e, w.cdf, w.lengths,
                                          w.offsets)
            assert rc == 0
            expect_body += lane.tolist()
            ends.append(len(expect_body))
        assert words.tolist() == [L] + ends + expect_body


def test_single_lane_is_standard_single_stream():
    """With one lane the payload after [1, W] is the plain single-stream rANS64 stream."""
    w = W.load("tiny")
    n = 3000
    ops = []
    for s, r in zip(w.symbols[:n].tolist(), w.indexes[:n].tolist()):
        row = w.cdf[r, : w.lengths[r]].tolist()
        ops += sm.operations(s, row, int(w.offsets[r]))
    stream = sm.encode_single(ops)
    rc, words = oracle.encode(w.symbols[:n], w.indexes[:n], w.cdf, w.lengths, w.offsets, 1)
    assert rc == 0
    assert words.tolist() == [1, len(stream)] + stream


def test_lane_partition_is_balanced():
    for n in (0, 1, 5, 16384, 1566720, 50135040, (1 << 40) + 3):
        for L in (1, 2, 3, 7, 64, 4096, 131072, 4294967295):
            begins = [oracle.lane_begin(n, L, j) for j in (0, 1, L // 2, L - 1, L)]
            assert begins[0] == 0 and begins[-1] == n
            assert begins == [(j * n) // L for j in (0, 1, L // 2, L - 1, L)]


# ---------------------------------------------------------------- bypass edges
@pytest.mark.parametrize("raw", list(W.EDGE_RAWS) + [2, 3, 14, 17, 4095, 4096, 65535, 65536])
def test_bypass_edge_values_round_trip(raw):
    cdf, lengths, offsets = single_table(ROW_C, offset=-1)
    mv = len(ROW_C) - 2
    v = W.raw_to_value(raw, mv)
    sym = np.asarray([0, v - 1, 1, v - 1, -1], dtype=np.int64)   # value = v + offset
    rc, words = oracle.encode(sym, np.zeros(5), cdf, lengths, offsets, 1)
    assert rc == 0
    rc, out = oracle.decode(words, np.zeros(5), cdf, lengths, offsets, 1)
    assert rc == 0 and out.tolist() == sym.tolist()
    assert words.tolist() == sm.encode(sym.tolist(), [0] * 5, [ROW_C], [-1], 1)


@pytest.mark.parametrize("v", [-(1 << 30) - 1, 3 + (1 << 30), -(1 << 31) + 2])
def test_bypass_out_of_range_is_rejected(v):
    cdf, lengths, offsets = single_table(ROW_C, offset=0)
    rc, _ = oracle.encode(np.asarray([0, v]), np.zeros(2), cdf, lengths, offsets, 1)
    assert rc == oracle.E_SYMBOL_RANGE


# ---------------------------------------------------------------- errors
def test_bad_tables_are_rejected():
    cdf, lengths, offsets = single_table(ROW_C)
    sym = np.zeros(4)
    idx = np.zeros(4)
    bad = [
        (np.asarray([[1, 20000, 50000, 65535, 65536]]), lengths),      # cdf[0] != 0
        (np.asarray([[0, 20000, 50000, 65535, 65535]]), lengths),      # terminal != 2^16
        (np.asarray([[0, 20000, 20000, 65535, 65536]]), lengths),      # zero frequency
        (np.asarray([[0, 50000, 20000, 65535, 65536]]), lengths),      # decreasing
        (cdf, np.asarray([2], np.int32)),                              # len < 3
        (cdf, np.asarray([6], np.int32)),                              # len > stride
    ]
    for c, l in bad:
        assert oracle.check_tables(c, l) == oracle.E_TABLE
        rc, _ = oracle.encode(sym, idx, c, l, offsets, 1)
        assert rc == oracle.E_TABLE


def test_bad_index_is_rejected():
    cdf, lengths, offsets = single_table(ROW_C)
    for bad in (-1, 1, 1 << 30):
        idx = np.asarray([0, 0, bad, 0])
        rc, _ = oracle.encode(np.zeros(4), idx, cdf, lengths, offsets, 2)
        assert rc == oracle.E_INDEX
        rc, words = oracle.encode(np.zeros(4), np.zeros(4), cdf, lengths, offsets, 2)
        rc, _ = oracle.decode(words, idx, cdf, lengths, offsets, 2)
        assert rc == oracle.E_INDEX


def test_capacity_too_small():
    w = W.load("tiny")
    rc, words = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, 64)
    assert rc == 0
    rc, _ = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, 64,
                          capacity=words.size - 1)
    assert rc == oracle.E_CAPACITY
    rc, again = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, 64,
                              capacity=words.size)
    assert rc == 0 and np.array_equal(again, words)


def test_corrupt_streams_are_rejected():
    w = W.load("tiny")
    L = 4
    rc, words = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, L)
    assert rc == 0

    def dec(s, lanes=L):
        return oracle.decode(np.asarray(s, np.uint32), w.indexes, w.cdf, w.lengths, w.offsets,
                             lanes)[0]

    assert dec(words) == 0
    assert dec(words, lanes=L + 1) == oracle.E_CORRUPT          # lane count mismatch
    s = words.copy(); s[0] = L + 1
    assert dec(s) == oracle.E_CORRUPT
    s = words.copy(); s[1], s[2] = s[2], s[1]                   # non-monotone ends
    assert dec(s) == oracle.E_CORRUPT
    assert dec(words[:-1]) == oracle.E_CORRUPT                  # stream shorter than header says
    # drop the last word of the last lane and fix the header: the lane runs short
    s = words[:-1].copy(); s[L] -= 1
    assert dec(s) == oracle.E_CORRUPT
    # an extra, never-read word at the end of the last lane fails the end check
    s = np.concatenate([words, [123]]).astype(np.uint32); s[L] += 1
    assert dec(s) == oracle.E_CORRUPT
    # a lane shorter than the two flush words
    s = words.copy(); s[1] = 1
    assert dec(s) == oracle.E_CORRUPT


def test_decoded_bypass_count_above_eight_is_corrupt():
    """A hand-made lane whose escape is followed by a group count of 9."""
    cdf, lengths, offsets = single_table([0, 32768, 65535, 65536])
    # state after the escape slot: x = 16*2^31 + 9 = 2^35 + 9 -> REG(65535, 1)
    x = ((1 << 35) + 9) * 65536 + 65535
    lane = [x & 0xFFFFFFFF, x >> 32]
    rc, _ = oracle.decode(np.asarray([1, 2] + lane, np.uint32), np.zeros(1), cdf, lengths,
                          offsets, 1)
    assert rc == oracle.E_CORRUPT


def test_entropy_of_y1080_payload_is_plausible():
    """Bits/symbol match the information content (2.55 expected; real latents give 1.76)."""
    w = W.load("y1080")
    rc, words = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, 4096)
    assert rc == 0
    payload_bits = 32.0 * (words.size - 1 - 4096)
    idx = w.indexes.astype(np.int64)
    v = w.symbols.astype(np.int64) - w.offsets[idx]
    mv = w.lengths[idx].astype(np.int64) - 2
    slot = np.where((v < 0) | (v >= mv), mv, v)
    f = w.cdf[idx, slot + 1].astype(np.int64) - w.cdf[idx, slot]
    info = float(np.sum(16.0 - np.log2(f)))          # bypass raw bits not included
    per_sym = payload_bits / w.n
    assert 2.3 < per_sym < 2.9
    assert info < payload_bits < info + 64 * 4096 + 0.05 * w.n


def test_oracle_does_not_touch_inputs():
    w = W.load("tiny")
    s0, i0 = w.symbols.copy(), w.indexes.copy()
    oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, 64)
    assert np.array_equal(s0, w.symbols) and np.array_equal(i0, w.indexes)


def test_log2_information_identity():
    """Sanity of the size-bound helper itself on a hand case: f=32768 costs 1 bit."""
    cdf, lengths, offsets = single_table([0, 32768, 65535, 65536])
    bits, puts = lane_information([0, 0, 2], [0, 0, 0], cdf, lengths, offsets)
    assert puts == 4 and math.isclose(bits, 1 + 1 + 16 + 4)
