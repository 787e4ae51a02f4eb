"""Run the quick oracle pins against a given build of the oracle library.

Exit status 0 means every pin held, 1 means at least one failed (a crash
also counts as a failure).  Used by test_oracle_mutants.py, which plants
deliberate mistakes in copies of the oracle source and expects each copy to
be caught.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from oracle import spec_model as sm  # noqa: E402
import workloads as W  # noqa: E402
from helpers import lane_information, lane_words_from_container, single_table, worked_cases  # noqa: E402


def pins(lib):
    failures = []
    for c in worked_cases():
        cdf, lengths, offsets = single_table(c["row"])
        n = len(c["symbols"])
        rc, words = oracle.encode(np.asarray(c["symbols"]), np.zeros(n), cdf, lengths, offsets,
                                  c["lanes"], lib=lib)
        if rc != 0 or words.tolist() != c["words"]:
            failures.append(f"worked encode {c['name']}")
        rc, out = oracle.decode(np.asarray(c["words"], np.uint32), np.zeros(n), cdf, lengths,
                                offsets, c["lanes"], lib=lib)
        if rc != 0 or out.tolist() != c["symbols"]:
            failures.append(f"worked decode {c['name']}")
    w = W.load("tiny")
    for L in (1, 3, 64):
        rc, words = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, L, lib=lib)
        if rc != 0:
            failures.append(f"tiny encode L={L} rc={rc}")
            continue
        rc, out = oracle.decode(words, w.indexes, w.cdf, w.lengths, w.offsets, L, lib=lib)
        if rc != 0 or not np.array_equal(out, w.symbols):
            failures.append(f"tiny round trip L={L}")
        ref = sm.encode(w.symbols[:600].tolist(), w.indexes[:600].tolist(),
                        [w.cdf[r, : w.lengths[r]].tolist() for r in range(w.num_tables)],
                        w.offsets.tolist(), 3)
        rc, sub = oracle.encode(w.symbols[:600], w.indexes[:600], w.cdf, w.lengths, w.offsets, 3,
                                lib=lib)
        if rc != 0 or sub.tolist() != ref:
            failures.append("spec model agreement")
        lanes = lane_words_from_container(words.tolist(), L)
        for j, ls in enumerate(lanes):
            b, e = (j * w.n) // L, ((j + 1) * w.n) // L
            bits, puts = lane_information(w.symbols[b:e], w.indexes[b:e], w.cdf, w.lengths,
                                          w.offsets)
            if not (bits + 32 - 9e-5 * puts < 32 * len(ls) <= bits + 64 + 9e-5 * puts):
                failures.append(f"size bound L={L} lane {j}")
                break
    # corrupt containers must be refused: a lane that runs short, and a lane
    # with a trailing word that is never read
    rc, words = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, 4, lib=lib)
    if rc == 0:
        short = words[:-1].copy()
        short[4] -= 1
        extra = np.concatenate([words, [7]]).astype(np.uint32)
        extra[4] += 1
        for bad, label in ((short, "short lane"), (extra, "extra word")):
            rc, _ = oracle.decode(bad, w.indexes, w.cdf, w.lengths, w.offsets, 4, lib=lib)
            if rc != oracle.E_CORRUPT:
                failures.append(f"corrupt container accepted: {label}")
    return failures


if __name__ == "__main__":
    lib = oracle.load(sys.argv[1])
    f = pins(lib)
    print("\n".join(f) if f else "all pins hold")
    sys.exit(1 if f else 0)
