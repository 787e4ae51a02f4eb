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
from helpers import (gaussian_row_by_integration, lane_information,  # noqa: E402
                     lane_words_from_container, latent_cases, LATENT_TABLE,
                     quantize_water_level, quantized_cases, single_table, worked_cases,
                     worked_splits, worked_interleaved, WORKED_ROWS)


def interleaved_pins(lib):
    failures = []
    cdf, lengths, offsets = single_table(WORKED_ROWS["A"])
    for c in worked_interleaved():
        n = len(c["symbols"])
        rc, words = oracle.encode_interleaved(np.asarray(c["symbols"]), np.zeros(n), cdf, lengths,
                                              offsets, c["streams"], c["width"], lib=lib)
        if rc != 0 or words.tolist() != c["words"]:
            failures.append(f"golden interleaved {c['name']}")
        rc, out = oracle.decode_interleaved(np.asarray(c["words"], np.uint32), np.zeros(n), cdf,
                                            lengths, offsets, c["streams"], c["width"], lib=lib)
        if rc != 0 or out.tolist() != c["symbols"]:
            failures.append(f"golden interleaved decode {c['name']}")
    w = W.load("tiny")
    for S, Wd in ((4, 64), (64, 1), (300, 8)):
        rc, words = oracle.encode_interleaved(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets,
                                              S, Wd, lib=lib)
        rc2, out = oracle.decode_interleaved(words, w.indexes, w.cdf, w.lengths, w.offsets, S, Wd,
                                             lib=lib)
        if rc or rc2 or not np.array_equal(out, w.symbols):
            failures.append(f"interleaved round trip S={S} W={Wd}")
    return failures


def split_pins(lib):
    failures = []
    cases = {c["name"]: c for c in worked_cases()}
    for name, pieces, recs in worked_splits():
        c = cases[name]
        cdf, lengths, offsets = single_table(c["row"])
        n = len(c["symbols"])
        rc, words, meta = oracle.encode_split(np.asarray(c["symbols"]), np.zeros(n), cdf, lengths,
                                              offsets, c["lanes"], pieces, lib=lib)
        if rc != 0 or words.tolist() != c["words"] or meta.reshape(-1, 3).tolist() != recs:
            failures.append(f"golden split records {name} P={pieces}")
        rc, out = oracle.decode_split(np.asarray(c["words"], np.uint32), np.asarray(recs, np.uint32),
                                      np.zeros(n), cdf, lengths, offsets, c["lanes"], pieces,
                                      lib=lib)
        if rc != 0 or out.tolist() != c["symbols"]:
            failures.append(f"golden split decode {name} P={pieces}")
    w = W.load("tiny")
    for L, P in ((64, 4), (7, 8), (300, 2)):
        rc, words, meta = oracle.encode_split(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets,
                                              L, P, lib=lib)
        rc0, plain = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, L, lib=lib)
        if rc or rc0 or not np.array_equal(words, plain):
            failures.append(f"split container differs L={L} P={P}")
            continue
        rc, out = oracle.decode_split(words, meta, w.indexes, w.cdf, w.lengths, w.offsets, L, P,
                                      lib=lib)
        if rc != 0 or not np.array_equal(out, w.symbols):
            failures.append(f"split round trip L={L} P={P}")
        bad = meta.copy()
        bad[L // 2, P // 2 - 1, 0] ^= 1
        rc, _ = oracle.decode_split(words, bad, w.indexes, w.cdf, w.lengths, w.offsets, L, P,
                                    lib=lib)
        if rc != oracle.E_CORRUPT:
            failures.append(f"altered split record accepted L={L} P={P}")
    return failures


def latent_pins(lib):
    failures = []
    syms, idxs = latent_cases()
    rc, sym, _ = oracle.latent_symbols([c[0] for c in syms], [c[1] for c in syms],
                                       np.ones(len(syms)), LATENT_TABLE, lib=lib)
    if rc != 0 or sym.tolist() != [c[2] for c in syms]:
        failures.append("golden latent symbols")
    rc, _, idx = oracle.latent_symbols(np.zeros(len(idxs)), np.zeros(len(idxs)),
                                       [c[0] for c in idxs], LATENT_TABLE, lib=lib)
    if rc != 0 or idx.tolist() != [c[1] for c in idxs]:
        failures.append("golden latent indexes")
    rc, out = oracle.dequantize(np.array([0, 1, -1], np.int32),
                                np.array([0.25, -0.5, 0.5], np.float32), lib=lib)
    if rc != 0 or out.tolist() != [0.25, 0.5, -0.5]:
        failures.append("dequantize")
    return failures


def table_pins(lib):
    from scipy.special import ndtri
    tail_z = float(ndtri(1.0 - 5e-10))
    failures = []
    for name, pmf, cdf in quantized_cases():
        rc, got = oracle.quantize_pmf(pmf, lib=lib)
        if rc != 0 or got.tolist() != cdf:
            failures.append(f"golden quantisation {name}")
    rng = np.random.default_rng(11)
    for trial in range(60):
        m = int(rng.integers(2, 12))
        p = rng.dirichlet(np.ones(m)) * rng.uniform(0.5, 2.0)
        p = np.minimum(p, 1.0)
        rc, got = oracle.quantize_pmf(p, lib=lib)
        if rc != 0 or not np.array_equal(np.diff(got.astype(np.int64)), quantize_water_level(p)):
            failures.append(f"closed-form quantisation trial {trial}")
            break
    for K, z in ((8, tail_z), (12, 1.0)):
        scales = np.exp(np.log(0.11) + (np.log(256.0) - np.log(0.11)) * np.arange(K) / (K - 1))
        stride = 2 * int(np.ceil(scales[-1] * z)) + 3
        rc, cdf, lengths, offsets = oracle.gaussian_tables(scales, z, stride, lib=lib)
        if rc != 0:
            failures.append(f"gaussian K={K} rc={rc}")
            continue
        for r, s in enumerate(scales):
            ref, off, _ = gaussian_row_by_integration(float(s), z)
            n = int(lengths[r])
            if (n != len(ref) or int(offsets[r]) != off or cdf[r, :n].tolist() != ref
                    or np.any(cdf[r, n:] != 65536)):
                failures.append(f"gaussian K={K} row {r}")
                break
    if oracle.gaussian_tables(np.array([2.0]), tail_z, 28, lib=lib)[0] != oracle.E_TABLE:
        failures.append("gaussian row longer than the stride accepted")
    return failures


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
    f = pins(lib) + table_pins(lib) + latent_pins(lib) + split_pins(lib) + interleaved_pins(lib)
    print("\n".join(f) if f else "all pins hold")
    sys.exit(1 if f else 0)
