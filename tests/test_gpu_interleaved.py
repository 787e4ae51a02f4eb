"""GPU parity of interleaved streams (64 states per stream, one shared cursor).

For each case the GPU container must equal the oracle's word for word, the
GPU must decode the oracle's container back to the input, and each side
decodes the other's.  Cases: the hand-derived two-state pattern scaled to 64
states (all lanes escaping in one step), streams shorter than 64 symbols,
ragged last steps, every config at several stream counts, and corrupt
containers refused like the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

# Blocks hold 4 streams below 2048, 8 from 2048 and 16 from 4096: 2047 and
# 4095 sit just below a boundary; "tiny" at 4096 gives streams of 4 symbols,
# "z" at 4100 and "y4kx8" at 5000 a partly filled last block.
CASES = [("tiny", 1), ("tiny", 4), ("tiny", 255), ("tiny", 300), ("z", 4), ("z", 1531),
         ("y1080", 64), ("y1080", 1024), ("y1080x16", 1024), ("y4kx8", 2048),
         ("tiny", 2047), ("z", 4095),
         ("tiny", 4096), ("z", 4100), ("y1080x16", 4096), ("y4kx8", 5000)]

_cache = {}


def _workload(name):
    if name not in _cache:
        import gpu_util as G
        w = W.load(name)
        _cache.clear()
        _cache[name] = (w, G.tables_of(w), G.to_dev(w.symbols), G.to_dev(w.indexes))
    return _cache[name]


def _gpu_encode(sym, idx, tables, S):
    import torch
    import gpu_util as G
    stream, nw, st = G.B.encode_interleaved(sym, idx, tables, S)
    torch.cuda.synchronize()
    return int(st.item()), stream[: int(nw.item())].cpu().numpy().view(np.uint32).copy()


def _gpu_decode(words, idx, tables, S):
    import torch
    import gpu_util as G
    s = torch.from_numpy(np.asarray(words, np.uint32).view(np.int32).copy()).to(G.DEV)
    out, st = G.B.decode_interleaved(s, idx, tables, S)
    torch.cuda.synchronize()
    return int(st.item()), out.cpu().numpy()


@pytest.mark.parametrize("name,S", CASES, ids=[f"{n}-S{s}" for n, s in CASES])
def test_interleaved_matches_oracle(name, S):
    import gpu_util as G
    w, tables, sym, idx = _workload(name)
    G.say(f"[interleaved] {name} streams={S}: oracle")
    rc, ref = oracle.encode_interleaved(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, S, 64)
    assert rc == 0
    G.say(f"[interleaved] {name} streams={S}: gpu encode")
    st, got = _gpu_encode(sym, idx, tables, S)
    assert st == 0
    if not np.array_equal(got, ref):
        n = min(got.size, ref.size)
        bad = np.flatnonzero(got[:n] != ref[:n])
        pytest.fail(f"sizes {got.size}/{ref.size}; {bad.size} words differ, first at "
                    f"{bad[0] if bad.size else n}")
    G.say(f"[interleaved] {name} streams={S}: gpu decode of the oracle's container")
    st, out = _gpu_decode(ref, idx, tables, S)
    assert st == 0 and np.array_equal(out, w.symbols)


def test_escapes_in_every_lane():
    """Row A of the worked streams: symbols 2 and -1 alternating (escapes in
    every lane of every step, words emitted in many slots)."""
    import gpu_util as G
    from helpers import single_table
    cdf, lengths, offsets = single_table([0, 32768, 65535, 65536])
    syms = np.tile(np.array([2, -1, 7, -9, 0, 1, 300, -4000], np.int32), 1000)
    idx = np.zeros(syms.size, np.int32)
    tables = G.B.Tables.from_numpy(cdf, lengths, offsets, G.DEV)
    for S in (1, 3, 40):
        G.say(f"[interleaved] escapes S={S}")
        rc, ref = oracle.encode_interleaved(syms, idx, cdf, lengths, offsets, S, 64)
        st, got = _gpu_encode(G.to_dev(syms), G.to_dev(idx), tables, S)
        assert rc == 0 and st == 0 and np.array_equal(got, ref)
        st, out = _gpu_decode(ref, G.to_dev(idx), tables, S)
        assert st == 0 and np.array_equal(out, syms)


def test_corrupt_containers_like_the_oracle():
    import gpu_util as G
    w, tables, sym, idx = _workload("tiny")
    S = 4
    rc, ref = oracle.encode_interleaved(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, S, 64)
    rng = np.random.default_rng(9)
    cases = [ref[:-1].copy(), np.concatenate([ref, [5]]).astype(np.uint32)]
    cases[0][S] -= 1
    cases[1][S] += 1
    for k in range(6):
        c = ref.copy()
        c[int(rng.integers(1 + S, c.size))] ^= np.uint32(1 << int(rng.integers(0, 32)))
        cases.append(c)
    for c in cases:
        G.say("[interleaved] corrupt container")
        rco, outo = oracle.decode_interleaved(c, w.indexes, w.cdf, w.lengths, w.offsets, S, 64)
        st, out = _gpu_decode(c, idx, tables, S)
        assert (st == 0) == (rco == 0), (st, rco)
        if st == 0:
            assert np.array_equal(out, outo)
    st, _ = _gpu_decode(ref, idx, tables, S + 1)
    assert st == oracle.E_CORRUPT


def test_prepared_interleaved_calls_code_many_tensors():
    """One preparation, then interleaved encodes and decodes of several
    tensors and stream counts (4-wave, 8-wave and 16-wave blocks) on that
    workspace; each container equals the oracle's.  A table count that does
    not match the prepared set is refused on the device, and a full call on
    the same workspace replaces the prepared set."""
    import torch
    import gpu_util as G
    B = G.B
    w, tables, sym, idx = _workload("tiny")
    n = w.n
    wz = W.load("z")
    tz = G.tables_of(wz)
    # one workspace for both table sets (its regions are sized by rows and stride)
    lib = B.load()
    ws = torch.zeros(max(lib.rans_interleaved_workspace_bytes(n, 4096, tables.num_tables,
                                                              tables.stride),
                         lib.rans_interleaved_workspace_bytes(16384, 64, tz.num_tables, tz.stride)),
                     dtype=torch.uint8, device=G.DEV)
    B.prepare_tables(tables, ws)
    for lo, hi, S in ((0, 16384, 4096), (5000, 16384, 2048), (100, 9000, 33), (7, 8, 1)):
        G.say(f"[il-prepared] [{lo},{hi}) streams={S}")
        rc, ref = oracle.encode_interleaved(w.symbols[lo:hi], w.indexes[lo:hi], w.cdf, w.lengths,
                                            w.offsets, S, 64)
        assert rc == 0
        stream, nw, st = B.encode_interleaved(sym[lo:hi].contiguous(), idx[lo:hi].contiguous(),
                                              tables, S, workspace=ws, prepared=True)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        assert np.array_equal(stream[: int(nw.item())].cpu().numpy().view(np.uint32), ref)
        out, st = B.decode_interleaved(stream, idx[lo:hi].contiguous(), tables, S, workspace=ws,
                                       prepared=True)
        torch.cuda.synchronize()
        assert int(st.item()) == 0 and np.array_equal(out.cpu().numpy(), w.symbols[lo:hi])
    G.say("[il-prepared] table count differs from the prepared set")
    wrong = B.Tables.from_numpy(w.cdf[:7], w.lengths[:7], w.offsets[:7], G.DEV)
    _, _, st = B.encode_interleaved(sym, idx, wrong, 4, workspace=ws, prepared=True)
    torch.cuda.synchronize()
    assert int(st.item()) == B.NAME_TO_CODE["RANS_E_ARG"]
    G.say("[il-prepared] a full call with other tables, then prepared calls with them")
    zsym, zidx = G.to_dev(wz.symbols[:16384]), G.to_dev(wz.indexes[:16384])
    rc, zref = oracle.encode_interleaved(wz.symbols[:16384], wz.indexes[:16384], wz.cdf,
                                         wz.lengths, wz.offsets, 64, 64)
    for prepared in (False, True):
        stream, nw, st = B.encode_interleaved(zsym, zidx, tz, 64, workspace=ws, prepared=prepared)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        assert np.array_equal(stream[: int(nw.item())].cpu().numpy().view(np.uint32), zref)


def test_encode_refused_up_front_copies_nothing():
    """An encode refused before coding (a zero-frequency row) reports
    RANS_E_TABLE; its streams' word counts are cleared, so the header and
    copy kernels never work from counts an earlier call left in the
    workspace, and the copy writes nothing.  A valid call on the same
    workspace afterwards still matches the oracle."""
    import torch
    import gpu_util as G
    B = G.B
    w, tables, sym, idx = _workload("tiny")
    S = 4096
    ws = torch.zeros(B.load().rans_interleaved_workspace_bytes(w.n, S, tables.num_tables,
                                                               tables.stride),
                     dtype=torch.uint8, device=G.DEV)
    rc, ref = oracle.encode_interleaved(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, S, 64)
    G.say("[il-refused] a valid encode leaves word counts in the workspace")
    stream, nw, st = B.encode_interleaved(sym, idx, tables, S, workspace=ws)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    bad_cdf = w.cdf.copy()
    bad_cdf[3, 2] = bad_cdf[3, 1]   # a zero frequency: the row is invalid
    bad = B.Tables.from_numpy(bad_cdf, w.lengths, w.offsets, G.DEV)
    G.say("[il-refused] the same call with an invalid row")
    sentinel = torch.full_like(stream, 0x5A5A5A5A)
    out, nw2, st = B.encode_interleaved(sym, idx, bad, S, workspace=ws, stream_out=sentinel)
    torch.cuda.synchronize()
    assert int(st.item()) == B.NAME_TO_CODE["RANS_E_TABLE"]
    # the payload area is untouched (the header words may be written)
    assert bool((out[1 + S:] == 0x5A5A5A5A).all())
    G.say("[il-refused] a valid encode afterwards")
    stream, nw, st = B.encode_interleaved(sym, idx, tables, S, workspace=ws)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(stream[: int(nw.item())].cpu().numpy().view(np.uint32), ref)
