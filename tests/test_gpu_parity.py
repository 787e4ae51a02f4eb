"""GPU parity: the HIP coder against the CPU oracle, byte for byte.

Every synthetic workload runs at its own lane counts and at one lane (the
standard single stream; on the batches that puts 25M or 50M symbols in one
lane and its scratch spans 100-400 MB), and tiny and z also at 2, 3, 7, 255,
n and n + 5 lanes (ragged partitions and empty lanes).  For each case the GPU encode must equal
the oracle's container word for word, the GPU must decode the oracle's
container back to the input, and each side decodes the other's stream.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny", L) for L in (64, 1, 2, 3, 7, 255, 16384, 16389)
] + [
    ("z", L) for L in (256, 1, 2, 3, 7, 255, 97920, 97925)
] + [
    ("y1080", 4096), ("y1080", 1), ("y1080", 977),
    ("y1080x16", 65536), ("y1080x16", 1),
    ("y4kx8", 1024), ("y4kx8", 16384), ("y4kx8", 131072), ("y4kx8", 1),
]

_cache = {}


def _workload(name):
    if name not in _cache:
        import gpu_util as G
        w = W.load(name)
        _cache.clear()
        _cache[name] = (w, G.tables_of(w), G.to_dev(w.symbols), G.to_dev(w.indexes))
    return _cache[name]


@pytest.mark.parametrize("name,lanes", CASES, ids=[f"{n}-L{L}" for n, L in CASES])
def test_encode_decode_match_oracle(name, lanes):
    import gpu_util as G
    w, tables, sym, idx = _workload(name)
    G.say(f"[parity] {name} n={w.n} lanes={lanes}: oracle encode")
    rc, ref = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, lanes)
    assert rc == 0
    G.say(f"[parity] {name} lanes={lanes}: gpu encode")
    st, got, nw = G.gpu_encode(sym, idx, tables, lanes)
    assert st == 0, f"encode status {st}"
    assert nw == ref.size, f"container size {nw} != oracle {ref.size}"
    if not np.array_equal(got, ref):
        bad = np.flatnonzero(got != ref)
        pytest.fail(f"{bad.size} words differ, first at {bad[0]}: {got[bad[0]]:#x} != {ref[bad[0]]:#x}")
    G.say(f"[parity] {name} lanes={lanes}: gpu decode of the oracle stream")
    st, out = G.gpu_decode(ref, idx, tables)
    assert st == 0, f"decode status {st}"
    assert np.array_equal(out, w.symbols)
    G.say(f"[parity] {name} lanes={lanes}: oracle decode of the gpu stream")
    rc, back = oracle.decode(got, w.indexes, w.cdf, w.lengths, w.offsets, lanes)
    assert rc == 0 and np.array_equal(back, w.symbols)


def test_empty_input_and_more_lanes_than_symbols():
    import gpu_util as G
    w, tables, sym, idx = _workload("tiny")
    for n, lanes in ((0, 1), (0, 5), (3, 8), (5, 5), (1, 64), (130, 129)):
        G.say(f"[edge] n={n} lanes={lanes}")
        rc, ref = oracle.encode(w.symbols[:n], w.indexes[:n], w.cdf, w.lengths, w.offsets, lanes)
        st, got, nw = G.gpu_encode(sym[:n], idx[:n], tables, lanes)
        assert rc == 0 and st == 0
        assert np.array_equal(got, ref)
        st, out = G.gpu_decode(ref, idx[:n], tables)
        assert st == 0 and np.array_equal(out, w.symbols[:n])


def test_bypass_edges_and_extremes():
    """Every zig-zag boundary and both 2^30 limits, on tiny, z and the 4-slot hand row."""
    import gpu_util as G
    rows = np.full((2, 5), 65536, np.int32)
    rows[0, :4] = [0, 32768, 65535, 65536]
    rows[1, :5] = [0, 1, 2, 65535, 65536]
    lengths = np.array([4, 5], np.int32)
    offsets = np.array([0, -7], np.int32)
    raws = list(W.EDGE_RAWS) + [2, 3, 14, 17, 4095, 4096, 65535, 65536, 1 << 20]
    syms, idxs = [], []
    for r in (0, 1):
        mv = lengths[r] - 2
        for raw in raws:
            syms.append(W.raw_to_value(raw, mv) + offsets[r])
            idxs.append(r)
        syms += [offsets[r], offsets[r] + mv - 1]
        idxs += [r, r]
    syms = np.array(syms * 7, np.int64).astype(np.int32)
    idxs = np.array(idxs * 7, np.int32)
    tables = G.B.Tables.from_numpy(rows, lengths, offsets, G.DEV)
    for lanes in (1, 3, 64):
        G.say(f"[bypass edges] lanes={lanes}")
        rc, ref = oracle.encode(syms, idxs, rows, lengths, offsets, lanes)
        assert rc == 0
        st, got, _ = G.gpu_encode(G.to_dev(syms), G.to_dev(idxs), tables, lanes)
        assert st == 0 and np.array_equal(got, ref)
        st, out = G.gpu_decode(ref, G.to_dev(idxs), tables)
        assert st == 0 and np.array_equal(out, syms)


def test_extreme_offsets():
    """Rows whose coded range reaches the int32 limits (values offset + slot
    that may not fit int32 take the general path on both sides)."""
    import gpu_util as G
    imax, imin = 2**31 - 1, -2**31
    rows = np.full((4, 6), 65536, np.int32)
    rows[:, :6] = [0, 1000, 30000, 60000, 65000, 65536]
    lengths = np.array([6, 6, 6, 6], np.int32)
    offsets = np.array([imax - 1, imin, imax - 3, imax], np.int32)
    syms, idxs = [], []
    for r, vals in ((0, [imax - 1, imax, imax - 2, imax - 1000, imax - 2**20]),
                    (1, [imin, imin + 1, imin + 3, imin + 4, imin + 100]),
                    (2, [imax - 3, imax - 2, imax - 1, imax, imax - 700]),
                    (3, [imax, imax - 1, imax - 9])):
        syms += vals
        idxs += [r] * len(vals)
    rng = np.random.default_rng(11)
    order = rng.permutation(np.repeat(np.arange(len(syms)), 40))
    syms = np.array(syms, np.int64)[order].astype(np.int32)
    idxs = np.array(idxs, np.int32)[order]
    tables = G.B.Tables.from_numpy(rows, lengths, offsets, G.DEV)
    for lanes in (1, 5, 64):
        G.say(f"[extreme offsets] lanes={lanes}")
        rc, ref = oracle.encode(syms, idxs, rows, lengths, offsets, lanes)
        assert rc == 0
        st, got, _ = G.gpu_encode(G.to_dev(syms), G.to_dev(idxs), tables, lanes)
        assert st == 0 and np.array_equal(got, ref)
        st, out = G.gpu_decode(ref, G.to_dev(idxs), tables)
        assert st == 0 and np.array_equal(out, syms)
    # s - offset wraps to a small value mod 2^32: still out of range
    bad = syms.copy()
    k = int(np.flatnonzero(idxs == 3)[0])
    bad[k] = imin
    rc, _ = oracle.encode(bad, idxs, rows, lengths, offsets, 8)
    st, _, _ = G.gpu_encode(G.to_dev(bad), G.to_dev(idxs), tables, 8)
    assert rc == oracle.E_SYMBOL_RANGE and st == rc


def test_wide_rows_uniform_symbols():
    """Uniform symbols over the widest rows: most steps miss the lookup pair
    (on both sides of it) or escape."""
    import gpu_util as G
    cdf, lengths, offsets, _ = W.gaussian_table_set(64)
    rng = np.random.default_rng(5)
    n = 40000
    idxs = rng.integers(56, 64, n).astype(np.int32)
    mv = lengths[idxs] - 2
    v = (rng.random(n) * (mv + 40)).astype(np.int64) - 20
    syms = (v + offsets[idxs]).astype(np.int32)
    tables = G.B.Tables.from_numpy(cdf, lengths, offsets, G.DEV)
    for lanes in (64, 1000):
        G.say(f"[wide rows] lanes={lanes}")
        rc, ref = oracle.encode(syms, idxs, cdf, lengths, offsets, lanes)
        assert rc == 0
        st, got, _ = G.gpu_encode(G.to_dev(syms), G.to_dev(idxs), tables, lanes)
        assert st == 0 and np.array_equal(got, ref)
        st, out = G.gpu_decode(ref, G.to_dev(idxs), tables)
        assert st == 0 and np.array_equal(out, syms)


def test_workspace_reuse_across_lane_counts():
    """One workspace, calls with growing and shrinking wave counts: every
    call must find its look-back flags zero, whatever earlier calls with
    other lane counts left in the workspace."""
    import gpu_util as G
    w, tables, sym, idx = _workload("tiny")
    for lanes in (64, 1000, 7, 4096, 2048, 16384, 300, 5000):
        G.say(f"[reuse] lanes={lanes}")
        rc, ref = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, lanes)
        st, got, _ = G.gpu_encode(sym, idx, tables, lanes)
        assert rc == 0 and st == 0 and np.array_equal(got, ref)


def test_repeat_calls_are_identical_and_workspace_is_reusable():
    import gpu_util as G
    w, tables, sym, idx = _workload("tiny")
    first = None
    for k in range(3):
        G.say(f"[repeat] call {k}")
        st, got, _ = G.gpu_encode(sym, idx, tables, 64)
        assert st == 0
        if first is None:
            first = got
        assert np.array_equal(got, first)
        st, out = G.gpu_decode(got, idx, tables)
        assert st == 0 and np.array_equal(out, w.symbols)


def test_prepared_tables_code_many_tensors():
    import torch
    import gpu_util as G
    w, tables, sym, idx = _workload("tiny")
    B = G.B
    n = w.n
    ws = B.workspace_for(G.DEV).get(B.workspace_bytes(n, 64, tables.num_tables, tables.stride))
    B.prepare_tables(tables, ws)
    for lo, hi, lanes in ((0, 5000, 16), (5000, 16384, 33), (100, 101, 1)):
        G.say(f"[prepared] [{lo},{hi}) lanes={lanes}")
        rc, ref = oracle.encode(w.symbols[lo:hi], w.indexes[lo:hi], w.cdf, w.lengths, w.offsets,
                                lanes)
        stream, nwords, status = B.encode_with_indexes(sym[lo:hi].contiguous(),
                                                       idx[lo:hi].contiguous(), tables, lanes,
                                                       workspace=ws, prepared=True)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        got = stream[: int(nwords.item())].cpu().numpy().view(np.uint32)
        assert np.array_equal(got, ref)
        out, status = B.decode_with_indexes(stream, idx[lo:hi].contiguous(), tables,
                                            workspace=ws, prepared=True)
        assert int(status.item()) == 0
        assert np.array_equal(out.cpu().numpy(), w.symbols[lo:hi])


def test_full_and_prepared_calls_share_a_workspace():
    """The *_with_indexes entry points leave their tables prepared in the
    workspace for later *_prepared calls, and a stand-alone preparation of
    other tables is replaced by the next full call.  Two table sets of
    different row counts and widths alternate on one workspace."""
    import torch
    import gpu_util as G
    B = G.B
    wt, tt, st_sym, st_idx = _workload("tiny")
    tiny = (wt, tt, st_sym, st_idx)
    wz = W.load("z")
    tz = G.tables_of(wz)
    z = (wz, tz, G.to_dev(wz.symbols), G.to_dev(wz.indexes))
    nbytes = max(B.workspace_bytes(w.n, 256, t.num_tables, t.stride) for w, t, _, _ in (tiny, z))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=G.DEV)
    refs = {}
    for w, t, _, _ in (tiny, z):
        rc, refs[w.name] = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, 256)
        assert rc == 0
    for step, (w, t, sym, idx), prepared in (
            (0, tiny, False), (1, tiny, True), (2, z, False), (3, z, True), (4, tiny, False),
            (5, z, False), (6, z, True)):
        G.say(f"[shared-ws] step {step}: {w.name} prepared={prepared}")
        stream, nwords, status = B.encode_with_indexes(sym, idx, t, 256, workspace=ws,
                                                       prepared=prepared)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        got = stream[: int(nwords.item())].cpu().numpy().view(np.uint32)
        assert np.array_equal(got, refs[w.name])
        out, status = B.decode_with_indexes(stream, idx, t, workspace=ws, prepared=prepared)
        assert int(status.item()) == 0
        assert np.array_equal(out.cpu().numpy(), w.symbols)
    G.say("[shared-ws] stand-alone preparation replaced by the next full call")
    B.prepare_tables(tiny[1], ws)
    stream, nwords, status = B.encode_with_indexes(z[2], z[3], tz, 256, workspace=ws)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(stream[: int(nwords.item())].cpu().numpy().view(np.uint32), refs["z"])


# ------------------------------------------------------------------- errors
def test_bad_index_reports_status():
    import gpu_util as G
    w, tables, sym, idx = _workload("tiny")
    bad = w.indexes.copy()
    bad[1234] = 8
    G.say("[errors] bad index encode")
    st, _, _ = G.gpu_encode(sym, G.to_dev(bad), tables, 64)
    assert st == oracle.E_INDEX
    rc, ref = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, 64)
    bad[99] = -1
    G.say("[errors] bad index decode")
    st, _ = G.gpu_decode(ref, G.to_dev(bad), tables)
    assert st == oracle.E_INDEX
    G.say("[errors] clean call after errors")
    st, got, _ = G.gpu_encode(sym, idx, tables, 64)
    assert st == 0 and np.array_equal(got, ref)


def test_symbol_out_of_range_reports_status():
    import gpu_util as G
    w, tables, sym, idx = _workload("tiny")
    s = w.symbols.copy()
    r = int(w.indexes[77])
    s[77] = np.int32(int(w.offsets[r]) - (1 << 30) - 1)
    G.say("[errors] symbol out of range")
    st, _, _ = G.gpu_encode(G.to_dev(s), idx, tables, 64)
    assert st == oracle.E_SYMBOL_RANGE


def test_bad_table_reports_status():
    import gpu_util as G
    w, _, sym, idx = _workload("tiny")
    cdf = w.cdf.copy()
    cdf[3, 5] = cdf[3, 4]          # zero frequency
    tables = G.B.Tables.from_numpy(cdf, w.lengths, w.offsets, G.DEV)
    G.say("[errors] bad table")
    st, _, _ = G.gpu_encode(sym, idx, tables, 64)
    assert st == oracle.E_TABLE
    lengths = w.lengths.copy()
    lengths[2] = 2
    tables = G.B.Tables.from_numpy(w.cdf, lengths, w.offsets, G.DEV)
    st, _, _ = G.gpu_encode(sym, idx, tables, 64)
    assert st == oracle.E_TABLE


def test_capacity_too_small_reports_status_and_stays_in_bounds():
    import gpu_util as G
    w, tables, sym, idx = _workload("tiny")
    rc, ref = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, 64)
    for cap in (ref.size - 1, 65 + 100, ref.size // 2):
        G.say(f"[errors] capacity {cap}")
        st, _, nw = G.gpu_encode(sym, idx, tables, 64, capacity=cap)
        assert st == oracle.E_CAPACITY and nw == ref.size
    st, got, _ = G.gpu_encode(sym, idx, tables, 64, capacity=ref.size)
    assert st == 0 and np.array_equal(got, ref)


def test_corrupt_streams_report_status():
    import gpu_util as G
    w, tables, sym, idx = _workload("tiny")
    L = 4
    rc, words = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, L)
    G.say("[errors] corrupt streams")
    assert G.gpu_decode(words, idx, tables)[0] == 0
    # the lane count in the header word: one more or one fewer lane, none,
    # more lanes than the container has words, above the lane limit
    for bad_L in (L + 1, L - 1, 0, words.size, (1 << 22) + 1):
        s = words.copy(); s[0] = bad_L
        assert G.gpu_decode(s, idx, tables)[0] == oracle.E_CORRUPT, bad_L
    s = words.copy(); s[1], s[2] = s[2], s[1]
    assert G.gpu_decode(s, idx, tables)[0] == oracle.E_CORRUPT
    assert G.gpu_decode(words[:-1], idx, tables)[0] == oracle.E_CORRUPT
    s = words[:-1].copy(); s[L] -= 1
    assert G.gpu_decode(s, idx, tables)[0] == oracle.E_CORRUPT
    s = np.concatenate([words, [123]]).astype(np.uint32); s[L] += 1
    assert G.gpu_decode(s, idx, tables)[0] == oracle.E_CORRUPT
    s = words.copy(); s[1] = 1
    assert G.gpu_decode(s, idx, tables)[0] == oracle.E_CORRUPT
    rng = np.random.default_rng(3)
    for k in range(8):
        s = words.copy()
        pos = int(rng.integers(1 + L, s.size))
        s[pos] ^= np.uint32(1 << int(rng.integers(0, 32)))
        st, out = G.gpu_decode(s, idx, tables)
        rco, outo = oracle.decode(s, w.indexes, w.cdf, w.lengths, w.offsets, int(s[0]))
        # both sides agree on acceptance; where both accept, outputs agree
        assert (st == 0) == (rco == 0)
        if st == 0:
            assert np.array_equal(out, outo)
    assert G.gpu_decode(words, idx, tables)[0] == 0


# ------------------------------------------------- table sets over the LDS budget
def _wide_table_set(K, lengths, seed):
    """K rows of the given lengths (stride = the longest), each a random pmf
    with every frequency at least 1, escape slot included."""
    rng = np.random.default_rng(seed)
    stride = int(max(lengths))
    cdf = np.full((K, stride), 65536, np.int32)
    for r, n in enumerate(lengths):
        p = rng.dirichlet(np.full(n - 1, 0.7))
        f = np.maximum(1, np.floor(p * (65536 - (n - 1)))).astype(np.int64)
        f[int(np.argmax(f))] += 65536 - int(f.sum())
        cdf[r, :n] = np.concatenate([[0], np.cumsum(f)])
    offsets = rng.integers(-2000, 2000, K).astype(np.int32)
    return cdf, np.asarray(lengths, np.int32), offsets


def _symbols_for(cdf, lengths, offsets, n, seed):
    rng = np.random.default_rng(seed)
    K = lengths.size
    idx = rng.integers(0, K, n).astype(np.int32)
    u = rng.random(n)
    sym = np.empty(n, np.int64)
    for r in range(K):
        sel = np.flatnonzero(idx == r)
        c = cdf[r, : lengths[r] - 1].astype(np.float64) / 65536.0   # slot starts
        sym[sel] = np.searchsorted(c, u[sel], side="right") - 1 + offsets[r]
    esc = rng.random(n) < 0.01
    sym[esc] += np.where(rng.random(int(esc.sum())) < 0.5, -1, 1) * (lengths[idx[esc]] + 1000)
    return sym.astype(np.int32), idx


@pytest.mark.parametrize("kind", ["both_global", "encoder_global"])
def test_table_sets_over_the_lds_budget(kind):
    """Sets whose packed form does not fit LDS are read from the workspace:
    64 rows of 3133 entries (both sets over budget), and 16 rows of 2500
    (the encoder set, 4 bytes a slot, over budget; the decoder set fits).
    Lane, split-record and interleaved containers must equal the oracle's
    word for word, and each decodes back."""
    import torch
    import gpu_util as G
    B = G.B
    if kind == "both_global":
        cdf, lengths, offsets = _wide_table_set(64, [3133] * 64, 41)
    else:
        cdf, lengths, offsets = _wide_table_set(16, [2500] * 16, 42)
    sym, idx = _symbols_for(cdf, lengths, offsets, 120_001, 43)
    tables = B.Tables.from_numpy(cdf, lengths, offsets, G.DEV)
    dsym, didx = G.to_dev(sym), G.to_dev(idx)
    for lanes in (1, 97, 4096):
        G.say(f"[over-budget] {kind} lanes={lanes}")
        rc, ref = oracle.encode(sym, idx, cdf, lengths, offsets, lanes)
        assert rc == 0
        st, got, nw = G.gpu_encode(dsym, didx, tables, lanes)
        assert st == 0 and nw == ref.size and np.array_equal(got, ref)
        st, out = G.gpu_decode(ref, didx, tables)
        assert st == 0 and np.array_equal(out, sym)
    G.say(f"[over-budget] {kind} split records")
    rc, sref, rmeta = oracle.encode_split(sym, idx, cdf, lengths, offsets, 97, 4)
    stream, nwords, meta, status = B.encode_with_splits(dsym, didx, tables, 97, 4)
    torch.cuda.synchronize()
    assert rc == 0 and int(status.item()) == 0
    assert np.array_equal(meta.cpu().numpy().view(np.uint32).reshape(rmeta.shape), rmeta)
    out, status = B.decode_with_splits(stream, meta, didx, tables, 4)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and np.array_equal(out.cpu().numpy(), sym)
    for S in (3, 64):
        G.say(f"[over-budget] {kind} interleaved S={S}")
        rc, iref = oracle.encode_interleaved(sym, idx, cdf, lengths, offsets, S, 64)
        istream, inw, ist = B.encode_interleaved(dsym, didx, tables, S)
        torch.cuda.synchronize()
        assert rc == 0 and int(ist.item()) == 0
        assert np.array_equal(istream[: int(inw.item())].cpu().numpy().view(np.uint32), iref)
        out, st2 = B.decode_interleaved(istream, didx, tables, S)
        torch.cuda.synchronize()
        assert int(st2.item()) == 0 and np.array_equal(out.cpu().numpy(), sym)
