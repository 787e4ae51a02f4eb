"""GPU parity at the ABI's limits (include/rans_hip.h): the most lanes,
interleaved streams, split pieces, table rows and row length a call takes,
and the most symbols.

Each case but the last compares the GPU container with the oracle's word for
word and decodes the oracle's container on the GPU.  At RANS_MAX_SYMBOLS
symbols (2^28, generated on the device) the oracle codes a sample of lanes
one by one (a lane's words do not depend on the other lanes), each compared
with that lane's words in the GPU container, and the whole container must
decode back to the input on the GPU.
"""
from __future__ import annotations

import os
import re

import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "rans_hip.h")


def _limit(name: str) -> int:
    text = open(HEADER).read()
    m = re.search(rf"#define {name} \(?(\d+)(ull|u)?( << (\d+)\))?", text)
    assert m, name
    v = int(m.group(1))
    return v << int(m.group(4)) if m.group(4) else v


MAX_LANES = _limit("RANS_MAX_LANES")
MAX_STREAMS = _limit("RANS_MAX_STREAMS")
MAX_PIECES = _limit("RANS_MAX_PIECES")
MAX_TABLES = _limit("RANS_MAX_TABLES")
MAX_STRIDE = _limit("RANS_MAX_STRIDE")
MAX_SYMBOLS = _limit("RANS_MAX_SYMBOLS")


def test_limits_read_from_the_header():
    assert (MAX_LANES, MAX_STREAMS, MAX_PIECES) == (1 << 22, 1 << 16, 64)
    assert (MAX_TABLES, MAX_STRIDE, MAX_SYMBOLS) == (4096, 16384, 1 << 28)


def _symbols(cdf, lengths, offsets, n, seed, escapes=0.01):
    """Seeded symbols drawn from each row's own pmf, a share of them moved
    out of the coded range (bypass)."""
    rng = np.random.default_rng(seed)
    K = lengths.size
    idx = rng.integers(0, K, n).astype(np.int32)
    u = rng.random(n)
    sym = np.empty(n, np.int64)
    order = np.argsort(idx, kind="stable")
    bounds = np.searchsorted(idx[order], np.arange(K + 1))
    for r in range(K):
        sel = order[bounds[r]:bounds[r + 1]]
        if sel.size:
            starts = cdf[r, : lengths[r] - 1].astype(np.float64) / 65536.0
            sym[sel] = np.searchsorted(starts, u[sel], side="right") - 1 + offsets[r]
    esc = rng.random(n) < escapes
    sym[esc] += np.where(rng.random(int(esc.sum())) < 0.5, -1, 1) * (lengths[idx[esc]] + 300)
    return sym.astype(np.int32), idx


def _random_rows(lengths, seed):
    """Rows of the given lengths (stride = the longest), each a random pmf
    with every frequency at least 1, escape slot included."""
    rng = np.random.default_rng(seed)
    K, stride = len(lengths), int(max(lengths))
    cdf = np.full((K, stride), 65536, np.int32)
    for r, n in enumerate(lengths):
        p = rng.dirichlet(np.full(n - 1, 0.7))
        f = np.maximum(1, np.floor(p * (65536 - (n - 1)))).astype(np.int64)
        f[int(np.argmax(f))] += 65536 - int(f.sum())
        cdf[r, :n] = np.concatenate([[0], np.cumsum(f)])
    offsets = rng.integers(-2000, 2000, K).astype(np.int32)
    return cdf, np.asarray(lengths, np.int32), offsets


def _lane_round_trip(cdf, lengths, offsets, sym, idx, lanes, what):
    import gpu_util as G
    tables = G.B.Tables.from_numpy(cdf, lengths, offsets, G.DEV)
    dsym, didx = G.to_dev(sym), G.to_dev(idx)
    G.say(f"[limits] {what}: oracle, n={sym.size} lanes={lanes}")
    rc, ref = oracle.encode(sym, idx, cdf, lengths, offsets, lanes)
    assert rc == 0
    G.say(f"[limits] {what}: gpu encode")
    st, got, nw = G.gpu_encode(dsym, didx, tables, lanes)
    assert st == 0 and nw == ref.size and np.array_equal(got, ref)
    G.say(f"[limits] {what}: gpu decode of the oracle's container")
    st, out = G.gpu_decode(ref, didx, tables)
    assert st == 0 and np.array_equal(out, sym)
    return tables, dsym, didx


@pytest.mark.parametrize("n", [2 * MAX_LANES + 12345, MAX_LANES - 3],
                         ids=["2L+12345", "L-3"])
def test_lane_container_at_the_lane_limit(n):
    """RANS_MAX_LANES lanes: a ragged partition of about two symbols a lane,
    and fewer symbols than lanes (empty lanes)."""
    w = W.load("tiny")
    sym, idx = _symbols(w.cdf, w.lengths, w.offsets, n, 7101)
    _lane_round_trip(w.cdf, w.lengths, w.offsets, sym, idx, MAX_LANES, "max lanes")


def test_interleaved_at_the_stream_limit():
    """RANS_MAX_STREAMS interleaved streams, each two steps and a bit."""
    import torch
    import gpu_util as G
    w = W.load("tiny")
    n = MAX_STREAMS * 64 * 2 + 4321
    sym, idx = _symbols(w.cdf, w.lengths, w.offsets, n, 7102)
    tables = G.tables_of(w)
    dsym, didx = G.to_dev(sym), G.to_dev(idx)
    G.say(f"[limits] max streams: oracle, n={n} S={MAX_STREAMS}")
    rc, ref = oracle.encode_interleaved(sym, idx, w.cdf, w.lengths, w.offsets, MAX_STREAMS, 64)
    assert rc == 0
    G.say("[limits] max streams: gpu encode")
    stream, nw, st = G.B.encode_interleaved(dsym, didx, tables, MAX_STREAMS)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and int(nw.item()) == ref.size
    assert np.array_equal(stream[: ref.size].cpu().numpy().view(np.uint32), ref)
    G.say("[limits] max streams: gpu decode of the oracle's container")
    s = torch.from_numpy(ref.view(np.int32).copy()).to(G.DEV)
    out, st = G.B.decode_interleaved(s, didx, tables, MAX_STREAMS)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and np.array_equal(out.cpu().numpy(), sym)


@pytest.mark.parametrize("lanes", [7, 200])
def test_split_records_at_the_piece_limit(lanes):
    """RANS_MAX_PIECES pieces a lane: about 700 symbols a lane, and 25 (most
    pieces empty)."""
    import torch
    import gpu_util as G
    w = W.load("tiny")
    sym, idx = _symbols(w.cdf, w.lengths, w.offsets, 5000, 7103)
    tables = G.tables_of(w)
    dsym, didx = G.to_dev(sym), G.to_dev(idx)
    G.say(f"[limits] max pieces: lanes={lanes}")
    rc, ref, rmeta = oracle.encode_split(sym, idx, w.cdf, w.lengths, w.offsets, lanes, MAX_PIECES)
    assert rc == 0
    stream, nwords, meta, status = G.B.encode_with_splits(dsym, didx, tables, lanes, MAX_PIECES)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(stream[: int(nwords.item())].cpu().numpy().view(np.uint32), ref)
    assert np.array_equal(meta.cpu().numpy().view(np.uint32).reshape(rmeta.shape), rmeta)
    s = torch.from_numpy(ref.view(np.int32).copy()).to(G.DEV)
    m = torch.from_numpy(rmeta.view(np.int32).copy()).to(G.DEV)
    out, status = G.B.decode_with_splits(s, m, didx, tables, MAX_PIECES)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and np.array_equal(out.cpu().numpy(), sym)


def test_table_set_at_the_row_limit():
    """RANS_MAX_TABLES rows of 3 to 40 entries."""
    rng = np.random.default_rng(7104)
    lengths = rng.integers(3, 41, MAX_TABLES).tolist()
    cdf, lengths, offsets = _random_rows(lengths, 7105)
    sym, idx = _symbols(cdf, lengths, offsets, 300_000, 7106)
    for lanes in (1, 1000):
        _lane_round_trip(cdf, lengths, offsets, sym, idx, lanes, "max rows")


def test_rows_at_the_stride_limit():
    """Rows of RANS_MAX_STRIDE entries (16,382 ordinary slots each)."""
    cdf, lengths, offsets = _random_rows([MAX_STRIDE] * 3, 7107)
    sym, idx = _symbols(cdf, lengths, offsets, 200_000, 7108)
    for lanes in (1, 100):
        _lane_round_trip(cdf, lengths, offsets, sym, idx, lanes, "max stride")


def test_most_symbols_sampled_lanes():
    """RANS_MAX_SYMBOLS symbols (made on the device from a seeded generator)
    in 65,521 lanes: sampled lanes equal the oracle's coding of their
    symbols, and the whole container decodes back to the input."""
    import torch
    import gpu_util as G
    w = W.load("tiny")
    tables = G.tables_of(w)
    n, L = MAX_SYMBOLS, 65521
    g = torch.Generator(device=G.DEV)
    g.manual_seed(7109)
    K = int(w.lengths.size)
    G.say(f"[limits] max symbols: generating n={n}")
    idx = torch.randint(0, K, (n,), generator=g, device=G.DEV, dtype=torch.int32)
    mv = torch.from_numpy(w.lengths - 2).to(G.DEV)[idx.long()]
    off = torch.from_numpy(w.offsets).to(G.DEV)[idx.long()]
    u = torch.rand(n, generator=g, device=G.DEV)
    v = (u * mv.float()).long().clamp_(max=mv.long() - 1)
    esc = torch.rand(n, generator=g, device=G.DEV) < 0.005
    side = torch.rand(n, generator=g, device=G.DEV) < 0.5
    v = torch.where(esc, torch.where(side, -v - 1, mv.long() + v), v)
    sym = (v + off.long()).to(torch.int32)
    del mv, off, u, v, esc, side
    G.say("[limits] max symbols: gpu encode")
    stream, nwords, status = G.B.encode_with_indexes(sym, idx, tables, L)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    header = stream[: 1 + L].cpu().numpy().view(np.uint32).astype(np.int64)
    assert header[0] == L and int(nwords.item()) == 1 + L + int(header[L])
    rng = np.random.default_rng(7110)
    sample = sorted({0, 1, L // 2, L - 2, L - 1, *rng.integers(0, L, 11).tolist()})
    for j in sample:
        b, e = oracle.lane_begin(n, L, j), oracle.lane_begin(n, L, j + 1)
        s_h = sym[b:e].cpu().numpy()
        i_h = idx[b:e].cpu().numpy()
        rc, ref = oracle.encode_lane(s_h, i_h, 0, e - b, w.cdf, w.lengths, w.offsets)
        assert rc == 0
        lo = 1 + L + (int(header[j]) if j else 0)
        hi = 1 + L + int(header[1 + j])
        got = stream[lo:hi].cpu().numpy().view(np.uint32)
        assert np.array_equal(got, ref), f"lane {j} differs"
    G.say("[limits] max symbols: gpu decode")
    out, status = G.B.decode_with_indexes(stream, idx, tables)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(out, sym)
