"""Randomised GPU parity: seeded random table sets, lane counts, sizes and symbols.

Each case draws a table set (row count, lengths, offsets, pmfs from a few
shapes including near-uniform and spiky ones), symbols from the rows'
densities with out-of-range values mixed in (both signs, up to the 2^30
distance limit and just past it), and a lane count from 1 to beyond the
symbol count.  The GPU container must equal the oracle's word for word (or
both must report the same error), the GPU must decode the oracle's stream,
and the split-record and interleaved containers must match the oracle's too.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu


def _table_set(rng):
    K = int(rng.choice([1, 2, 7, 64, 300]))
    stride = int(rng.choice([3, 5, 40, 700]))
    rows, lengths, offsets = [], [], []
    for _ in range(K):
        n = int(rng.integers(3, stride + 1))
        kind = int(rng.integers(0, 3))
        if kind == 0:
            p = rng.dirichlet(np.full(n - 1, 0.3))
        elif kind == 1:
            p = np.ones(n - 1)
        else:
            p = np.full(n - 1, 1e-6)
            p[int(rng.integers(0, n - 1))] = 1.0
        f = np.maximum(1, np.floor(p / p.sum() * (65536 - (n - 1)))).astype(np.int64)
        f[int(np.argmax(f))] += 65536 - int(f.sum())
        cdf = np.concatenate([[0], np.cumsum(f)])
        row = np.full(stride, 65536, np.int32)
        row[:n] = cdf
        rows.append(row)
        lengths.append(n)
        offsets.append(int(rng.integers(-40, 40)))
    return np.stack(rows), np.array(lengths, np.int32), np.array(offsets, np.int32)


def _symbols(rng, cdf, lengths, offsets, n):
    K = lengths.size
    idx = rng.integers(0, K, n).astype(np.int32)
    sym = np.empty(n, np.int64)
    for r in range(K):
        sel = np.flatnonzero(idx == r)
        if sel.size == 0:
            continue
        f = np.diff(cdf[r, : lengths[r]].astype(np.int64))[:-1].astype(np.float64)
        p = f / f.sum() if f.size and f.sum() > 0 else None
        v = rng.choice(max(1, f.size), sel.size, p=p) if p is not None else np.zeros(sel.size)
        sym[sel] = v + offsets[r]
    esc = rng.random(n) < 0.02
    dist = np.floor(2.0 ** rng.uniform(0, 29.9, n)).astype(np.int64)
    sign = np.where(rng.random(n) < 0.5, -1, 1)
    sym = np.where(esc, offsets[idx] + np.where(sign < 0, -dist, lengths[idx] - 2 + dist), sym)
    return np.clip(sym, -2**31, 2**31 - 1).astype(np.int32), idx


@pytest.mark.parametrize("seed", range(24))
def test_random_case(seed):
    import torch
    import gpu_util as G
    rng = np.random.default_rng(1000 + seed)
    cdf, lengths, offsets = _table_set(rng)
    n = int(rng.choice([0, 1, 63, 1000, 20000, 150000]))
    lanes = int(rng.choice([1, 2, 63, 64, 65, 1000, 4096])) if n else int(rng.integers(1, 9))
    sym, idx = _symbols(rng, cdf, lengths, offsets, n)
    if seed % 6 == 5 and n:
        sym[int(rng.integers(0, n))] = offsets[idx[0]] - (1 << 30) - 5   # beyond the range limit
    G.say(f"[random] seed {seed}: K={lengths.size} stride={cdf.shape[1]} n={n} lanes={lanes}")
    tables = G.B.Tables.from_numpy(cdf, lengths, offsets, G.DEV)
    rc, ref = oracle.encode(sym, idx, cdf, lengths, offsets, lanes)
    st, got, nw = G.gpu_encode(G.to_dev(sym), G.to_dev(idx), tables, lanes)
    assert st == rc, (st, rc)
    if rc != 0:
        return
    assert nw == ref.size and np.array_equal(got, ref)
    st, out = G.gpu_decode(ref, G.to_dev(idx), tables)
    assert st == 0 and np.array_equal(out, sym)
    # split records at a random piece count
    P = int(rng.choice([2, 4, 16]))
    rc, _, rmeta = oracle.encode_split(sym, idx, cdf, lengths, offsets, lanes, P)
    stream, nwords, meta, status = G.B.encode_with_splits(G.to_dev(sym), G.to_dev(idx), tables,
                                                           lanes, P)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(meta.cpu().numpy().view(np.uint32).reshape(rmeta.shape), rmeta)
    out, status = G.B.decode_with_splits(stream, meta, G.to_dev(idx), tables, P)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and np.array_equal(out.cpu().numpy(), sym)
    # interleaved streams
    # (4096 and more streams run the 16-wave blocks)
    S = int(rng.choice([max(1, min(lanes, 300)), 4096, 4111]))
    rc, iref = oracle.encode_interleaved(sym, idx, cdf, lengths, offsets, S, 64)
    istream, inw, ist = G.B.encode_interleaved(G.to_dev(sym), G.to_dev(idx), tables, S)
    torch.cuda.synchronize()
    assert rc == 0 and int(ist.item()) == 0
    assert np.array_equal(istream[: int(inw.item())].cpu().numpy().view(np.uint32), iref)
    out, st2 = G.B.decode_interleaved(istream, G.to_dev(idx), tables, S)
    torch.cuda.synchronize()
    assert int(st2.item()) == 0 and np.array_equal(out.cpu().numpy(), sym)
