"""GPU parity of split records (decode parallelism beyond the lane count).

For each case the GPU encode must give the oracle's container and split
records word for word, the GPU must decode the oracle's container piece by
piece from the oracle's records back to the input, and altered records must
be refused as corrupt by both sides.  Cases cover many empty pieces (3 lanes
of 16,384 symbols cut in 16 or 64; lanes shorter than the piece count),
ragged pieces, the 1080p latent at 2, 4 and 8 pieces and a 4K batch.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

CASES = [("tiny", 64, 2), ("tiny", 64, 64), ("tiny", 3, 16), ("tiny", 16389, 4),
         ("z", 256, 4), ("z", 97925, 2), ("y1080", 4096, 2), ("y1080", 4096, 4),
         ("y1080", 4096, 8), ("y1080", 977, 64), ("y4kx8", 16384, 4)]

_cache = {}


def _workload(name):
    if name not in _cache:
        import gpu_util as G
        w = W.load(name)
        _cache.clear()
        _cache[name] = (w, G.tables_of(w), G.to_dev(w.symbols), G.to_dev(w.indexes))
    return _cache[name]


@pytest.mark.parametrize("name,lanes,pieces", CASES, ids=[f"{n}-L{L}-P{P}" for n, L, P in CASES])
def test_split_records_and_piecewise_decode(name, lanes, pieces):
    import torch
    import gpu_util as G
    w, tables, sym, idx = _workload(name)
    G.say(f"[splits] {name} lanes={lanes} pieces={pieces}: oracle")
    rc, ref, rmeta = oracle.encode_split(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, lanes,
                                         pieces)
    assert rc == 0
    G.say(f"[splits] {name} lanes={lanes} pieces={pieces}: gpu encode")
    stream, nwords, meta, status = G.B.encode_with_splits(sym, idx, tables, lanes, pieces)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    got = stream[: int(nwords.item())].cpu().numpy().view(np.uint32)
    assert np.array_equal(got, ref), "container differs"
    gm = meta.cpu().numpy().view(np.uint32).reshape(rmeta.shape)
    bad = np.argwhere(gm != rmeta)
    assert bad.size == 0, f"{len(bad)} record words differ, first at {bad[0].tolist()}"
    G.say(f"[splits] {name} lanes={lanes} pieces={pieces}: gpu decode from oracle records")
    s = torch.from_numpy(ref.view(np.int32).copy()).to(G.DEV)
    m = torch.from_numpy(rmeta.view(np.int32).copy()).to(G.DEV)
    out, status = G.B.decode_with_splits(s, m, idx, tables, pieces)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(out.cpu().numpy(), w.symbols)


def test_altered_records_are_refused_like_the_oracle():
    import torch
    import gpu_util as G
    w, tables, sym, idx = _workload("tiny")
    L, P = 64, 4
    rc, ref, rmeta = oracle.encode_split(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, L, P)
    assert rc == 0
    s = torch.from_numpy(ref.view(np.int32).copy()).to(G.DEV)
    for j, c, k, delta in ((3, 0, 0, 1), (10, 1, 1, 1 << 7), (20, 2, 2, 1), (30, 1, 2, -1),
                           (40, 0, 2, 1 << 30), (63, 2, 0, 1 << 31)):
        bad = rmeta.astype(np.int64)
        bad[j, c, k] = (bad[j, c, k] + delta) % (1 << 32)
        bad = bad.astype(np.uint32)
        G.say(f"[splits] altered record lane {j} cut {c + 1} word {k}")
        rco, _ = oracle.decode_split(ref, bad, w.indexes, w.cdf, w.lengths, w.offsets, L, P)
        m = torch.from_numpy(bad.view(np.int32).copy()).to(G.DEV)
        out, status = G.B.decode_with_splits(s, m, idx, tables, P)
        torch.cuda.synchronize()
        assert rco == oracle.E_CORRUPT and int(status.item()) == oracle.E_CORRUPT


def test_one_piece_matches_the_plain_calls():
    import torch
    import gpu_util as G
    w, tables, sym, idx = _workload("z")
    G.say("[splits] one piece")
    stream, nwords, meta, status = G.B.encode_with_splits(sym, idx, tables, 256, 1)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and meta.numel() == 0
    rc, ref = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, 256)
    assert np.array_equal(stream[: int(nwords.item())].cpu().numpy().view(np.uint32), ref)
    out, status = G.B.decode_with_splits(stream, meta, idx, tables, 1)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and np.array_equal(out.cpu().numpy(), w.symbols)
