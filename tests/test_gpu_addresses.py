"""Every kernel family on buffers whose device addresses have bit 31 of their
low 32 bits set.

Buffer descriptors are built from a 64-bit base split into two 32-bit
halves; a half widened with sign extension would corrupt the high half of
exactly such addresses (a mistake of this kind once sent the fused encoder
outside its arrays).  Here every array a call touches -- inputs, outputs,
tables and workspace -- is carved from one large allocation at offsets
whose addresses lie in the upper half of a 4 GiB window, and each result is
compared with the oracle's.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TABLE64 = np.exp(np.linspace(np.log(0.11), np.log(256.0), 64)).astype(np.float32)


class Arena:
    """Slices of one device allocation, all at addresses whose low word is at
    least 2^31 (the window [2^31, 2^32) of some 4 GiB span)."""

    def __init__(self, need_bytes: int):
        import torch
        import gpu_util as G
        self.buf = torch.empty((1 << 32) + need_bytes + 4096, dtype=torch.uint8, device=G.DEV)
        base = self.buf.data_ptr()
        self.off = ((1 << 31) - (base & 0xFFFFFFFF)) % (1 << 32)
        self.end = self.off + (1 << 31)
        assert need_bytes < (1 << 31)

    def take(self, n, dtype):
        import torch
        itemsize = torch.empty(0, dtype=dtype).element_size()
        nbytes = max(1, n) * itemsize
        t = self.buf[self.off:self.off + nbytes].view(dtype)[:n]
        assert (t.data_ptr() & 0x80000000) and self.off + nbytes <= self.end
        self.off = (self.off + nbytes + 255) // 256 * 256
        return t

    def put(self, a, dtype):
        import torch
        import gpu_util as G
        src = torch.from_numpy(np.ascontiguousarray(a)).to(G.DEV, dtype)
        t = self.take(src.numel(), dtype).view(src.shape)
        t.copy_(src)
        return t


def _tables(ar, w):
    import torch
    import gpu_util as G
    return G.B.Tables(ar.put(w.cdf, torch.int32), ar.put(w.lengths, torch.int32),
                      ar.put(w.offsets, torch.int32))


@pytest.mark.parametrize("lanes", [4096, 1024])
def test_lane_coders_and_splits_at_high_addresses(lanes):
    import torch
    import gpu_util as G
    # (1024 lanes decode on the one-decoding-wave path, 4096 on eight waves)
    G.say(f"[addresses] lane encode, decode, split decode (y1080, {lanes} lanes)")
    w = W.load("y1080")
    pieces = 4
    ar = Arena(256 << 20)
    tables = _tables(ar, w)
    sym, idx = ar.put(w.symbols, torch.int32), ar.put(w.indexes, torch.int32)
    cap = G.B.encode_bound_words(w.n, lanes)
    stream = ar.take(cap, torch.int32)
    nw, st = ar.take(1, torch.int64), ar.take(1, torch.int32)
    ws = ar.take(G.B.workspace_bytes(w.n, lanes, tables.num_tables, tables.stride), torch.uint8)
    ws.zero_()
    G.B.encode_with_indexes(sym, idx, tables, lanes, stream_out=stream, stream_words=nw, status=st,
                            workspace=ws)
    G.B.check(st)
    got = stream[: int(nw.item())].cpu().numpy().view(np.uint32)
    rc, ref = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, lanes)
    assert rc == 0 and np.array_equal(got, ref)
    out = ar.take(w.n, torch.int32)
    G.B.decode_with_indexes(stream, idx, tables, symbols_out=out, status=st, workspace=ws)
    G.B.check(st)
    assert np.array_equal(out.cpu().numpy(), w.symbols)
    meta = ar.take(3 * lanes * (pieces - 1), torch.int32).view(lanes, pieces - 1, 3)
    _, nw2, _, st3 = G.B.encode_with_splits(sym, idx, tables, lanes, pieces, stream_out=stream,
                                            split_out=meta, workspace=ws)
    G.B.check(st3)
    assert int(nw2.item()) == int(nw.item())
    rc, _, ometa = oracle.encode_split(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, lanes,
                                       pieces)
    assert rc == 0 and np.array_equal(meta.cpu().numpy().view(np.uint32).reshape(-1),
                                      ometa.reshape(-1))
    out.zero_()
    _, st4 = G.B.decode_with_splits(stream, meta, idx, tables, pieces, symbols_out=out,
                                    workspace=ws)
    G.B.check(st4)
    assert np.array_equal(out.cpu().numpy(), w.symbols)


def test_interleaved_and_fused_at_high_addresses():
    import torch
    import gpu_util as G
    G.say("[addresses] interleaved encode, fused encode, decode (1080p y, 4096 streams)")
    rc, cdf, lengths, offsets = oracle.gaussian_tables(TABLE64.astype(np.float64),
                                                       6.109410204869238, 3133)
    assert rc == 0
    n, S = 192 * 68 * 120, 4096
    rng = np.random.default_rng(8)
    scales = np.exp(rng.uniform(np.log(0.11), np.log(40.0), n)).astype(np.float32)
    m = (rng.standard_normal(n) * 2).astype(np.float32)
    y = (m + rng.standard_normal(n).astype(np.float32) * scales).astype(np.float32)
    rc, osym, oidx = oracle.latent_symbols(y, m, scales, TABLE64)
    rc2, ref = oracle.encode_interleaved(osym, oidx, cdf, lengths, offsets, S, 64)
    assert rc == 0 and rc2 == 0
    ar = Arena(256 << 20)
    tables = G.B.Tables(ar.put(cdf, torch.int32), ar.put(lengths, torch.int32),
                        ar.put(offsets, torch.int32))
    lib = G.B.load()
    cap = int(lib.rans_interleaved_bound_words(n, S))
    ws = ar.take(int(lib.rans_interleaved_workspace_bytes(n, S, 64, 3133)), torch.uint8)
    ws.zero_()
    dy, dm, ds, dt = (ar.put(a, torch.float32) for a in (y, m, scales, TABLE64))
    sym, idx = ar.take(n, torch.int32), ar.take(n, torch.int32)
    G.B.latent_symbols(dy, dm, ds, dt, symbols_out=sym, indexes_out=idx)
    assert np.array_equal(sym.cpu().numpy(), osym) and np.array_equal(idx.cpu().numpy(), oidx)
    for fused in (False, True):
        stream = ar.take(cap, torch.int32)
        if fused:
            stream, nw, st = G.B.encode_interleaved_latent(dy, dm, ds, dt, tables, S,
                                                           stream_out=stream, workspace=ws)
        else:
            stream, nw, st = G.B.encode_interleaved(sym, idx, tables, S, stream_out=stream,
                                                    workspace=ws)
        G.B.check(st)
        got = stream[: int(nw.item())].cpu().numpy().view(np.uint32)
        assert np.array_equal(got, ref), f"fused={fused}"
        out = ar.take(n, torch.int32)
        out, st2 = G.B.decode_interleaved(stream, idx, tables, S, symbols_out=out, workspace=ws)
        G.B.check(st2)
        assert np.array_equal(out.cpu().numpy(), osym)
    y_hat = ar.take(n, torch.float32)
    G.B.dequantize(sym, dm, out=y_hat)
    rc, oy = oracle.dequantize(osym, m)
    assert rc == 0 and np.array_equal(y_hat.cpu().numpy().view(np.int32), oy.view(np.int32))


def test_table_builder_at_high_addresses():
    import torch
    import gpu_util as G
    G.say("[addresses] device table builder (64 Gaussian rows)")
    rc, cdf, lengths, offsets = oracle.gaussian_tables(TABLE64.astype(np.float64),
                                                       6.109410204869238, 3133)
    assert rc == 0
    ar = Arena(16 << 20)
    sc = ar.put(TABLE64.astype(np.float64), torch.float64)
    dcdf, dlen, doff = ar.take(64 * 3133, torch.int32), ar.take(64, torch.int32), ar.take(64, torch.int32)
    rs = ar.take(64, torch.int32)
    rc = G.B.load().rans_gaussian_tables(G.B._ptr(sc), 64, 6.109410204869238, 3133,
                                         G.B._ptr(dcdf), G.B._ptr(dlen), G.B._ptr(doff),
                                         G.B._ptr(rs), G.B._stream(G.DEV))
    assert rc == 0
    torch.cuda.synchronize()
    assert not rs.cpu().numpy().any()
    assert np.array_equal(dcdf.cpu().numpy().reshape(64, 3133), cdf)
    assert np.array_equal(dlen.cpu().numpy(), lengths) and np.array_equal(doff.cpu().numpy(), offsets)
