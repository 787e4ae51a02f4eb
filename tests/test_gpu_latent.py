"""GPU parity of the latent front end and dequantisation against the oracle.

Hand-derived cases on both the 16-byte and the 4-byte access paths, seeded
latents of the 1080p y shape (and ragged sizes) with a 64-scale table, an
unsorted table, a table holding NaN, a one-entry table, and the whole chain
latent -> symbols and indexes -> device-built tables -> encode -> decode ->
dequantise against the same chain on the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from helpers import LATENT_TABLE, latent_cases

pytestmark = pytest.mark.gpu

TABLE64 = np.exp(np.linspace(np.log(0.11), np.log(256.0), 64)).astype(np.float32)


def _dev(a, dtype=None):
    import torch
    import gpu_util as G
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(G.DEV) if dtype is None else t.to(G.DEV, dtype)


def _gpu_front(y, mean, scale, table, offset=0):
    """Run the front end on device copies placed `offset` floats into their
    buffers (offset 1 forces the 4-byte path)."""
    import torch
    import gpu_util as G
    n = len(y)
    bufs = []
    for a in (y, mean, scale):
        b = torch.zeros(n + 4, dtype=torch.float32, device=G.DEV)
        b[offset:offset + n] = _dev(np.asarray(a, np.float32))
        bufs.append(b[offset:offset + n])
    so = torch.full((n + 4,), 77, dtype=torch.int32, device=G.DEV)
    io = torch.full((n + 4,), 77, dtype=torch.int32, device=G.DEV)
    sym, idx = G.B.latent_symbols(*bufs, _dev(np.asarray(table, np.float32)),
                                  symbols_out=so[offset:offset + n],
                                  indexes_out=io[offset:offset + n])
    torch.cuda.synchronize()
    s, i = so.cpu().numpy(), io.cpu().numpy()
    assert np.all(s[:offset] == 77) and np.all(s[offset + n:] == 77)
    assert np.all(i[:offset] == 77) and np.all(i[offset + n:] == 77)
    return s[offset:offset + n], i[offset:offset + n]


@pytest.mark.parametrize("offset", [0, 1])
def test_golden_cases(offset):
    import gpu_util as G
    syms, idxs = latent_cases()
    G.say(f"[latent] golden offset={offset}")
    k = max(len(syms), len(idxs))
    y = np.zeros(k, np.float32); m = np.zeros(k, np.float32); s = np.ones(k, np.float32)
    y[:len(syms)] = [c[0] for c in syms]; m[:len(syms)] = [c[1] for c in syms]
    s[:len(idxs)] = [c[0] for c in idxs]
    sym, idx = _gpu_front(y, m, s, LATENT_TABLE, offset)
    assert sym[:len(syms)].tolist() == [c[2] for c in syms]
    assert idx[:len(idxs)].tolist() == [c[1] for c in idxs]


def _random_latent(n, seed):
    rng = np.random.default_rng(seed)
    y = (rng.standard_normal(n) * rng.choice([0.3, 3.0, 200.0], n)).astype(np.float32)
    m = (rng.standard_normal(n) * 2).astype(np.float32)
    s = np.exp(rng.uniform(np.log(0.01), np.log(400.0), n)).astype(np.float32)
    y[:257] = np.round(y[:257]) + np.float32(0.5)
    m[:257] = 0
    if n >= 306:
        s[:64] = TABLE64
        s[64:70] = [np.nan, np.inf, 0.0, -1.0, 1e-30, 3e38]
        y[300:306] = [np.nan, np.inf, -np.inf, 3e9, -3e9, 2147483520]
    return y, m, s


@pytest.mark.parametrize("n,offset", [(1566720, 0), (1566723, 0), (100003, 1), (1, 0), (5, 1)])
def test_random_latents(n, offset):
    import gpu_util as G
    y, m, s = _random_latent(n, n)
    G.say(f"[latent] random n={n} offset={offset}")
    sym, idx = _gpu_front(y, m, s, TABLE64, offset)
    rc, osym, oidx = oracle.latent_symbols(y, m, s, TABLE64)
    assert rc == 0
    assert np.array_equal(sym, osym) and np.array_equal(idx, oidx)


@pytest.mark.parametrize("name", ["unsorted", "nan_entry", "one_entry", "ties", "two_nan",
                                  "two_sorted", "negative", "one_cell"])
def test_other_tables(name):
    import gpu_util as G
    rng = np.random.default_rng(3)
    table = {"unsorted": rng.permutation(TABLE64),
             "nan_entry": np.where(np.arange(64) == 17, np.nan, TABLE64),
             "two_nan": np.array([np.nan, 1.0]),
             "two_sorted": np.array([0.5, 1.0]),
             "negative": np.linspace(-3.0, 40.0, 64),
             "one_cell": np.linspace(1.0, 1.05, 64),
             "one_entry": TABLE64[:1],
             "ties": np.repeat(TABLE64[::4], 4)}[name].astype(np.float32)
    y, m, s = _random_latent(20011, 5)
    G.say(f"[latent] table {name}")
    sym, idx = _gpu_front(y, m, s, table)
    rc, osym, oidx = oracle.latent_symbols(y, m, s, table)
    assert rc == 0 and np.array_equal(sym, osym) and np.array_equal(idx, oidx)


@pytest.mark.parametrize("n,offset", [(1566720, 0), (1003, 0), (7, 0), (1001, 1)])
def test_dequantize(n, offset):
    import torch
    import gpu_util as G
    rng = np.random.default_rng(n)
    q = rng.integers(-2**31, 2**31, n, dtype=np.int64).astype(np.int32)
    q[: n // 2] = rng.integers(-40, 40, n // 2)
    q[:4] = [2**31 - 1, -2**31, 16777217, -16777217]
    m = (rng.standard_normal(n) * 3).astype(np.float32)
    G.say(f"[latent] dequantize n={n} offset={offset}")
    qb = torch.zeros(n + 4, dtype=torch.int32, device=G.DEV)
    qb[offset:offset + n] = _dev(q)
    mb = torch.zeros(n + 4, dtype=torch.float32, device=G.DEV)
    mb[offset:offset + n] = _dev(m)
    ob = torch.full((n + 4,), 5.0, dtype=torch.float32, device=G.DEV)
    G.B.dequantize(qb[offset:offset + n], mb[offset:offset + n], out=ob[offset:offset + n])
    torch.cuda.synchronize()
    o = ob.cpu().numpy()
    assert np.all(o[:offset] == 5.0) and np.all(o[offset + n:] == 5.0)
    rc, ref = oracle.dequantize(q, m)
    assert rc == 0 and np.array_equal(o[offset:offset + n].view(np.int32), ref.view(np.int32))


def test_latent_chain_matches_the_oracle_chain():
    """latent -> symbols, indexes -> (device-built tables) -> encode -> decode ->
    dequantise, against the same chain on the oracle."""
    import torch
    import gpu_util as G
    from scipy.special import ndtri
    C, H, W = 192, 68, 120
    n = C * H * W
    rng = np.random.default_rng(42)
    scales = np.exp(rng.uniform(np.log(0.11), np.log(40.0), n)).astype(np.float32)
    m = (rng.standard_normal(n) * 2).astype(np.float32)
    y = (m + rng.standard_normal(n).astype(np.float32) * scales).astype(np.float32)
    tail_z = float(ndtri(1.0 - 5e-10))
    table64 = TABLE64.astype(np.float64)
    G.say("[latent] chain: tables")
    tables, st = G.B.gaussian_tables(_dev(table64), tail_z, 3133)
    G.B.check_rows(st)
    G.say("[latent] chain: front end")
    sym, idx = G.B.latent_symbols(_dev(y), _dev(m), _dev(scales), _dev(TABLE64))
    G.say("[latent] chain: encode")
    stream, nwords, status = G.B.encode_with_indexes(sym, idx, tables, 4096)
    G.B.check(status)
    G.say("[latent] chain: decode + dequantise")
    out, status = G.B.decode_with_indexes(stream, idx, tables)
    G.B.check(status)
    y_hat = G.B.dequantize(out, _dev(m)).cpu().numpy()
    words = stream[: int(nwords.item())].cpu().numpy().view(np.uint32)
    # the same chain on the oracle
    rc, ocdf, olen, ooff = oracle.gaussian_tables(table64, tail_z, 3133)
    rc2, osym, oidx = oracle.latent_symbols(y, m, scales, TABLE64)
    rc3, owords = oracle.encode(osym, oidx, ocdf, olen, ooff, 4096)
    rc4, oout = oracle.decode(owords, oidx, ocdf, olen, ooff, 4096)
    rc5, oy = oracle.dequantize(oout, m)
    assert rc == rc2 == rc3 == rc4 == rc5 == 0
    assert np.array_equal(words, owords)
    assert np.array_equal(y_hat.view(np.int32), oy.view(np.int32))
    assert np.max(np.abs(y_hat - y)) <= 0.5 + 1e-3 * np.max(np.abs(y))
