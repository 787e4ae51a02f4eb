"""GPU parity of the front end fused into the interleaved encoder.

rans_encode_interleaved_latent must give, word for word, the container the
oracle chain gives: oracle.latent_symbols (symbol = rint(y - mean), index
from the scale table), then oracle.encode_interleaved (64 states a stream).
Cases: the 1080p y shape (192 x 68 x 120) at 4096 streams and at one
stream, ragged sizes, an empty latent, saturating and NaN values (the status
must match the oracle's), unsorted / tied / NaN-holding / two-entry scale
tables, one with negative entries (no index lookup table) and one packed
into a single lookup cell (long forward scans), a one-row set, a table set
over the LDS budget (the global-table path), and two prepared calls in a row
on one workspace.  The GPU's own two-pass path
(front end, then encode) must agree too.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

TABLE64 = np.exp(np.linspace(np.log(0.11), np.log(256.0), 64)).astype(np.float32)
TAIL_Z = 6.109410204869238   # the standard-normal quantile of 1 - 5e-10
WIDTH = 64


def _dev(a, dtype=None):
    import torch
    import gpu_util as G
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(G.DEV) if dtype is None else t.to(G.DEV, dtype)


def _tables(scales, stride):
    """Gaussian rows for the scales, built by the oracle (the coding tables are
    an input here; their device build has its own tests)."""
    import gpu_util as G
    rc, cdf, lengths, offsets = oracle.gaussian_tables(np.asarray(scales, np.float64), TAIL_Z,
                                                       stride)
    assert rc == 0
    return (cdf, lengths, offsets), G.B.Tables.from_numpy(cdf, lengths, offsets, G.DEV)


def _latent(n, seed, spread=40.0):
    rng = np.random.default_rng(seed)
    scales = np.exp(rng.uniform(np.log(0.11), np.log(spread), n)).astype(np.float32)
    m = (rng.standard_normal(n) * 2).astype(np.float32)
    y = (m + rng.standard_normal(n).astype(np.float32) * scales).astype(np.float32)
    return y, m, scales


def _oracle_chain(y, m, s, table, host_tables, streams):
    rc, sym, idx = oracle.latent_symbols(y, m, s, table)
    assert rc == 0
    return oracle.encode_interleaved(sym, idx, *host_tables, streams, WIDTH)


def _gpu_fused(y, m, s, table, tables, streams, canary=True):
    import torch
    import gpu_util as G
    n = len(y)
    cap = int(G.B.load().rans_interleaved_bound_words(n, streams))
    out = torch.full((cap + 64,), 0x5A5A5A5A, dtype=torch.int32, device=G.DEV)
    stream, nw, st = G.B.encode_interleaved_latent(_dev(y), _dev(m), _dev(s), _dev(table), tables,
                                                   streams, stream_out=out[:cap])
    torch.cuda.synchronize()
    host = out.cpu().numpy().view(np.uint32)
    if canary:
        assert np.all(host[cap:] == 0x5A5A5A5A), "write past the stream capacity"
    return int(st.item()), host[: int(nw.item())].copy()


@pytest.mark.parametrize("n,streams", [(192 * 68 * 120, 4096), (192 * 68 * 120, 1),
                                       (1566723, 7), (100003, 64), (4097, 4096), (5, 3), (0, 2)])
def test_fused_matches_the_oracle_chain(n, streams):
    import gpu_util as G
    G.say(f"[fused] n={n} streams={streams}")
    host_tables, tables = _tables(TABLE64, 3133)
    y, m, s = _latent(n, 1000 + n)
    st, got = _gpu_fused(y, m, s, TABLE64, tables, streams)
    rc, ref = _oracle_chain(y, m, s, TABLE64, host_tables, streams)
    assert rc == 0 and st == 0
    assert np.array_equal(got, ref)


def test_fused_equals_the_two_pass_gpu_path():
    import torch
    import gpu_util as G
    G.say("[fused] against the GPU two-pass path")
    n, streams = 300007, 512
    _, tables = _tables(TABLE64, 3133)
    y, m, s = _latent(n, 77)
    st, got = _gpu_fused(y, m, s, TABLE64, tables, streams)
    sym, idx = G.B.latent_symbols(_dev(y), _dev(m), _dev(s), _dev(TABLE64))
    stream, nw, st2 = G.B.encode_interleaved(sym, idx, tables, streams)
    torch.cuda.synchronize()
    two = stream[: int(nw.item())].cpu().numpy().view(np.uint32)
    assert st == 0 and int(st2.item()) == 0 and np.array_equal(got, two)


@pytest.mark.parametrize("what", ["nan_y", "huge", "nan_scale_inf"])
def test_fused_edge_values_status(what):
    import gpu_util as G
    G.say(f"[fused] edge values {what}")
    host_tables, tables = _tables(TABLE64, 3133)
    y, m, s = _latent(20011, 9)
    if what == "nan_y":
        y[12345] = np.nan            # symbol INT32_MIN: out of range
    elif what == "huge":
        y[777] = np.float32(3e9)     # saturates to INT32_MAX
    else:
        s[100:106] = [np.nan, np.inf, -np.inf, 0.0, -1.0, 3e38]   # indexes only: valid
        y[200:204] = [np.float32(0.5), np.float32(-0.5), np.float32(1.5), np.float32(2.5)]
        m[200:204] = 0
    st, got = _gpu_fused(y, m, s, TABLE64, tables, 64)
    rc, ref = _oracle_chain(y, m, s, TABLE64, host_tables, 64)
    assert st == rc
    if what == "nan_scale_inf":
        assert rc == 0 and np.array_equal(got, ref)
    else:
        assert rc == oracle.E_SYMBOL_RANGE


@pytest.mark.parametrize("name", ["unsorted", "ties", "nan_entry", "one_row", "two_nan",
                                  "two_sorted", "negative", "one_cell"])
def test_fused_other_scale_tables(name):
    import gpu_util as G
    rng = np.random.default_rng(11)
    table = {"unsorted": rng.permutation(TABLE64),
             "ties": np.repeat(TABLE64[::4], 4),
             "nan_entry": np.where(np.arange(64) == 17, np.nan, TABLE64),
             "two_nan": np.array([np.nan, 1.0]),
             "two_sorted": np.array([0.5, 1.0]),
             "negative": np.linspace(-3.0, 40.0, 64),
             "one_cell": np.linspace(1.0, 1.05, 64),
             "one_row": TABLE64[40:41]}[name].astype(np.float32)
    # the coding rows come from a positive finite copy of the table (one row
    # per entry)
    rows = np.where(np.isfinite(table) & (table > 0), table, np.float32(1.0))
    G.say(f"[fused] scale table {name}")
    host_tables, tables = _tables(rows, 3133)
    y, m, s = _latent(50021, 21)
    st, got = _gpu_fused(y, m, s, table, tables, 128)
    rc, ref = _oracle_chain(y, m, s, table, host_tables, 128)
    assert rc == 0 and st == 0 and np.array_equal(got, ref)


def test_fused_table_set_over_the_lds_budget():
    import gpu_util as G
    G.say("[fused] 300 rows, stride 3133 (tables read from the workspace)")
    table = np.exp(np.linspace(np.log(0.11), np.log(256.0), 300)).astype(np.float32)
    host_tables, tables = _tables(table, 3133)
    assert int(host_tables[1].astype(np.int64).sum()) * 4 > 160 * 1024
    y, m, s = _latent(200003, 31, spread=256.0)
    st, got = _gpu_fused(y, m, s, table, tables, 256)
    rc, ref = _oracle_chain(y, m, s, table, host_tables, 256)
    assert rc == 0 and st == 0 and np.array_equal(got, ref)


def test_fused_prepared_twice_on_one_workspace():
    import torch
    import gpu_util as G
    G.say("[fused] prepared, two calls")
    host_tables, tables = _tables(TABLE64, 3133)
    lib = G.B.load()
    n0, streams = 400009, 1024
    ws = torch.zeros(int(lib.rans_interleaved_workspace_bytes(n0, streams, 64, 3133)),
                     dtype=torch.uint8, device=G.DEV)
    G.B.prepare_tables(tables, ws)
    for n in (n0, 12345):
        y, m, s = _latent(n, n)
        stream, nw, st = G.B.encode_interleaved_latent(_dev(y), _dev(m), _dev(s), _dev(TABLE64),
                                                       tables, streams, workspace=ws,
                                                       prepared=True)
        torch.cuda.synchronize()
        got = stream[: int(nw.item())].cpu().numpy().view(np.uint32)
        rc, ref = _oracle_chain(y, m, s, TABLE64, host_tables, streams)
        assert rc == 0 and int(st.item()) == 0 and np.array_equal(got, ref)


def test_fused_decodes_back_to_the_front_end_symbols():
    import torch
    import gpu_util as G
    G.say("[fused] decode of the fused container")
    n, streams = 192 * 68 * 120, 4096
    _, tables = _tables(TABLE64, 3133)
    y, m, s = _latent(n, 5)
    stream, nw, st = G.B.encode_interleaved_latent(_dev(y), _dev(m), _dev(s), _dev(TABLE64),
                                                   tables, streams)
    G.B.check(st)
    rc, sym, idx = oracle.latent_symbols(y, m, s, TABLE64)
    out, st2 = G.B.decode_interleaved(stream, _dev(idx), tables, streams)
    G.B.check(st2)
    assert rc == 0 and np.array_equal(out.cpu().numpy(), sym)
    torch.cuda.synchronize()
