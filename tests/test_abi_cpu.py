"""The C ABI without a GPU: the library loads, exports every function the public
header declares, sizes its buffers as documented and rejects bad arguments on
the host before any launch."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rans_hip.h")


@pytest.fixture(scope="module")
def lib():
    from learned_image_compression_amd import binding as B
    from learned_image_compression_amd import build as hip_build
    if not os.path.exists(B.LIBRARY):
        hip_build.build()
    return B.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rans_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert len(names) == 23, names
    from learned_image_compression_amd import binding as B
    assert sorted(B.EXPORTS) == names
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(-8, 1):
        assert lib.rans_status_string(code).decode() not in ("", "unknown status")
    assert lib.rans_status_string(-100).decode() == "unknown status"


def test_bounds(lib):
    for n, L in ((0, 1), (16384, 64), (1566720, 4096), (50135040, 131072)):
        assert lib.rans_encode_bound_words(n, L) == 1 + L + 2 * n + 4 * L
        ws = lib.rans_workspace_bytes(n, L, 64, 3133)
        # header + look-back flags (one per wave, 2^16 at most) + decoder and
        # encoder table regions (at least 143 KiB and 111 KiB, and room for 64
        # rows of 3133 entries: 2 bytes an entry and 512 bucket entries a row,
        # 4 bytes an entry) + 2n+4L words of lane scratch
        tables = max(143 * 1024, 2 * 64 * 3133 + 2 * 64 * 512) + max(110 * 1024, 4 * 64 * 3133)
        assert ws >= 256 + 8 * (1 << 16) + tables + 4 * (2 * n + 4 * L)
        assert ws % 4 == 0
    # table regions grow with rows and stride up to the largest set
    small = lib.rans_workspace_bytes(0, 1, 8, 16)
    big = lib.rans_workspace_bytes(0, 1, 4096, 16384)
    assert big - small >= 6 * 4096 * 16384


def _encode(lib, **kw):
    args = dict(symbols=1, indexes=1, n=10, cdf=1, lengths=1, offsets=1, K=8, stride=3133,
                lanes=4, stream=1, cap=1000, words=1, status=1, ws=256, ws_bytes=1 << 30,
                hstream=0)
    args.update(kw)
    v = ctypes.c_void_p
    return lib.rans_encode_with_indexes(
        v(args["symbols"]), v(args["indexes"]), args["n"], v(args["cdf"]), v(args["lengths"]),
        v(args["offsets"]), args["K"], args["stride"], args["lanes"], v(args["stream"]),
        args["cap"], v(args["words"]), v(args["status"]), v(args["ws"]), args["ws_bytes"],
        v(args["hstream"]))


def _decode(lib, **kw):
    args = dict(stream=1, cap=1000, indexes=1, n=10, cdf=1, lengths=1, offsets=1, K=8,
                stride=3133, symbols=1, status=1, ws=256, ws_bytes=1 << 30, hstream=0)
    args.update(kw)
    v = ctypes.c_void_p
    return lib.rans_decode_with_indexes(
        v(args["stream"]), args["cap"], v(args["indexes"]), args["n"], v(args["cdf"]),
        v(args["lengths"]), v(args["offsets"]), args["K"], args["stride"],
        v(args["symbols"]), v(args["status"]), v(args["ws"]), args["ws_bytes"],
        v(args["hstream"]))


@pytest.mark.parametrize("kw,code", [
    (dict(lanes=0), -1),
    (dict(symbols=0), -1),
    (dict(indexes=0), -1),
    (dict(stream=0), -1),
    (dict(words=0), -1),
    (dict(status=0), -1),
    (dict(cap=4), -1),                  # smaller than the 1 + L header
    (dict(cdf=0), -1),
    (dict(K=0), -2),
    (dict(K=4097), -2),
    (dict(stride=2), -2),
    (dict(stride=16385), -2),
    (dict(ws=0), -7),
    (dict(ws=128), -7),                 # not 256-byte aligned
    (dict(ws_bytes=1000), -7),
    (dict(n=1 << 41), -1),
    (dict(n=(1 << 28) + 1), -1),        # above RANS_MAX_SYMBOLS
    (dict(lanes=(1 << 22) + 1), -1),    # above RANS_MAX_LANES
])
def test_encode_rejects_bad_arguments_on_host(lib, kw, code):
    assert _encode(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(stream=0), -1),
    (dict(indexes=0), -1),
    (dict(symbols=0), -1),
    (dict(status=0), -1),
    (dict(cap=0), -1),                  # not even the lane-count word
    (dict(offsets=0), -1),
    (dict(K=0), -2),
    (dict(stride=20000), -2),
    (dict(ws=0), -7),
    (dict(ws=64), -7),
    (dict(ws_bytes=4096), -7),
    (dict(n=(1 << 28) + 1), -1),
])
def test_decode_rejects_bad_arguments_on_host(lib, kw, code):
    assert _decode(lib, **kw) == code


def test_zero_symbols_may_pass_null_arrays(lib):
    # n = 0 with null symbol/index pointers passes host validation; with a
    # null workspace the call stops at the workspace check, before any launch
    assert _encode(lib, n=0, symbols=0, indexes=0, ws=0) == -7
    assert _decode(lib, n=0, symbols=0, indexes=0, ws=0) == -7


def test_binding_refuses_to_run_without_library(tmp_path):
    from learned_image_compression_amd import binding as B
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        B.load(str(tmp_path / "missing.so"))


def _gauss(lib, **kw):
    a = dict(scales=1, K=64, tail_z=6.1, stride=3133, cdf=1, lengths=1, offsets=1, status=1,
             hstream=0)
    a.update(kw)
    return lib.rans_gaussian_tables(a["scales"], a["K"], a["tail_z"], a["stride"], a["cdf"],
                                    a["lengths"], a["offsets"], a["status"], a["hstream"])


def _pmfs(lib, **kw):
    a = dict(pmf=1, lengths=1, K=8, pmf_stride=256, stride=258, cdf=1, cdf_lengths=1, status=1,
             hstream=0)
    a.update(kw)
    return lib.rans_quantize_pmfs(a["pmf"], a["lengths"], a["K"], a["pmf_stride"], a["stride"],
                                  a["cdf"], a["cdf_lengths"], a["status"], a["hstream"])


@pytest.mark.parametrize("kw", [
    dict(scales=0), dict(cdf=0), dict(lengths=0), dict(offsets=0), dict(status=0),
    dict(K=0), dict(K=4097), dict(stride=2), dict(stride=16385),
    dict(tail_z=0.0), dict(tail_z=-1.0), dict(tail_z=float("nan")), dict(tail_z=float("inf")),
])
def test_gaussian_tables_reject_bad_arguments_on_host(lib, kw):
    assert _gauss(lib, **kw) == -1


@pytest.mark.parametrize("kw", [
    dict(pmf=0), dict(lengths=0), dict(cdf=0), dict(cdf_lengths=0), dict(status=0),
    dict(K=0), dict(K=4097), dict(pmf_stride=1), dict(stride=2), dict(stride=16385),
])
def test_quantize_pmfs_reject_bad_arguments_on_host(lib, kw):
    assert _pmfs(lib, **kw) == -1


@pytest.mark.parametrize("kw,code", [
    (dict(table=0), -1), (dict(K=0), -1), (dict(K=4097), -1),
    (dict(y=0), -1), (dict(means=0), -1), (dict(scales=0), -1), (dict(sym=0), -1),
    (dict(idx=0), -1),
    (dict(n=0, y=0, means=0, scales=0, sym=0, idx=0), 0),   # nothing to do, no launch
])
def test_latent_symbols_host_checks(lib, kw, code):
    a = dict(y=1, means=1, scales=1, n=100, table=1, K=64, sym=1, idx=1)
    a.update(kw)
    assert lib.rans_latent_symbols(a["y"], a["means"], a["scales"], a["n"], a["table"], a["K"],
                                   a["sym"], a["idx"], 0) == code


@pytest.mark.parametrize("kw,code", [
    (dict(sym=0), -1), (dict(means=0), -1), (dict(out=0), -1),
    (dict(n=0, sym=0, means=0, out=0), 0),
])
def test_dequantize_host_checks(lib, kw, code):
    a = dict(sym=1, means=1, n=100, out=1)
    a.update(kw)
    assert lib.rans_dequantize(a["sym"], a["means"], a["n"], a["out"], 0) == code


@pytest.mark.parametrize("pieces,meta,code", [(0, 1, -1), (3, 1, -1), (128, 1, -1), (4, 0, -1)])
def test_split_calls_check_pieces_on_host(lib, pieces, meta, code):
    assert lib.rans_encode_with_splits(1, 1, 10, 1, 1, 1, 8, 3133, 4, pieces, 1, 1000, 1, meta, 1,
                                       256, 1 << 30, 0) == code
    assert lib.rans_decode_with_splits(1, 1000, 1, 10, 1, 1, 1, 8, 3133, pieces, meta, 1000, 1,
                                       1, 256, 1 << 30, 0) == code


def test_interleaved_sizes(lib):
    for n, S in ((0, 1), (16384, 4), (1566720, 2048), (50135040, 65536)):
        assert lib.rans_interleaved_bound_words(n, S) == 1 + S + 2 * n + 256 * S
        ws = lib.rans_interleaved_workspace_bytes(n, S, 64, 3133)
        # header, flags, table regions, per-stream scratch (2 m + 256 words),
        # and word counts
        assert ws >= 256 + 8 * (1 << 16) + 254 * 1024 + 4 * (2 * n + 256 * S) + 4 * S
        assert ws == lib.rans_workspace_bytes(0, 1, 64, 3133) - 16 + \
            ((4 * (2 * n + 256 * S) + 255) // 256) * 256 + 4 * S


@pytest.mark.parametrize("kw,code", [
    (dict(S=0), -1), (dict(S=(1 << 16) + 1), -1), (dict(stream=0), -1), (dict(words=0), -1),
    (dict(status=0), -1), (dict(symbols=0), -1), (dict(cap=4), -1), (dict(K=0), -2),
    (dict(ws=0), -7), (dict(ws=128), -7), (dict(ws_bytes=4096), -7),
])
def test_encode_interleaved_host_checks(lib, kw, code):
    a = dict(symbols=1, indexes=1, n=10, cdf=1, lengths=1, offsets=1, K=8, stride=3133, S=4,
             stream=1, cap=1000, words=1, status=1, ws=256, ws_bytes=1 << 30)
    a.update(kw)
    assert lib.rans_encode_interleaved(a["symbols"], a["indexes"], a["n"], a["cdf"], a["lengths"],
                                       a["offsets"], a["K"], a["stride"], a["S"], a["stream"],
                                       a["cap"], a["words"], a["status"], a["ws"], a["ws_bytes"],
                                       0) == code


@pytest.mark.parametrize("kw,code", [
    (dict(S=0), -1), (dict(S=(1 << 16) + 1), -1), (dict(stream=0), -1), (dict(status=0), -1),
    (dict(out=0), -1), (dict(cap=2), -1), (dict(stride=20000), -2), (dict(ws=0), -7),
])
def test_decode_interleaved_host_checks(lib, kw, code):
    a = dict(stream=1, cap=1000, indexes=1, n=10, cdf=1, lengths=1, offsets=1, K=8, stride=3133,
             S=4, out=1, status=1, ws=256, ws_bytes=1 << 30)
    a.update(kw)
    assert lib.rans_decode_interleaved(a["stream"], a["cap"], a["indexes"], a["n"], a["cdf"],
                                       a["lengths"], a["offsets"], a["K"], a["stride"], a["S"],
                                       a["out"], a["status"], a["ws"], a["ws_bytes"], 0) == code


@pytest.mark.parametrize("kw,code", [
    (dict(S=0), -1), (dict(S=(1 << 16) + 1), -1), (dict(stream=0), -1), (dict(words=0), -1),
    (dict(status=0), -1), (dict(symbols=0), -1), (dict(indexes=0), -1), (dict(cap=4), -1),
    (dict(n=(1 << 40)), -1), (dict(K=0), -2), (dict(K=(1 << 20)), -2), (dict(stride=2), -2),
    (dict(stride=16385), -2), (dict(ws=0), -7), (dict(ws=128), -7), (dict(ws_bytes=4096), -7),
])
def test_encode_interleaved_prepared_host_checks(lib, kw, code):
    a = dict(symbols=1, indexes=1, n=10, K=8, stride=3133, S=4, stream=1, cap=1000, words=1,
             status=1, ws=256, ws_bytes=1 << 30)
    a.update(kw)
    assert lib.rans_encode_interleaved_prepared(a["symbols"], a["indexes"], a["n"], a["K"],
                                                a["stride"], a["S"], a["stream"], a["cap"],
                                                a["words"], a["status"], a["ws"], a["ws_bytes"],
                                                0) == code


@pytest.mark.parametrize("kw,code", [
    (dict(S=0), -1), (dict(S=(1 << 16) + 1), -1), (dict(stream=0), -1), (dict(status=0), -1),
    (dict(out=0), -1), (dict(indexes=0), -1), (dict(cap=2), -1), (dict(n=(1 << 40)), -1),
    (dict(K=0), -2), (dict(stride=2), -2), (dict(ws=0), -7), (dict(ws=128), -7),
    (dict(ws_bytes=4096), -7),
])
def test_decode_interleaved_prepared_host_checks(lib, kw, code):
    a = dict(stream=1, cap=1000, indexes=1, n=10, K=8, stride=3133, S=4, out=1, status=1, ws=256,
             ws_bytes=1 << 30)
    a.update(kw)
    assert lib.rans_decode_interleaved_prepared(a["stream"], a["cap"], a["indexes"], a["n"],
                                                a["K"], a["stride"], a["S"], a["out"], a["status"],
                                                a["ws"], a["ws_bytes"], 0) == code
