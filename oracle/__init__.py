"""CPU oracle for indexed rANS64 coding -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  ``rans_oracle.c`` is the plain single-threaded
reference (linear-scan decode, exact integer division); ``spec_model.py`` is
a second model in Python integers used for exhaustive brute force.  The
oracle shares no code with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "rans_oracle.c")
LIBRARY = os.path.join(HERE, "librans_oracle.so")

OK, E_ARG, E_TABLE, E_INDEX, E_SYMBOL_RANGE, E_CAPACITY, E_CORRUPT = 0, -1, -2, -3, -4, -5, -6

_lock = threading.Lock()
_lib = None


def build(source: str = SOURCE, out: str = LIBRARY, extra_flags=()) -> str:
    """Compile the oracle with the host C compiler (no GPU involved)."""
    tmp = f"{out}.tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-Werror", "-shared", "-fPIC",
           *extra_flags, source, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(lib):
    i32p = ctypes.POINTER(ctypes.c_int32)
    u32p = ctypes.POINTER(ctypes.c_uint32)
    u64p = ctypes.POINTER(ctypes.c_uint64)
    u64, i32, u32 = ctypes.c_uint64, ctypes.c_int32, ctypes.c_uint32
    lib.oracle_lane_begin.argtypes = [u64, u32, u32]
    lib.oracle_lane_begin.restype = u64
    lib.oracle_check_tables.argtypes = [i32p, i32p, i32, i32]
    lib.oracle_check_tables.restype = ctypes.c_int
    lib.oracle_encode_lane.argtypes = [i32p, i32p, u64, u64, i32p, i32p, i32p, i32, i32,
                                       u32p, u64, u64p]
    lib.oracle_encode_lane.restype = ctypes.c_int
    lib.oracle_decode_lane.argtypes = [u32p, u64, i32p, u64, u64, i32p, i32p, i32p, i32, i32,
                                       i32p]
    lib.oracle_decode_lane.restype = ctypes.c_int
    lib.oracle_encode.argtypes = [i32p, i32p, u64, i32p, i32p, i32p, i32, i32, u32,
                                  u32p, u64, u64p]
    lib.oracle_encode.restype = ctypes.c_int
    lib.oracle_decode.argtypes = [u32p, u64, i32p, u64, i32p, i32p, i32p, i32, i32, u32, i32p]
    lib.oracle_decode.restype = ctypes.c_int
    f64p = ctypes.POINTER(ctypes.c_double)
    f64 = ctypes.c_double
    lib.oracle_quantize_pmf.argtypes = [f64p, i32, i32p]
    lib.oracle_quantize_pmf.restype = ctypes.c_int
    lib.oracle_gaussian_row.argtypes = [f64, f64, i32, i32p, i32p, i32p]
    lib.oracle_gaussian_row.restype = ctypes.c_int
    lib.oracle_gaussian_tables.argtypes = [f64p, i32, f64, i32, i32p, i32p, i32p]
    lib.oracle_gaussian_tables.restype = ctypes.c_int
    lib.oracle_encode_split.argtypes = [i32p, i32p, u64, i32p, i32p, i32p, i32, i32, u32, u32,
                                        u32p, u64, u64p, u32p]
    lib.oracle_encode_split.restype = ctypes.c_int
    lib.oracle_decode_split.argtypes = [u32p, u64, i32p, u64, i32p, i32p, i32p, i32, i32, u32,
                                        u32, u32p, i32p]
    lib.oracle_decode_split.restype = ctypes.c_int
    lib.oracle_encode_interleaved.argtypes = [i32p, i32p, u64, i32p, i32p, i32p, i32, i32, u32,
                                              u32, u32p, u64, u64p]
    lib.oracle_encode_interleaved.restype = ctypes.c_int
    lib.oracle_decode_interleaved.argtypes = [u32p, u64, i32p, u64, i32p, i32p, i32p, i32, i32,
                                              u32, u32, i32p]
    lib.oracle_decode_interleaved.restype = ctypes.c_int
    f32p = ctypes.POINTER(ctypes.c_float)
    lib.oracle_latent_symbols.argtypes = [f32p, f32p, f32p, u64, f32p, i32, i32p, i32p]
    lib.oracle_latent_symbols.restype = ctypes.c_int
    lib.oracle_dequantize.argtypes = [i32p, f32p, u64, f32p]
    lib.oracle_dequantize.restype = ctypes.c_int
    return lib


def load(path: str | None = None):
    """Load the compiled oracle (building it from source if absent or stale)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if (not os.path.exists(LIBRARY)
                    or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE)):
                build()
            _lib = _bind(ctypes.CDLL(LIBRARY))
    return _lib


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _tables(cdf, lengths, offsets):
    cdf = np.ascontiguousarray(cdf, dtype=np.int32)
    lengths = np.ascontiguousarray(lengths, dtype=np.int32)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    if cdf.ndim != 2:
        raise ValueError("cdf must be [K, stride]")
    return cdf, lengths, offsets


def lane_begin(n: int, lanes: int, j: int, lib=None) -> int:
    lib = lib or load()
    return int(lib.oracle_lane_begin(n, lanes, j))


def check_tables(cdf, lengths, lib=None) -> int:
    lib = lib or load()
    cdf = np.ascontiguousarray(cdf, dtype=np.int32)
    lengths = np.ascontiguousarray(lengths, dtype=np.int32)
    return int(lib.oracle_check_tables(_ptr(cdf, ctypes.c_int32), _ptr(lengths, ctypes.c_int32),
                                       cdf.shape[0], cdf.shape[1]))


def encode(symbols, indexes, cdf, lengths, offsets, lanes: int, capacity: int | None = None,
           lib=None):
    """Return (status, words) where words is the uint32 container (empty on error)."""
    lib = lib or load()
    symbols = np.ascontiguousarray(symbols, dtype=np.int32)
    indexes = np.ascontiguousarray(indexes, dtype=np.int32)
    cdf, lengths, offsets = _tables(cdf, lengths, offsets)
    n = symbols.size
    if capacity is None:
        capacity = 1 + 3 * lanes + 10 * n
    out = np.zeros(max(capacity, 1), dtype=np.uint32)
    total = ctypes.c_uint64(0)
    rc = lib.oracle_encode(_ptr(symbols, ctypes.c_int32), _ptr(indexes, ctypes.c_int32), n,
                           _ptr(cdf, ctypes.c_int32), _ptr(lengths, ctypes.c_int32),
                           _ptr(offsets, ctypes.c_int32), cdf.shape[0], cdf.shape[1], lanes,
                           _ptr(out, ctypes.c_uint32), capacity, ctypes.byref(total))
    if rc != OK:
        return int(rc), out[:0] if rc != E_CAPACITY else out[: min(capacity, total.value)]
    return 0, out[: total.value].copy()


def decode(stream, indexes, cdf, lengths, offsets, lanes: int, lib=None):
    """Return (status, symbols)."""
    lib = lib or load()
    stream = np.ascontiguousarray(stream, dtype=np.uint32)
    indexes = np.ascontiguousarray(indexes, dtype=np.int32)
    cdf, lengths, offsets = _tables(cdf, lengths, offsets)
    out = np.zeros(max(indexes.size, 1), dtype=np.int32)
    rc = lib.oracle_decode(_ptr(stream, ctypes.c_uint32), stream.size,
                           _ptr(indexes, ctypes.c_int32), indexes.size,
                           _ptr(cdf, ctypes.c_int32), _ptr(lengths, ctypes.c_int32),
                           _ptr(offsets, ctypes.c_int32), cdf.shape[0], cdf.shape[1], lanes,
                           _ptr(out, ctypes.c_int32))
    return int(rc), out[: indexes.size]


def encode_lane(symbols, indexes, begin, end, cdf, lengths, offsets, lib=None):
    """One lane stream (no container header) for positions [begin, end)."""
    lib = lib or load()
    symbols = np.ascontiguousarray(symbols, dtype=np.int32)
    indexes = np.ascontiguousarray(indexes, dtype=np.int32)
    cdf, lengths, offsets = _tables(cdf, lengths, offsets)
    cap = 2 + 10 * (end - begin)
    out = np.zeros(cap, dtype=np.uint32)
    words = ctypes.c_uint64(0)
    rc = lib.oracle_encode_lane(_ptr(symbols, ctypes.c_int32), _ptr(indexes, ctypes.c_int32),
                                begin, end, _ptr(cdf, ctypes.c_int32),
                                _ptr(lengths, ctypes.c_int32), _ptr(offsets, ctypes.c_int32),
                                cdf.shape[0], cdf.shape[1], _ptr(out, ctypes.c_uint32), cap,
                                ctypes.byref(words))
    return int(rc), out[: words.value].copy() if rc == OK else out[:0]


def decode_lane(lane_words, indexes, begin, end, cdf, lengths, offsets, lib=None):
    lib = lib or load()
    lane_words = np.ascontiguousarray(lane_words, dtype=np.uint32)
    indexes = np.ascontiguousarray(indexes, dtype=np.int32)
    cdf, lengths, offsets = _tables(cdf, lengths, offsets)
    out = np.zeros(max(indexes.size, 1), dtype=np.int32)
    rc = lib.oracle_decode_lane(_ptr(lane_words, ctypes.c_uint32), lane_words.size,
                                _ptr(indexes, ctypes.c_int32), begin, end,
                                _ptr(cdf, ctypes.c_int32), _ptr(lengths, ctypes.c_int32),
                                _ptr(offsets, ctypes.c_int32), cdf.shape[0], cdf.shape[1],
                                _ptr(out, ctypes.c_int32))
    return int(rc), out[begin:end].copy()


def quantize_pmf(pmf, lib=None):
    """Return (status, cdf) for one pmf row (alphabet then escape slot)."""
    lib = lib or load()
    pmf = np.ascontiguousarray(pmf, dtype=np.float64)
    cdf = np.zeros(pmf.size + 1, dtype=np.int32)
    rc = lib.oracle_quantize_pmf(_ptr(pmf, ctypes.c_double), pmf.size, _ptr(cdf, ctypes.c_int32))
    return int(rc), cdf


def gaussian_tables(scales, tail_z: float, stride: int, lib=None):
    """Return (status, cdf [K, stride], lengths [K], offsets [K]) for one row per scale."""
    lib = lib or load()
    scales = np.ascontiguousarray(scales, dtype=np.float64)
    K = scales.size
    cdf = np.zeros((K, stride), dtype=np.int32)
    lengths = np.zeros(K, dtype=np.int32)
    offsets = np.zeros(K, dtype=np.int32)
    rc = lib.oracle_gaussian_tables(_ptr(scales, ctypes.c_double), K, float(tail_z), stride,
                                    _ptr(cdf, ctypes.c_int32), _ptr(lengths, ctypes.c_int32),
                                    _ptr(offsets, ctypes.c_int32))
    return int(rc), cdf, lengths, offsets


def latent_symbols(y, means, scales, scale_table, lib=None):
    """Return (status, symbols int32, indexes int32) of the latent front end."""
    lib = lib or load()
    y = np.ascontiguousarray(y, dtype=np.float32)
    means = np.ascontiguousarray(means, dtype=np.float32)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    table = np.ascontiguousarray(scale_table, dtype=np.float32)
    n = y.size
    sym = np.zeros(max(n, 1), dtype=np.int32)
    idx = np.zeros(max(n, 1), dtype=np.int32)
    f32 = ctypes.c_float
    rc = lib.oracle_latent_symbols(_ptr(y, f32), _ptr(means, f32), _ptr(scales, f32), n,
                                   _ptr(table, f32), table.size, _ptr(sym, ctypes.c_int32),
                                   _ptr(idx, ctypes.c_int32))
    return int(rc), sym[:n], idx[:n]


def dequantize(symbols, means, lib=None):
    """Return (status, y_hat float32)."""
    lib = lib or load()
    symbols = np.ascontiguousarray(symbols, dtype=np.int32)
    means = np.ascontiguousarray(means, dtype=np.float32)
    out = np.zeros(max(symbols.size, 1), dtype=np.float32)
    rc = lib.oracle_dequantize(_ptr(symbols, ctypes.c_int32), _ptr(means, ctypes.c_float),
                               symbols.size, _ptr(out, ctypes.c_float))
    return int(rc), out[: symbols.size]


def encode_split(symbols, indexes, cdf, lengths, offsets, lanes: int, pieces: int,
                 capacity: int | None = None, lib=None):
    """Return (status, words, split_meta uint32 [lanes, pieces - 1, 3])."""
    lib = lib or load()
    symbols = np.ascontiguousarray(symbols, dtype=np.int32)
    indexes = np.ascontiguousarray(indexes, dtype=np.int32)
    cdf, lengths, offsets = _tables(cdf, lengths, offsets)
    n = symbols.size
    if capacity is None:
        capacity = 1 + 3 * lanes + 10 * n
    out = np.zeros(max(capacity, 1), dtype=np.uint32)
    meta = np.zeros(max(3 * lanes * (pieces - 1), 1), dtype=np.uint32)
    total = ctypes.c_uint64(0)
    rc = lib.oracle_encode_split(_ptr(symbols, ctypes.c_int32), _ptr(indexes, ctypes.c_int32), n,
                                 _ptr(cdf, ctypes.c_int32), _ptr(lengths, ctypes.c_int32),
                                 _ptr(offsets, ctypes.c_int32), cdf.shape[0], cdf.shape[1],
                                 lanes, pieces, _ptr(out, ctypes.c_uint32), capacity,
                                 ctypes.byref(total), _ptr(meta, ctypes.c_uint32))
    meta = meta[: 3 * lanes * (pieces - 1)].reshape(lanes, pieces - 1, 3)
    if rc != OK:
        return int(rc), out[:0], meta
    return 0, out[: total.value].copy(), meta


def decode_split(stream, split_meta, indexes, cdf, lengths, offsets, lanes: int, pieces: int,
                 lib=None):
    """Return (status, symbols) decoding piece by piece from the split records."""
    lib = lib or load()
    stream = np.ascontiguousarray(stream, dtype=np.uint32)
    meta = np.ascontiguousarray(split_meta, dtype=np.uint32).reshape(-1)
    if meta.size == 0:
        meta = np.zeros(1, dtype=np.uint32)
    indexes = np.ascontiguousarray(indexes, dtype=np.int32)
    cdf, lengths, offsets = _tables(cdf, lengths, offsets)
    out = np.zeros(max(indexes.size, 1), dtype=np.int32)
    rc = lib.oracle_decode_split(_ptr(stream, ctypes.c_uint32), stream.size,
                                 _ptr(indexes, ctypes.c_int32), indexes.size,
                                 _ptr(cdf, ctypes.c_int32), _ptr(lengths, ctypes.c_int32),
                                 _ptr(offsets, ctypes.c_int32), cdf.shape[0], cdf.shape[1],
                                 lanes, pieces, _ptr(meta, ctypes.c_uint32),
                                 _ptr(out, ctypes.c_int32))
    return int(rc), out[: indexes.size]


def encode_interleaved(symbols, indexes, cdf, lengths, offsets, streams: int, width: int,
                       capacity: int | None = None, lib=None):
    """Return (status, words) of the interleaved-stream container."""
    lib = lib or load()
    symbols = np.ascontiguousarray(symbols, dtype=np.int32)
    indexes = np.ascontiguousarray(indexes, dtype=np.int32)
    cdf, lengths, offsets = _tables(cdf, lengths, offsets)
    n = symbols.size
    if capacity is None:
        capacity = 1 + streams * (1 + 2 * width) + 10 * n
    out = np.zeros(max(capacity, 1), dtype=np.uint32)
    total = ctypes.c_uint64(0)
    rc = lib.oracle_encode_interleaved(_ptr(symbols, ctypes.c_int32), _ptr(indexes, ctypes.c_int32),
                                       n, _ptr(cdf, ctypes.c_int32), _ptr(lengths, ctypes.c_int32),
                                       _ptr(offsets, ctypes.c_int32), cdf.shape[0], cdf.shape[1],
                                       streams, width, _ptr(out, ctypes.c_uint32), capacity,
                                       ctypes.byref(total))
    if rc != OK:
        return int(rc), out[:0]
    return 0, out[: total.value].copy()


def decode_interleaved(stream, indexes, cdf, lengths, offsets, streams: int, width: int, lib=None):
    """Return (status, symbols)."""
    lib = lib or load()
    stream = np.ascontiguousarray(stream, dtype=np.uint32)
    indexes = np.ascontiguousarray(indexes, dtype=np.int32)
    cdf, lengths, offsets = _tables(cdf, lengths, offsets)
    out = np.zeros(max(indexes.size, 1), dtype=np.int32)
    rc = lib.oracle_decode_interleaved(_ptr(stream, ctypes.c_uint32), stream.size,
                                       _ptr(indexes, ctypes.c_int32), indexes.size,
                                       _ptr(cdf, ctypes.c_int32), _ptr(lengths, ctypes.c_int32),
                                       _ptr(offsets, ctypes.c_int32), cdf.shape[0], cdf.shape[1],
                                       streams, width, _ptr(out, ctypes.c_int32))
    return int(rc), out[: indexes.size]
