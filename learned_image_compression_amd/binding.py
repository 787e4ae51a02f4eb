"""ctypes binding of librans_hip.so: argument marshalling only.

Torch tensors provide device memory and the current HIP stream; every step of
the coder runs in the library's kernels.  There is no CPU path: if the
library is missing this module raises instead of falling back.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "librans_hip.so")

STATUS = {
    0: "RANS_OK",
    -1: "RANS_E_ARG",
    -2: "RANS_E_TABLE",
    -3: "RANS_E_INDEX",
    -4: "RANS_E_SYMBOL_RANGE",
    -5: "RANS_E_CAPACITY",
    -6: "RANS_E_CORRUPT",
    -7: "RANS_E_WORKSPACE",
    -8: "RANS_E_HIP",
}
NAME_TO_CODE = {v: k for k, v in STATUS.items()}

# every symbol the public header declares
EXPORTS = (
    "rans_encode_bound_words",
    "rans_workspace_bytes",
    "rans_encode_with_indexes",
    "rans_decode_with_indexes",
    "rans_prepare_tables",
    "rans_encode_prepared",
    "rans_decode_prepared",
    "rans_gaussian_tables",
    "rans_quantize_pmfs",
    "rans_latent_symbols",
    "rans_encode_with_splits",
    "rans_interleaved_bound_words",
    "rans_interleaved_workspace_bytes",
    "rans_encode_interleaved",
    "rans_decode_interleaved",
    "rans_encode_interleaved_prepared",
    "rans_decode_interleaved_prepared",
    "rans_decode_with_splits",
    "rans_dequantize",
    "rans_encode_noalloc",
    "rans_encode_interleaved_latent",
    "rans_encode_interleaved_latent_prepared",
    "rans_status_string",
)


class RansError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = int(code)
        super().__init__(f"{where}: {STATUS.get(self.code, self.code)} "
                         f"({_status_text(self.code)})")


_lock = threading.Lock()
_lib = None


def _status_text(code: int) -> str:
    try:
        return load().rans_status_string(int(code)).decode()
    except Exception:  # pragma: no cover - library missing
        return "?"


def load(path: str | None = None):
    """Load the compiled HIP library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIBRARY
        if not os.path.exists(p):
            raise RuntimeError(
                f"{p} is missing: build it with `python -m learned_image_compression_amd.build` "
                "(hipcc, gfx950); there is no CPU fallback")
        lib = ctypes.CDLL(p)
        vp, u64, i32, u32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_uint32
        lib.rans_encode_bound_words.argtypes = [u64, u32]
        lib.rans_encode_bound_words.restype = u64
        lib.rans_workspace_bytes.argtypes = [u64, u32, i32, i32]
        lib.rans_workspace_bytes.restype = u64
        lib.rans_encode_with_indexes.argtypes = [vp, vp, u64, vp, vp, vp, i32, i32, u32, vp, u64,
                                                 vp, vp, vp, u64, vp]
        lib.rans_encode_with_indexes.restype = ctypes.c_int
        lib.rans_decode_with_indexes.argtypes = [vp, u64, vp, u64, vp, vp, vp, i32, i32, vp, vp,
                                                 vp, u64, vp]
        lib.rans_decode_with_indexes.restype = ctypes.c_int
        lib.rans_prepare_tables.argtypes = [vp, vp, vp, i32, i32, vp, u64, vp]
        lib.rans_prepare_tables.restype = ctypes.c_int
        lib.rans_encode_prepared.argtypes = [vp, vp, u64, i32, i32, u32, vp, u64, vp, vp, vp, u64,
                                             vp]
        lib.rans_encode_prepared.restype = ctypes.c_int
        lib.rans_decode_prepared.argtypes = [vp, u64, vp, u64, i32, i32, vp, vp, vp, u64, vp]
        lib.rans_decode_prepared.restype = ctypes.c_int
        f64 = ctypes.c_double
        lib.rans_gaussian_tables.argtypes = [vp, i32, f64, i32, vp, vp, vp, vp, vp]
        lib.rans_gaussian_tables.restype = ctypes.c_int
        lib.rans_quantize_pmfs.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp]
        lib.rans_quantize_pmfs.restype = ctypes.c_int
        lib.rans_encode_with_splits.argtypes = [vp, vp, u64, vp, vp, vp, i32, i32, u32, u32, vp,
                                                u64, vp, vp, vp, vp, u64, vp]
        lib.rans_encode_with_splits.restype = ctypes.c_int
        lib.rans_decode_with_splits.argtypes = [vp, u64, vp, u64, vp, vp, vp, i32, i32, u32, vp,
                                                u64, vp, vp, vp, u64, vp]
        lib.rans_decode_with_splits.restype = ctypes.c_int
        lib.rans_interleaved_bound_words.argtypes = [u64, u32]
        lib.rans_interleaved_bound_words.restype = u64
        lib.rans_interleaved_workspace_bytes.argtypes = [u64, u32, i32, i32]
        lib.rans_interleaved_workspace_bytes.restype = u64
        lib.rans_encode_interleaved.argtypes = [vp, vp, u64, vp, vp, vp, i32, i32, u32, vp, u64,
                                                vp, vp, vp, u64, vp]
        lib.rans_encode_interleaved.restype = ctypes.c_int
        lib.rans_decode_interleaved.argtypes = [vp, u64, vp, u64, vp, vp, vp, i32, i32, u32, vp,
                                                vp, vp, u64, vp]
        lib.rans_decode_interleaved.restype = ctypes.c_int
        lib.rans_encode_interleaved_prepared.argtypes = [vp, vp, u64, i32, i32, u32, vp, u64, vp,
                                                         vp, vp, u64, vp]
        lib.rans_encode_interleaved_prepared.restype = ctypes.c_int
        lib.rans_decode_interleaved_prepared.argtypes = [vp, u64, vp, u64, i32, i32, u32, vp, vp,
                                                         vp, u64, vp]
        lib.rans_decode_interleaved_prepared.restype = ctypes.c_int
        lib.rans_latent_symbols.argtypes = [vp, vp, vp, u64, vp, i32, vp, vp, vp]
        lib.rans_latent_symbols.restype = ctypes.c_int
        lib.rans_dequantize.argtypes = [vp, vp, u64, vp, vp]
        lib.rans_dequantize.restype = ctypes.c_int
        lib.rans_encode_noalloc.argtypes = [vp, vp, u64, vp, vp, vp, i32, i32, u32, vp, u64, vp,
                                            vp, vp]
        lib.rans_encode_noalloc.restype = ctypes.c_int
        lib.rans_encode_interleaved_latent.argtypes = [vp, vp, vp, u64, vp, vp, vp, vp, i32, i32,
                                                       u32, vp, u64, vp, vp, vp, u64, vp]
        lib.rans_encode_interleaved_latent.restype = ctypes.c_int
        lib.rans_encode_interleaved_latent_prepared.argtypes = [vp, vp, vp, u64, vp, i32, i32, u32,
                                                                vp, u64, vp, vp, vp, u64, vp]
        lib.rans_encode_interleaved_latent_prepared.restype = ctypes.c_int
        lib.rans_status_string.argtypes = [ctypes.c_int]
        lib.rans_status_string.restype = ctypes.c_char_p
        if path is None:
            _lib = lib
        return lib


def encode_bound_words(n: int, lanes: int) -> int:
    return int(load().rans_encode_bound_words(n, lanes))


def workspace_bytes(n: int, lanes: int, num_tables: int, stride: int) -> int:
    return int(load().rans_workspace_bytes(n, lanes, num_tables, stride))


def decode_workspace_bytes(num_tables: int, stride: int) -> int:
    """Workspace a decode needs: everything before the encoder's scratch."""
    return int(load().rans_workspace_bytes(0, 1, num_tables, stride))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, dtype, device, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class Workspace:
    """Zero-filled device workspace, grown (re-zeroed) on demand.

    The default workspaces are kept per (device, stream): calls that share a
    workspace must not overlap in time, and calls on one stream never do.
    Growing a workspace replaces it with a new zero-filled buffer, which drops
    any table set prepared in it (a later ``prepared=True`` call then reports
    RANS_E_ARG); callers that prepare tables once pass their own workspace.
    """

    def __init__(self, device):
        self.device = torch.device(device)
        self.buf = None

    def get(self, nbytes: int) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes:
            # 256-byte alignment: the caching allocator aligns blocks to 512 bytes
            self.buf = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=self.device)
            assert self.buf.data_ptr() % 256 == 0
        return self.buf


_workspaces: dict = {}


def workspace_for(device) -> Workspace:
    """The default workspace of `device` for its current stream."""
    device = torch.device(device)
    index = device.index if device.index is not None else torch.cuda.current_device()
    stream = torch.cuda.current_stream(torch.device("cuda", index)).cuda_stream
    key = (index, stream)
    with _lock:
        if key not in _workspaces:
            _workspaces[key] = Workspace(torch.device("cuda", index))
        return _workspaces[key]


class Tables:
    """A CDF table set on the device (int32 cdf[K, stride], lengths[K], offsets[K])."""

    def __init__(self, cdf: torch.Tensor, lengths: torch.Tensor, offsets: torch.Tensor):
        device = cdf.device
        for t, name in ((cdf, "cdf"), (lengths, "cdf_lengths"), (offsets, "offsets")):
            _need(t, torch.int32, device, name)
        if cdf.dim() != 2 or lengths.numel() != cdf.shape[0] or offsets.numel() != cdf.shape[0]:
            raise ValueError("cdf must be [K, stride] with K lengths and K offsets")
        self.cdf, self.lengths, self.offsets = cdf, lengths, offsets
        self.device = device

    @property
    def num_tables(self) -> int:
        return int(self.cdf.shape[0])

    @property
    def stride(self) -> int:
        return int(self.cdf.shape[1])

    @classmethod
    def from_numpy(cls, cdf, lengths, offsets, device="cuda"):
        return cls(torch.as_tensor(cdf, dtype=torch.int32).to(device).contiguous(),
                   torch.as_tensor(lengths, dtype=torch.int32).to(device).contiguous(),
                   torch.as_tensor(offsets, dtype=torch.int32).to(device).contiguous())


def _check_rc(rc: int, where: str):
    if rc != 0:
        raise RansError(rc, where)


def encode_with_indexes(symbols: torch.Tensor, indexes: torch.Tensor, tables: Tables,
                        num_lanes: int, *, stream_out: torch.Tensor | None = None,
                        stream_words: torch.Tensor | None = None,
                        status: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                        prepared: bool = False):
    """Enqueue an encode; returns (stream int32 words, stream_words int64[1], status int32[1]).

    Nothing is synchronised: read status/stream_words after the stream is done
    (``check(status)``).  ``prepared=True`` reuses tables already packed into
    ``workspace`` by :func:`prepare_tables`.
    """
    device = tables.device
    _need(symbols, torch.int32, device, "symbols")
    _need(indexes, torch.int32, device, "indexes")
    n = symbols.numel()
    if indexes.numel() != n:
        raise ValueError("symbols and indexes differ in size")
    lib = load()
    if stream_out is None:
        stream_out = torch.empty(encode_bound_words(n, num_lanes), dtype=torch.int32, device=device)
    _need(stream_out, torch.int32, device, "stream_out")
    if stream_words is None:
        stream_words = torch.zeros(1, dtype=torch.int64, device=device)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=device)
    ws = workspace if workspace is not None else workspace_for(device).get(
        workspace_bytes(n, num_lanes, tables.num_tables, tables.stride))
    st = _stream(device)
    if prepared:
        rc = lib.rans_encode_prepared(_ptr(symbols), _ptr(indexes), n, tables.num_tables,
                                      tables.stride, num_lanes, _ptr(stream_out),
                                      stream_out.numel(), _ptr(stream_words), _ptr(status),
                                      _ptr(ws), ws.numel(), st)
    else:
        rc = lib.rans_encode_with_indexes(_ptr(symbols), _ptr(indexes), n, _ptr(tables.cdf),
                                          _ptr(tables.lengths), _ptr(tables.offsets),
                                          tables.num_tables, tables.stride, num_lanes,
                                          _ptr(stream_out), stream_out.numel(), _ptr(stream_words),
                                          _ptr(status), _ptr(ws), ws.numel(), st)
    _check_rc(rc, "rans_encode_with_indexes")
    return stream_out, stream_words, status


def encode_noalloc(symbols: torch.Tensor, indexes: torch.Tensor, tables: Tables, num_lanes: int,
                   stream_out: torch.Tensor, stream_words: torch.Tensor, status: torch.Tensor):
    """Enqueue an encode that allocates nothing: the library's fixed per-device
    scratch array serves as the workspace (``rans_encode_noalloc``).  All
    buffers are the caller's; calls on one GPU must not overlap in time."""
    device = tables.device
    _need(symbols, torch.int32, device, "symbols")
    _need(indexes, torch.int32, device, "indexes")
    _need(stream_out, torch.int32, device, "stream_out")
    _need(stream_words, torch.int64, device, "stream_words")
    _need(status, torch.int32, device, "status")
    n = symbols.numel()
    if indexes.numel() != n:
        raise ValueError("symbols and indexes differ in size")
    rc = load().rans_encode_noalloc(_ptr(symbols), _ptr(indexes), n, _ptr(tables.cdf),
                                    _ptr(tables.lengths), _ptr(tables.offsets), tables.num_tables,
                                    tables.stride, num_lanes, _ptr(stream_out), stream_out.numel(),
                                    _ptr(stream_words), _ptr(status), _stream(device))
    _check_rc(rc, "rans_encode_noalloc")
    return stream_out, stream_words, status


def decode_with_indexes(stream: torch.Tensor, indexes: torch.Tensor, tables: Tables, *,
                        symbols_out: torch.Tensor | None = None,
                        status: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                        capacity_words: int | None = None, prepared: bool = False):
    """Enqueue a decode; returns (symbols int32[n], status int32[1]).  The lane
    count comes from the container's first word."""
    device = tables.device
    _need(stream, torch.int32, device, "stream")
    _need(indexes, torch.int32, device, "indexes")
    n = indexes.numel()
    lib = load()
    if symbols_out is None:
        symbols_out = torch.empty(n, dtype=torch.int32, device=device)
    _need(symbols_out, torch.int32, device, "symbols_out")
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=device)
    cap = stream.numel() if capacity_words is None else int(capacity_words)
    ws = workspace if workspace is not None else workspace_for(device).get(
        decode_workspace_bytes(tables.num_tables, tables.stride))
    st = _stream(device)
    if prepared:
        rc = lib.rans_decode_prepared(_ptr(stream), cap, _ptr(indexes), n, tables.num_tables,
                                      tables.stride, _ptr(symbols_out), _ptr(status),
                                      _ptr(ws), ws.numel(), st)
    else:
        rc = lib.rans_decode_with_indexes(_ptr(stream), cap, _ptr(indexes), n, _ptr(tables.cdf),
                                          _ptr(tables.lengths), _ptr(tables.offsets),
                                          tables.num_tables, tables.stride,
                                          _ptr(symbols_out), _ptr(status), _ptr(ws), ws.numel(),
                                          st)
    _check_rc(rc, "rans_decode_with_indexes")
    return symbols_out, status


def prepare_tables(tables: Tables, workspace: torch.Tensor):
    rc = load().rans_prepare_tables(_ptr(tables.cdf), _ptr(tables.lengths), _ptr(tables.offsets),
                                    tables.num_tables, tables.stride, _ptr(workspace),
                                    workspace.numel(), _stream(tables.device))
    _check_rc(rc, "rans_prepare_tables")


def check(status: torch.Tensor, where: str = "device"):
    """Synchronise on the status word and raise RansError if it is non-zero."""
    code = int(status.item())
    if code != 0:
        raise RansError(code, where)


def gaussian_tables(scales: torch.Tensor, tail_z: float, cdf_stride: int):
    """Enqueue the build of one discretised Gaussian CDF row per scale.

    ``scales`` is a float64 device tensor [K]; returns (Tables, row_status
    int32 [K]).  Nothing is synchronised: a row whose status is non-zero was
    not built (``check_rows(row_status)``).
    """
    device = scales.device
    _need(scales, torch.float64, device, "scales")
    K = scales.numel()
    cdf = torch.empty((K, cdf_stride), dtype=torch.int32, device=device)
    lengths = torch.empty(K, dtype=torch.int32, device=device)
    offsets = torch.empty(K, dtype=torch.int32, device=device)
    status = torch.empty(K, dtype=torch.int32, device=device)
    rc = load().rans_gaussian_tables(_ptr(scales), K, float(tail_z), cdf_stride, _ptr(cdf),
                                     _ptr(lengths), _ptr(offsets), _ptr(status), _stream(device))
    _check_rc(rc, "rans_gaussian_tables")
    return Tables(cdf, lengths, offsets), status


def quantize_pmfs(pmf: torch.Tensor, pmf_lengths: torch.Tensor, cdf_stride: int):
    """Enqueue the 16-bit quantisation of pmf rows (float64 [K, S], alphabet then
    escape slot; int32 lengths [K]); returns (cdf [K, cdf_stride], cdf_lengths [K],
    row_status [K])."""
    device = pmf.device
    _need(pmf, torch.float64, device, "pmf")
    _need(pmf_lengths, torch.int32, device, "pmf_lengths")
    if pmf.dim() != 2 or pmf_lengths.numel() != pmf.shape[0]:
        raise ValueError("pmf must be [K, S] with K lengths")
    K = pmf.shape[0]
    cdf = torch.empty((K, cdf_stride), dtype=torch.int32, device=device)
    lengths = torch.empty(K, dtype=torch.int32, device=device)
    status = torch.empty(K, dtype=torch.int32, device=device)
    rc = load().rans_quantize_pmfs(_ptr(pmf), _ptr(pmf_lengths), K, pmf.shape[1], cdf_stride,
                                   _ptr(cdf), _ptr(lengths), _ptr(status), _stream(device))
    _check_rc(rc, "rans_quantize_pmfs")
    return cdf, lengths, status


def check_rows(row_status: torch.Tensor, where: str = "table build"):
    """Synchronise on per-row statuses and raise RansError for the first failed row."""
    st = row_status.cpu()
    bad = torch.nonzero(st).flatten()
    if bad.numel():
        raise RansError(int(st[bad[0]]), f"{where}: row {int(bad[0])}")


def latent_symbols(y: torch.Tensor, means: torch.Tensor, scales: torch.Tensor,
                   scale_table: torch.Tensor, *, symbols_out: torch.Tensor | None = None,
                   indexes_out: torch.Tensor | None = None):
    """Enqueue the front end: (symbols, indexes) int32 of rint(y - means) and the
    table index of each scale (float32 device tensors of one size; float32 table)."""
    device = y.device
    for t, name in ((y, "y"), (means, "means"), (scales, "scales"), (scale_table, "scale_table")):
        _need(t, torch.float32, device, name)
    n = y.numel()
    if means.numel() != n or scales.numel() != n:
        raise ValueError("y, means and scales differ in size")
    if symbols_out is None:
        symbols_out = torch.empty(n, dtype=torch.int32, device=device)
    if indexes_out is None:
        indexes_out = torch.empty(n, dtype=torch.int32, device=device)
    _need(symbols_out, torch.int32, device, "symbols_out")
    _need(indexes_out, torch.int32, device, "indexes_out")
    if symbols_out.numel() != n or indexes_out.numel() != n:
        raise ValueError("output sizes differ from the input")
    rc = load().rans_latent_symbols(_ptr(y), _ptr(means), _ptr(scales), n, _ptr(scale_table),
                                    scale_table.numel(), _ptr(symbols_out), _ptr(indexes_out),
                                    _stream(device))
    _check_rc(rc, "rans_latent_symbols")
    return symbols_out, indexes_out


def dequantize(symbols: torch.Tensor, means: torch.Tensor, *, out: torch.Tensor | None = None):
    """Enqueue y_hat = symbols + means (float32)."""
    device = symbols.device
    _need(symbols, torch.int32, device, "symbols")
    _need(means, torch.float32, device, "means")
    n = symbols.numel()
    if means.numel() != n:
        raise ValueError("symbols and means differ in size")
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=device)
    _need(out, torch.float32, device, "out")
    if out.numel() != n:
        raise ValueError("output size differs from the input")
    rc = load().rans_dequantize(_ptr(symbols), _ptr(means), n, _ptr(out), _stream(device))
    _check_rc(rc, "rans_dequantize")
    return out


def encode_with_splits(symbols: torch.Tensor, indexes: torch.Tensor, tables: Tables,
                       num_lanes: int, pieces: int, *, stream_out: torch.Tensor | None = None,
                       split_out: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Enqueue an encode that also writes split records (int32 [lanes, pieces - 1, 3]);
    returns (stream, stream_words, split_records, status)."""
    device = tables.device
    _need(symbols, torch.int32, device, "symbols")
    _need(indexes, torch.int32, device, "indexes")
    n = symbols.numel()
    if indexes.numel() != n:
        raise ValueError("symbols and indexes differ in size")
    if stream_out is None:
        stream_out = torch.empty(encode_bound_words(n, num_lanes), dtype=torch.int32,
                                 device=device)
    if split_out is None:
        split_out = torch.empty((num_lanes, max(pieces - 1, 0), 3), dtype=torch.int32,
                                device=device)
    _need(stream_out, torch.int32, device, "stream_out")
    _need(split_out, torch.int32, device, "split_out")
    if split_out.numel() < 3 * num_lanes * max(pieces - 1, 0):
        raise ValueError("split_out too small")
    stream_words = torch.zeros(1, dtype=torch.int64, device=device)
    status = torch.zeros(1, dtype=torch.int32, device=device)
    ws = workspace if workspace is not None else workspace_for(device).get(
        workspace_bytes(n, num_lanes, tables.num_tables, tables.stride))
    rc = load().rans_encode_with_splits(
        _ptr(symbols), _ptr(indexes), n, _ptr(tables.cdf), _ptr(tables.lengths),
        _ptr(tables.offsets), tables.num_tables, tables.stride, num_lanes, pieces,
        _ptr(stream_out), stream_out.numel(), _ptr(stream_words), _ptr(split_out), _ptr(status),
        _ptr(ws), ws.numel(), _stream(device))
    _check_rc(rc, "rans_encode_with_splits")
    return stream_out, stream_words, split_out, status


def decode_with_splits(stream: torch.Tensor, split_records: torch.Tensor, indexes: torch.Tensor,
                       tables: Tables, pieces: int, *,
                       symbols_out: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None,
                       capacity_words: int | None = None):
    """Enqueue a decode of every lane as `pieces` pieces; returns (symbols, status).
    The lane count comes from the container; the records must cover it."""
    device = tables.device
    _need(stream, torch.int32, device, "stream")
    _need(split_records, torch.int32, device, "split_records")
    _need(indexes, torch.int32, device, "indexes")
    n = indexes.numel()
    if symbols_out is None:
        symbols_out = torch.empty(n, dtype=torch.int32, device=device)
    _need(symbols_out, torch.int32, device, "symbols_out")
    status = torch.zeros(1, dtype=torch.int32, device=device)
    cap = stream.numel() if capacity_words is None else int(capacity_words)
    ws = workspace if workspace is not None else workspace_for(device).get(
        decode_workspace_bytes(tables.num_tables, tables.stride))
    rc = load().rans_decode_with_splits(
        _ptr(stream), cap, _ptr(indexes), n, _ptr(tables.cdf), _ptr(tables.lengths),
        _ptr(tables.offsets), tables.num_tables, tables.stride, pieces,
        _ptr(split_records), split_records.numel(), _ptr(symbols_out), _ptr(status), _ptr(ws),
        ws.numel(), _stream(device))
    _check_rc(rc, "rans_decode_with_splits")
    return symbols_out, status


def encode_interleaved(symbols: torch.Tensor, indexes: torch.Tensor, tables: Tables,
                       num_streams: int, *, stream_out: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None, prepared: bool = False):
    """Enqueue an interleaved-stream encode (64 states per stream); returns
    (stream int32 words, stream_words int64[1], status int32[1]).
    ``prepared=True`` reuses tables already packed into ``workspace`` by
    :func:`prepare_tables`."""
    device = tables.device
    _need(symbols, torch.int32, device, "symbols")
    _need(indexes, torch.int32, device, "indexes")
    n = symbols.numel()
    if indexes.numel() != n:
        raise ValueError("symbols and indexes differ in size")
    lib = load()
    if stream_out is None:
        stream_out = torch.empty(int(lib.rans_interleaved_bound_words(n, num_streams)),
                                 dtype=torch.int32, device=device)
    _need(stream_out, torch.int32, device, "stream_out")
    stream_words = torch.zeros(1, dtype=torch.int64, device=device)
    status = torch.zeros(1, dtype=torch.int32, device=device)
    ws = workspace if workspace is not None else workspace_for(device).get(
        int(lib.rans_interleaved_workspace_bytes(n, num_streams, tables.num_tables,
                                                 tables.stride)))
    if prepared:
        rc = lib.rans_encode_interleaved_prepared(_ptr(symbols), _ptr(indexes), n,
                                                  tables.num_tables, tables.stride, num_streams,
                                                  _ptr(stream_out),
                                                  stream_out.numel(), _ptr(stream_words),
                                                  _ptr(status), _ptr(ws), ws.numel(),
                                                  _stream(device))
    else:
        rc = lib.rans_encode_interleaved(_ptr(symbols), _ptr(indexes), n, _ptr(tables.cdf),
                                         _ptr(tables.lengths), _ptr(tables.offsets),
                                         tables.num_tables, tables.stride, num_streams,
                                         _ptr(stream_out), stream_out.numel(), _ptr(stream_words),
                                         _ptr(status), _ptr(ws), ws.numel(), _stream(device))
    _check_rc(rc, "rans_encode_interleaved")
    return stream_out, stream_words, status


def encode_interleaved_latent(y: torch.Tensor, means: torch.Tensor, scales: torch.Tensor,
                              scale_table: torch.Tensor, tables: Tables, num_streams: int, *,
                              stream_out: torch.Tensor | None = None,
                              workspace: torch.Tensor | None = None, prepared: bool = False):
    """Enqueue the front end fused into the interleaved encode: the container
    of ``encode_interleaved(*latent_symbols(y, means, scales, scale_table))``
    with no symbol or index array in between (float32 device tensors of one
    size; ``scale_table`` holds one scale per table row).  Returns (stream int32
    words, stream_words int64[1], status int32[1])."""
    device = tables.device
    for t, name in ((y, "y"), (means, "means"), (scales, "scales"), (scale_table, "scale_table")):
        _need(t, torch.float32, device, name)
    n = y.numel()
    if means.numel() != n or scales.numel() != n:
        raise ValueError("y, means and scales differ in size")
    if scale_table.numel() != tables.num_tables:
        raise ValueError("the scale table needs one scale per table row")
    lib = load()
    if stream_out is None:
        stream_out = torch.empty(int(lib.rans_interleaved_bound_words(n, num_streams)),
                                 dtype=torch.int32, device=device)
    _need(stream_out, torch.int32, device, "stream_out")
    stream_words = torch.zeros(1, dtype=torch.int64, device=device)
    status = torch.zeros(1, dtype=torch.int32, device=device)
    ws = workspace if workspace is not None else workspace_for(device).get(
        int(lib.rans_interleaved_workspace_bytes(n, num_streams, tables.num_tables,
                                                 tables.stride)))
    if prepared:
        rc = lib.rans_encode_interleaved_latent_prepared(
            _ptr(y), _ptr(means), _ptr(scales), n, _ptr(scale_table), tables.num_tables,
            tables.stride, num_streams, _ptr(stream_out), stream_out.numel(), _ptr(stream_words),
            _ptr(status), _ptr(ws), ws.numel(), _stream(device))
    else:
        rc = lib.rans_encode_interleaved_latent(
            _ptr(y), _ptr(means), _ptr(scales), n, _ptr(scale_table), _ptr(tables.cdf),
            _ptr(tables.lengths), _ptr(tables.offsets), tables.num_tables, tables.stride,
            num_streams, _ptr(stream_out), stream_out.numel(), _ptr(stream_words), _ptr(status),
            _ptr(ws), ws.numel(), _stream(device))
    _check_rc(rc, "rans_encode_interleaved_latent")
    return stream_out, stream_words, status


def decode_interleaved(stream: torch.Tensor, indexes: torch.Tensor, tables: Tables,
                       num_streams: int, *, symbols_out: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None,
                       capacity_words: int | None = None, prepared: bool = False):
    """Enqueue an interleaved-stream decode; returns (symbols, status).
    ``prepared=True`` reuses tables already packed into ``workspace``."""
    device = tables.device
    _need(stream, torch.int32, device, "stream")
    _need(indexes, torch.int32, device, "indexes")
    n = indexes.numel()
    lib = load()
    if symbols_out is None:
        symbols_out = torch.empty(n, dtype=torch.int32, device=device)
    _need(symbols_out, torch.int32, device, "symbols_out")
    status = torch.zeros(1, dtype=torch.int32, device=device)
    cap = stream.numel() if capacity_words is None else int(capacity_words)
    ws = workspace if workspace is not None else workspace_for(device).get(
        decode_workspace_bytes(tables.num_tables, tables.stride))
    if prepared:
        rc = lib.rans_decode_interleaved_prepared(_ptr(stream), cap, _ptr(indexes), n,
                                                  tables.num_tables, tables.stride, num_streams,
                                                  _ptr(symbols_out), _ptr(status), _ptr(ws),
                                                  ws.numel(), _stream(device))
    else:
        rc = lib.rans_decode_interleaved(_ptr(stream), cap, _ptr(indexes), n, _ptr(tables.cdf),
                                         _ptr(tables.lengths), _ptr(tables.offsets),
                                         tables.num_tables, tables.stride, num_streams,
                                         _ptr(symbols_out), _ptr(status), _ptr(ws), ws.numel(),
                                         _stream(device))
    _check_rc(rc, "rans_decode_interleaved")
    return symbols_out, status
