"""Helpers for the GPU parity tests (import only inside gpu-marked tests)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from learned_image_compression_amd import binding as B

DEV = torch.device("cuda:0")


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def tables_of(w):
    return B.Tables.from_numpy(w.cdf, w.lengths, w.offsets, DEV)


def to_dev(a, dtype=torch.int32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV, dtype)


def gpu_encode(symbols, indexes, tables, lanes, capacity=None, canary=True):
    """Encode on the GPU; returns (status, words as np.uint32, total words)."""
    n = int(symbols.numel())
    bound = B.encode_bound_words(n, lanes)
    cap = bound if capacity is None else capacity
    out = torch.full((cap + 64,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    stream, nwords, status = B.encode_with_indexes(symbols, indexes, tables, lanes,
                                                   stream_out=out[:cap])
    torch.cuda.synchronize()
    st = int(status.item())
    nw = int(nwords.item())
    host = out.cpu().numpy().view(np.uint32)
    if canary:
        assert np.all(host[cap:] == 0x5A5A5A5A), "write past the stream capacity"
    return st, host[: min(nw, cap)].copy(), nw


def gpu_decode(words, indexes, tables, capacity=None):
    """Decode on the GPU from host words (the lane count is the container's own);
    returns (status, symbols as np.int32)."""
    n = int(indexes.numel())
    s = torch.from_numpy(np.asarray(words, dtype=np.uint32).view(np.int32).copy()).to(DEV)
    out = torch.full((n + 64,), 0x3C3C3C3C, dtype=torch.int32, device=DEV)
    sym, status = B.decode_with_indexes(s, indexes, tables, symbols_out=out[:n],
                                        capacity_words=capacity)
    torch.cuda.synchronize()
    host = out.cpu().numpy()
    assert np.all(host[n:] == 0x3C3C3C3C), "write past the symbol output"
    return int(status.item()), host[:n].copy()
