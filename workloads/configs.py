"""Seeded synthetic workloads for the indexed rANS coder.

The pages measure real ``mbt2018_mean`` (quality 3) latents of one
1920x1088 image (kompressor README, "Getting Started" and "Benchmarks";
BENCHMARKS.md preamble): a ``y`` latent of 192x68x120 = 1,566,720 symbols
coded with 64 Gaussian CDF rows, and a factorised ``z`` latent.  Neither the
weights nor the latents are available, so these generators stand in for them
with the same shapes, table counts and row lengths, and with symbol
statistics drawn from the tables' own densities.  Every array is produced
from ``numpy.random.default_rng(seed)`` in a fixed draw order, so the oracle
and the GPU path consume identical inputs.

This module only draws inputs; it holds none of the coder's arithmetic.
"""
from __future__ import annotations

import dataclasses
import math
import os

import numpy as np
from scipy.ndimage import gaussian_filter1d
from scipy.special import ndtr

from .tables import (
    gaussian_half_width,
    gaussian_table_set,
    logistic_table_set,
)

# raw (zig-zagged) values that sit on nibble boundaries and at the int32 limit
EDGE_RAWS = (0, 1, 15, 16, 255, 256, (1 << 28) - 1, 1 << 28, (1 << 31) - 1, (1 << 31) - 2)


@dataclasses.dataclass
class Workload:
    name: str
    symbols: np.ndarray   # int32 [n]
    indexes: np.ndarray   # int32 [n]
    cdf: np.ndarray       # int32 [K, stride]
    lengths: np.ndarray   # int32 [K]
    offsets: np.ndarray   # int32 [K]
    lanes: tuple          # lane counts this workload is run at

    @property
    def n(self) -> int:
        return int(self.symbols.size)

    @property
    def num_tables(self) -> int:
        return int(self.cdf.shape[0])

    @property
    def stride(self) -> int:
        return int(self.cdf.shape[1])


def raw_to_value(raw: int, mv: int) -> int:
    """Coded-slot value v that the zig-zag escape maps to ``raw``."""
    return -(raw + 1) // 2 if raw & 1 else mv + raw // 2


def smooth_field(rng, C, H, W, sigma=3.0):
    """Per-channel N(0,1) noise, separable Gaussian blur (reflect, 4 sigma), re-standardised."""
    u = rng.standard_normal((C, H, W))
    u = gaussian_filter1d(u, sigma, axis=1, mode="reflect", truncate=4.0)
    u = gaussian_filter1d(u, sigma, axis=2, mode="reflect", truncate=4.0)
    u -= u.mean(axis=(1, 2), keepdims=True)
    u /= u.std(axis=(1, 2), keepdims=True)
    return u


def _gaussian_symbols(rng, idx, scales, lengths, offsets):
    s = scales[idx]
    half = (lengths[idx].astype(np.int64) - 3) // 2
    x = np.rint(rng.standard_normal(idx.shape) * s)
    return np.clip(x, -half, half).astype(np.int64)


def _force_bypass(rng, sym, idx, lengths, offsets, frac, edge_raws=()):
    """Move a seeded fraction of positions outside their row's coded range."""
    n = sym.size
    m = int(round(frac * n))
    if m == 0:
        return sym
    pos = rng.choice(n, size=m, replace=False)
    d = np.floor(2.0 ** rng.uniform(0.0, 20.0, size=m)).astype(np.int64)
    below = rng.random(m) < 0.5
    r = idx[pos]
    off = offsets[r].astype(np.int64)
    mv = lengths[r].astype(np.int64) - 2
    v = np.where(below, -d, mv - 1 + d)
    for k, raw in enumerate(edge_raws[:m]):
        v[k] = raw_to_value(int(raw), int(mv[k]))
    sym[pos] = v + off
    return sym


def make_tiny(seed=1):
    cdf, lengths, offsets, scales = gaussian_table_set(8)
    rng = np.random.default_rng(seed)
    n = 16384
    idx = rng.integers(0, 8, size=n)
    sym = _gaussian_symbols(rng, idx, scales, lengths, offsets)
    sym = _force_bypass(rng, sym, idx, lengths, offsets, 0.01, EDGE_RAWS)
    return Workload("tiny", sym.astype(np.int32), idx.astype(np.int32),
                    cdf, lengths, offsets, (64, 1, 2, 3, 7, 255, n, n + 5))


def make_z(seed=2):
    C, H, W = 192, 17, 30
    rng = np.random.default_rng(seed)
    scales = rng.uniform(0.5, 8.0, size=C)
    cdf, lengths, offsets = logistic_table_set(scales, stride=64)
    idx = np.repeat(np.arange(C), H * W)
    u = rng.random(idx.size)
    u = np.clip(u, 1e-12, 1 - 1e-12)
    x = scales[idx] * np.log(u / (1.0 - u))  # logistic(0, s) by inversion
    sym = np.rint(x).astype(np.int64)
    n = idx.size
    return Workload("z", sym.astype(np.int32), idx.astype(np.int32),
                    cdf, lengths, offsets, (256, 1, 2, 3, 7, 255, n, n + 5))


_Y_TABLES = None


def y_tables():
    global _Y_TABLES
    if _Y_TABLES is None:
        _Y_TABLES = gaussian_table_set(64)
    return _Y_TABLES


def _y_latent(seed, C, H, W, index_map, bypass_frac):
    cdf, lengths, offsets, scales = y_tables()
    rng = np.random.default_rng(seed)
    u = smooth_field(rng, C, H, W)
    idx = index_map(u).reshape(-1).astype(np.int64)
    sym = _gaussian_symbols(rng, idx, scales, lengths, offsets)
    sym = _force_bypass(rng, sym, idx, lengths, offsets, bypass_frac)
    return sym, idx


def _y1080_index(u):
    return np.clip(np.rint(20.0 + 10.0 * u), 0, 63)


def _y4k_index(u):
    p = ndtr(u)
    low = np.floor(9.0 * p / 0.8)
    high = 9.0 + np.minimum(54.0, np.floor(55.0 * (p - 0.8) / 0.2))
    return np.where(p < 0.8, low, high)


def make_y1080(seed=3):
    cdf, lengths, offsets, _ = y_tables()
    sym, idx = _y_latent(seed, 192, 68, 120, _y1080_index, 0.001)
    return Workload("y1080", sym.astype(np.int32), idx.astype(np.int32),
                    cdf, lengths, offsets, (4096, 1))


def make_y1080x16():
    cdf, lengths, offsets, _ = y_tables()
    parts = [_y_latent(1000 + b, 192, 68, 120, _y1080_index, 0.001) for b in range(16)]
    sym = np.concatenate([p[0] for p in parts])
    idx = np.concatenate([p[1] for p in parts])
    return Workload("y1080x16", sym.astype(np.int32), idx.astype(np.int32),
                    cdf, lengths, offsets, (65536, 1))


def make_y4kx8():
    cdf, lengths, offsets, _ = y_tables()
    parts = [_y_latent(2000 + b, 192, 136, 240, _y4k_index, 0.005) for b in range(8)]
    sym = np.concatenate([p[0] for p in parts])
    idx = np.concatenate([p[1] for p in parts])
    return Workload("y4kx8", sym.astype(np.int32), idx.astype(np.int32),
                    cdf, lengths, offsets, (1024, 16384, 131072))


MAKERS = {
    "tiny": make_tiny,
    "z": make_z,
    "y1080": make_y1080,
    "y1080x16": make_y1080x16,
    "y4kx8": make_y4kx8,
}

_CACHE_VERSION = 1


def _cache_dir():
    d = os.environ.get("LIC_AMD_CACHE", os.path.join("/tmp", "lic_amd_workloads"))
    os.makedirs(d, exist_ok=True)
    return d


def load(name: str, cache: bool = True) -> Workload:
    """Build (or read back from a local .npz cache) one named workload."""
    maker = MAKERS[name]
    path = os.path.join(_cache_dir(), f"{name}_v{_CACHE_VERSION}.npz")
    if cache and os.path.exists(path):
        with np.load(path, allow_pickle=False) as z:
            return Workload(name, z["symbols"], z["indexes"], z["cdf"], z["lengths"],
                            z["offsets"], tuple(int(v) for v in z["lanes"]))
    w = maker()
    if cache:
        tmp = path + f".tmp{os.getpid()}.npz"
        np.savez(tmp, symbols=w.symbols, indexes=w.indexes, cdf=w.cdf, lengths=w.lengths,
                 offsets=w.offsets, lanes=np.asarray(w.lanes, dtype=np.int64))
        os.replace(tmp, path)
    return w
