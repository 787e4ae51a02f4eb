"""Synthetic 16-bit quantised CDF tables (inputs to the coder, not part of it).

The pages describe the tables the coder consumes but not how the codec built
them: the y latent of the 1080p mean-scale hyperprior is coded with 64 CDF
rows whose marshalled form holds 200,512 int32 entries (kompressor
BENCHMARKS.md, section 4, ``cdf.tolist() (200512 elements)``), and torch_ans
describes a row as the alphabet plus an escape slot for bypass coding plus the
terminal entry (torch_ans page, "Range limit" under ``rans*_push`` and the
alias-sampling note under "Performance Tuning").

This module builds such tables from closed-form densities:

* a zero-mean Gaussian per scale, discretised on integer bins
  ``[v-1/2, v+1/2)`` over ``v in [-c, c]`` with ``c = ceil(s * z)`` where
  ``z = Phi^-1(1 - 5e-10)`` (two-sided tail mass 1e-9); with 64 scales
  log-spaced over 0.11..256 the longest row is 3133 = 200512 / 64 entries;
* a zero-mean logistic per channel (factorised hyperprior ``z``), same
  binning, half-width ``min(30, ceil(s * ln(2e9)))`` so a row has at most 63
  entries.

The probability outside ``[-c-1/2, c+1/2)`` becomes the escape slot.  A pmf
is quantised to 16 bits by rounding half-to-even, raising every frequency to
at least 1, then moving the surplus (or deficit) one unit at a time onto the
currently largest frequency (lowest slot on ties; never below 1) until the
row sums to 2**16.  Rows are returned in the layout the coder takes:
``cdf[K, stride]`` int32 with ``cdf[r, 0] = 0``, ``cdf[r, len-1] = 65536``,
padding entries set to 65536, plus ``lengths[K]`` and ``offsets[K]``.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import ndtr, ndtri

PRECISION = 16
TOTAL = 1 << PRECISION
GAUSS_TAIL_Z = float(ndtri(1.0 - 5e-10))          # 6.10941...
LOGISTIC_TAIL_Z = math.log((1.0 - 5e-10) / 5e-10)  # 21.4164...


def quantise_pmf(pmf: np.ndarray) -> np.ndarray:
    """Quantise a pmf (alphabet + escape slot, summing to 1) to 16-bit frequencies."""
    p = np.asarray(pmf, dtype=np.float64)
    f = np.rint(p * TOTAL).astype(np.int64)  # numpy rint rounds half to even
    f = np.maximum(f, 1)
    excess = int(f.sum()) - TOTAL
    while excess != 0:
        k = int(np.argmax(f))  # first index of the maximum
        if excess > 0:
            if f[k] <= 1:
                raise ValueError("cannot remove surplus: every frequency is 1")
            f[k] -= 1
            excess -= 1
        else:
            f[k] += 1
            excess += 1
    return f


def freqs_to_cdf(f: np.ndarray) -> np.ndarray:
    cdf = np.zeros(len(f) + 1, dtype=np.int64)
    np.cumsum(f, out=cdf[1:])
    assert cdf[-1] == TOTAL
    return cdf


def _pack(rows, offsets, stride=None):
    lengths = np.array([len(r) for r in rows], dtype=np.int32)
    if stride is None:
        stride = int(lengths.max())
    cdf = np.full((len(rows), stride), TOTAL, dtype=np.int32)
    for k, r in enumerate(rows):
        cdf[k, : len(r)] = r
    return cdf, lengths, np.asarray(offsets, dtype=np.int32)


def gaussian_scales(K: int, lo: float = 0.11, hi: float = 256.0) -> np.ndarray:
    k = np.arange(K, dtype=np.float64)
    return np.exp(math.log(lo) + (math.log(hi) - math.log(lo)) * k / (K - 1))


def gaussian_half_width(s: float) -> int:
    return int(math.ceil(s * GAUSS_TAIL_Z))


def gaussian_table_set(K: int, stride: int | None = None):
    """K discretised zero-mean Gaussians, scales log-spaced over 0.11..256."""
    scales = gaussian_scales(K)
    rows, offs = [], []
    for s in scales:
        c = gaussian_half_width(float(s))
        v = np.arange(-c, c + 1, dtype=np.float64)
        p = ndtr((v + 0.5) / s) - ndtr((v - 0.5) / s)
        pmf = np.concatenate([p, [max(0.0, 1.0 - p.sum())]])
        rows.append(freqs_to_cdf(quantise_pmf(pmf)))
        offs.append(-c)
    cdf, lengths, offsets = _pack(rows, offs, stride)
    return cdf, lengths, offsets, scales


def _sigmoid(x):
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def logistic_half_width(s: float) -> int:
    return min(30, int(math.ceil(s * LOGISTIC_TAIL_Z)))


def logistic_table_set(scales: np.ndarray, stride: int = 64):
    """One discretised zero-mean logistic row per channel scale."""
    rows, offs = [], []
    for s in np.asarray(scales, dtype=np.float64):
        c = logistic_half_width(float(s))
        v = np.arange(-c, c + 1, dtype=np.float64)
        p = _sigmoid((v + 0.5) / s) - _sigmoid((v - 0.5) / s)
        pmf = np.concatenate([p, [max(0.0, 1.0 - p.sum())]])
        rows.append(freqs_to_cdf(quantise_pmf(pmf)))
        offs.append(-c)
    return _pack(rows, offs, stride)
