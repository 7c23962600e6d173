"""Oracle: size accounting -- entropy, payload identity, per-batch optimum.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

Page basis: "Single-Stage Huffman Encoder for ML Compression", Key
contributions and Results (the fixed codebook is compared with per-shard
Huffman coding and with the Shannon bound) and Methodology step 5 (the
comparison also includes plain 8-bit storage).

Readings: "per-shard Huffman" = an optimal codebook built from the evaluated
batch's own histogram (same length limit, no clamp); the Shannon bound of a
batch = n * H with H the empirical entropy of its byte histogram.
"""

from __future__ import annotations

import math

import numpy as np

from .huffman import package_merge_lengths


def entropy_bits(hist) -> float:
    """Empirical entropy H = -sum p log2 p of a histogram, in bits per symbol (float64)."""
    h = np.asarray(hist, dtype=np.float64)
    n = h.sum()
    if n == 0:
        return 0.0
    p = h[h > 0] / n
    return float(-(p * np.log2(p)).sum())


def payload_bits_identity(hist, lengths) -> int:
    """sum over s of f[s] * len[s]: the payload bits any encoder of this data must produce."""
    h = [int(x) for x in np.asarray(hist, dtype=np.uint64)]
    ln = [int(x) for x in np.asarray(lengths)]
    return sum(a * b for a, b in zip(h, ln))


def per_batch_optimal_bits(hist, max_len: int = 16) -> int:
    """Payload bits of the optimal (length-limited) code built from this histogram itself."""
    return payload_bits_identity(hist, package_merge_lengths(hist, max_len))


def shannon_bits(hist) -> float:
    h = np.asarray(hist, dtype=np.float64)
    return float(h.sum()) * entropy_bits(hist)


def gaussian_entropy_bits(sigma: float) -> float:
    """Differential entropy of N(0, sigma^2) in bits: a closed form the rounded data approaches."""
    return 0.5 * math.log2(2 * math.pi * math.e * sigma * sigma)
