"""Pins of the oracle's histogram and codebook construction (CPU only).

Each check ties the oracle to something other than itself: brute-force
enumeration, a textbook heap Huffman, the Kraft identity, closed forms and
hand-derived worked examples.
"""

import collections
import heapq
import itertools
import math

import numpy as np
import pytest

import oracle
from oracle.huffman import package_merge_lengths, canonical_codes, kraft_sum_scaled, codebook_frequencies
from golden_examples import load as load_golden


# ----------------------------------------------------------------------------- histogram

@pytest.mark.parametrize("n,alpha,seed", [(0, 256, 0), (1, 256, 1), (1000, 3, 2), (4097, 256, 3), (65536, 17, 4)])
def test_histogram_counts_by_hand(n, alpha, seed):
    x = np.random.default_rng(seed).integers(0, alpha, n, dtype=np.uint8)
    h = oracle.histogram(x)
    ref = collections.Counter(int(v) for v in x)
    assert h.dtype == np.uint64 and h.shape == (256,)
    assert int(h.sum()) == n
    for s in range(256):
        assert int(h[s]) == ref.get(s, 0)


def test_codebook_frequencies_sum_and_clamp():
    a = np.zeros(256, np.uint64)
    b = np.zeros(256, np.uint64)
    a[3], a[4] = 5, 7
    b[4], b[200] = 1, 2
    f = codebook_frequencies([a, b], min_freq=1)
    assert f[3] == 5 and f[4] == 8 and f[200] == 2
    assert int((f == 1).sum()) == 253  # every other byte value raised to 1
    g = codebook_frequencies([a, b], min_freq=0)
    assert int((g == 0).sum()) == 253


# ----------------------------------------------------------------------------- brute force

def _feasible_vectors(m, L):
    vecs = np.array(list(itertools.product(range(1, L + 1), repeat=m)), dtype=np.int64)
    kraft = (2.0 ** (-vecs)).sum(axis=1)
    return vecs[kraft <= 1.0 + 1e-12]


def _random_freqs(rng, m, count):
    out = []
    for i in range(count):
        kind = i % 4
        if kind == 0:
            f = rng.integers(1, 10, m)  # many ties
        elif kind == 1:
            f = rng.integers(1, 1_000_000, m)
        elif kind == 2:
            f = 2 ** rng.integers(0, 20, m)  # extreme skew, ties in powers
        else:
            f = np.maximum(1, (rng.pareto(1.0, m) * 10).astype(np.int64))
        out.append(f)
    return np.array(out, dtype=np.int64)


@pytest.mark.parametrize("m", [2, 3, 4, 5, 6, 7])
def test_package_merge_is_optimal_brute_force(m):
    rng = np.random.default_rng(1000 + m)
    Lmin = max(1, math.ceil(math.log2(m)))
    for L in range(Lmin, m):
        vecs = _feasible_vectors(m, L)
        freqs = _random_freqs(rng, m, 300 if m >= 7 else 1000)
        best = (vecs.astype(np.float64) @ freqs.T.astype(np.float64)).min(axis=0)
        syms = rng.choice(256, m, replace=False)
        for f, b in zip(freqs, best):
            full = np.zeros(256, np.uint64)
            full[syms] = f
            ln = package_merge_lengths(full, L)
            assert np.all(ln[syms] >= 1) and np.all(ln[syms] <= L)
            assert int((ln > 0).sum()) == m
            assert kraft_sum_scaled(ln, 16) <= 1 << 16
            cost = int((ln[syms].astype(np.int64) * f).sum())
            assert cost == int(b), (m, L, f, ln[syms])


def _heap_huffman_lengths(freq):
    """Textbook Huffman with heapq; returns {symbol: depth}."""
    heap = [(int(f), i, (s,)) for i, (s, f) in enumerate(freq.items())]
    heapq.heapify(heap)
    depth = {s: 0 for s in freq}
    tick = len(heap)
    while len(heap) > 1:
        f1, _, a = heapq.heappop(heap)
        f2, _, b = heapq.heappop(heap)
        for s in a + b:
            depth[s] += 1
        heapq.heappush(heap, (f1 + f2, tick, a + b))
        tick += 1
    return depth


def test_cost_matches_textbook_huffman_when_limit_slack():
    rng = np.random.default_rng(7)
    checked = 0
    for trial in range(300):
        m = int(rng.integers(2, 257))
        syms = rng.choice(256, m, replace=False)
        f = rng.integers(1, 50_000, m) if trial % 2 else rng.integers(1, 6, m)
        freq = {int(s): int(v) for s, v in zip(syms, f)}
        depth = _heap_huffman_lengths(freq)
        if max(depth.values()) > 16:
            continue
        full = np.zeros(256, np.uint64)
        full[syms] = f
        ln = package_merge_lengths(full, 16)
        cost_pm = sum(int(ln[s]) * v for s, v in freq.items())
        cost_heap = sum(depth[s] * v for s, v in freq.items())
        assert cost_pm == cost_heap
        checked += 1
    assert checked > 250


def test_kraft_equality_and_monotone():
    rng = np.random.default_rng(11)
    for trial in range(200):
        m = int(rng.integers(2, 257))
        syms = rng.choice(256, m, replace=False)
        f = rng.integers(1, 1 << int(rng.integers(1, 40)), m, dtype=np.int64)
        full = np.zeros(256, np.uint64)
        full[syms] = f
        L = int(rng.integers(max(8, math.ceil(math.log2(m))), 17))
        ln = package_merge_lengths(full, L)
        assert kraft_sum_scaled(ln, 16) == 1 << 16  # complete code
        order = np.argsort(-f, kind="stable")
        for a, b in zip(order[:-1], order[1:]):
            if f[a] > f[b]:
                assert ln[syms[a]] <= ln[syms[b]]


@pytest.mark.parametrize("k", [1, 2, 3, 5, 8])
def test_equal_frequencies_closed_form(k):
    full = np.zeros(256, np.uint64)
    full[: 1 << k] = 12345
    ln = package_merge_lengths(full, 16)
    assert np.all(ln[: 1 << k] == k) and np.all(ln[1 << k:] == 0)


def test_dyadic_closed_form_reaches_entropy():
    # F proportional to 2^-k_i with sum(2^-k_i) = 1 -> len_i = k_i exactly, avg = H.
    ks = [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16, 16]
    full = np.zeros(256, np.uint64)
    syms = np.random.default_rng(5).choice(256, len(ks), replace=False)
    for s, k in zip(syms, ks):
        full[s] = 1 << (16 - k)
    ln = package_merge_lengths(full, 16)
    assert [int(ln[s]) for s in syms] == ks
    n = int(full.sum())
    avg = oracle.payload_bits_identity(full, ln) / n
    assert abs(avg - oracle.entropy_bits(full)) < 1e-12


def test_entropy_bracket_on_build_histograms():
    rng = np.random.default_rng(21)
    for sigma in (2.0, 5.0, 20.0, 60.0):
        x = np.clip(np.rint(rng.normal(0, sigma, 200_000)), -128, 127).astype(np.int8).view(np.uint8)
        h = oracle.histogram(x)
        ln = package_merge_lengths(h, 16)
        avg = oracle.payload_bits_identity(h, ln) / x.size
        H = oracle.entropy_bits(h)
        assert H <= avg < H + 1


def test_single_and_empty_alphabets():
    full = np.zeros(256, np.uint64)
    assert np.all(package_merge_lengths(full, 16) == 0)
    full[0x07] = 99
    ln = package_merge_lengths(full, 16)
    assert ln[0x07] == 1 and int(ln.sum()) == 1
    full[:] = 1
    with pytest.raises(ValueError):
        package_merge_lengths(full, 7)  # 256 symbols cannot fit in 7 bits
    assert np.all(package_merge_lengths(full, 8) == 8)


# ----------------------------------------------------------------------------- canonical codes

def _check_prefix_free(ln, cd):
    words = [format(int(cd[s]), f"0{int(ln[s])}b") for s in range(256) if ln[s] > 0]
    for a in words:
        for b in words:
            if a is not b and a != b:
                assert not b.startswith(a)
    assert len(set(words)) == len(words)


def test_canonical_codes_properties():
    rng = np.random.default_rng(3)
    for trial in range(40):
        m = int(rng.integers(2, 257))
        syms = rng.choice(256, m, replace=False)
        full = np.zeros(256, np.uint64)
        full[syms] = rng.integers(1, 10_000, m)
        ln = package_merge_lengths(full, 16)
        cd = canonical_codes(ln)
        _check_prefix_free(ln, cd)
        lmax = int(ln.max())
        last = max((s for s in range(256) if ln[s] == lmax))
        assert int(cd[last]) == (1 << lmax) - 1  # complete code ends in all ones
        for L in range(1, 17):
            same = [s for s in range(256) if ln[s] == L]
            vals = [int(cd[s]) for s in same]
            assert vals == list(range(vals[0], vals[0] + len(vals))) if vals else True


def test_uniform_codebook_is_identity():
    ln = np.full(256, 8, np.uint8)
    assert np.array_equal(canonical_codes(ln), np.arange(256, dtype=np.uint32))


def test_golden_codebooks():
    for ex in load_golden():
        ln = package_merge_lengths(ex["freq"], ex["max_len"])
        assert np.array_equal(ln, ex["lengths"]), ex["name"]
        cd = canonical_codes(ln)
        for s, bits in ex["codes"].items():
            assert format(int(cd[s]), f"0{int(ln[s])}b") == bits, (ex["name"], s)
