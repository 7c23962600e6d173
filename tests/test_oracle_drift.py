"""Pins of the codebook refresh rule (oracle/drift.py).

The page ("Single-Stage Huffman Encoder for ML Compression", Limitations and
future work, distribution drift) leaves the refresh rule open; the pins below
fix the rule's arithmetic with values derived by hand from closed forms:

* a uniform histogram's optimal 256-symbol code is all 8 bits (Kraft equality
  with 256 equal lengths), so a uniform 8-bit code is never refreshed;
* a byte with more than half the mass gets a 1-bit code in an optimal code, so
  against an all-8-bit code the batch costs exactly 8x the optimum: the
  decision flips between tol = 7 000 000 - 1 ppm and 7 000 000 ppm.
"""

import numpy as np
import pytest

import oracle

U8 = np.full(256, 8, np.uint8)


def test_uniform_code_on_uniform_data_is_kept():
    h = np.full(256, 1000, np.uint64)
    r, use, bc, bo = oracle.drift_check(h, U8, 16, 0)
    assert not r and bc == bo == 8 * 256 * 1000
    assert np.array_equal(use, U8)


@pytest.mark.parametrize("n", [300, 10_000, 1 << 24])
def test_dominant_byte_boundary(n):
    h = np.zeros(256, np.uint64)
    h[0] = n  # more than the other 255 clamped counts together
    r1, use1, bc, bo = oracle.drift_check(h, U8, 16, 7_000_000 - 1)
    assert bc == 8 * n and bo == n  # 1-bit code for byte 0
    assert r1 and use1[0] == 1
    r2, use2, _, _ = oracle.drift_check(h, U8, 16, 7_000_000)
    assert not r2 and np.array_equal(use2, U8)


def test_uncodable_byte_forces_refresh():
    cur = U8.copy()
    cur[5] = 0
    cur[6] = 7  # keeps Kraft at most 1: one 7-bit code replaces two 8-bit ones
    h = np.full(256, 3, np.uint64)
    r, use, bc, bo = oracle.drift_check(h, cur, 16, 10**12)
    assert r and bc is None and use[5] > 0
    assert oracle.payload_bits_or_none(h, use) == bo


def test_rule_over_a_drifting_sequence():
    rng = np.random.default_rng(3)
    hists = []
    for k in range(12):
        sigma = 8 + 4 * k
        x = np.clip(np.rint(rng.normal(0, sigma, 50_000)), -128, 127).astype(np.int8).view(np.uint8)
        hists.append(oracle.histogram(x))
    first = oracle.package_merge_lengths(oracle.codebook_frequencies(hists[:1], 1), 16)
    for tol in (0, 20_000, 10**9):
        steps = oracle.adaptive_codebooks(hists, first, 16, tol)
        cur = first
        for h, (r, use, bc, bo) in zip(hists, steps):
            assert bc == oracle.payload_bits_or_none(h, cur)
            # a refresh codes the batch at its clamped optimum, never worse
            if r:
                assert oracle.payload_bits_or_none(h, use) == bo <= bc
            else:
                assert np.array_equal(use, cur)
            # the clamped optimum is never below the unclamped one
            assert bo >= oracle.per_batch_optimal_bits(h, 16)
            cur = use
    never = oracle.adaptive_codebooks(hists, first, 16, 10**9)
    assert not any(r for r, *_ in never)
    always = oracle.adaptive_codebooks(hists, first, 16, 0)
    assert sum(r for r, *_ in always) >= 6  # sigma grows every batch
    # an identical batch right after a refresh keeps the new codebook
    again = oracle.adaptive_codebooks([hists[5], hists[5]], first, 16, 0)
    assert again[0][0] and not again[1][0]
