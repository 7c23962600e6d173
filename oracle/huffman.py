"""Oracle: symbol statistics and the canonical, length-limited Huffman codebook.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

Page basis
----------
* "Single-Stage Huffman Encoder for ML Compression", Overview: classic Huffman
  coding of a tensor shard is three steps -- frequency analysis, codebook
  generation, codebook transmission.
* Same page, Methodology steps 1-3: count the 8-bit symbol frequencies of a few
  warm-up batches, take their average distribution, build the Huffman codebook
  once from it.
* "Lossless Compression for LLM Tensor Incremental Snapshots", Technical
  framework steps 2-3 (frequency statistics of the byte groups, Huffman tree
  and coding) and Key design item 2 (an efficient Huffman-tree construction).

Readings (the pages give no parameters; their Key design section says so):
* "average distribution" = the integer SUM of the warm-up histograms (Huffman
  comparisons are invariant to a common positive scale), then every symbol's
  frequency is raised to at least ``min_freq`` so a fixed codebook covers all
  256 byte values;
* codes are limited to ``max_len`` bits and are OPTIMAL under that limit
  (package-merge; no heuristic length adjustment);
* ties are broken by one fixed rule (below) so the length vector is unique;
* code words are CANONICAL, so the codebook is fully described by its lengths.
"""

from __future__ import annotations

import numpy as np

NSYM = 256


def histogram(sym: np.ndarray) -> np.ndarray:
    """f[s] = number of positions i with sym[i] == s, for s in 0..255 (uint64).

    Frequency analysis step ("Single-Stage Huffman Encoder ...", Overview;
    "Lossless Compression ... Snapshots", Technical framework step 2).
    """
    sym = np.ascontiguousarray(sym).view(np.uint8).ravel()
    return np.bincount(sym, minlength=NSYM).astype(np.uint64)


def codebook_frequencies(hists, min_freq: int = 1) -> np.ndarray:
    """Frequencies a fixed codebook is built from.

    "Single-Stage Huffman Encoder ...", Methodology steps 1-2: statistics of
    warm-up batches are combined into one average distribution.  Reading: the
    combination is the integer sum (a common scale does not change any Huffman
    decision), after which F[s] = max(F[s], min_freq).  ``min_freq = 0`` keeps
    the raw sum (per-tensor mode: absent symbols get no code).
    """
    hists = [np.asarray(h, dtype=np.uint64) for h in hists]
    total = np.zeros(NSYM, dtype=np.uint64)
    for h in hists:
        if h.shape != (NSYM,):
            raise ValueError("histogram must have 256 bins")
        total += h
    if min_freq > 0:
        total = np.maximum(total, np.uint64(min_freq))
    return total


def package_merge_lengths(freq, max_len: int = 16) -> np.ndarray:
    """Optimal code lengths under sum(F*len) with 1 <= len <= max_len (uint8[256]).

    Huffman-tree step ("Lossless Compression ... Snapshots", Technical
    framework step 3, Key design item 2), written as the package-merge
    solution of the coin-collector problem (Larmore & Hirschberg, 1990):

    * every coded symbol (F > 0) owns one coin of weight F[s] at each of the
      denominations 2^-1 .. 2^-max_len; the codeword length of s is the number
      of its coins in the cheapest coin set of total face value m - 1;
    * the list at the smallest denomination is the coins sorted by
      (weight, symbol); moving up one denomination, consecutive pairs of the
      current list are packaged (an odd last item is dropped) and the packages
      are merged with a fresh copy of the coins;
    * after max_len - 1 such steps the first 2m - 2 items of the list are the
      optimal set.

    Tie rule (the pages are silent; this fixes a unique answer): coins are
    ordered by (weight, symbol value); when a coin and a package weigh the
    same, the coin comes first; each source keeps its own order.

    Every list item carries the vector of coin counts per symbol it contains,
    so the result is read off directly -- O(max_len * m^2), slow and plain.
    Special cases: m = 0 -> all zero; m = 1 -> that symbol gets length 1;
    m > 2^max_len -> ValueError.
    """
    freq = [int(x) for x in np.asarray(freq, dtype=np.uint64).ravel()]
    if len(freq) != NSYM:
        raise ValueError("freq must have 256 entries")
    if not 1 <= max_len <= 16:
        raise ValueError("max_len must be in 1..16")
    lengths = np.zeros(NSYM, dtype=np.uint8)
    coded = [s for s in range(NSYM) if freq[s] > 0]
    m = len(coded)
    if m == 0:
        return lengths
    if m == 1:
        lengths[coded[0]] = 1
        return lengths
    if m > (1 << max_len):
        raise ValueError("too many coded symbols for max_len")

    order = sorted(coded, key=lambda s: (freq[s], s))
    coins = []
    for s in order:
        v = np.zeros(NSYM, dtype=np.int64)
        v[s] = 1
        coins.append((freq[s], v))

    current = list(coins)
    for _ in range(max_len - 1):
        packages = []
        for j in range(len(current) // 2):
            a, b = current[2 * j], current[2 * j + 1]
            packages.append((a[0] + b[0], a[1] + b[1]))
        merged = []
        i = k = 0
        while i < len(coins) or k < len(packages):
            if k == len(packages) or (i < len(coins) and coins[i][0] <= packages[k][0]):
                merged.append(coins[i])
                i += 1
            else:
                merged.append(packages[k])
                k += 1
        current = merged

    chosen = current[: 2 * m - 2]
    count = np.zeros(NSYM, dtype=np.int64)
    for _, v in chosen:
        count += v
    assert np.all(count[coded] >= 1) and np.all(count <= max_len)
    lengths[:] = count.astype(np.uint8)
    return lengths


def canonical_codes(lengths) -> np.ndarray:
    """Canonical code words for a length vector (uint32[256], right-aligned).

    Reading: the codebook exchanged and stored is the length vector alone; the
    code words follow the canonical rule (Schwartz & Kallick, 1964): sort the
    coded symbols by (length, symbol value); the first gets the all-zero code
    of its length; each next code is (previous code + 1) shifted left by the
    growth in length.  Bits are emitted most-significant first.
    """
    lengths = np.asarray(lengths, dtype=np.int64).ravel()
    if lengths.shape != (NSYM,):
        raise ValueError("lengths must have 256 entries")
    codes = np.zeros(NSYM, dtype=np.uint32)
    coded = sorted((int(lengths[s]), s) for s in range(NSYM) if lengths[s] > 0)
    code = 0
    prev_len = None
    for ln, s in coded:
        if prev_len is None:
            code = 0
        else:
            code = (code + 1) << (ln - prev_len)
        if code >= (1 << ln):
            raise ValueError("length vector violates the Kraft inequality")
        codes[s] = code
        prev_len = ln
    return codes


def kraft_sum_scaled(lengths, max_len: int = 16) -> int:
    """sum over coded symbols of 2^(max_len - len): equals 2^max_len iff the code is complete."""
    lengths = np.asarray(lengths, dtype=np.int64).ravel()
    return int(sum(1 << (max_len - int(l)) for l in lengths if l > 0))
