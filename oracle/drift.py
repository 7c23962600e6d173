"""Oracle: codebook refresh under distribution drift -- TEST INFRASTRUCTURE.

(See ``oracle/__init__.py`` for the rules this package obeys.)

Page basis: "Single-Stage Huffman Encoder for ML Compression", Limitations
and future work, first item: a fixed codebook assumes stationary symbol
statistics, a large shift (e.g. a change of domain) can cost compression, and
an adaptive refresh mechanism is left open.

Reading (the page gives no rule; this is the one taken here):

* a batch is coded with the current fixed codebook unless that costs more
  than a tolerance over the best fixed codebook for the batch itself;
* "best fixed codebook for the batch" = package-merge lengths (same length
  limit) on the batch histogram clamped to frequency >= 1, i.e. built the way
  every fixed codebook is built (Methodology steps 1-2), so a refreshed
  codebook still codes every byte value;
* cost = payload bits, sum over s of f[s] * len[s] (a byte the current code
  cannot code makes the current cost infinite);
* refresh  <=>  bits_cur * 10^6 > bits_opt * (10^6 + tol_ppm), in integers,
  so both implementations take the same decision exactly;
* on refresh the batch is coded with the new codebook, which then stays
  current for the following batches.
"""

from __future__ import annotations

import numpy as np

from .huffman import NSYM, codebook_frequencies, package_merge_lengths


def payload_bits_or_none(hist, lengths):
    """sum f[s]*len[s]; None when some byte with f[s] > 0 has no code word."""
    h = [int(x) for x in np.asarray(hist, dtype=np.uint64).ravel()]
    ln = [int(x) for x in np.asarray(lengths).ravel()]
    if len(h) != NSYM or len(ln) != NSYM:
        raise ValueError("histogram and lengths have 256 entries")
    total = 0
    for f, l in zip(h, ln):
        if f and not l:
            return None
        total += f * l
    return total


def drift_check(hist, cur_lengths, max_len: int = 16, tol_ppm: int = 0):
    """One batch's decision: (refresh, lengths to code it with, bits_cur, bits_opt).

    bits_cur is None when the current codebook cannot code the batch."""
    if tol_ppm < 0:
        raise ValueError("tol_ppm must be >= 0")
    best = package_merge_lengths(codebook_frequencies([np.asarray(hist, dtype=np.uint64)], 1), max_len)
    bits_opt = payload_bits_or_none(hist, best)
    bits_cur = payload_bits_or_none(hist, cur_lengths)
    refresh = bits_cur is None or bits_cur * 1_000_000 > bits_opt * (1_000_000 + int(tol_ppm))
    use = best if refresh else np.asarray(cur_lengths, dtype=np.uint8).copy()
    return bool(refresh), use, bits_cur, bits_opt


def adaptive_codebooks(hists, first_lengths, max_len: int = 16, tol_ppm: int = 0):
    """Run the rule over a sequence of batch histograms.

    Returns a list of (refresh, lengths used, bits_cur, bits_opt), one per batch."""
    cur = np.asarray(first_lengths, dtype=np.uint8).copy()
    out = []
    for h in hists:
        r, use, bc, bo = drift_check(h, cur, max_len, tol_ppm)
        out.append((r, use, bc, bo))
        cur = use
    return out
