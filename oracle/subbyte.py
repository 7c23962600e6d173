"""Oracle: 4-bit tensors, coded as packed pairs or as a 16-symbol alphabet.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

Page basis: "Single-Stage Huffman Encoder for ML Compression", Limitations and
future work (quantisation granularity): the method is built for 8-bit tensors
and extending it to 4-bit data is left open.

Readings (the pages fix no layout or alphabet for 4-bit data):
* a 4-bit tensor is stored two values per byte, value 2i in bits 0-3 and value
  2i+1 in bits 4-7 (two's complement);
* "packed pairs": each byte -- the ordered pair of 4-bit values -- is one
  symbol of the usual 256-symbol alphabet, so the byte codec (histogram,
  codebook, encode, decode) applies unchanged;
* "16-symbol codes": each 4-bit value is a symbol of its own, coded with a
  length-limited optimal code over 16 symbols.  Only its size is computed here,
  to compare the two readings: concatenating two 16-symbol code words gives a
  prefix code on pairs, so the optimal pair code is never longer than the
  16-symbol code when the latter's words are at most half the pair limit
  (``pair_bound_holds`` states exactly that).
"""

from __future__ import annotations

import numpy as np

from .huffman import package_merge_lengths
from .metrics import payload_bits_identity


def nibbles(packed) -> np.ndarray:
    """The 4-bit values (as 0..15) in tensor order: low nibble of byte i, then its high nibble."""
    b = np.ascontiguousarray(packed).view(np.uint8).ravel()
    out = np.empty(2 * b.size, dtype=np.uint8)
    out[0::2] = b & 0x0F
    out[1::2] = b >> 4
    return out


def nibble_histogram(packed) -> np.ndarray:
    """f[v] = number of 4-bit values equal to v (v in 0..15), over both halves of every byte.

    Returned with 256 bins (bins 16..255 zero) so the 256-symbol code builder
    takes it as is.
    """
    return np.bincount(nibbles(packed), minlength=256).astype(np.uint64)


def nibble_code_lengths(packed, max_len: int = 8) -> np.ndarray:
    """Optimal code lengths of the 16-symbol reading (only values that occur get a code)."""
    return package_merge_lengths(nibble_histogram(packed), max_len)


def nibble_code_bits(packed, max_len: int = 8) -> int:
    """Payload bits of the whole tensor under the 16-symbol reading."""
    h = nibble_histogram(packed)
    return payload_bits_identity(h, package_merge_lengths(h, max_len))


def pair_code_bits(packed, max_len: int = 16) -> int:
    """Payload bits of the whole tensor under the packed-pair reading (optimal for this tensor)."""
    h = np.bincount(np.ascontiguousarray(packed).view(np.uint8).ravel(), minlength=256).astype(np.uint64)
    return payload_bits_identity(h, package_merge_lengths(h, max_len))


def pair_bound_holds(packed, pair_max_len: int = 16) -> bool:
    """pair_code_bits(L) <= nibble_code_bits(L // 2): the concatenation argument above."""
    return pair_code_bits(packed, pair_max_len) <= nibble_code_bits(packed, pair_max_len // 2)
