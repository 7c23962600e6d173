"""CPU oracle of the Huffman byte codec -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.

A plain, slow, obviously-correct numpy / pure-Python implementation of every
step on the coding path:

* ``huffman``   -- histogram, codebook frequencies, length-limited optimal code
                   lengths (package-merge), canonical code assignment;
* ``stream``    -- chunked stream format, two independent encoders (bit-string
                   definition and vectorised numpy) and two independent decoders
                   (bit-by-bit canonical and lock-step lookup table);
* ``bytegroup`` -- byte grouping (bf16: high / low byte planes; fp32: four
                   byte planes) and the two-stream container;
* ``metrics``   -- entropy, compressed-size identities and per-batch optimum;
* ``drift``     -- the codebook refresh rule under distribution drift;
* ``subbyte``   -- 4-bit tensors: packed pairs against 16-symbol codes.

Sources: "Single-Stage Huffman Encoder for ML Compression" (summary page of
arXiv 2601.10673; sections Overview and Methodology) and "Lossless Compression
for LLM Tensor Incremental Snapshots" (summary page of arXiv 2505.09810;
sections Technical framework, Key design and the original abstract).  Every
function cites the passage it follows; where the pages are silent the reading
taken is stated in the docstring.

Rules this package obeys:

* Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
  ``bench.py`` may import it.  The library never calls it; there is no CPU
  fallback anywhere in the product path.
* It shares no code, table, constant generator or helper with the HIP library
  (``lossless_entropy_coding_byte_amd``) and imports nothing from it.
* Parity status: every function here is pinned by ``tests/test_oracle_*.py``
  against brute force, closed forms, library routines or hand-derived worked
  examples (``tests/golden/``); none is "parity unpinned".
"""

from .huffman import (
    histogram,
    codebook_frequencies,
    package_merge_lengths,
    canonical_codes,
    kraft_sum_scaled,
)
from .stream import (
    OracleError,
    CorruptStream,
    UncodedSymbol,
    num_chunks,
    table_bytes,
    encoded_bound,
    header_bytes,
    count_bytes,
    lanes_per_chunk,
    lane_symbol_counts,
    lane_positions,
    count_span,
    encode_bitstring,
    encode,
    decode_bitwise,
    decode,
    chunk_word_counts,
    lane_bit_counts,
    parse_table,
)
from .bytegroup import (split_bf16, merge_bf16, encode_bf16, decode_bf16, container_bytes, parse_container,
                        snapshot_delta, apply_delta, split_fp32, merge_fp32, encode_fp32, decode_fp32)
from . import subbyte
from .metrics import entropy_bits, payload_bits_identity, per_batch_optimal_bits
from .drift import payload_bits_or_none, drift_check, adaptive_codebooks

__all__ = [
    "histogram", "codebook_frequencies", "package_merge_lengths", "canonical_codes",
    "kraft_sum_scaled", "OracleError", "CorruptStream", "UncodedSymbol", "num_chunks",
    "table_bytes", "header_bytes", "count_bytes", "lanes_per_chunk", "lane_symbol_counts", "lane_positions", "count_span", "encoded_bound", "encode_bitstring", "encode", "decode_bitwise", "decode",
    "chunk_word_counts", "lane_bit_counts", "parse_table", "split_bf16", "merge_bf16", "encode_bf16", "decode_bf16",
    "container_bytes", "parse_container", "entropy_bits", "payload_bits_identity",
    "per_batch_optimal_bits", "snapshot_delta", "apply_delta", "payload_bits_or_none", "drift_check",
    "adaptive_codebooks", "split_fp32", "merge_fp32", "encode_fp32", "decode_fp32", "subbyte",
]
