"""The block-by-block comparison used by the full-size parity tests (CPU only).

A long stream is checked chunk run by chunk run against the oracle's streams
of those runs alone.  This holds because chunks are independent: a run's
offset table is the long stream's entries minus the run's first payload word,
and its unit metadata and payload words are slices of the long stream.  The
checks below show the comparison accepts the oracle's own long stream and
rejects a change in any part of it.
"""

import numpy as np
import pytest

import oracle
import oracle_jobs
import workloads


@pytest.fixture(autouse=True)
def small_blocks(monkeypatch):
    monkeypatch.setattr(oracle_jobs, "BLOCK_SYMBOLS", 1 << 16)


@pytest.mark.parametrize("n,chunk", [(300_007, 4096), (1 << 18, 16384), (200_000, 65536)])
def test_blocks_reassemble_the_long_stream(n, chunk):
    x = workloads.skewed_bytes(5, n, 6.0)
    ln = oracle.package_merge_lengths(oracle.codebook_frequencies([oracle.histogram(x)], 1), 16)
    whole, _ = oracle.encode(x, ln, oracle.canonical_codes(ln), chunk)
    blocks = oracle_jobs.encode_blocks(x, ln, chunk)
    assert len(blocks) >= 2 or chunk > (1 << 16)
    assert oracle_jobs.check_blocks(whole, n, chunk, blocks) == oracle.num_chunks(n, chunk)


def test_blocks_catch_any_changed_part():
    n, chunk = 300_007, 4096
    x = workloads.skewed_bytes(6, n, 6.0)
    ln = oracle.package_merge_lengths(oracle.codebook_frequencies([oracle.histogram(x)], 1), 16)
    whole, _ = oracle.encode(x, ln, oracle.canonical_codes(ln), chunk)
    blocks = oracle_jobs.encode_blocks(x, ln, chunk)
    nc = oracle.num_chunks(n, chunk)
    a, _ = oracle.count_span(n, chunk, 0, nc - (nc % 2))
    hb = oracle.header_bytes(n, chunk)
    for where in (4 * (nc // 2), a + 3, hb + 5, whole.size - 1):
        bad = whole.copy()
        bad[where] ^= 0x10
        with pytest.raises(AssertionError):
            oracle_jobs.check_blocks(bad, n, chunk, blocks)
