"""Oracle work of the full-size parity tests, run in worker processes.

The workers are forked from a server process that the test session starts
before anything touches the GPU (``tests/conftest.py``); they import numpy,
the oracle and the input recipes only.  Each job regenerates or receives its
inputs and returns the oracle's stream(s), so the parent only compares bytes.

Layout helpers at the bottom slice a stream of many chunks into the part that
belongs to a run of whole chunks, using the oracle's own layout functions, so
that one long stream can be compared block by block with the oracle's
streams of its blocks.
"""

from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

_CTX = None
BLOCK_SYMBOLS = 1 << 24  # oracle calls cover at most this many symbols (whole chunks)


def start_server() -> None:
    """Start the fork server (call before the GPU is initialised)."""
    global _CTX
    if _CTX is not None:
        return
    ctx = mp.get_context("forkserver")
    ctx.set_forkserver_preload(["numpy", "oracle", "workloads", "oracle_jobs"])
    from multiprocessing import forkserver

    forkserver.ensure_running()
    _CTX = ctx


def workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def pool():
    if _CTX is None:
        raise RuntimeError("the oracle worker server was not started before the GPU was initialised")
    return _CTX.Pool(workers())


# ----------------------------------------------------------------------------- jobs

def encode(args):
    """(symbols, lengths, chunk) -> (oracle stream, payload bits)."""
    import oracle

    sym, lengths, chunk = args
    s, bits = oracle.encode(sym, lengths, oracle.canonical_codes(lengths), chunk)
    return s, bits


def encode_blocks(sym, lengths, chunk):
    """Oracle streams of consecutive blocks of whole chunks: [(first symbol, symbols, stream)]."""
    import oracle

    cd = oracle.canonical_codes(lengths)
    step = max(chunk, BLOCK_SYMBOLS // chunk * chunk)
    return [(i, min(step, sym.size - i), oracle.encode(sym[i:i + step], lengths, cd, chunk)[0])
            for i in range(0, sym.size, step)]


def drift_batch(args):
    """Batch k of the drift stream: (k, symbols, histogram, block streams)."""
    import workloads

    k, lengths, chunk = args
    x = workloads.int8_drift_batch(k)
    h = np.bincount(x, minlength=256).astype(np.uint64)
    return k, x, h, encode_blocks(x, lengths, chunk)


def delta_snapshots(j):
    """Block j of the snapshot workload: (j, W0, W1) as uint16 (the recipe of ``workloads.bf16_delta``)."""
    import workloads

    w0 = workloads.bf16_bits(workloads.rng(4, 0, j).normal(0.0, 0.02, workloads.BLOCK).astype(np.float32))
    noise = workloads.rng(4, 1, j).normal(0.0, 1e-4, workloads.BLOCK).astype(np.float32)
    w1 = workloads.bf16_bits(workloads.bf16_to_f32(w0) + noise)
    return j, w0, w1


def plane_blocks(args):
    """(offset, plane symbols, lengths, chunk) -> (offset, block streams)."""
    off, sym, lengths, chunk = args
    return off, encode_blocks(sym, lengths, chunk)


# ----------------------------------------------------------------------------- stream slicing

def compare_chunk_run(stream, n, chunk, c0, ref, ref_n):
    """Check that chunks [c0, c0 + nc(ref_n)) of `stream` (n symbols) are the
    oracle stream `ref` of those chunks' symbols: offset table (shifted by the
    run's first payload word), lane word counts, payload words."""
    import oracle

    nc = oracle.num_chunks(n, chunk)
    nb = oracle.num_chunks(ref_n, chunk)
    table = stream[: 4 * nc].view("<u4")
    base = int(table[c0 - 1]) if c0 else 0
    rt = ref[: 4 * nb].view("<u4").astype(np.int64)
    got = table[c0:c0 + nb].astype(np.int64) - base
    if not np.array_equal(got, rt):
        bad = int(np.argmax(got != rt))
        raise AssertionError(f"offset table differs at chunk {c0 + bad}")
    a, b = oracle.count_span(n, chunk, c0, c0 + nb)
    ra, rb = oracle.count_span(ref_n, chunk, 0, nb)
    if not np.array_equal(stream[a:b], ref[ra:rb]):
        raise AssertionError(f"lane word counts differ in chunks [{c0}, {c0 + nb})")
    hb, rhb = oracle.header_bytes(n, chunk), oracle.header_bytes(ref_n, chunk)
    W = int(rt[-1])
    if ref.size != rhb + 4 * W:
        raise AssertionError("oracle block stream has an unexpected size")
    if not np.array_equal(stream[hb + 4 * base: hb + 4 * (base + W)], ref[rhb:]):
        raise AssertionError(f"payload differs in chunks [{c0}, {c0 + nb})")
    return nb


def check_blocks(stream, n, chunk, blocks, offset=0):
    """compare_chunk_run over [(first symbol, symbols, oracle stream)], the
    first symbols counted from `offset`; returns the number of chunks covered."""
    covered = 0
    for i, m, ref in blocks:
        first = offset + i
        assert first % chunk == 0
        covered += compare_chunk_run(stream, n, chunk, first // chunk, ref, m)
    return covered
