"""C-ABI library on the CPU: every declared symbol is exported, and the host-only
functions (codebook builder, sizes, container header) agree with the oracle."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import lossless_entropy_coding_byte_amd as lecb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "lecb.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lecb_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = lecb.load()
    declared = _declared_functions()
    assert len(declared) >= 20
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(lecb.exported_symbols()) == declared  # the binding mirrors the header 1:1
    assert lecb.lecb_abi_version() == 3


def test_sizes_match_oracle():
    for n in (0, 1, 255, 256, 4096, 4097, 123457, 1 << 20):
        for chunk in (256, 1024, 4096, 16384, 65536):
            assert lecb.lecb_num_chunks(n, chunk) == oracle.num_chunks(n, chunk)
            hb = oracle.header_bytes(n, chunk) if n else 0
            assert lecb.lecb_header_bytes(n, chunk) == hb
            assert lecb.lecb_encoded_bound(n, chunk, 16) == oracle.encoded_bound(n, chunk, 16)
    assert lecb.lecb_num_chunks(100, 300) == 0  # not a power of two
    assert lecb.lecb_encoded_bound(100, 4096, 17) == 0


def test_workspace_bytes_contract():
    """The workspace holds, per stream (two), a 64-byte header and one 64-bit
    slot per chunk plus four more (the encoder's ranges: at most the chunks + 3),
    then 256 bytes for the headers of a third and fourth stream; every part is
    256-byte aligned."""
    for n in (0, 1, 4096, 123457, 1 << 20, 1 << 26):
        for chunk in (256, 4096, 16384, 65536):
            nc = -(-n // chunk)
            part = -(-(64 + 8 * (nc + 4)) // 256) * 256
            ws = lecb.lecb_workspace_bytes(n, chunk)
            assert ws == 2 * part + 256, (n, chunk)
            assert ws % 256 == 0
    assert lecb.lecb_workspace_bytes(1000, 300) == 0
    assert lecb.lecb_workspace_bytes(1000, 128) == 0


def _random_hist(rng, kind):
    h = np.zeros(256, np.uint64)
    m = int(rng.integers(1, 257))
    syms = rng.choice(256, m, replace=False)
    if kind == 0:
        h[syms] = rng.integers(1, 8, m)  # ties everywhere
    elif kind == 1:
        h[syms] = rng.integers(1, 1 << 30, m)
    elif kind == 2:
        h[syms] = 1 << rng.integers(0, 40, m)  # power-of-two ties, deep trees
    elif kind == 3:
        h[syms] = np.maximum(1, (rng.pareto(0.7, m) * 3).astype(np.int64))
    else:
        x = np.clip(np.rint(rng.normal(0, rng.uniform(0.5, 60), 5000)), -128, 127).astype(np.int8)
        h = oracle.histogram(x.view(np.uint8))
    return h


@pytest.mark.parametrize("kind", range(5))
def test_builder_matches_oracle_on_random_histograms(kind):
    rng = np.random.default_rng(77 + kind)
    for trial in range(2000 if kind < 4 else 500):
        h = _random_hist(rng, kind)
        m = int((h > 0).sum())
        lo = max(1, int(np.ceil(np.log2(max(m, 2)))))
        L = int(rng.integers(lo, 17))
        min_freq = int(rng.integers(0, 2)) if trial % 3 == 0 else 0
        if min_freq:
            L = max(L, 8)
        F = oracle.codebook_frequencies([h], min_freq)
        ref_len = oracle.package_merge_lengths(F, L)
        cb = lecb.lecb_build_codebook(h, L, min_freq)
        assert np.array_equal(cb.lengths(), ref_len), (kind, trial, L)
        ref_codes = oracle.canonical_codes(ref_len)
        assert np.array_equal(cb.codes()[ref_len > 0], ref_codes[ref_len > 0])
        assert cb.num_coded == int((ref_len > 0).sum())


def test_builder_on_workload_histograms():
    import workloads

    warm = [oracle.histogram(workloads.int8_fixed(r)) for r in (1, 2, 3, 4)]
    F = oracle.codebook_frequencies(warm, 1)
    cb = lecb.lecb_build_codebook(np.sum(warm, axis=0, dtype=np.uint64), 16, 1)
    assert np.array_equal(cb.lengths(), oracle.package_merge_lengths(F, 16))
    x = workloads.bf16_weights(1 << 18)
    for plane in oracle.split_bf16(x):
        h = oracle.histogram(plane)
        assert np.array_equal(lecb.lecb_build_codebook(h, 16, 0).lengths(), oracle.package_merge_lengths(h, 16))


def test_builder_errors():
    with pytest.raises(lecb.LecbError) as e:
        lecb.lecb_build_codebook(np.zeros(256, np.uint64), 16, 0)
    assert e.value.status == lecb.LECB_ERR_NO_SYMBOLS
    with pytest.raises(lecb.LecbError) as e:
        lecb.lecb_build_codebook(np.ones(256, np.uint64), 7, 0)
    assert e.value.status == lecb.LECB_ERR_NO_SYMBOLS
    with pytest.raises(lecb.LecbError) as e:
        lecb.lecb_build_codebook(np.ones(256, np.uint64), 17, 0)
    assert e.value.status == lecb.LECB_ERR_INVALID_ARG
    bad = np.zeros(256, np.uint8)
    bad[:3] = 1  # three 1-bit codes violate Kraft
    with pytest.raises(lecb.LecbError):
        lecb.lecb_codebook_from_lengths(bad)


def test_container_header_golden_bytes():
    from golden_examples import load_container

    f, head = load_container()
    got = lecb.lecb_container_write_header(f["n"], f["chunk"], f["max_len"], f["len_hi"], f["len_lo"],
                                           f["bytes_hi"], f["bytes_lo"])
    assert np.array_equal(got, head)
    back = lecb.lecb_container_read_header(head)
    assert (back["n"], back["bytes_hi"], back["bytes_lo"]) == (f["n"], f["bytes_hi"], f["bytes_lo"])
    assert np.array_equal(back["len_hi"], f["len_hi"]) and np.array_equal(back["len_lo"], f["len_lo"])


def test_container_header_matches_oracle():
    x = np.random.default_rng(3).integers(0, 65536, 5000, dtype=np.uint16)
    enc = oracle.encode_bf16(x, 4096)
    ref = oracle.container_bytes(enc)[: lecb.CONTAINER_HEADER_BYTES]
    got = lecb.lecb_container_write_header(x.size, 4096, 16, enc["len_hi"], enc["len_lo"],
                                           enc["stream_hi"].size, enc["stream_lo"].size)
    assert np.array_equal(got, ref)
    back = lecb.lecb_container_read_header(got)
    assert back["n"] == x.size and back["bytes_lo"] == enc["stream_lo"].size
    assert np.array_equal(back["len_hi"], enc["len_hi"])


def test_stream_stats_match_oracle():
    import workloads

    x = workloads.int8_fixed(0)
    warm = np.sum([oracle.histogram(workloads.int8_fixed(r)) for r in (1, 2, 3, 4)], axis=0, dtype=np.uint64)
    ln = oracle.package_merge_lengths(oracle.codebook_frequencies([warm], 1), 16)
    h = oracle.histogram(x)
    st = lecb.lecb_stream_stats(h, ln, 16)
    assert st["n"] == x.size and st["uncoded"] == 0
    assert st["payload_bits"] == oracle.payload_bits_identity(h, ln)
    assert st["optimal_bits"] == oracle.per_batch_optimal_bits(h, 16)
    assert abs(st["shannon_bits"] - oracle.metrics.shannon_bits(h)) < 1e-6 * st["shannon_bits"]
    ln2 = ln.copy()
    ln2[int(np.argmax(h))] = 0
    assert lecb.lecb_stream_stats(h, ln2, 16)["uncoded"] == int(h.max())


def test_drift_check_matches_oracle():
    """The C refresh rule takes the oracle's decision, bits and lengths on a
    drifting sequence of int8 batches and on hand-made edge cases."""
    rng = np.random.default_rng(11)
    hists = []
    for k in range(10):
        x = np.clip(np.rint(rng.normal(0, 6 + 5 * k, 40_000)), -128, 127).astype(np.int8).view(np.uint8)
        hists.append(oracle.histogram(x))
    first = oracle.package_merge_lengths(oracle.codebook_frequencies(hists[:1], 1), 16)
    for tol in (0, 5_000, 50_000, 10**9):
        cur_o = first
        cur_c = lecb.lecb_codebook_from_lengths(first)
        cur_c.max_len = 16
        for h in hists:
            r_o, use_o, bc_o, bo_o = oracle.drift_check(h, cur_o, 16, tol)
            r_c, use_c, bc_c, bo_c = lecb.lecb_drift_check(h, cur_c, 16, tol)
            assert (r_c, bc_c, bo_c) == (r_o, bc_o, bo_o)
            assert np.array_equal(use_c.lengths(), use_o)
            cur_o, cur_c = use_o, use_c
    # uncodable byte
    cur = np.full(256, 8, np.uint8)
    cur[5], cur[6] = 0, 7
    h = np.full(256, 3, np.uint64)
    r, use, bc, bo = lecb.lecb_drift_check(h, lecb.lecb_codebook_from_lengths(cur), 16, 10**9)
    assert r and bc is None and use.lengths()[5] > 0
    # exact boundary: a dominant byte against an all-8-bit code costs 8x the optimum
    h = np.zeros(256, np.uint64)
    h[0] = 10_000
    u8 = lecb.lecb_codebook_from_lengths(np.full(256, 8, np.uint8))
    assert lecb.lecb_drift_check(h, u8, 16, 6_999_999)[0]
    assert not lecb.lecb_drift_check(h, u8, 16, 7_000_000)[0]
