"""Pins of the oracle's stream format, encoders and decoders (CPU only)."""

import numpy as np
import pytest

import oracle
from oracle.huffman import package_merge_lengths, canonical_codes
from oracle.stream import encode, encode_bitstring, decode, decode_bitwise, CorruptStream, UncodedSymbol
from golden_examples import load as load_golden
import workloads


def _codebook(x, clamp=False, max_len=16):
    h = oracle.histogram(x)
    if clamp:
        h = np.maximum(h, 1)
    ln = package_merge_lengths(h, max_len)
    return ln, canonical_codes(ln)


CASES = [
    # (name, n, chunk, generator)
    ("empty", 0, 256, lambda n: np.zeros(0, np.uint8)),
    ("one", 1, 256, lambda n: np.array([200], np.uint8)),
    ("lt_chunk", 100, 256, lambda n: workloads.uniform_bytes(1, n)),
    ("ragged", 3 * 256 + 17, 256, lambda n: workloads.skewed_bytes(2, n)),
    ("exact", 4 * 1024, 1024, lambda n: workloads.uniform_bytes(3, n, 5)),
    ("all_equal", 2000, 512, lambda n: np.full(n, 9, np.uint8)),
    ("two_syms", 1500, 256, lambda n: workloads.uniform_bytes(4, n, 2)),
    ("gauss", 5000, 4096, lambda n: workloads.q8(np.random.default_rng(9).normal(0, 20, n))),
]


@pytest.mark.parametrize("name,n,chunk,gen", CASES, ids=[c[0] for c in CASES])
def test_two_encoders_and_two_decoders_agree(name, n, chunk, gen):
    x = gen(n)
    ln, cd = _codebook(x, clamp=(name == "gauss"))
    s1, b1 = encode_bitstring(x, ln, cd, chunk)
    s2, b2 = encode(x, ln, cd, chunk)
    assert np.array_equal(s1, s2) and b1 == b2
    assert b1 == oracle.payload_bits_identity(oracle.histogram(x), ln)
    assert s1.size == oracle.header_bytes(n, chunk) + 4 * int(oracle.chunk_word_counts(x, ln, chunk).sum())
    assert s1.size <= oracle.encoded_bound(n, chunk, 16)
    y1 = decode_bitwise(s1, ln, chunk, n)
    y2 = decode(s1, ln, chunk, n)
    assert np.array_equal(y1, x) and np.array_equal(y2, x)


def test_uniform_code_closed_form_byteswap():
    # All 256 lengths 8 -> code[s] = s; each payload word holds 4 input bytes MSB first,
    # so the payload is the input with every aligned 4-byte group reversed.
    x = workloads.uniform_bytes(5, 4096 * 3)
    ln = np.full(256, 8, np.uint8)
    s, bits = encode(x, ln, canonical_codes(ln), 4096)
    tb = oracle.header_bytes(x.size, 4096)
    assert bits == 8 * x.size
    assert np.array_equal(s[tb:], x.view(">u4").astype("<u4").view(np.uint8))
    assert list(s[:12].view("<u4")) == [1024, 2048, 3072]


def test_golden_streams():
    for ex in load_golden():
        if "input" not in ex:
            continue
        ln = package_merge_lengths(ex["freq"], ex["max_len"])
        cd = canonical_codes(ln)
        for enc in (encode_bitstring, encode):
            s, bits = enc(ex["input"], ln, cd, ex["chunk"])
            assert np.array_equal(s, ex["stream"]), (ex["name"], enc.__name__, s)
            assert bits == ex["payload_bits"]
        for dec in (decode_bitwise, decode):
            assert np.array_equal(dec(ex["stream"], ln, ex["chunk"], ex["input"].size), ex["input"])


def test_long_codes_and_boundary_straddling():
    # A codebook with 16-bit codes: many words straddle, exercises the split path.
    f = np.array([max(1, (1 << 30) >> s) for s in range(256)], np.uint64)
    ln = package_merge_lengths(f, 16)
    assert int(ln.max()) == 16
    cd = canonical_codes(ln)
    x = workloads.uniform_bytes(8, 3000)
    s1, _ = encode_bitstring(x, ln, cd, 1024)
    s2, _ = encode(x, ln, cd, 1024)
    assert np.array_equal(s1, s2)
    assert np.array_equal(decode(s2, ln, 1024, x.size), x)


def test_uncoded_symbol_raises():
    x = np.array([1, 2, 3], np.uint8)
    ln = np.zeros(256, np.uint8)
    ln[1] = ln[2] = 1
    with pytest.raises(UncodedSymbol):
        encode(x, ln, canonical_codes(ln), 256)
    with pytest.raises(UncodedSymbol):
        encode_bitstring(x, ln, canonical_codes(ln), 256)


def _corruptions():
    x = workloads.skewed_bytes(10, 5000)
    ln, cd = _codebook(x)
    s, _ = encode(x, ln, cd, 1024)
    return x, ln, s


def test_corrupt_streams_detected():
    x, ln, s = _corruptions()
    n, chunk = x.size, 1024
    tb = oracle.header_bytes(n, chunk)
    gb = oracle.table_bytes(n, chunk)
    bad = []
    t = s.copy(); t[0:4] = np.array([0, 0, 0, 0], np.uint8); bad.append(("zero end", t))
    t = s.copy(); e = t[:20].view("<u4").copy(); e[1], e[2] = e[2], e[1]; t[:20] = e.view(np.uint8); bad.append(("non-monotone", t))
    bad.append(("truncated", s[:-4].copy()))
    bad.append(("extra word", np.concatenate([s, np.zeros(4, np.uint8)])))
    t = s.copy(); t[4 * 5] = 1; bad.append(("table padding", t))
    # flip the lowest bit of chunk 0's last word: it is padding (chunk 0 ends mid-word by construction below)
    ends = s[:4 * 5].view("<u4")
    bits0 = int(oracle.stream.chunk_bit_counts(x[:chunk], ln, chunk)[0])
    if bits0 % 32:
        t = s.copy(); off = tb + 4 * (int(ends[0]) - 1); t[off] |= 1; bad.append(("padding bit", t))
    # gap section: chunk 0 has K = 4 units; change the gap of unit 1, then its padding nibble area
    t = s.copy(); t[gb] ^= 0x10; bad.append(("gap value", t))
    t = s.copy(); t[tb - 1] = 0x01; bad.append(("gap padding", t))
    for name, t in bad:
        with pytest.raises(CorruptStream):
            decode(t, ln, chunk, n)
        with pytest.raises(CorruptStream):
            decode_bitwise(t, ln, chunk, n)


def test_incomplete_code_rejects_unmatched_prefix():
    ln = np.zeros(256, np.uint8)
    ln[7] = 1  # only code word is "0"
    s = np.zeros(36, np.uint8)
    s[0] = 1
    s[35] = 0x80  # first payload bit is 1: no code word matches
    with pytest.raises(CorruptStream):
        decode(s, ln, 4096, 3)
    with pytest.raises(CorruptStream):
        decode_bitwise(s, ln, 4096, 3)


def test_chunks_are_independent():
    # The payload of chunk c depends only on chunk c's bytes: encoding a chunk alone
    # gives the same words as its slice of the whole stream.
    x = workloads.skewed_bytes(12, 10 * 512 + 33, sigma=30)
    ln, cd = _codebook(x)
    s, _ = encode(x, ln, cd, 512)
    nc = oracle.num_chunks(x.size, 512)
    tb = oracle.header_bytes(x.size, 512)
    gb = oracle.table_bytes(x.size, 512)
    ends = s[:4 * nc].view("<u4").astype(np.int64)
    starts = np.concatenate([[0], ends[:-1]])
    for c in range(nc):
        one, _ = encode(x[c * 512:(c + 1) * 512], ln, cd, 512)
        assert np.array_equal(one[32:], s[tb + 4 * starts[c]: tb + 4 * ends[c]])
        assert one[16] == s[gb + c]  # K = 2 nibbles per chunk = one gap byte per chunk


def test_gaps_point_at_code_word_starts():
    # Every nonzero gap lands on a code-word start (or the data end) that is not word-aligned.
    x = workloads.skewed_bytes(13, 20 * 4096 + 100, sigma=25)
    ln, cd = _codebook(x)
    s, _ = encode(x, ln, cd, 4096)
    starts, ends, gaps, payload = oracle.parse_table(s, x.size, 4096)
    assert gaps.shape == (21, 16) and np.all(gaps[:, 0] == 0) and gaps.max() <= 15
    assert (gaps > 0).mean() > 0.5  # most unit boundaries fall inside a code word
    for c in range(starts.size):
        lens = ln[x[c * 4096:(c + 1) * 4096]].astype(np.int64)
        bnd = set(np.concatenate([[0], np.cumsum(lens)]).tolist())
        for j, w in enumerate(oracle.stream.unit_starts(int(ends[c] - starts[c]), 4096)):
            p = 32 * int(w) + int(gaps[c, j])
            assert p in bnd
            assert not any(q in bnd for q in range(32 * int(w), p))
