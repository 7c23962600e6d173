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


def test_uniform_code_closed_form_block_transpose():
    # All 256 lengths 8 -> code[s] = s, so every word holds 4 input bytes MSB first
    # (the aligned 4-byte group reversed).  Chunk 4096 -> 16 lanes of 256 bytes; every
    # pair takes 16 bits, so each lane reads word k >= 2 before pair 2(k-1) and all
    # lanes read in step: the chunk's payload is word k of lanes 0..15, k = 0..63.
    # Lane j's word k is word k%4 of block (k//4)*16 + j, so the payload is the
    # chunk's byte-reversed words with the block index and the word-in-lane swapped.
    x = workloads.uniform_bytes(5, 4096 * 3)
    ln = np.full(256, 8, np.uint8)
    s, bits = encode(x, ln, canonical_codes(ln), 4096)
    tb = oracle.header_bytes(x.size, 4096)
    assert bits == 8 * x.size
    natural = x.view(">u4").astype(np.int64).reshape(3, 16, 16, 4)   # chunk, block row, lane, word
    k, j = np.meshgrid(np.arange(64), np.arange(16), indexing="ij")
    want = natural[:, k // 4, j, k % 4]                               # chunk, k, j
    assert np.array_equal(s[tb:].view("<u4").astype(np.int64), want.ravel())
    assert list(s[:12].view("<u4")) == [1024, 2048, 3072]
    assert np.all(s[16:16 + 3 * 32].view("<u2") == 64)               # 64 words per lane


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
    n, chunk = x.size, 1024            # 5 chunks of 4 lanes, the last one 904 symbols
    tb = oracle.header_bytes(n, chunk)
    gb = oracle.table_bytes(n, chunk)
    bad = []
    t = s.copy(); t[0:4] = np.array([0, 0, 0, 0], np.uint8); bad.append(("zero end", t))
    t = s.copy(); e = t[:20].view("<u4").copy(); e[1], e[2] = e[2], e[1]; t[:20] = e.view(np.uint8); bad.append(("non-monotone", t))
    bad.append(("truncated", s[:-4].copy()))
    bad.append(("extra word", np.concatenate([s, np.zeros(4, np.uint8)])))
    t = s.copy(); t[4 * 5] = 1; bad.append(("table padding", t))
    # word counts: move one word from lane 0 to lane 1 of chunk 0 (same chunk total)
    t = s.copy(); u = t[gb:gb + 4].view("<u2").copy(); u[0] -= 1; u[1] += 1
    t[gb:gb + 4] = u.view(np.uint8); bad.append(("word count moved", t))
    # one word more for lane 0 and one less in the chunk's last word ... the totals disagree
    t = s.copy(); u = t[gb:gb + 2].view("<u2").copy(); u[0] += 1
    t[gb:gb + 2] = u.view(np.uint8); bad.append(("word count total", t))
    t = s.copy(); t[tb - 1] = 0x01; bad.append(("word count padding", t))
    for name, t in bad:
        with pytest.raises(CorruptStream):
            decode(t, ln, chunk, n)
        with pytest.raises(CorruptStream):
            decode_bitwise(t, ln, chunk, n)


def test_corrupt_padding_and_empty_lanes():
    # Golden B7 (chunk 512, 2 lanes): lane 1's last word is 16 zero code bits and 16
    # bits of padding, and it is the chunk's last word; its lowest bit is padding.
    ex = next(e for e in load_golden() if e["name"].startswith("B7"))
    ln, n, s = ex["lengths"], ex["input"].size, ex["stream"]
    t = s.copy(); t[-4] |= 1
    # B6 (chunk 1024, 300 symbols): lane 3 of 4 holds 64 symbols; give it no words and
    # lane 2 one more (same total) -> a lane with symbols and no words
    b6 = next(e for e in load_golden() if e["name"].startswith("B6"))
    u = b6["stream"].copy(); u[16 + 4] += 1; u[16 + 6] = 0
    # a chunk of 300 symbols at chunk 4096 has lanes 1..15 empty: B1-like stream with a
    # word moved to an empty lane
    b1 = next(e for e in load_golden() if e["name"] == "B1 no ties, one chunk")
    v = b1["stream"].copy(); v[16] = 0; v[18] = 1
    for stream, lens, nn, ch in ((t, ln, n, ex["chunk"]), (u, b6["lengths"], 300, 1024),
                                 (v, b1["lengths"], b1["input"].size, 4096)):
        with pytest.raises(CorruptStream):
            decode(stream, lens, ch, nn)
        with pytest.raises(CorruptStream):
            decode_bitwise(stream, lens, ch, nn)


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
    # gives the same words and unit counts as its slice of the whole stream.
    x = workloads.skewed_bytes(12, 10 * 512 + 33, sigma=30)
    ln, cd = _codebook(x)
    s, _ = encode(x, ln, cd, 512)
    nc = oracle.num_chunks(x.size, 512)
    tb = oracle.header_bytes(x.size, 512)
    ends = s[:4 * nc].view("<u4").astype(np.int64)
    starts = np.concatenate([[0], ends[:-1]])
    for c in range(nc):
        piece = x[c * 512:(c + 1) * 512]
        one, _ = encode(piece, ln, cd, 512)
        assert np.array_equal(one[32:], s[tb + 4 * starts[c]: tb + 4 * ends[c]])
        a, b = oracle.count_span(x.size, 512, c, c + 1)
        a1, b1 = oracle.count_span(piece.size, 512, 0, 1)
        assert np.array_equal(one[a1:b1], s[a:b])  # G = 2 counts per chunk


def test_lane_counts_are_the_lanes_words():
    # Block b (16 symbols) of chunk c belongs to lane b mod 16 (chunk 4096); a lane's
    # count is ceil(sum of its code lengths / 32).  Checked with explicit loops over
    # the blocks, independently of the encoder's sorting.
    n, chunk = 20 * 4096 + 100, 4096
    x = workloads.skewed_bytes(13, n, sigma=25)
    ln, cd = _codebook(x)
    s, bits = encode(x, ln, cd, chunk)
    starts, ends, counts, payload = oracle.parse_table(s, n, chunk)
    assert counts.shape == (21, 16)
    lens = ln[x].astype(np.int64)
    lane_bits = np.zeros((21, 16), np.int64)
    for c in range(21):
        for b in range(0, min(chunk, n - c * chunk), 16):
            lane_bits[c, (b // 16) % 16] += lens[c * chunk + b: min(c * chunk + b + 16, n)].sum()
    assert np.array_equal(counts, (lane_bits + 31) // 32)
    assert lane_bits.sum() == bits
    assert np.array_equal(ends - starts, counts.sum(axis=1))
    # the last chunk's 100 symbols: blocks 0..5 full and 4 symbols in block 6 -> lanes 0..6
    assert np.array_equal(oracle.lane_symbol_counts(n, chunk)[20], [16] * 6 + [4] + [0] * 9)
    assert np.all(counts[20, 7:] == 0) and np.all(counts[20, :7] > 0)


@pytest.mark.parametrize("n,chunk,L", [(1000003, 4096, 16), (5000, 1024, 9), (300, 256, 12), (65536 * 2 + 7, 65536, 16)])
def test_encoded_bound_is_reached(n, chunk, L):
    # The bound is the size of the stream in which every symbol has an L-bit code
    # word (rounded up to 16 bytes): a codebook with an L-bit code and an input made
    # of that symbol reaches it; no stream of a code with lengths <= L exceeds it.
    f = np.array([max(1, (1 << 40) >> min(s, 39)) for s in range(256)], np.uint64)
    ln = package_merge_lengths(f, L)
    assert int(ln.max()) == L
    sym = int(np.argmax(ln))
    x = np.full(n, sym, np.uint8)
    s, bits = encode(x, ln, canonical_codes(ln), chunk)
    assert bits == L * n
    assert oracle.encoded_bound(n, chunk, L) == (s.size + 15) // 16 * 16
    y = workloads.uniform_bytes(14, n)
    assert encode(y, ln, canonical_codes(ln), chunk)[0].size <= oracle.encoded_bound(n, chunk, L)


def test_encoded_bound_hand_value():
    # n = 1000003, chunk 4096, L = 16: nc = 245 chunks (244 full + 579 symbols);
    # table align16(980) = 992 bytes; unit counts 245 * 16 * 2 = 7840 bytes
    # (already a multiple of 16); words 244 * 4096*16/32 + ceil(579*16/32) =
    # 499712 + 290 = 500002 -> 2000008 bytes; 992 + 7840 + 2000008 = 2008840
    # = 125552 * 16 + 8, rounded up to 2008848.
    assert oracle.encoded_bound(1000003, 4096, 16) == 2008848
    # chunk 256, L = 9, n = 1000: nc = 4 (3 full + 232); table 16; counts 4*1*2 = 8 -> 16;
    # words 3 * ceil(256*9/32) + ceil(232*9/32) = 3*72 + 66 = 282 -> 1128; 16 + 16 + 1128
    # = 1160 = 72 * 16 + 8, rounded up to 1168.
    assert oracle.encoded_bound(1000, 256, 9) == 1168
    # chunk 4096, L = 3, n = 4136: chunk 0 = 16 lanes x 256 x 3 bits = 24 words each
    # (384); chunk 1 = 40 symbols = blocks 0, 1 (16 each, lanes 0 and 1: 48 bits -> 2
    # words) and block 2 (8 symbols, lane 2: 24 bits -> 1 word) = 5 words (a per-chunk
    # rounding would give ceil(120/32) = 4).  389 words = 1556 bytes; table 16, counts
    # 2*16*2 = 64: 1636 -> 1648.
    assert oracle.encoded_bound(4136, 4096, 3) == 1648
