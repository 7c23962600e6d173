"""Oracle: the chunked Huffman stream -- format, two encoders, two decoders.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

Page basis
----------
* "Single-Stage Huffman Encoder for ML Compression", Methodology step 4: every
  tensor is coded directly with a codebook computed beforehand, with no
  per-tensor analysis and no codebook in the stream.
* "Lossless Compression for LLM Tensor Incremental Snapshots", Technical
  framework: Huffman coding of the byte groups and the reverse path (read,
  Huffman-decode, restore the byte groups); Key design item 3: the work is cut
  into independent tasks that run in parallel.

The pages fix no stream layout.  Reading (stream format v1), chosen before any
kernel and followed bit for bit by the library:

* ``n`` symbols are cut into ``nc = ceil(n / chunk)`` chunks; chunk c holds
  symbols ``[c*chunk, min((c+1)*chunk, n))`` -- the independent work unit;
* a chunk's bits are its symbols' code words concatenated in order, MOST
  significant bit first, starting at bit 31 of a fresh 32-bit word and filling
  downwards; the chunk's last word is zero-padded; words are stored
  little-endian; chunks follow each other with no gap;
* decode units: a chunk of Wc payload words is cut at K = max(1, chunk // 256)
  word-aligned bit positions s_j = 32 * floor(j * Wc / K), j = 0..K-1; the
  GAP of unit j is the distance in bits from s_j to the first code-word
  boundary at or after s_j (boundaries = code-word starts and the end of the
  chunk's data); it is always 0..15 because no code word exceeds 16 bits.
  The gaps let a decoder start K independent decoders per chunk at exact
  code-word starts (the "gap array" of Yamamoto et al., 2020 -- prior art, not
  on the pages; the pages' Key design item 3 asks for independent parallel
  tasks);
* stream = ``u32 end[nc]`` (end[c] = index, counted in payload words, one past
  chunk c's last word; chunk c spans words [end[c-1], end[c]) with
  end[-1] = 0) || zero bytes up to a 16-byte boundary || gap nibbles
  (nibble i = c*K + j is the low half of byte i//2 when i is even, the high
  half when odd) || zero bytes up to a 16-byte boundary || ``u32 payload[W]``
  with W = end[nc-1];
  size = align16(4*nc) + align16(ceil(nc*K/2)) + 4*W;  n = 0 -> empty stream;
* nothing else is stored: chunk size, n and the codebook travel outside
  (the fixed codebook is never transmitted, per Methodology step 4).
"""

from __future__ import annotations

import numpy as np

NSYM = 256


class OracleError(Exception):
    """Base class of the oracle's coding errors."""


class CorruptStream(OracleError):
    """The stream cannot be the output of ``encode`` for these arguments."""


class UncodedSymbol(OracleError):
    """The input holds a byte value that has no code word (length 0)."""


def _align16(x: int) -> int:
    return (x + 15) // 16 * 16


def num_chunks(n: int, chunk: int) -> int:
    return -(-int(n) // int(chunk))


def units_per_chunk(chunk: int) -> int:
    return max(1, int(chunk) // 256)


def table_bytes(n: int, chunk: int) -> int:
    return _align16(4 * num_chunks(n, chunk))


def gap_bytes(n: int, chunk: int) -> int:
    return _align16(-(-num_chunks(n, chunk) * units_per_chunk(chunk) // 2))


def header_bytes(n: int, chunk: int) -> int:
    """Bytes before the payload: offset table and gap nibbles, each padded to 16 bytes."""
    return table_bytes(n, chunk) + gap_bytes(n, chunk)


def unit_meta_span(n: int, chunk: int, c0: int, c1: int):
    """Byte range [a, b) of the stream that holds the per-unit metadata of chunks
    [c0, c1) (unit j of chunk c is entry c*K + j); the range must cover whole bytes."""
    K = units_per_chunk(chunk)
    if (c0 * K) % 2 or (c1 * K) % 2:
        raise ValueError("these chunks do not cover whole bytes of gap nibbles")
    tb = table_bytes(n, chunk)
    return tb + c0 * K // 2, tb + c1 * K // 2


def encoded_bound(n: int, chunk: int, max_len: int = 16) -> int:
    """Largest possible stream size (every symbol at max_len bits plus one padding word per
    chunk), rounded up to a multiple of 16 bytes."""
    nc = num_chunks(n, chunk)
    if nc == 0:
        return 0
    return _align16(header_bytes(n, chunk) + 4 * (-(-int(n) * int(max_len) // 32) + nc))


def unit_starts(words: int, chunk: int) -> np.ndarray:
    """Word index of each decode-unit boundary of a chunk with ``words`` payload words."""
    K = units_per_chunk(chunk)
    return (np.arange(K, dtype=np.int64) * int(words)) // K


def _gap_of(boundaries, s):
    """First element of the sorted ``boundaries`` at or after bit s, minus s."""
    i = int(np.searchsorted(boundaries, s, side="left"))
    return int(boundaries[i]) - s


def _pack_nibbles(gaps: np.ndarray, nbytes: int) -> np.ndarray:
    g = np.zeros(2 * nbytes, dtype=np.uint8)
    g[: gaps.size] = gaps
    return (g[0::2] | (g[1::2] << 4)).astype(np.uint8)


def _unpack_nibbles(raw: np.ndarray) -> np.ndarray:
    out = np.empty(2 * raw.size, dtype=np.uint8)
    out[0::2] = raw & 0xF
    out[1::2] = raw >> 4
    return out


def _check_args(sym, lengths, chunk):
    sym = np.ascontiguousarray(sym).view(np.uint8).ravel()
    lengths = np.asarray(lengths, dtype=np.int64).ravel()
    if lengths.shape != (NSYM,):
        raise ValueError("lengths must have 256 entries")
    if chunk <= 0:
        raise ValueError("chunk must be positive")
    return sym, lengths


# --------------------------------------------------------------------------
# encoder (i): the definition, one character per bit.  Small inputs only.
# --------------------------------------------------------------------------

def _assemble(n, chunk, ends, gaps, payload_words):
    nc = num_chunks(n, chunk)
    table = np.zeros(table_bytes(n, chunk) // 4, dtype="<u4")
    table[:nc] = ends
    gap = _pack_nibbles(np.asarray(gaps, dtype=np.uint8), gap_bytes(n, chunk))
    payload = np.asarray(payload_words, dtype=np.uint64).astype("<u4")
    return np.concatenate([table.view(np.uint8), gap, payload.view(np.uint8)])


def encode_bitstring(sym, lengths, codes, chunk: int):
    """Encode by writing every code word as a '0'/'1' string (the definition).

    Returns (stream bytes as uint8 array, payload_bits).
    """
    sym, lengths = _check_args(sym, lengths, chunk)
    codes = np.asarray(codes, dtype=np.int64).ravel()
    n = sym.size
    nc = num_chunks(n, chunk)
    if nc == 0:
        return np.zeros(0, dtype=np.uint8), 0
    words, ends, gaps = [], [], []
    payload_bits = 0
    for c in range(nc):
        parts = []
        for s in sym[c * chunk: min((c + 1) * chunk, n)]:
            ln = int(lengths[s])
            if ln == 0:
                raise UncodedSymbol(f"byte {int(s)} has no code")
            parts.append(format(int(codes[s]), f"0{ln}b"))
        bits = "".join(parts)
        payload_bits += len(bits)
        boundaries = [0]
        for part in parts:
            boundaries.append(boundaries[-1] + len(part))  # starts of the next word, then the data end
        bits += "0" * (-len(bits) % 32)
        nwords = len(bits) // 32
        for w in unit_starts(nwords, chunk):
            s_j = 32 * int(w)
            gaps.append(min(b for b in boundaries if b >= s_j) - s_j)
        for i in range(0, len(bits), 32):
            words.append(int(bits[i:i + 32], 2))
        ends.append(len(words))
    if len(words) >= 1 << 32:
        raise OverflowError("payload too large for 32-bit word offsets")
    return _assemble(n, chunk, ends, gaps, words), payload_bits


# --------------------------------------------------------------------------
# encoder (ii): vectorised numpy, blocks of whole chunks.
# --------------------------------------------------------------------------

def chunk_bit_counts(sym, lengths, chunk: int) -> np.ndarray:
    """bits[c] = sum of the code lengths of chunk c's symbols (int64[nc])."""
    sym, lengths = _check_args(sym, lengths, chunk)
    n = sym.size
    nc = num_chunks(n, chunk)
    bits = np.zeros(nc, dtype=np.int64)
    block = max(1, (1 << 22) // chunk) * chunk
    for start in range(0, n, block):
        ln = lengths[sym[start:start + block]]
        if np.any(ln == 0):
            bad = int(sym[start:start + block][np.argmax(ln == 0)])
            raise UncodedSymbol(f"byte {bad} has no code")
        c0 = start // chunk
        idx = np.arange(ln.size, dtype=np.int64) // chunk
        bits[c0:c0 + idx[-1] + 1] = np.bincount(idx, weights=ln).astype(np.int64)
    return bits


def chunk_word_counts(sym, lengths, chunk: int) -> np.ndarray:
    """words[c] = ceil(bits[c] / 32): payload words chunk c occupies."""
    return (chunk_bit_counts(sym, lengths, chunk) + 31) // 32


def encode(sym, lengths, codes, chunk: int):
    """Vectorised encoder.  Returns (stream bytes as uint8 array, payload_bits).

    For every symbol i of chunk c: g = 32*start_word(c) + (bits of the chunk's
    earlier symbols); its code word goes to word g>>5 starting (MSB-first) at
    bit 31-(g&31), spilling into the next word when it crosses the boundary.
    Fields of distinct symbols are disjoint, so each word is the plain SUM of
    its fields; sums stay below 2^32 and are exact in float64 bincount.
    Gaps: for each unit boundary S (global bit), the first code-word start at
    or after S inside the same chunk, else the chunk's data end.
    """
    sym, lengths = _check_args(sym, lengths, chunk)
    codes = np.asarray(codes, dtype=np.int64).ravel()
    n = sym.size
    nc = num_chunks(n, chunk)
    if nc == 0:
        return np.zeros(0, dtype=np.uint8), 0
    K = units_per_chunk(chunk)
    bits = chunk_bit_counts(sym, lengths, chunk)
    words = (bits + 31) // 32
    ends = np.cumsum(words)
    W = int(ends[-1])
    if W >= 1 << 32:
        raise OverflowError("payload too large for 32-bit word offsets")
    starts = ends - words
    data_end = 32 * starts + bits  # global bit just past each chunk's last code word
    unit_bit = 32 * (starts[:, None] + (np.arange(K, dtype=np.int64)[None, :] * words[:, None]) // K)
    gaps = np.full((nc, K), -1, dtype=np.int64)
    payload = np.zeros(W + 1, dtype=np.float64)
    block = max(1, (1 << 22) // chunk) * chunk
    for start in range(0, n, block):
        s = sym[start:start + block]
        ln = lengths[s]
        cd = codes[s]
        cid = (start + np.arange(s.size, dtype=np.int64)) // chunk
        incl = np.cumsum(ln)
        excl = incl - ln
        first = np.searchsorted(cid, cid, side="left")  # index of each chunk's first symbol in the block
        pos = excl - excl[first]
        g = 32 * starts[cid] + pos
        w = g >> 5
        b = g & 31
        shift = 32 - b - ln
        fits = shift >= 0
        hi = np.where(fits, cd << np.maximum(shift, 0), cd >> np.maximum(-shift, 0))
        lo = np.where(fits, 0, (cd << np.maximum(32 + shift, 0)) & 0xFFFFFFFF)
        payload += np.bincount(w, weights=hi.astype(np.float64), minlength=W + 1)
        payload += np.bincount(w + 1, weights=lo.astype(np.float64), minlength=W + 2)[: W + 1]
        # gaps of the unit boundaries of this block's chunks
        c0, c1 = int(cid[0]), int(cid[-1]) + 1
        S = unit_bit[c0:c1]
        i = np.searchsorted(g, S.ravel(), side="left").reshape(S.shape)
        inside = (i < g.size)
        inside[inside] &= cid[i[inside]] == np.arange(c0, c1)[:, None].repeat(K, 1)[inside]
        nxt = np.where(inside, g[np.minimum(i, g.size - 1)], data_end[c0:c1, None])
        gaps[c0:c1] = nxt - S
    assert np.all((gaps >= 0) & (gaps <= 15))
    payload = payload[:W].astype(np.uint64)
    assert np.all(payload < (1 << 32))
    return _assemble(n, chunk, ends, gaps.ravel(), payload), int(bits.sum())


# --------------------------------------------------------------------------
# decoding
# --------------------------------------------------------------------------

def parse_table(stream, n: int, chunk: int):
    """Validate the layout; return (starts, ends, gaps[nc, K], payload words as uint64)."""
    stream = np.ascontiguousarray(stream).view(np.uint8).ravel()
    nc = num_chunks(n, chunk)
    K = units_per_chunk(chunk)
    if nc == 0:
        if stream.size != 0:
            raise CorruptStream("non-empty stream for n = 0")
        z = np.zeros(0, np.int64)
        return z, z, np.zeros((0, K), np.int64), np.zeros(0, np.uint64)
    tb = table_bytes(n, chunk)
    hb = header_bytes(n, chunk)
    if stream.size < hb or (stream.size - hb) % 4:
        raise CorruptStream("stream shorter than its header or not whole words")
    ends = stream[: 4 * nc].view("<u4").astype(np.int64)
    if np.any(stream[4 * nc: tb] != 0):
        raise CorruptStream("non-zero table padding")
    nib = _unpack_nibbles(stream[tb:hb])
    if np.any(nib[nc * K:] != 0):
        raise CorruptStream("non-zero gap padding")
    gaps = nib[: nc * K].astype(np.int64).reshape(nc, K)
    W = (stream.size - hb) // 4
    starts = np.concatenate([[0], ends[:-1]])
    if np.any(ends <= starts):
        raise CorruptStream("offset table not strictly increasing")
    if int(ends[-1]) != W:
        raise CorruptStream("offset table disagrees with the stream size")
    payload = stream[hb:].view("<u4").astype(np.uint64)
    return starts, ends, gaps, payload


def _check_gaps(starts, ends, gaps, boundary_lists, chunk):
    """Every stored gap must equal the distance to the first boundary at or after its unit start."""
    for c in range(starts.size):
        b = np.asarray(boundary_lists[c], dtype=np.int64)
        for j, w in enumerate(unit_starts(int(ends[c] - starts[c]), chunk)):
            if _gap_of(b, 32 * int(w)) != int(gaps[c, j]):
                raise CorruptStream("gap disagrees with the code-word boundaries")


def _canonical_tables(lengths):
    """first_code, count per length and the symbols in canonical order."""
    lengths = np.asarray(lengths, dtype=np.int64).ravel()
    order = sorted((int(lengths[s]), s) for s in range(NSYM) if lengths[s] > 0)
    count = [0] * 17
    for ln, _ in order:
        count[ln] += 1
    first = [0] * 17
    index = [0] * 17
    code = 0
    idx = 0
    for ln in range(1, 17):
        code <<= 1
        first[ln] = code
        index[ln] = idx
        code += count[ln]
        idx += count[ln]
    return first, count, index, [s for _, s in order]


def decode_bitwise(stream, lengths, chunk: int, n: int) -> np.ndarray:
    """Decoder (i): canonical prefix matching one bit at a time.  Small inputs only.

    A code word of length l is recognised when the l bits read so far, as an
    integer v, satisfy first[l] <= v < first[l] + count[l]; its symbol is the
    (v - first[l])-th symbol of length l in canonical order.
    """
    lengths = np.asarray(lengths, dtype=np.int64).ravel()
    starts, ends, gaps, payload = parse_table(stream, n, chunk)
    first, count, index, syms = _canonical_tables(lengths)
    out = np.zeros(n, dtype=np.uint8)
    boundary_lists = []
    for c in range(starts.size):
        words = payload[starts[c]:ends[c]]
        bitstr = "".join(format(int(w), "032b") for w in words)
        p = 0
        bl = [0]
        for k in range(min(chunk, n - c * chunk)):
            v = 0
            ln = 0
            while True:
                if p >= len(bitstr):
                    raise CorruptStream("code word runs past the end of its chunk")
                v = (v << 1) | (bitstr[p] == "1")
                p += 1
                ln += 1
                if ln > 16:
                    raise CorruptStream("no code word matches")
                if count[ln] and first[ln] <= v < first[ln] + count[ln]:
                    out[c * chunk + k] = syms[index[ln] + v - first[ln]]
                    break
            bl.append(p)
        if (len(bitstr) - p) >= 32:
            raise CorruptStream("chunk holds more words than its symbols need")
        if "1" in bitstr[p:]:
            raise CorruptStream("non-zero padding after the last code word")
        boundary_lists.append(bl)
    _check_gaps(starts, ends, gaps, boundary_lists, chunk)
    return out


def _lookup_table(lengths, codes):
    """65536-entry table indexed by the next 16 bits: (symbol, length); length 0 = no code word."""
    lengths = np.asarray(lengths, dtype=np.int64).ravel()
    codes = np.asarray(codes, dtype=np.int64).ravel()
    sym_of = np.zeros(1 << 16, dtype=np.uint8)
    len_of = np.zeros(1 << 16, dtype=np.int64)
    for s in range(NSYM):
        ln = int(lengths[s])
        if ln:
            lo = int(codes[s]) << (16 - ln)
            hi = (int(codes[s]) + 1) << (16 - ln)
            if np.any(len_of[lo:hi]):
                raise ValueError("codes are not prefix-free")
            sym_of[lo:hi] = s
            len_of[lo:hi] = ln
    return sym_of, len_of


def decode(stream, lengths, chunk: int, n: int, codes=None) -> np.ndarray:
    """Decoder (ii): all chunks advance one symbol per step through a 16-bit lookup table.

    The gaps are not needed to decode sequentially; they are checked afterwards
    against the code-word boundaries the decode found.
    """
    from .huffman import canonical_codes

    lengths = np.asarray(lengths, dtype=np.int64).ravel()
    if codes is None:
        codes = canonical_codes(lengths)
    starts, ends, gaps, payload = parse_table(stream, n, chunk)
    nc = starts.size
    out = np.zeros(n, dtype=np.uint8)
    if nc == 0:
        return out
    K = units_per_chunk(chunk)
    sym_of, len_of = _lookup_table(lengths, codes)
    words = np.concatenate([payload, np.zeros(2, dtype=np.uint64)])
    pos = starts * 32
    endbit = ends * 32
    m = np.minimum(chunk, n - np.arange(nc, dtype=np.int64) * chunk)
    base = np.arange(nc, dtype=np.int64) * chunk
    # unit boundaries (global bits) and the first code-word boundary found at or after each
    wc = ends - starts
    ubit = 32 * (starts[:, None] + (np.arange(K, dtype=np.int64)[None, :] * wc[:, None]) // K)
    found = np.full((nc, K), -1, dtype=np.int64)

    def mark(act, p):
        # a boundary at p settles every unit boundary in (previous boundary, p]
        sub = ubit[act] if not isinstance(act, slice) else ubit
        f = found[act] if not isinstance(act, slice) else found
        hit = (f < 0) & (sub <= p[:, None])
        f[hit] = np.broadcast_to(p[:, None], f.shape)[hit]
        if isinstance(act, slice):
            found[:] = f
        else:
            found[act] = f

    mark(slice(None), pos.copy())
    for k in range(int(m.max())):
        act = np.nonzero(m > k)[0] if m[-1] <= k else slice(None)
        p = pos[act]
        w = p >> 5
        window = (words[w] << np.uint64(32)) | words[w + 1]
        peek = (window >> (np.uint64(48) - (p & 31).astype(np.uint64))) & np.uint64(0xFFFF)
        ln = len_of[peek.astype(np.int64)]
        if np.any(ln == 0):
            raise CorruptStream("no code word matches")
        if np.any(p + ln > endbit[act]):
            raise CorruptStream("code word runs past the end of its chunk")
        out[base[act] + k] = sym_of[peek.astype(np.int64)]
        pos[act] = p + ln
        mark(act, pos[act])
    if np.any(endbit - pos >= 32):
        raise CorruptStream("chunk holds more words than its symbols need")
    rest = endbit - pos
    last = words[ends - 1]
    mask = (np.uint64(1) << rest.astype(np.uint64)) - np.uint64(1)
    if np.any(last & mask):
        raise CorruptStream("non-zero padding after the last code word")
    if np.any(found - ubit != gaps):
        raise CorruptStream("gap disagrees with the code-word boundaries")
    return out
