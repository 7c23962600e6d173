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

The pages fix no stream layout.  Reading (stream format v2), chosen before the
kernels that follow it and followed bit for bit by the library:

* ``n`` symbols are cut into ``nc = ceil(n / chunk)`` chunks; chunk c holds
  symbols ``[c*chunk, min((c+1)*chunk, n))`` -- the independent work unit;
* a chunk's bits are its symbols' code words concatenated in order, MOST
  significant bit first, starting at bit 31 of a fresh 32-bit word and filling
  downwards; the chunk's last word is zero-padded; words are stored
  little-endian; chunks follow each other with no gap;
* decode units: a chunk is cut into K = ceil(chunk / 256) units of 256
  consecutive symbols (the last one shorter when the chunk is not a multiple
  of 256, units past n empty); ULEN[c*K + j] = the number of code bits of
  unit j of chunk c.  Unit j's code words start at bit sum(ULEN[c*K : c*K+j])
  of the chunk, so a decoder can start K independent decoders per chunk, each
  at a known bit and a known output position (the pages' Key design item 3
  asks for independent parallel tasks; storing per-part bit counts is our
  reading, not the pages');
* stream = ``u32 end[nc]`` (end[c] = index, counted in payload words, one past
  chunk c's last word; chunk c spans words [end[c-1], end[c]) with
  end[-1] = 0) || zero bytes up to a 16-byte boundary || ``u16 ULEN[nc*K]``
  (little-endian) || zero bytes up to a 16-byte boundary || ``u32 payload[W]``
  with W = end[nc-1];
  size = align16(4*nc) + align16(2*nc*K) + 4*W;  n = 0 -> empty stream;
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


UNIT = 256  # symbols per decode unit


def units_per_chunk(chunk: int) -> int:
    return -(-int(chunk) // UNIT)


def table_bytes(n: int, chunk: int) -> int:
    return _align16(4 * num_chunks(n, chunk))


def ulen_bytes(n: int, chunk: int) -> int:
    return _align16(2 * num_chunks(n, chunk) * units_per_chunk(chunk))


def header_bytes(n: int, chunk: int) -> int:
    """Bytes before the payload: offset table and unit bit counts, each padded to 16 bytes."""
    return table_bytes(n, chunk) + ulen_bytes(n, chunk)


def unit_meta_span(n: int, chunk: int, c0: int, c1: int):
    """Byte range [a, b) of the stream that holds the unit bit counts of chunks [c0, c1)."""
    K = units_per_chunk(chunk)
    tb = table_bytes(n, chunk)
    return tb + 2 * c0 * K, tb + 2 * c1 * K


def encoded_bound(n: int, chunk: int, max_len: int = 16) -> int:
    """Largest stream any code with lengths <= max_len can give, rounded up to 16 bytes:
    chunk c of m_c symbols takes at most ceil(m_c * max_len / 32) words, reached when
    every symbol has a max_len-bit code word."""
    nc = num_chunks(n, chunk)
    if nc == 0:
        return 0
    full, last = nc - 1, int(n) - (nc - 1) * int(chunk)
    words = full * -(-int(chunk) * int(max_len) // 32) + -(-last * int(max_len) // 32)
    return _align16(header_bytes(n, chunk) + 4 * words)


def unit_ranges(n: int, chunk: int):
    """(first symbol, end symbol) of every unit, as int64[nc, K] arrays (empty units: first == end)."""
    nc = num_chunks(n, chunk)
    K = units_per_chunk(chunk)
    c = np.arange(nc, dtype=np.int64)[:, None]
    j = np.arange(K, dtype=np.int64)[None, :]
    chunk_end = np.minimum((c + 1) * chunk, n)
    first = np.minimum(c * chunk + j * UNIT, chunk_end)
    end = np.minimum(first + UNIT, chunk_end)
    return first, end


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

def _assemble(n, chunk, ends, ulen, payload_words):
    nc = num_chunks(n, chunk)
    table = np.zeros(table_bytes(n, chunk) // 4, dtype="<u4")
    table[:nc] = ends
    units = np.zeros(ulen_bytes(n, chunk) // 2, dtype="<u2")
    units[: nc * units_per_chunk(chunk)] = np.asarray(ulen, dtype=np.int64).ravel()
    payload = np.asarray(payload_words, dtype=np.uint64).astype("<u4")
    return np.concatenate([table.view(np.uint8), units.view(np.uint8), payload.view(np.uint8)])


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
    K = units_per_chunk(chunk)
    words, ends, ulen = [], [], []
    payload_bits = 0
    for c in range(nc):
        chunk_syms = sym[c * chunk: min((c + 1) * chunk, n)]
        bits = ""
        for j in range(K):
            unit = ""
            for s in chunk_syms[j * UNIT:(j + 1) * UNIT]:
                ln = int(lengths[s])
                if ln == 0:
                    raise UncodedSymbol(f"byte {int(s)} has no code")
                unit += format(int(codes[s]), f"0{ln}b")
            ulen.append(len(unit))
            bits += unit
        payload_bits += len(bits)
        bits += "0" * (-len(bits) % 32)
        for i in range(0, len(bits), 32):
            words.append(int(bits[i:i + 32], 2))
        ends.append(len(words))
    if len(words) >= 1 << 32:
        raise OverflowError("payload too large for 32-bit word offsets")
    return _assemble(n, chunk, ends, ulen, words), payload_bits


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
    Unit bit counts: the code lengths summed per unit (symbol i of chunk c is
    in unit (i - c*chunk) // 256).
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
    ulen = np.zeros(nc * K, dtype=np.int64)
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
        # bit counts of the units of this block's symbols
        uid = cid * K + ((start + np.arange(s.size, dtype=np.int64)) - cid * chunk) // UNIT
        u0 = int(uid[0])
        part = np.bincount(uid - u0, weights=ln).astype(np.int64)
        ulen[u0:u0 + part.size] += part
    assert np.all(ulen <= UNIT * 16)
    payload = payload[:W].astype(np.uint64)
    assert np.all(payload < (1 << 32))
    return _assemble(n, chunk, ends, ulen, payload), int(bits.sum())


# --------------------------------------------------------------------------
# decoding
# --------------------------------------------------------------------------

def parse_table(stream, n: int, chunk: int):
    """Validate the layout; return (starts, ends, ulen[nc, K], payload words as uint64)."""
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
    if np.any(stream[tb + 2 * nc * K: hb] != 0):
        raise CorruptStream("non-zero unit-count padding")
    ulen = stream[tb: tb + 2 * nc * K].view("<u2").astype(np.int64).reshape(nc, K)
    W = (stream.size - hb) // 4
    starts = np.concatenate([[0], ends[:-1]])
    if np.any(ends <= starts):
        raise CorruptStream("offset table not strictly increasing")
    if int(ends[-1]) != W:
        raise CorruptStream("offset table disagrees with the stream size")
    payload = stream[hb:].view("<u4").astype(np.uint64)
    return starts, ends, ulen, payload


def _check_units(ulen, unit_bits):
    """The stored unit bit counts must be the bits the decode found for each unit."""
    if not np.array_equal(np.asarray(unit_bits, dtype=np.int64).reshape(ulen.shape), ulen):
        raise CorruptStream("unit bit count disagrees with the code words")


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
    starts, ends, ulen, payload = parse_table(stream, n, chunk)
    first, count, index, syms = _canonical_tables(lengths)
    K = units_per_chunk(chunk)
    out = np.zeros(n, dtype=np.uint8)
    unit_bits = np.zeros(ulen.shape, dtype=np.int64)
    for c in range(starts.size):
        words = payload[starts[c]:ends[c]]
        bitstr = "".join(format(int(w), "032b") for w in words)
        p = 0
        at = [0]  # bit position at every unit boundary
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
            if (k + 1) % UNIT == 0:
                at.append(p)
        at += [p] * (K + 1 - len(at))
        unit_bits[c] = np.diff(at[:K + 1])
        if (len(bitstr) - p) >= 32:
            raise CorruptStream("chunk holds more words than its symbols need")
        if "1" in bitstr[p:]:
            raise CorruptStream("non-zero padding after the last code word")
    _check_units(ulen, unit_bits)
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

    The unit bit counts are not needed to decode sequentially; they are checked
    afterwards against the positions the decode reached at the unit boundaries.
    """
    from .huffman import canonical_codes

    lengths = np.asarray(lengths, dtype=np.int64).ravel()
    if codes is None:
        codes = canonical_codes(lengths)
    starts, ends, ulen, payload = parse_table(stream, n, chunk)
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
    at = np.zeros((nc, K + 1), dtype=np.int64)  # bit position at every unit boundary
    at[:, 0] = pos
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
        if (k + 1) % UNIT == 0:
            at[act, (k + 1) // UNIT] = pos[act]
    # boundaries at or after a chunk's last symbol are its end position
    done = np.arange(K + 1)[None, :] >= (-(-m // UNIT))[:, None]
    at = np.where(done, pos[:, None], at)
    if np.any(endbit - pos >= 32):
        raise CorruptStream("chunk holds more words than its symbols need")
    rest = endbit - pos
    last = words[ends - 1]
    mask = (np.uint64(1) << rest.astype(np.uint64)) - np.uint64(1)
    if np.any(last & mask):
        raise CorruptStream("non-zero padding after the last code word")
    _check_units(ulen, np.diff(at, axis=1))
    return out
