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

The pages fix no stream layout.  Reading (stream format v3), chosen before the
kernels that follow it and followed bit for bit by the library:

* ``n`` symbols are cut into ``nc = ceil(n / chunk)`` chunks; chunk c holds
  symbols ``[c*chunk, min((c+1)*chunk, n))`` -- the independent work unit;
* lanes: a chunk is coded as G = min(max(chunk // 256, 1), 16) interleaved
  lanes (the pages' independent parallel tasks, Key design item 3).  The
  chunk's symbols are cut into blocks of 16 (the last one shorter); block b
  belongs to lane b mod G, so lane j holds blocks j, j+G, j+2G, ... in order;
* a lane's bits are its symbols' code words concatenated in order, MOST
  significant bit first, cut into 32-bit words (the last one zero-padded):
  lane j takes N_j = ceil(bits_j / 32) words;
* word order inside the chunk: the order in which a lane-parallel decoder
  reads them.  Every lane reads its words 0 and 1 before decoding (first all
  lanes' words 0, then all lanes' words 1, in lane order, each only if the lane
  has it); then the lane decodes its symbols two at a time, and its word
  k >= 2 is read just before the first pair (symbols 2p and 2p+1 of the lane)
  whose first bit lies at or after bit 32*(k-1) of the lane's string, i.e.
  once word k-2 is used up.  Words read before the same pair follow lane order;
  pairs are taken in increasing p.  A lane holds two words at a time, so a
  pair (at most 32 bits) always has its bits at hand;
* stream = ``u32 end[nc]`` (end[c] = index, counted in payload words, one past
  chunk c's last word; chunk c spans words [end[c-1], end[c]) with
  end[-1] = 0) || zero bytes up to a 16-byte boundary || ``u16 NW[nc*G]``
  (NW[c*G + j] = N_j of lane j of chunk c; 0 for a lane with no symbols) ||
  zero bytes up to a 16-byte boundary || ``u32 payload[W]`` (little-endian)
  with W = end[nc-1];  size = align16(4*nc) + align16(2*nc*G) + 4*W;
  n = 0 -> empty stream;
* nothing else is stored: chunk size, n and the codebook travel outside
  (the fixed codebook is never transmitted, per Methodology step 4).

Which lane a block goes to, the lane word counts and the read order are our
reading (the pages ask for independent parallel pieces, not for a layout).
"""

from __future__ import annotations

import numpy as np

NSYM = 256
BLOCK = 16       # symbols per block
LANE_MIN = 256   # a chunk has one lane per 256 symbols ...
LANES_MAX = 16   # ... and at most 16 lanes


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


def lanes_per_chunk(chunk: int) -> int:
    return min(max(int(chunk) // LANE_MIN, 1), LANES_MAX)


def table_bytes(n: int, chunk: int) -> int:
    return _align16(4 * num_chunks(n, chunk))


def count_bytes(n: int, chunk: int) -> int:
    return _align16(2 * num_chunks(n, chunk) * lanes_per_chunk(chunk))


def header_bytes(n: int, chunk: int) -> int:
    """Bytes before the payload: offset table and lane word counts, each padded to 16 bytes."""
    return table_bytes(n, chunk) + count_bytes(n, chunk)


def count_span(n: int, chunk: int, c0: int, c1: int):
    """Byte range [a, b) of the stream that holds the lane word counts of chunks [c0, c1)."""
    G = lanes_per_chunk(chunk)
    tb = table_bytes(n, chunk)
    return tb + 2 * c0 * G, tb + 2 * c1 * G


def lane_symbol_counts(n: int, chunk: int) -> np.ndarray:
    """int64[nc, G]: how many symbols each lane of each chunk holds."""
    nc = num_chunks(n, chunk)
    G = lanes_per_chunk(chunk)
    c = np.arange(nc, dtype=np.int64)[:, None]
    j = np.arange(G, dtype=np.int64)[None, :]
    m = np.minimum(int(chunk), int(n) - c * int(chunk))      # symbols of the chunk
    full, rest = m // BLOCK, m % BLOCK                         # whole blocks, symbols of the short one
    whole = np.maximum(0, (full - j + G - 1) // G)             # blocks b < full with b % G == j
    return whole * BLOCK + np.where((full % G == j) & (rest > 0), rest, 0)


def lane_positions(m: int, G: int):
    """For the m symbols of one chunk: (lane, index within the lane) of every symbol."""
    i = np.arange(int(m), dtype=np.int64)
    b = i // BLOCK
    return b % G, (b // G) * BLOCK + i % BLOCK


def encoded_bound(n: int, chunk: int, max_len: int = 16) -> int:
    """Largest stream any code with lengths <= max_len can give, rounded up to 16 bytes:
    a lane of m symbols takes at most ceil(m * max_len / 32) words, reached when every
    symbol has a max_len-bit code word."""
    if num_chunks(n, chunk) == 0:
        return 0
    m = lane_symbol_counts(n, chunk)
    words = int(((m * int(max_len) + 31) // 32).sum())
    return _align16(header_bytes(n, chunk) + 4 * words)


def _check_args(sym, lengths, chunk):
    sym = np.ascontiguousarray(sym).view(np.uint8).ravel()
    lengths = np.asarray(lengths, dtype=np.int64).ravel()
    if lengths.shape != (NSYM,):
        raise ValueError("lengths must have 256 entries")
    if chunk <= 0:
        raise ValueError("chunk must be positive")
    return sym, lengths


def _assemble(n, chunk, ends, counts, payload_words):
    nc = num_chunks(n, chunk)
    table = np.zeros(table_bytes(n, chunk) // 4, dtype="<u4")
    table[:nc] = ends
    cnt = np.zeros(count_bytes(n, chunk) // 2, dtype="<u2")
    counts = np.asarray(counts, dtype=np.int64).ravel()
    if counts.size and int(counts.max()) >= 1 << 16:
        raise OverflowError("a lane has more words than a u16 count holds")
    cnt[: nc * lanes_per_chunk(chunk)] = counts
    payload = np.asarray(payload_words, dtype=np.uint64).astype("<u4")
    return np.concatenate([table.view(np.uint8), cnt.view(np.uint8), payload.view(np.uint8)])


def _read_round(pair_start_bits, k: int) -> int:
    """When a lane reads its word k: -2 and -1 for words 0 and 1 (before decoding), else the
    first pair p whose first bit pair_start_bits[p] is at or after bit 32*(k-1)."""
    if k < 2:
        return k - 2
    for p, b in enumerate(pair_start_bits):
        if b >= 32 * (k - 1):
            return p
    raise AssertionError("a lane's last word is always read")  # shown in the format note


# --------------------------------------------------------------------------
# encoder (i): the definition, one character per bit.  Small inputs only.
# --------------------------------------------------------------------------

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
    G = lanes_per_chunk(chunk)
    words, ends, counts = [], [], []
    payload_bits = 0
    for c in range(nc):
        chunk_syms = sym[c * chunk: min((c + 1) * chunk, n)]
        reads = []   # (round, lane, word value)
        for j in range(G):
            lane = [s for i, s in enumerate(chunk_syms) if (i // BLOCK) % G == j]
            bits, starts = "", []
            for s in lane:
                ln = int(lengths[s])
                if ln == 0:
                    raise UncodedSymbol(f"byte {int(s)} has no code")
                starts.append(len(bits))
                bits += format(int(codes[s]), f"0{ln}b")
            payload_bits += len(bits)
            bits += "0" * (-len(bits) % 32)
            lane_words = [int(bits[i:i + 32], 2) for i in range(0, len(bits), 32)]
            counts.append(len(lane_words))
            pair_starts = starts[0::2]
            for k, w in enumerate(lane_words):
                reads.append((_read_round(pair_starts, k), j, w))
        reads.sort(key=lambda r: (r[0], r[1]))
        words += [w for _, _, w in reads]
        ends.append(len(words))
    if len(words) >= 1 << 32:
        raise OverflowError("payload too large for 32-bit word offsets")
    return _assemble(n, chunk, ends, counts, words), payload_bits


# --------------------------------------------------------------------------
# encoder (ii): vectorised numpy, blocks of whole chunks.
# --------------------------------------------------------------------------

def _lane_layout(chunk: int, start: int, size: int):
    """For symbols [start, start+size) (whole chunks): global lane id (chunk*G + lane) and
    index within the lane of every symbol."""
    G = lanes_per_chunk(chunk)
    i = start + np.arange(size, dtype=np.int64)
    c = i // chunk
    r = i - c * chunk
    b = r // BLOCK
    return c * G + b % G, (b // G) * BLOCK + r % BLOCK


def lane_bit_counts(sym, lengths, chunk: int) -> np.ndarray:
    """bits[c, j] = sum of the code lengths of lane j of chunk c (int64[nc, G])."""
    sym, lengths = _check_args(sym, lengths, chunk)
    n = sym.size
    nc = num_chunks(n, chunk)
    G = lanes_per_chunk(chunk)
    bits = np.zeros(nc * G, dtype=np.int64)
    block = max(1, (1 << 22) // chunk) * chunk
    for start in range(0, n, block):
        ln = lengths[sym[start:start + block]]
        if np.any(ln == 0):
            bad = int(sym[start:start + block][np.argmax(ln == 0)])
            raise UncodedSymbol(f"byte {bad} has no code")
        lane, _ = _lane_layout(chunk, start, ln.size)
        l0 = int(lane.min())
        part = np.bincount(lane - l0, weights=ln).astype(np.int64)
        bits[l0:l0 + part.size] += part
    return bits.reshape(nc, G)


def chunk_bit_counts(sym, lengths, chunk: int) -> np.ndarray:
    """bits[c] = sum of the code lengths of chunk c's symbols (int64[nc])."""
    return lane_bit_counts(sym, lengths, chunk).sum(axis=1)


def chunk_word_counts(sym, lengths, chunk: int) -> np.ndarray:
    """words[c] = sum over the chunk's lanes of ceil(bits / 32): payload words chunk c occupies."""
    return ((lane_bit_counts(sym, lengths, chunk) + 31) // 32).sum(axis=1)


def encode(sym, lengths, codes, chunk: int):
    """Vectorised encoder.  Returns (stream bytes as uint8 array, payload_bits).

    1. Every symbol's lane and index within the lane; symbols sorted by (lane,
       index) give every lane's string; a symbol's bit offset g in its lane is
       the sum of the lengths before it.
    2. The lanes' words laid out lane after lane: the code word of a symbol at
       lane offset g goes to word g>>5 of its lane starting (MSB-first) at bit
       31-(g&31), spilling into the next word when it crosses the boundary.
       Fields of distinct symbols are disjoint, so each word is the plain SUM of
       its fields (exact in float64 bincount: sums stay below 2^32).
    3. Every word's read round (-2, -1, or the pair p found by a sorted search
       over the lane's pair-start offsets), then the words of each chunk sorted
       by (round, lane).
    """
    sym, lengths = _check_args(sym, lengths, chunk)
    codes = np.asarray(codes, dtype=np.int64).ravel()
    n = sym.size
    nc = num_chunks(n, chunk)
    if nc == 0:
        return np.zeros(0, dtype=np.uint8), 0
    G = lanes_per_chunk(chunk)
    lane_bits = lane_bit_counts(sym, lengths, chunk).ravel()
    nw = (lane_bits + 31) // 32                       # words per lane
    ends = np.cumsum(nw.reshape(nc, G).sum(axis=1))
    W = int(ends[-1])
    if W >= 1 << 32:
        raise OverflowError("payload too large for 32-bit word offsets")
    chunk_first = np.concatenate([[0], ends[:-1]])
    payload = np.empty(W, dtype=np.uint64)
    block = max(1, (1 << 22) // chunk) * chunk
    for start in range(0, n, block):
        s = sym[start:start + block]
        lane, t = _lane_layout(chunk, start, s.size)
        order = np.lexsort((t, lane))                 # lane strings, symbol after symbol
        lane, t, s = lane[order], t[order], s[order]
        ln = lengths[s]
        cd = codes[s]
        l0 = int(lane[0])
        lanes = np.arange(l0, int(lane[-1]) + 1)      # the block's lanes that hold symbols
        lw = nw[lanes]
        lane_word0 = np.concatenate([[0], np.cumsum(lw)[:-1]])   # lane-after-lane layout
        excl = np.cumsum(ln) - ln
        first_of_lane = np.searchsorted(lane, lanes, side="left")
        g = excl - np.concatenate([excl, [0]])[first_of_lane][lane - l0]   # bit offset in the lane
        w = lane_word0[lane - l0] + (g >> 5)
        b = g & 31
        shift = 32 - b - ln
        fits = shift >= 0
        hi = np.where(fits, cd << np.maximum(shift, 0), cd >> np.maximum(-shift, 0))
        lo = np.where(fits, 0, (cd << np.maximum(32 + shift, 0)) & 0xFFFFFFFF)
        total = int(lw.sum())
        words = np.bincount(w, weights=hi.astype(np.float64), minlength=total + 1)
        words += np.bincount(w + 1, weights=lo.astype(np.float64), minlength=total + 2)[: total + 1]
        words = words[:total].astype(np.uint64)
        assert np.all(words < (1 << 32))
        # read round of every word (lane-after-lane order)
        wl = np.repeat(lanes, lw)                                    # lane of each word
        k = np.arange(total, dtype=np.int64) - np.repeat(lane_word0, lw)
        even = (t % 2) == 0                                          # pair starts
        ek = lane[even] * (1 << 24) + g[even]                        # sorted: lane, then offset
        q = wl * (1 << 24) + 32 * (k - 1)
        p = np.searchsorted(ek, q, side="left") - np.searchsorted(ek, wl * (1 << 24), side="left")
        rnd = np.where(k < 2, k - 2, p)
        chunk_of = wl // G
        dest = np.lexsort((wl, rnd, chunk_of))                       # by chunk, round, lane
        out_at = int(chunk_first[int(chunk_of[0])])
        payload[out_at:out_at + total] = words[dest]
    return _assemble(n, chunk, ends, nw, payload), int(lane_bits.sum())


# --------------------------------------------------------------------------
# decoding
# --------------------------------------------------------------------------

def parse_table(stream, n: int, chunk: int):
    """Validate the layout; return (starts, ends, word counts int64[nc, G], payload as uint64)."""
    stream = np.ascontiguousarray(stream).view(np.uint8).ravel()
    nc = num_chunks(n, chunk)
    G = lanes_per_chunk(chunk)
    if nc == 0:
        if stream.size != 0:
            raise CorruptStream("non-empty stream for n = 0")
        z = np.zeros(0, np.int64)
        return z, z, np.zeros((0, G), np.int64), np.zeros(0, np.uint64)
    tb = table_bytes(n, chunk)
    hb = header_bytes(n, chunk)
    if stream.size < hb or (stream.size - hb) % 4:
        raise CorruptStream("stream shorter than its header or not whole words")
    ends = stream[: 4 * nc].view("<u4").astype(np.int64)
    if np.any(stream[4 * nc: tb] != 0):
        raise CorruptStream("non-zero table padding")
    if np.any(stream[tb + 2 * nc * G: hb] != 0):
        raise CorruptStream("non-zero word-count padding")
    counts = stream[tb: tb + 2 * nc * G].view("<u2").astype(np.int64).reshape(nc, G)
    W = (stream.size - hb) // 4
    starts = np.concatenate([[0], ends[:-1]])
    if np.any(ends <= starts):
        raise CorruptStream("offset table not strictly increasing")
    if int(ends[-1]) != W:
        raise CorruptStream("offset table disagrees with the stream size")
    if np.any(counts.sum(axis=1) != ends - starts):
        raise CorruptStream("lane word counts disagree with the chunk's words")
    if np.any((counts == 0) != (lane_symbol_counts(n, chunk) == 0)):
        raise CorruptStream("a lane with symbols has no words, or an empty lane has words")
    payload = stream[hb:].view("<u4").astype(np.uint64)
    return starts, ends, counts, payload


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
    """Decoder (i): the read order replayed chunk by chunk, lane by lane, and canonical
    prefix matching one bit at a time.  Small inputs only.

    A code word of length l is recognised when the l bits read so far, as an
    integer v, satisfy first[l] <= v < first[l] + count[l]; its symbol is the
    (v - first[l])-th symbol of length l in canonical order.
    """
    lengths = np.asarray(lengths, dtype=np.int64).ravel()
    starts, ends, counts, payload = parse_table(stream, n, chunk)
    first, count, index, syms = _canonical_tables(lengths)
    G = lanes_per_chunk(chunk)
    out = np.zeros(n, dtype=np.uint8)
    for c in range(starts.size):
        m = min(chunk, n - c * chunk)
        lane_of, t_of = lane_positions(m, G)
        mj = [int(np.sum(lane_of == j)) for j in range(G)]
        cw = [int(x) for x in payload[starts[c]:ends[c]]]
        taken = 0
        bits = [""] * G          # the words each lane has read, as one bit string
        pos = [0] * G            # next bit of each lane
        decoded = [[] for _ in range(G)]

        def read(j):
            nonlocal taken
            if taken >= len(cw):
                raise CorruptStream("a lane reads past its chunk's words")
            bits[j] += format(cw[taken], "032b")
            taken += 1

        for k in (0, 1):
            for j in range(G):
                if counts[c, j] > k:
                    read(j)
        for p in range(-(-max(mj) // 2)):
            for j in range(G):
                k = len(bits[j]) // 32
                if 2 * p < mj[j] and k < counts[c, j] and pos[j] >= 32 * (k - 1):
                    read(j)
            for j in range(G):
                for _ in range(max(0, min(2, mj[j] - 2 * p))):
                    v = 0
                    ln = 0
                    while True:
                        if pos[j] >= len(bits[j]):
                            raise CorruptStream("code word runs past the words the lane has read")
                        v = (v << 1) | (bits[j][pos[j]] == "1")
                        pos[j] += 1
                        ln += 1
                        if ln > 16:
                            raise CorruptStream("no code word matches")
                        if count[ln] and first[ln] <= v < first[ln] + count[ln]:
                            decoded[j].append(syms[index[ln] + v - first[ln]])
                            break
        for j in range(G):
            if len(bits[j]) != 32 * counts[c, j]:
                raise CorruptStream("a lane's last word is never read")
            if len(bits[j]) - pos[j] >= 32:
                raise CorruptStream("lane holds more words than its symbols need")
            if "1" in bits[j][pos[j]:]:
                raise CorruptStream("non-zero padding after a lane's last code word")
        for i in range(m):
            out[c * chunk + i] = decoded[lane_of[i]][t_of[i]]
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
    """Decoder (ii): every lane of every chunk advances one pair per step.

    Before each pair the lanes that have used up a word read the next one; the
    chunk's read cursor hands them consecutive payload words in lane order.
    Symbols come from a 16-bit lookup table over each lane's words so far.
    """
    from .huffman import canonical_codes

    lengths = np.asarray(lengths, dtype=np.int64).ravel()
    if codes is None:
        codes = canonical_codes(lengths)
    starts, ends, counts, payload = parse_table(stream, n, chunk)
    nc = starts.size
    out = np.zeros(n, dtype=np.uint8)
    if nc == 0:
        return out
    G = lanes_per_chunk(chunk)
    sym_of, len_of = _lookup_table(lengths, codes)
    mj = lane_symbol_counts(n, chunk).ravel()             # symbols per lane
    N = counts.ravel()
    L = nc * G
    lane = np.arange(L, dtype=np.int64)
    cid = lane // G
    buf = np.zeros((L, int(N.max()) + 2), dtype=np.uint64)  # words read so far (zeros after)
    got = np.zeros(L, dtype=np.int64)                      # words read
    bit = np.zeros(L, dtype=np.int64)                      # next bit
    cursor = starts.copy()                                 # next payload word of each chunk

    def read(want):
        # lanes in `want` read their next word; a chunk's readers take consecutive words
        f = want.reshape(nc, G).astype(np.int64)
        at = (cursor[:, None] + np.cumsum(f, axis=1) - f).ravel()[want]
        if np.any(at >= ends[cid[want]]):
            raise CorruptStream("a lane reads past its chunk's words")
        buf[want, got[want]] = payload[at]
        got[want] += 1
        cursor[:] += f.sum(axis=1)

    read(N > 0)
    read(N > 1)
    base = cid * chunk
    for p in range(-(-int(mj.max()) // 2)):
        read((mj > 2 * p) & (got < N) & (bit >= 32 * (got - 1)))
        for h in (0, 1):
            a = np.nonzero(mj > 2 * p + h)[0]
            b = bit[a]
            w = b >> 5
            window = (buf[a, w] << np.uint64(32)) | buf[a, w + 1]
            peek = ((window >> (np.uint64(48) - (b & 31).astype(np.uint64))) & np.uint64(0xFFFF)).astype(np.int64)
            ln = len_of[peek]
            if np.any(ln == 0):
                raise CorruptStream("no code word matches")
            if np.any(b + ln > 32 * got[a]):
                raise CorruptStream("code word runs past the words the lane has read")
            t = 2 * p + h                                   # index within the lane
            blk = (t // BLOCK) * G + a % G                  # block of the chunk it sits in
            out[base[a] + blk * BLOCK + t % BLOCK] = sym_of[peek]
            bit[a] = b + ln
    if np.any(got != N):
        raise CorruptStream("a lane's last word is never read")
    if np.any(32 * N - bit >= 32):
        raise CorruptStream("lane holds more words than its symbols need")
    rest = 32 * N - bit
    last = buf[lane, np.maximum(N - 1, 0)]
    mask = (np.uint64(1) << rest.astype(np.uint64)) - np.uint64(1)
    if np.any(last & mask):
        raise CorruptStream("non-zero padding after a lane's last code word")
    return out
