"""Oracle: byte grouping (bf16: two planes, fp32: four) and the two-stream container.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

Page basis: "Lossless Compression for LLM Tensor Incremental Snapshots",
Technical framework step 1 (byte grouping before coding) and its reverse path
(byte-group restore after Huffman decoding); the original abstract names
byte grouping as the data preparation that LMC builds on.

Readings:
* the summary's wording ("combining bytes into larger units") contradicts the
  standard meaning of byte grouping for floating-point data; we take the
  standard one: a bf16 tensor (little-endian 16-bit words) is split into a
  HIGH-byte plane (bits 15..8: sign, exponent, top mantissa bit) and a
  LOW-byte plane (bits 7..0), and each plane is Huffman-coded on its own;
* per-tensor mode = the classic three steps of "Single-Stage Huffman Encoder
  for ML Compression", Overview: each plane gets its own histogram and its own
  optimal codebook (no frequency clamp), and the codebook is transmitted -- as
  its 256 code lengths, the codes being canonical.

Container v1 (little-endian):
    0   magic  b"LECB"
    4   u16 version = 1
    6   u16 kind = 1            (bf16, two byte planes)
    8   u64 n                   (elements)
    16  u32 chunk
    20  u32 max_len
    24  u8  len_hi[256]
    280 u8  len_lo[256]
    536 u64 bytes_hi
    544 u64 bytes_lo
    552 zero padding to 560
    560 stream_hi, zero-padded to a 16-byte boundary, then stream_lo
"""

from __future__ import annotations

import struct

import numpy as np

from .huffman import histogram, package_merge_lengths, canonical_codes
from .stream import encode, decode, CorruptStream

HEADER_BYTES = 560
MAGIC = b"LECB"


def split_bf16(x) -> tuple[np.ndarray, np.ndarray]:
    """hi[i] = x[i] >> 8, lo[i] = x[i] & 0xFF for the 16-bit patterns x."""
    x = np.ascontiguousarray(x).view(np.uint16).ravel()
    return (x >> 8).astype(np.uint8), (x & 0xFF).astype(np.uint8)


def merge_bf16(hi, lo) -> np.ndarray:
    """x[i] = hi[i] << 8 | lo[i] (the byte-group restore)."""
    hi = np.asarray(hi, dtype=np.uint16)
    lo = np.asarray(lo, dtype=np.uint16)
    return ((hi << 8) | lo).astype(np.uint16)


def snapshot_delta(w0, w1) -> np.ndarray:
    """D[i] = W0[i] ^ W1[i] on the 16-bit patterns.

    "Lossless Compression for LLM Tensor Incremental Snapshots", Technical
    framework (incremental delta between consecutive checkpoints) and the
    original abstract.  Reading: the pages do not define the delta operator;
    the bitwise XOR of the stored bit patterns is taken (exactly invertible,
    no floating-point rounding)."""
    w0 = np.ascontiguousarray(w0).view(np.uint16).ravel()
    w1 = np.ascontiguousarray(w1).view(np.uint16).ravel()
    if w0.shape != w1.shape:
        raise ValueError("snapshots differ in size")
    return np.bitwise_xor(w0, w1)


def apply_delta(w0, d) -> np.ndarray:
    """W1[i] = W0[i] ^ D[i]: the later snapshot from the earlier one and the delta."""
    return snapshot_delta(w0, d)


def split_fp32(x) -> list[np.ndarray]:
    """Four byte planes of 32-bit patterns x, most significant first:
    plane p holds (x[i] >> (8 * (3 - p))) & 0xFF.

    Byte grouping with a 4-byte group ("Lossless Compression for LLM Tensor
    Incremental Snapshots", Technical framework step 1; Key design item 1
    makes the byte-group size a design choice).  Reading: the same per-byte
    planes as for bf16, one plane per byte position of the element."""
    x = np.ascontiguousarray(x).view(np.uint32).ravel()
    return [((x >> np.uint32(8 * (3 - p))) & np.uint32(0xFF)).astype(np.uint8) for p in range(4)]


def merge_fp32(planes) -> np.ndarray:
    """x[i] = sum over p of planes[p][i] << 8 * (3 - p) (the byte-group restore)."""
    if len(planes) != 4:
        raise ValueError("four planes expected")
    x = np.zeros(np.asarray(planes[0]).size, dtype=np.uint32)
    for p, plane in enumerate(planes):
        x |= np.asarray(plane, dtype=np.uint32) << np.uint32(8 * (3 - p))
    return x


def encode_fp32(x, chunk: int, max_len: int = 16) -> dict:
    """Per-tensor coding of a 32-bit tensor: per plane histogram, optimal codebook, stream."""
    planes = split_fp32(x)
    out = {"n": planes[0].size, "chunk": chunk, "max_len": max_len, "len": [], "stream": [], "bits": []}
    for plane in planes:
        ln = package_merge_lengths(histogram(plane), max_len)
        stream, bits = encode(plane, ln, canonical_codes(ln), chunk)
        out["len"].append(ln)
        out["stream"].append(stream)
        out["bits"].append(bits)
    return out


def decode_fp32(enc: dict) -> np.ndarray:
    n, chunk = enc["n"], enc["chunk"]
    return merge_fp32([decode(s, ln, chunk, n) for s, ln in zip(enc["stream"], enc["len"])])


def encode_bf16(x, chunk: int, max_len: int = 16) -> dict:
    """Per-tensor coding of one bf16 tensor: split, histogram, codebook and stream per plane."""
    hi, lo = split_bf16(x)
    out = {"n": hi.size, "chunk": chunk, "max_len": max_len}
    for name, plane in (("hi", hi), ("lo", lo)):
        ln = package_merge_lengths(histogram(plane), max_len)
        stream, bits = encode(plane, ln, canonical_codes(ln), chunk)
        out["len_" + name] = ln
        out["stream_" + name] = stream
        out["bits_" + name] = bits
    return out


def decode_bf16(enc: dict) -> np.ndarray:
    n, chunk = enc["n"], enc["chunk"]
    hi = decode(enc["stream_hi"], enc["len_hi"], chunk, n)
    lo = decode(enc["stream_lo"], enc["len_lo"], chunk, n)
    return merge_bf16(hi, lo)


def container_bytes(enc: dict) -> np.ndarray:
    """Serialise an ``encode_bf16`` result into container v1."""
    sh = np.asarray(enc["stream_hi"], dtype=np.uint8)
    sl = np.asarray(enc["stream_lo"], dtype=np.uint8)
    head = bytearray(HEADER_BYTES)
    struct.pack_into("<4sHHQII", head, 0, MAGIC, 1, 1, int(enc["n"]), int(enc["chunk"]), int(enc["max_len"]))
    head[24:280] = np.asarray(enc["len_hi"], dtype=np.uint8).tobytes()
    head[280:536] = np.asarray(enc["len_lo"], dtype=np.uint8).tobytes()
    struct.pack_into("<QQ", head, 536, sh.size, sl.size)
    pad = (-sh.size) % 16
    return np.concatenate([np.frombuffer(bytes(head), np.uint8), sh, np.zeros(pad, np.uint8), sl])


def parse_container(buf) -> dict:
    buf = np.ascontiguousarray(buf).view(np.uint8).ravel()
    if buf.size < HEADER_BYTES:
        raise CorruptStream("container shorter than its header")
    magic, ver, kind, n, chunk, max_len = struct.unpack_from("<4sHHQII", buf.tobytes()[:24])
    if magic != MAGIC or ver != 1 or kind != 1:
        raise CorruptStream("bad container header")
    bh, bl = struct.unpack_from("<QQ", buf.tobytes()[536:552])
    off_lo = HEADER_BYTES + bh + (-bh % 16)
    if buf.size != off_lo + bl:
        raise CorruptStream("container size disagrees with its header")
    return {
        "n": n, "chunk": chunk, "max_len": max_len,
        "len_hi": buf[24:280].copy(), "len_lo": buf[280:536].copy(),
        "stream_hi": buf[HEADER_BYTES:HEADER_BYTES + bh].copy(),
        "stream_lo": buf[off_lo:off_lo + bl].copy(),
    }
