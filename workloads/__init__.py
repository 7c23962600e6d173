"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module holds input recipes only -- random draws, rounding of the draws to
the tensor's storage type, and the snapshot delta that the snapshot workload
feeds to the coder.  It contains none of the coding arithmetic and imports
neither the library nor the oracle.

The pages measure on tensors that are not available here (Gemma 2B
activations and weight shards in "Single-Stage Huffman Encoder for ML
Compression", Results; LLM training checkpoints in "Lossless Compression for
LLM Tensor Incremental Snapshots", Experiment highlights).  These seeded
stand-ins take their shapes and value distributions from the workload list:

* ``int8_fixed``   1 Mi int8 symbols from round(N(0, 20^2)), four warm-up
                   batches from other seeds, chunk 4096;
* ``bf16_weights`` 64 Mi bf16 from N(0, 0.02^2) with 0.1 % outliers x20,
                   chunk 16384 (normal body plus outliers is the weight shape
                   the LLM.265 article describes);
* ``int8_acts``    [8, 2048, 2048] int8 from Laplace(0, b) with a per-channel
                   scale b ~ U(4, 32) on the last axis, chunk 4096;
* ``bf16_delta``   512 Mi bf16 XOR snapshot delta, W1 = bf16(W0 + N(0, 1e-4^2)),
                   chunk 65536;
* ``int8_drift``   64 batches of 64 Mi int8 from round(N(0, s_k^2)),
                   s_k = 10 + 30 k / 63, chunk 4096;
* ``int4_packed``  64 Mi int4 weights, two per byte (32 Mi bytes): N(0, 1)
                   values quantised per group of 128 with scale absmax / 7,
                   four warm-up batches from other seeds, chunk 4096 (a 4-bit
                   tensor; the pages name 4-bit data as open work);
* ``fp32_weights`` 64 Mi float32 from N(0, 0.02^2) with 0.1 % outliers x20
                   (the bf16_weights recipe kept in float32), chunk 16384.

RNG: ``numpy.random.default_rng([cfg, role, block])`` (PCG64).  Tensors are
drawn in blocks of 2^26 elements; block j uses ``block = j``.  ``scale`` < 1
shrinks the element count (whole blocks are cut at the end) for tests.
"""

from __future__ import annotations

import numpy as np

BLOCK = 1 << 26

CONFIGS = {
    "int8_fixed": dict(cfg=1, kind="u8", mode="fixed", n=1 << 20, chunk=4096),
    "bf16_weights": dict(cfg=2, kind="bf16", mode="pertensor", n=1 << 26, chunk=16384),
    "int8_acts": dict(cfg=3, kind="u8", mode="fixed", n=8 * 2048 * 2048, chunk=4096),
    "bf16_delta": dict(cfg=4, kind="bf16", mode="pertensor", n=1 << 29, chunk=65536),
    "int8_drift": dict(cfg=5, kind="u8", mode="fixed", n=1 << 32, chunk=4096),
    "int4_packed": dict(cfg=6, kind="u8", mode="fixed", n=1 << 25, chunk=4096),
    "fp32_weights": dict(cfg=7, kind="fp32", mode="pertensor", n=1 << 26, chunk=16384),
}


def rng(cfg: int, role: int, block: int) -> np.random.Generator:
    return np.random.default_rng([cfg, role, block])


def q8(x: np.ndarray) -> np.ndarray:
    """round half to even, clip to the int8 range, reinterpret as bytes."""
    return np.clip(np.rint(x), -128, 127).astype(np.int8).view(np.uint8)


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------- int8, fixed codebook

def int8_fixed(role: int = 0, n: int = 1 << 20) -> np.ndarray:
    """Eval batch (role 0) or warm-up batch (roles 1..4): round(N(0, 20^2)) as bytes."""
    return q8(rng(1, role, 0).normal(0.0, 20.0, n))


def int8_fixed_batch(block: int, n: int = 1 << 20) -> np.ndarray:
    """Independent eval batch number ``block`` (role 0); block 0 is ``int8_fixed(0, n)``."""
    return q8(rng(1, 0, block).normal(0.0, 20.0, n))


_C3_SHAPE = (8, 2048, 2048)


def int8_acts_scales() -> np.ndarray:
    return rng(3, 9, 0).uniform(4.0, 32.0, _C3_SHAPE[-1])


def int8_acts(role: int = 0, rows: int | None = None) -> np.ndarray:
    """Activations [8, 2048, 2048]: Laplace(0, 1) * b[channel] in float64, quantised; C-order bytes.

    ``rows`` (default 8*2048) limits the number of [2048]-channel rows drawn.
    """
    b = int8_acts_scales()
    r = _C3_SHAPE[0] * _C3_SHAPE[1] if rows is None else rows
    x = rng(3, role, 0).laplace(0.0, 1.0, (r, _C3_SHAPE[2])) * b
    return q8(x).ravel()


def drift_sigma(k: int) -> float:
    return 10.0 + 30.0 * k / 63.0


def int8_drift_batch(k: int, n: int = BLOCK) -> np.ndarray:
    """Batch k of the drift stream: round(N(0, s_k^2)) as bytes (role 0, block k)."""
    return q8(rng(5, 0, k).normal(0.0, drift_sigma(k), n))


# --------------------------------------------------------------------------- int4, two per byte

INT4_GROUP = 128


def int4_values(role: int = 0, count: int = 1 << 26) -> np.ndarray:
    """Signed 4-bit weights as int8 in -7..7: N(0, 1) draws quantised per group of
    INT4_GROUP consecutive values with scale = group absmax / 7 (round half to even).
    ``count`` is a multiple of INT4_GROUP."""
    x = rng(6, role, 0).normal(0.0, 1.0, count).reshape(-1, INT4_GROUP)
    scale = np.abs(x).max(axis=1, keepdims=True) / 7.0
    return np.clip(np.rint(x / scale), -8, 7).astype(np.int8).ravel()


def pack_int4(v: np.ndarray) -> np.ndarray:
    """Two 4-bit two's-complement values per byte: value 2i in bits 0-3, 2i+1 in bits 4-7."""
    u = (np.asarray(v, dtype=np.int8).view(np.uint8) & 0x0F).reshape(-1, 2)
    return (u[:, 0] | (u[:, 1] << 4)).astype(np.uint8)


def int4_packed(role: int = 0, nbytes: int = 1 << 25) -> np.ndarray:
    """Eval batch (role 0) or warm-up batch (roles 1..4) of packed int4 weights, as bytes."""
    return pack_int4(int4_values(role, 2 * nbytes))


# --------------------------------------------------------------------------- bf16, per tensor

def bf16_weights(n: int = 1 << 26) -> np.ndarray:
    """bf16 weights N(0, 0.02^2) with i.i.d. 0.1 % outliers scaled x20 in float32, as uint16."""
    out = np.empty(n, dtype=np.uint16)
    for j, s in enumerate(range(0, n, BLOCK)):
        m = min(BLOCK, n - s)
        g = rng(2, 0, j)
        w = g.normal(0.0, 0.02, m).astype(np.float32)
        u = g.random(m)
        w[u < 0.001] *= np.float32(20.0)
        out[s:s + m] = bf16_bits(w)
    return out


def fp32_weights(n: int = 1 << 26) -> np.ndarray:
    """float32 weights N(0, 0.02^2) with i.i.d. 0.1 % outliers scaled x20, as uint32 bit patterns."""
    out = np.empty(n, dtype=np.uint32)
    for j, s in enumerate(range(0, n, BLOCK)):
        m = min(BLOCK, n - s)
        g = rng(7, 0, j)
        w = g.normal(0.0, 0.02, m).astype(np.float32)
        u = g.random(m)
        w[u < 0.001] *= np.float32(20.0)
        out[s:s + m] = w.view(np.uint32)
    return out


def bf16_delta(n: int = 1 << 29, return_snapshots: bool = False):
    """Snapshot delta D = W0 xor W1 with W1 = bf16(f32(W0) + N(0, 1e-4^2)), as uint16."""
    d = np.empty(n, dtype=np.uint16)
    w0s = np.empty(n, dtype=np.uint16) if return_snapshots else None
    w1s = np.empty(n, dtype=np.uint16) if return_snapshots else None
    for j, s in enumerate(range(0, n, BLOCK)):
        m = min(BLOCK, n - s)
        w0 = bf16_bits(rng(4, 0, j).normal(0.0, 0.02, m).astype(np.float32))
        noise = rng(4, 1, j).normal(0.0, 1e-4, m).astype(np.float32)
        w1 = bf16_bits(bf16_to_f32(w0) + noise)
        d[s:s + m] = w0 ^ w1
        if return_snapshots:
            w0s[s:s + m] = w0
            w1s[s:s + m] = w1
    return (d, w0s, w1s) if return_snapshots else d


def uniform_bytes(seed: int, n: int, alphabet: int = 256) -> np.ndarray:
    """Uniform random bytes over 0..alphabet-1 (edge-case and small parity inputs)."""
    return np.random.default_rng([100, seed]).integers(0, alphabet, n, dtype=np.uint8)


def skewed_bytes(seed: int, n: int, sigma: float = 3.0) -> np.ndarray:
    """Heavily skewed bytes: round(N(0, sigma^2)) as int8 (a few dominant symbols)."""
    return q8(np.random.default_rng([101, seed]).normal(0.0, sigma, n))
