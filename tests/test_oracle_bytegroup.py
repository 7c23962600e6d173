"""Pins of the oracle's byte grouping, container and size accounting (CPU only)."""

import numpy as np
import torch

import oracle
import workloads
from golden_examples import load_container


def test_split_matches_torch_bf16_bit_view():
    x32 = np.random.default_rng(1).normal(0, 0.02, 10_000).astype(np.float32)
    t = torch.from_numpy(x32).to(torch.bfloat16)
    u16 = t.view(torch.int16).numpy().view(np.uint16)
    hi, lo = oracle.split_bf16(u16)
    b = u16.view(np.uint8).reshape(-1, 2)  # little-endian: byte 1 is the high byte
    assert np.array_equal(hi, b[:, 1]) and np.array_equal(lo, b[:, 0])
    assert np.array_equal(oracle.merge_bf16(hi, lo), u16)


def test_generator_bf16_rounding_matches_torch():
    x32 = np.random.default_rng(2).normal(0, 0.02, 100_000).astype(np.float32)
    x32[::7] *= 20
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(workloads.bf16_bits(x32), ref)


def test_bf16_container_round_trip_and_layout():
    x = workloads.bf16_weights(70_000)
    enc = oracle.encode_bf16(x, 16384)
    buf = oracle.container_bytes(enc)
    bh, bl = enc["stream_hi"].size, enc["stream_lo"].size
    assert buf.size == 560 + bh + (-bh % 16) + bl
    assert bytes(buf[:4]) == b"LECB"
    back = oracle.parse_container(buf)
    assert np.array_equal(oracle.decode_bf16(back), x)
    # byte grouping separates a compressible high plane from a nearly random low plane
    assert enc["bits_hi"] < 0.5 * 8 * x.size
    assert enc["bits_lo"] > 0.95 * 8 * x.size


def test_delta_planes():
    d, w0, w1 = workloads.bf16_delta(1 << 16, return_snapshots=True)
    assert np.array_equal(w0 ^ d, w1)
    hi, lo = oracle.split_bf16(d)
    assert (hi == 0).mean() > 0.95  # a small update rarely touches sign/exponent bits


def test_workload_entropy_closed_forms():
    # round(N(0, s^2)) has entropy close to the Gaussian differential entropy at these s.
    h = oracle.histogram(workloads.int8_fixed(0))
    assert abs(oracle.entropy_bits(h) - oracle.metrics.gaussian_entropy_bits(20.0)) < 0.01
    h10 = oracle.histogram(workloads.int8_drift_batch(0, 1 << 20))
    assert abs(oracle.entropy_bits(h10) - oracle.metrics.gaussian_entropy_bits(10.0)) < 0.01


def test_payload_identity_and_optimum():
    x = workloads.int8_fixed(0)
    warm = [oracle.histogram(workloads.int8_fixed(r)) for r in (1, 2, 3, 4)]
    F = oracle.codebook_frequencies(warm, 1)
    ln = oracle.package_merge_lengths(F, 16)
    h = oracle.histogram(x)
    fixed_bits = oracle.payload_bits_identity(h, ln)
    opt_bits = oracle.per_batch_optimal_bits(h, 16)
    shannon = oracle.metrics.shannon_bits(h)
    assert shannon <= opt_bits <= fixed_bits
    assert fixed_bits / opt_bits - 1 < 0.005  # the page's "within 0.5 % of per-shard Huffman" holds here
    assert fixed_bits / shannon - 1 < 0.01


def test_snapshot_delta_pins():
    """XOR delta: the identities that fix it (involution, zero on equal
    snapshots, bit-flip count) checked on random patterns and by hand."""
    import workloads
    rng = np.random.default_rng(5)
    w0 = rng.integers(0, 1 << 16, 10_001, dtype=np.uint16)
    w1 = rng.integers(0, 1 << 16, 10_001, dtype=np.uint16)
    d = oracle.snapshot_delta(w0, w1)
    assert np.array_equal(oracle.apply_delta(w0, d), w1)
    assert np.array_equal(oracle.apply_delta(w1, d), w0)
    assert not oracle.snapshot_delta(w0, w0).any()
    # by hand: 0x3F80 (1.0) and 0x4000 (2.0) differ in bits 14..7 -> 0x7F80
    assert int(oracle.snapshot_delta(np.array([0x3F80], np.uint16), np.array([0x4000], np.uint16))[0]) == 0x7F80
    # the snapshot workload's delta is this operator
    ds, w0s, w1s = workloads.bf16_delta(1 << 16, return_snapshots=True)
    assert np.array_equal(oracle.snapshot_delta(w0s, w1s), ds)


def test_fp32_planes_of_ieee_patterns():
    # IEEE 754 binary32 patterns (sign | 8-bit exponent | 23-bit fraction):
    # 1.0 = 0x3F800000, -2.5 = 0xC0200000, the float nearest pi = 0x40490FDB
    pats = np.array([0x3F800000, 0xC0200000, 0x40490FDB], np.uint32)
    assert np.array_equal(np.array([1.0, -2.5, np.pi], np.float32).view(np.uint32), pats)
    planes = oracle.split_fp32(pats)
    assert [p.tolist() for p in planes] == [[0x3F, 0xC0, 0x40], [0x80, 0x20, 0x49], [0x00, 0x00, 0x0F],
                                            [0x00, 0x00, 0xDB]]
    # little-endian bytes: plane p is byte 3 - p of the stored element
    b = pats.view(np.uint8).reshape(-1, 4)
    for p in range(4):
        assert np.array_equal(planes[p], b[:, 3 - p])
    assert np.array_equal(oracle.merge_fp32(planes), pats)


def test_fp32_upper_planes_are_the_bf16_planes():
    # a float32 whose low 16 bits are zero is a bf16 value: its two upper
    # planes are that bf16 value's high and low byte planes
    x32 = workloads.bf16_to_f32(workloads.bf16_weights(4096)).view(np.uint32)
    p = oracle.split_fp32(x32)
    hi, lo = oracle.split_bf16((x32 >> 16).astype(np.uint16))
    assert np.array_equal(p[0], hi) and np.array_equal(p[1], lo)
    assert not p[2].any() and not p[3].any()


def test_fp32_round_trip_and_plane_streams():
    x = workloads.fp32_weights(40_000)
    enc = oracle.encode_fp32(x, 4096)
    assert np.array_equal(oracle.decode_fp32(enc), x)
    planes = oracle.split_fp32(x)
    for p in range(4):
        assert enc["bits"][p] == oracle.payload_bits_identity(oracle.histogram(planes[p]), enc["len"][p])
    # the sign/exponent plane compresses, the low mantissa bytes hardly at all
    assert enc["bits"][0] < 4 * x.size and enc["bits"][3] > 7.9 * x.size


def test_container_header_golden_bytes():
    """The container header against hand-derived bytes (tests/golden/container_header.txt):
    every field at its offset, hi and lo tables and sizes distinguishable."""
    f, head = load_container()
    enc = {"n": f["n"], "chunk": f["chunk"], "max_len": f["max_len"], "len_hi": f["len_hi"],
           "len_lo": f["len_lo"], "stream_hi": np.zeros(f["bytes_hi"], np.uint8),
           "stream_lo": np.zeros(f["bytes_lo"], np.uint8)}
    buf = oracle.container_bytes(enc)
    assert np.array_equal(buf[:560], head)
    assert buf.size == f["total_bytes"]
    back = oracle.parse_container(buf)
    assert (back["n"], back["chunk"], back["max_len"]) == (f["n"], f["chunk"], f["max_len"])
    assert np.array_equal(back["len_hi"], f["len_hi"]) and np.array_equal(back["len_lo"], f["len_lo"])
    assert back["stream_hi"].size == f["bytes_hi"] and back["stream_lo"].size == f["bytes_lo"]
