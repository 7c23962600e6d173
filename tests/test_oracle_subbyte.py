"""Pins of the 4-bit readings (oracle/subbyte.py).

"Single-Stage Huffman Encoder for ML Compression", Limitations and future work
(quantisation granularity) leaves 4-bit data open.  The pins fix the two
readings with values derived by hand:

* byte layout: value 2i in the low nibble, 2i+1 in the high nibble;
* dyadic 4-bit distribution p = (1/2, 1/4, 1/8, 1/16, 1/16): the optimal code
  has lengths -log2 p = (1, 2, 3, 4, 4) (Kraft equality plus Gibbs' equality
  case), and with independent halves the pair code's lengths are the sums, so
  both readings cost the same number of bits;
* uniform bytes: 4 bits per value in both readings;
* equal halves (byte = v | v << 4): the pair reading costs exactly half;
* the concatenation bound, pair bits <= 16-symbol bits, on seeded data.
"""

import numpy as np
import pytest

import oracle
import workloads
from oracle import subbyte


def test_nibble_order_hand_example():
    packed = np.array([0x21, 0xF0, 0x07], np.uint8)
    assert subbyte.nibbles(packed).tolist() == [1, 2, 0, 15, 7, 0]
    h = subbyte.nibble_histogram(packed)
    assert h.shape == (256,) and h[0] == 2 and h[1] == 1 and h[2] == 1 and h[7] == 1 and h[15] == 1
    assert h.sum() == 6


def test_workload_packing_matches_nibble_order():
    # the workload's packer and the oracle's unpacker are written separately
    v = workloads.int4_values(3, 1024)
    assert v.min() >= -8 and v.max() <= 7
    # absmax of every group maps to +-7 exactly
    assert np.all(np.abs(v.reshape(-1, workloads.INT4_GROUP)).max(axis=1) == 7)
    packed = workloads.pack_int4(v)
    assert packed.size == 512
    assert np.array_equal(subbyte.nibbles(packed), (v.view(np.uint8) & 0x0F))


def _dyadic_pairs(scale: int) -> np.ndarray:
    f = {0: 8, 1: 4, 2: 2, 3: 1, 4: 1}
    out = []
    for a, fa in f.items():
        for b, fb in f.items():
            out += [a | (b << 4)] * (fa * fb * scale)
    return np.array(out, np.uint8)


@pytest.mark.parametrize("scale", [1, 3])
def test_dyadic_independent_halves_cost_the_same(scale):
    packed = _dyadic_pairs(scale)
    ln = subbyte.nibble_code_lengths(packed, 8)
    assert ln[:5].tolist() == [1, 2, 3, 4, 4] and not ln[5:].any()
    # 16 * scale pairs per unit of f(a): each value appears 2 * 16 * scale * f(v) times
    want = 2 * 16 * scale * (8 * 1 + 4 * 2 + 2 * 3 + 1 * 4 + 1 * 4)
    assert subbyte.nibble_code_bits(packed, 8) == want
    assert subbyte.pair_code_bits(packed, 16) == want
    pl = oracle.package_merge_lengths(oracle.histogram(packed), 16)
    for a in range(5):
        for b in range(5):
            assert pl[a | (b << 4)] == ln[a] + ln[b]


def test_uniform_bytes_four_bits_per_value():
    packed = np.arange(256, dtype=np.uint8).repeat(2)
    assert subbyte.nibble_code_bits(packed, 8) == 4 * 2 * packed.size
    assert subbyte.pair_code_bits(packed, 16) == 8 * packed.size


def test_equal_halves_pair_code_is_half():
    v = np.arange(16, dtype=np.uint8).repeat(5)
    packed = v | (v << 4)
    assert subbyte.nibble_code_bits(packed, 8) == 4 * 2 * packed.size
    assert subbyte.pair_code_bits(packed, 16) == 4 * packed.size


@pytest.mark.parametrize("kind", ["int4", "skewed", "uniform"])
def test_pair_bound_on_seeded_data(kind):
    if kind == "int4":
        packed = workloads.int4_packed(0, 1 << 16)
    elif kind == "skewed":
        packed = workloads.skewed_bytes(5, 1 << 14, 1.5)
    else:
        packed = workloads.uniform_bytes(6, 1 << 14)
    assert subbyte.pair_bound_holds(packed)
