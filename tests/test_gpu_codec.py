"""GPU parity of every kernel against the oracle, through the C ABI.

Bar: bit-exact streams, byte-exact round trips, exact histograms.  Sizes span
several chunks, several 4096-symbol tiles and a ragged tail.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
import oracle_jobs
import lossless_entropy_coding_byte_amd as lecb
from gpu_helpers import DEV, to_dev, codebook_for, gpu_encode, gpu_decode

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# ----------------------------------------------------------------------------- histogram

@pytest.mark.parametrize("n", [1, 15, 16, 17, 4096 * 3 + 5, 1_000_003])
def test_histogram_u8_exact(n):
    _say(f"hist u8 n={n}")
    x = workloads.skewed_bytes(n, n, sigma=30)
    h = torch.zeros(256, dtype=torch.int64, device=DEV)
    lecb.lecb_histogram(to_dev(x), h)
    assert np.array_equal(h.cpu().numpy().astype(np.uint64), oracle.histogram(x))
    lecb.lecb_histogram(to_dev(x), h, accumulate=True)
    assert np.array_equal(h.cpu().numpy().astype(np.uint64), 2 * oracle.histogram(x))


def test_histogram_single_value_plane():
    # every byte equal: all increments land in one bin
    x = np.full(3_000_017, 0, np.uint8)
    h = torch.zeros(256, dtype=torch.int64, device=DEV)
    lecb.lecb_histogram(to_dev(x), h)
    assert int(h[0]) == x.size and int(h.sum()) == x.size


@pytest.mark.parametrize("n", [1, 7, 8, 9, 100_001, 1 << 20])
def test_histogram_bf16_exact(n):
    _say(f"hist bf16 n={n}")
    x = workloads.bf16_weights(n)
    hh = torch.zeros(256, dtype=torch.int64, device=DEV)
    hl = torch.zeros(256, dtype=torch.int64, device=DEV)
    lecb.lecb_histogram_bf16(to_dev(x.view(np.int16)), hh, hl)
    hi, lo = oracle.split_bf16(x)
    assert np.array_equal(hh.cpu().numpy().astype(np.uint64), oracle.histogram(hi))
    assert np.array_equal(hl.cpu().numpy().astype(np.uint64), oracle.histogram(lo))


# ----------------------------------------------------------------------------- byte grouping

@pytest.mark.parametrize("n", [1, 15, 16, 17, 99_999, 1 << 20])
def test_split_merge_exact(n):
    x = workloads.bf16_weights(n)
    xd = to_dev(x.view(np.int16))
    hi = torch.empty(n, dtype=torch.uint8, device=DEV)
    lo = torch.empty(n, dtype=torch.uint8, device=DEV)
    lecb.lecb_split_bf16(xd, hi, lo)
    rh, rl = oracle.split_bf16(x)
    assert np.array_equal(hi.cpu().numpy(), rh) and np.array_equal(lo.cpu().numpy(), rl)
    back = torch.empty(n, dtype=torch.int16, device=DEV)
    lecb.lecb_merge_bf16(hi, lo, back)
    assert np.array_equal(back.cpu().numpy().view(np.uint16), x)


# ----------------------------------------------------------------------------- encode / decode

def _gauss(seed, n, sigma=20.0):
    return workloads.q8(np.random.default_rng([7, seed]).normal(0, sigma, n))


CASES = [
    # name, n, chunk, input maker, clamp
    ("one_symbol_one_chunk", 1, 4096, lambda n: np.array([77], np.uint8), True),
    ("tiny_lt_unit", 100, 256, lambda n: _gauss(1, n), True),
    ("ragged_256", 256 * 37 + 11, 256, lambda n: _gauss(2, n), True),
    ("ragged_1024", 1024 * 19 + 1000, 1024, lambda n: _gauss(3, n, 5.0), False),
    ("tiles_4096", 4096 * 25 + 4095, 4096, lambda n: _gauss(4, n), True),
    ("tiles_16384", 16384 * 9 + 77, 16384, lambda n: _gauss(5, n, 60.0), True),
    ("tiles_65536", 65536 * 5 + 12345, 65536, lambda n: _gauss(6, n, 2.0), False),
    ("all_equal", 50_000, 4096, lambda n: np.full(n, 200, np.uint8), False),
    ("two_symbols", 70_001, 1024, lambda n: workloads.uniform_bytes(9, n, 2), False),
    ("uniform_8bit", 4096 * 8, 4096, lambda n: workloads.uniform_bytes(10, n), False),
]


@pytest.mark.parametrize("name,n,chunk,gen,clamp", CASES, ids=[c[0] for c in CASES])
def test_encode_bit_exact_and_round_trip(name, n, chunk, gen, clamp):
    _say(f"encode/decode case={name} n={n} chunk={chunk}")
    x = gen(n)
    ln = codebook_for(x, clamp)
    ref, ref_bits = oracle.encode(x, ln, oracle.canonical_codes(ln), chunk)
    got, r, dcb = gpu_encode(x, ln, chunk)
    assert int(r["status"]) == 0, lecb.lecb_status_str(int(r["status"]))
    assert int(r["bytes"]) == ref.size
    assert int(r["payload_bits"]) == ref_bits
    assert np.array_equal(got, ref)
    y, rd = gpu_decode(ref, dcb, chunk, n)
    assert int(rd["status"]) == 0, lecb.lecb_status_str(int(rd["status"]))
    assert int(rd["payload_bits"]) == ref_bits
    assert np.array_equal(y, x)


def test_skewed_lanes_encode_exactly():
    """One lane of each chunk codes 1-bit code words while the other 15 code
    16-bit ones: the slow lane's words complete long after the others have
    taken hundreds of read positions, more than the encoder stages per group,
    so it codes those chunks again with direct stores.  The stream must still
    equal the oracle's."""
    f = np.array([max(1, (1 << 40) >> s) for s in range(256)], np.uint64)
    ln = oracle.package_merge_lengths(f, 16)
    long16 = np.flatnonzero(ln == 16)
    assert ln[0] == 1 and long16.size > 100
    chunk, nch = 4096, 6
    x = long16[workloads.uniform_bytes(77, chunk * nch + 1000, long16.size)].astype(np.uint8)
    blocks = x[: chunk * nch].reshape(nch, 16, 16, 16)              # chunk, block row, lane, symbol
    blocks[:, :, 0, :] = 0                                         # lane 0: the 1-bit code word
    got, r, _ = gpu_encode(x, ln, chunk)
    assert int(r["status"]) == 0
    ref, bits = oracle.encode(x, ln, oracle.canonical_codes(ln), chunk)
    assert np.array_equal(got, ref) and int(r["payload_bits"]) == bits


def test_long_codes_straddle_words():
    # geometric weights: code lengths up to 16, many code words cross word boundaries
    f = np.array([max(1, (1 << 30) >> s) for s in range(256)], np.uint64)
    ln = oracle.package_merge_lengths(f, 16)
    assert int(ln.max()) == 16
    x = workloads.uniform_bytes(11, 4096 * 6 + 333)
    ref, _ = oracle.encode(x, ln, oracle.canonical_codes(ln), 4096)
    got, r, dcb = gpu_encode(x, ln, 4096)
    assert np.array_equal(got, ref)
    y, rd = gpu_decode(ref, dcb, 4096, x.size)
    assert int(rd["status"]) == 0 and np.array_equal(y, x)


@pytest.mark.parametrize("max_len", [9, 11, 12, 13])
def test_length_limits(max_len):
    x = _gauss(12, 4096 * 4 + 1, 30.0)
    ln = codebook_for(x, True, max_len)
    assert int(ln.max()) == max_len
    ref, _ = oracle.encode(x, ln, oracle.canonical_codes(ln), 4096)
    got, r, dcb = gpu_encode(x, ln, 4096)
    assert np.array_equal(got, ref)
    y, rd = gpu_decode(ref, dcb, 4096, x.size)
    assert int(rd["status"]) == 0 and np.array_equal(y, x)


def test_empty_input():
    ln = codebook_for(np.arange(256, dtype=np.uint8), True)
    got, r, dcb = gpu_encode(np.zeros(0, np.uint8), ln, 4096)
    assert int(r["bytes"]) == 0 and int(r["status"]) == 0


def test_determinism_repeat_encode():
    x = _gauss(13, 4096 * 200 + 5)
    ln = codebook_for(x, True)
    a, _, _ = gpu_encode(x, ln, 4096)
    b, _, _ = gpu_encode(x, ln, 4096)
    assert np.array_equal(a, b)


def test_workspace_reuse_across_calls():
    # per-workgroup word totals and the exit counter must not leak between calls sharing a workspace
    x1 = _gauss(14, 4096 * 300 + 9)
    x2 = _gauss(15, 4096 * 120 + 1, 40.0)
    ln = codebook_for(np.concatenate([x1, x2]), True)
    cb = lecb.DeviceCodebook.upload(lecb.lecb_codebook_from_lengths(ln), DEV)
    ws = lecb.new_workspace(x1.size, 4096, DEV)
    for x in (x1, x2, x1, x2):
        out, res = lecb.encode_bytes(to_dev(x), cb, 4096, ws=ws)
        r = lecb.results_to_numpy(res)[0]
        ref, _ = oracle.encode(x, ln, oracle.canonical_codes(ln), 4096)
        assert np.array_equal(out[: int(r["bytes"])].cpu().numpy(), ref)


def test_cross_decode_gpu_stream_with_oracle():
    x = _gauss(16, 16384 * 3 + 5000, 25.0)
    ln = codebook_for(x, True)
    got, r, _ = gpu_encode(x, ln, 16384)
    assert np.array_equal(oracle.decode(got, ln, 16384, x.size), x)


# ----------------------------------------------------------------------------- bf16 planes

def test_plane_encode_matches_oracle():
    x = workloads.bf16_weights(200_003)
    hi, lo = oracle.split_bf16(x)
    xd = to_dev(x.view(np.int16))
    for plane, data in ((1, hi), (0, lo)):
        ln = codebook_for(data, False)
        ref, bits = oracle.encode(data, ln, oracle.canonical_codes(ln), 16384)
        dcb = lecb.DeviceCodebook.upload(lecb.lecb_codebook_from_lengths(ln), DEV)
        out = torch.empty(lecb.lecb_encoded_bound(x.size, 16384), dtype=torch.uint8, device=DEV)
        res = lecb.new_results(1, DEV)
        ws = lecb.new_workspace(x.size, 16384, DEV)
        lecb.lecb_encode_plane(xd, x.size, plane, dcb.blob, 16384, out, res, ws)
        r = lecb.results_to_numpy(res)[0]
        assert int(r["status"]) == 0 and int(r["payload_bits"]) == bits
        assert np.array_equal(out[: int(r["bytes"])].cpu().numpy(), ref)


@pytest.mark.parametrize("n,chunk", [(77, 256), (50_001, 1024), (200_003, 4096), (300_001, 16384),
                                     (100_000, 32768), ((1 << 20) + 77, 65536)])
def test_bf16_pair_encode_fixed_codebooks(n, chunk):
    """Both planes in one pass with codebooks from other data (every byte coded):
    each stream is bit-exact with the oracle and with the single-plane encode."""
    _say(f"bf16 pair encode n={n} chunk={chunk}")
    x = workloads.bf16_weights(n)
    warm = workloads.bf16_weights(1 << 16)
    hi_w, lo_w = oracle.split_bf16(warm)
    hi, lo = oracle.split_bf16(x)
    ln_hi = oracle.package_merge_lengths(oracle.codebook_frequencies([oracle.histogram(hi_w)], 1), 16)
    ln_lo = oracle.package_merge_lengths(oracle.codebook_frequencies([oracle.histogram(lo_w)], 1), 16)
    bh = lecb.DeviceCodebook.upload(lecb.lecb_codebook_from_lengths(ln_hi), DEV)
    bl = lecb.DeviceCodebook.upload(lecb.lecb_codebook_from_lengths(ln_lo), DEV)
    xd = to_dev(x.view(np.int16))
    cap = lecb.lecb_encoded_bound(n, chunk)
    oh = torch.empty(cap, dtype=torch.uint8, device=DEV)
    ol = torch.empty(cap, dtype=torch.uint8, device=DEV)
    res = lecb.new_results(2, DEV)
    ws = lecb.new_workspace(n, chunk, DEV)
    lecb.lecb_encode_bf16(xd, n, bh.blob, bl.blob, chunk, oh, ol, res, ws)
    r = lecb.results_to_numpy(res)
    for k, (data, ln, o) in enumerate(((hi, ln_hi, oh), (lo, ln_lo, ol))):
        ref, bits = oracle.encode(data, ln, oracle.canonical_codes(ln), chunk)
        assert int(r[k]["status"]) == 0 and int(r[k]["payload_bits"]) == bits
        assert np.array_equal(o[: int(r[k]["bytes"])].cpu().numpy(), ref)
    # the single-plane path gives the same bytes
    one = torch.empty(cap, dtype=torch.uint8, device=DEV)
    res1 = lecb.new_results(1, DEV)
    lecb.lecb_encode_plane(xd, n, 0, bl.blob, chunk, one, res1, ws)
    r1 = lecb.results_to_numpy(res1)[0]
    assert int(r1["bytes"]) == int(r[1]["bytes"])
    assert torch.equal(one[: int(r1["bytes"])], ol[: int(r1["bytes"])])


@pytest.mark.parametrize("n,chunk", [(77, 256), (200_003, 4096), ((1 << 20) + 77, 65536)])
def test_bf16_two_plane_decode(n, chunk):
    """One launch decodes both planes; each plane equals the oracle's, and a
    corrupt low stream is reported in the low result only."""
    _say(f"bf16 two-plane decode n={n} chunk={chunk}")
    x = workloads.bf16_weights(n)
    enc = oracle.encode_bf16(x, chunk)
    hi, lo = oracle.split_bf16(x)
    bh = lecb.DeviceCodebook.upload(lecb.lecb_codebook_from_lengths(enc["len_hi"]), DEV)
    bl = lecb.DeviceCodebook.upload(lecb.lecb_codebook_from_lengths(enc["len_lo"]), DEV)

    def dev_stream(a):
        buf = torch.zeros((a.size + 15) // 16 * 16 + 16, dtype=torch.uint8, device=DEV)
        buf[: a.size] = to_dev(a)
        return buf

    sh, sl = dev_stream(enc["stream_hi"]), dev_stream(enc["stream_lo"])
    oh = torch.empty((n + 15) // 16 * 16, dtype=torch.uint8, device=DEV)
    ol = torch.empty_like(oh)
    res = lecb.new_results(2, DEV)
    ws = lecb.new_workspace(n, chunk, DEV)
    lecb.lecb_decode_bf16_planes(sh, enc["stream_hi"].size, sl, enc["stream_lo"].size, bh.blob, bl.blob,
                                 chunk, n, oh, ol, res, ws)
    r = lecb.results_to_numpy(res)
    assert int(r[0]["status"]) == 0 and int(r[1]["status"]) == 0
    assert np.array_equal(oh[:n].cpu().numpy(), hi) and np.array_equal(ol[:n].cpu().numpy(), lo)
    bad = enc["stream_lo"].copy()
    bad[-1] ^= 0x01  # last payload word: a padding bit or a code bit changes
    sl2 = dev_stream(bad)
    lecb.lecb_decode_bf16_planes(sh, enc["stream_hi"].size, sl2, bad.size, bh.blob, bl.blob,
                                 chunk, n, oh, ol, res, ws)
    r = lecb.results_to_numpy(res)
    assert int(r[0]["status"]) == 0
    try:
        oracle.decode(bad, enc["len_lo"], chunk, n)
        lo_ok = True
    except oracle.CorruptStream:
        lo_ok = False
    assert (int(r[1]["status"]) == 0) == lo_ok
    if lo_ok:
        assert np.array_equal(ol[:n].cpu().numpy(), oracle.decode(bad, enc["len_lo"], chunk, n))


@pytest.mark.parametrize("n,chunk", [(1, 256), (300_001, 16384), (1 << 20, 65536)])
def test_bf16_pertensor_pipeline(n, chunk):
    _say(f"bf16 per-tensor n={n} chunk={chunk}")
    x = workloads.bf16_weights(n)
    ref = oracle.encode_bf16(x, chunk)
    xd = to_dev(x.view(np.int16))
    hist = torch.zeros(512, dtype=torch.int64, device=DEV)
    bh, bl = lecb.new_codebook_blob(DEV), lecb.new_codebook_blob(DEV)
    cap = lecb.lecb_encoded_bound(n, chunk)
    oh = torch.empty(cap, dtype=torch.uint8, device=DEV)
    ol = torch.empty(cap, dtype=torch.uint8, device=DEV)
    res = lecb.new_results(2, DEV)
    ws = lecb.new_workspace(n, chunk, DEV)
    cb_hi, cb_lo = lecb.lecb_encode_bf16_pertensor(xd, n, chunk, 16, hist, bh, bl, oh, ol, res, ws)
    r = lecb.results_to_numpy(res)
    assert np.array_equal(cb_hi.lengths(), ref["len_hi"]) and np.array_equal(cb_lo.lengths(), ref["len_lo"])
    assert np.array_equal(oh[: int(r[0]["bytes"])].cpu().numpy(), ref["stream_hi"])
    assert np.array_equal(ol[: int(r[1]["bytes"])].cpu().numpy(), ref["stream_lo"])
    out = torch.empty(n, dtype=torch.int16, device=DEV)
    res2 = lecb.new_results(2, DEV)
    lecb.lecb_decode_bf16(oh, int(r[0]["bytes"]), ol, int(r[1]["bytes"]), bh, bl, chunk, n, out, res2, ws)
    rr = lecb.results_to_numpy(res2)
    assert int(rr[0]["status"]) == 0 and int(rr[1]["status"]) == 0
    assert np.array_equal(out.cpu().numpy().view(np.uint16), x)


# ----------------------------------------------------------------------------- fused snapshot delta

@pytest.mark.parametrize("n,chunk", [(1, 256), (300_001, 16384), ((1 << 20) + 5, 65536)])
def test_fused_snapshot_delta(n, chunk):
    """Encode from (W0, W1) and decode to W1: the delta planes' histograms,
    codebooks and streams equal the oracle's for D = W0 ^ W1 (the XOR never
    materialised), and the decode reproduces W1 exactly."""
    _say(f"fused delta n={n} chunk={chunk}")
    d, w0, w1 = workloads.bf16_delta(n, return_snapshots=True)
    enc = oracle.encode_bf16(oracle.snapshot_delta(w0, w1), chunk)
    w0d, w1d = to_dev(w0.view(np.int16)), to_dev(w1.view(np.int16))
    hh = torch.zeros(256, dtype=torch.int64, device=DEV)
    hl = torch.zeros(256, dtype=torch.int64, device=DEV)
    lecb.lecb_histogram_bf16_delta(w0d, w1d, hh, hl)
    dh, dl = oracle.split_bf16(d)
    assert np.array_equal(hh.cpu().numpy().astype(np.uint64), oracle.histogram(dh))
    assert np.array_equal(hl.cpu().numpy().astype(np.uint64), oracle.histogram(dl))
    hist = torch.zeros(512, dtype=torch.int64, device=DEV)
    bh, bl = lecb.new_codebook_blob(DEV), lecb.new_codebook_blob(DEV)
    cap = lecb.lecb_encoded_bound(n, chunk)
    oh = torch.empty(cap, dtype=torch.uint8, device=DEV)
    ol = torch.empty(cap, dtype=torch.uint8, device=DEV)
    res = lecb.new_results(2, DEV)
    ws = lecb.new_workspace(n, chunk, DEV)
    cb_hi, cb_lo = lecb.lecb_encode_bf16_delta_pertensor(w0d, w1d, n, chunk, 16, hist, bh, bl, oh, ol, res, ws)
    assert np.array_equal(cb_hi.lengths(), enc["len_hi"]) and np.array_equal(cb_lo.lengths(), enc["len_lo"])
    r = lecb.results_to_numpy(res)
    assert int(r[0]["status"]) == 0 and int(r[1]["status"]) == 0
    assert np.array_equal(oh[: int(r[0]["bytes"])].cpu().numpy(), enc["stream_hi"])
    assert np.array_equal(ol[: int(r[1]["bytes"])].cpu().numpy(), enc["stream_lo"])
    out = torch.empty(n, dtype=torch.int16, device=DEV)
    rd = lecb.new_results(2, DEV)
    lecb.lecb_decode_bf16_delta_from_results(oh, ol, res, bh, bl, chunk, n, w0d, out, rd, ws)
    q = lecb.results_to_numpy(rd)
    assert int(q[0]["status"]) == 0 and int(q[1]["status"]) == 0
    assert np.array_equal(out.cpu().numpy().view(np.uint16), w1)
    out.zero_()
    lecb.lecb_decode_bf16_delta(oh, int(r[0]["bytes"]), ol, int(r[1]["bytes"]), bh, bl, chunk, n, w0d, out, rd, ws)
    assert np.array_equal(out.cpu().numpy().view(np.uint16), w1)


# ----------------------------------------------------------------------------- codebooks built on the device

def _test_histograms(seed, count):
    r = np.random.default_rng(seed)
    out = []
    for t in range(count):
        kind = t % 6
        if kind == 0:
            h = r.integers(0, 1000, 256)
        elif kind == 1:
            h = np.zeros(256, np.int64)
            h[r.integers(0, 256, r.integers(1, 8))] = r.integers(1, 50)
        elif kind == 2:
            h = (r.pareto(1.0, 256) * 10).astype(np.int64)
        elif kind == 3:
            h = np.full(256, 7)
            h[: r.integers(0, 256)] = 0
        elif kind == 4:
            h = (2.0 ** r.integers(0, 40, 256)).astype(np.int64)
            h[r.random(256) < 0.3] = 0
        else:
            h = r.integers(0, 3, 256)
        out.append(h.astype(np.uint64))
    return out


@pytest.mark.parametrize("max_len,min_freq", [(16, 0), (16, 1), (12, 0), (9, 1), (8, 0), (1, 0)])
def test_device_codebook_build_matches_host(max_len, min_freq):
    """The device builder's codebook blob equals, byte for byte, the blob of the
    host builder + upload (lengths, codes, tables); where no code exists the
    device codebook has no code word.  Lengths also against the oracle."""
    hists = _test_histograms(40 + max_len, 48)
    for g in range(0, len(hists), 4):
        group = hists[g:g + 4]
        hd = to_dev(np.concatenate(group).view(np.int64))
        blobs = [lecb.new_codebook_blob(DEV) for _ in group]
        lecb.lecb_build_codebook_device(hd, blobs, max_len, min_freq)
        for h, blob in zip(group, blobs):
            F = oracle.codebook_frequencies([h], min_freq)
            m = int((F > 0).sum())
            got = lecb.lecb_codebook_download(blob)
            if m == 0 or m > (1 << max_len):
                assert not got.lengths().any()
                continue
            assert np.array_equal(got.lengths(), oracle.package_merge_lengths(F, max_len))
            ref = lecb.new_codebook_blob(DEV)
            lecb.lecb_codebook_upload(lecb.lecb_build_codebook(h, max_len, min_freq), ref)
            assert torch.equal(blob, ref)


def test_device_codebook_special_cases():
    cases = [np.zeros(256, np.uint64)]
    one = np.zeros(256, np.uint64); one[77] = 5; cases.append(one)
    two = np.zeros(256, np.uint64); two[3] = 1; two[200] = 1 << 40; cases.append(two)
    cases.append(np.ones(256, np.uint64))
    hd = to_dev(np.concatenate(cases).view(np.int64))
    blobs = [lecb.new_codebook_blob(DEV) for _ in cases]
    for g in range(0, 4):
        lecb.lecb_build_codebook_device(hd[256 * g:], blobs[g:g + 1], 16, 0)
    ln = [lecb.lecb_codebook_download(b).lengths() for b in blobs]
    assert not ln[0].any()
    assert ln[1][77] == 1 and ln[1].sum() == 1
    assert ln[2][3] == 1 and ln[2][200] == 1 and ln[2].sum() == 2
    assert np.all(ln[3] == 8)
    # empty codebook: an encode with it reports the uncoded byte
    xd = torch.zeros(4096, dtype=torch.uint8, device=DEV)
    out = torch.empty(lecb.lecb_encoded_bound(4096, 4096), dtype=torch.uint8, device=DEV)
    res = lecb.new_results(1, DEV)
    lecb.lecb_encode(xd, 4096, blobs[0], 4096, out, res, lecb.new_workspace(4096, 4096, DEV))
    assert int(lecb.results_to_numpy(res)[0]["status"]) == lecb.LECB_ERR_UNCODED_SYMBOL


@pytest.mark.parametrize("n,chunk", [(1, 256), (300_001, 16384), ((1 << 20) + 3, 65536)])
def test_pertensor_nosync_entries(n, chunk):
    """bf16, snapshot-delta and fp32 per-tensor encodes with device-built
    codebooks: streams and lengths equal the oracle's."""
    _say(f"per-tensor nosync n={n} chunk={chunk}")
    cap = lecb.lecb_encoded_bound(n, chunk)
    ws = lecb.new_workspace(n, chunk, DEV)
    # bf16
    x = workloads.bf16_weights(n)
    ref = oracle.encode_bf16(x, chunk)
    hist = torch.zeros(512, dtype=torch.int64, device=DEV)
    bh, bl = lecb.new_codebook_blob(DEV), lecb.new_codebook_blob(DEV)
    oh = torch.empty(cap, dtype=torch.uint8, device=DEV)
    ol = torch.empty(cap, dtype=torch.uint8, device=DEV)
    res = lecb.new_results(2, DEV)
    lecb.lecb_encode_bf16_pertensor_nosync(to_dev(x.view(np.int16)), n, chunk, 16, hist, bh, bl, oh, ol, res, ws)
    r = lecb.results_to_numpy(res)
    assert np.array_equal(lecb.lecb_codebook_download(bh).lengths(), ref["len_hi"])
    assert np.array_equal(lecb.lecb_codebook_download(bl).lengths(), ref["len_lo"])
    assert np.array_equal(oh[: int(r[0]["bytes"])].cpu().numpy(), ref["stream_hi"])
    assert np.array_equal(ol[: int(r[1]["bytes"])].cpu().numpy(), ref["stream_lo"])
    # snapshot delta from the two snapshots
    d, w0, w1 = workloads.bf16_delta(n, return_snapshots=True)
    ref = oracle.encode_bf16(d, chunk)
    lecb.lecb_encode_bf16_delta_pertensor_nosync(to_dev(w0.view(np.int16)), to_dev(w1.view(np.int16)), n, chunk,
                                                 16, hist, bh, bl, oh, ol, res, ws)
    r = lecb.results_to_numpy(res)
    assert np.array_equal(oh[: int(r[0]["bytes"])].cpu().numpy(), ref["stream_hi"])
    assert np.array_equal(ol[: int(r[1]["bytes"])].cpu().numpy(), ref["stream_lo"])
    # fp32
    x = workloads.fp32_weights(n)
    ref = oracle.encode_fp32(x, chunk)
    h4 = torch.zeros(1024, dtype=torch.int64, device=DEV)
    blobs = [lecb.new_codebook_blob(DEV) for _ in range(4)]
    outs = [torch.empty(cap, dtype=torch.uint8, device=DEV) for _ in range(4)]
    res4 = lecb.new_results(4, DEV)
    lecb.lecb_encode_fp32_pertensor_nosync(to_dev(x.view(np.int32)), n, chunk, 16, h4, blobs, outs, res4, ws)
    r = lecb.results_to_numpy(res4)
    for p in range(4):
        assert int(r[p]["status"]) == 0
        assert np.array_equal(lecb.lecb_codebook_download(blobs[p]).lengths(), ref["len"][p])
        assert np.array_equal(outs[p][: int(r[p]["bytes"])].cpu().numpy(), ref["stream"][p])


# ----------------------------------------------------------------------------- 32-bit elements, four planes

@pytest.mark.parametrize("n", [1, 3, 4099, 1 << 20])
def test_histogram_and_merge_fp32_exact(n):
    _say(f"fp32 histogram/merge n={n}")
    x = workloads.fp32_weights(n)
    xd = to_dev(x.view(np.int32))
    hist = torch.zeros(1024, dtype=torch.int64, device=DEV)
    lecb.lecb_histogram_fp32(xd, hist)
    h = hist.cpu().numpy().astype(np.uint64)
    planes = oracle.split_fp32(x)
    for p in range(4):
        assert np.array_equal(h[256 * p:256 * (p + 1)], oracle.histogram(planes[p])), p
    lecb.lecb_histogram_fp32(xd, hist, accumulate=True)
    assert np.array_equal(hist.cpu().numpy().astype(np.uint64), 2 * h)
    pd = [to_dev(pl) for pl in planes]
    out = torch.empty(n, dtype=torch.int32, device=DEV)
    lecb.lecb_merge_fp32(pd, out)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), x)


@pytest.mark.parametrize("n,chunk", [(1, 256), (5000, 4096), (300_001, 16384), ((1 << 20) + 7, 65536)])
def test_fp32_pertensor_pipeline(n, chunk):
    """Four byte planes: histograms, codebooks and all four streams equal the
    oracle's; both decode entries restore the 32-bit elements exactly."""
    _say(f"fp32 per-tensor n={n} chunk={chunk}")
    x = workloads.fp32_weights(n)
    ref = oracle.encode_fp32(x, chunk)
    xd = to_dev(x.view(np.int32))
    hist = torch.zeros(1024, dtype=torch.int64, device=DEV)
    blobs = [lecb.new_codebook_blob(DEV) for _ in range(4)]
    cap = lecb.lecb_encoded_bound(n, chunk)
    outs = [torch.empty(cap, dtype=torch.uint8, device=DEV) for _ in range(4)]
    res = lecb.new_results(4, DEV)
    ws = lecb.new_workspace(n, chunk, DEV)
    cbs = lecb.lecb_encode_fp32_pertensor(xd, n, chunk, 16, hist, blobs, outs, res, ws)
    r = lecb.results_to_numpy(res)
    for p in range(4):
        assert int(r[p]["status"]) == 0, p
        assert np.array_equal(cbs[p].lengths(), ref["len"][p]), p
        assert int(r[p]["payload_bits"]) == ref["bits"][p], p
        assert np.array_equal(outs[p][: int(r[p]["bytes"])].cpu().numpy(), ref["stream"][p]), p
    out = torch.empty(n, dtype=torch.int32, device=DEV)
    rd = lecb.new_results(4, DEV)
    lecb.lecb_decode_fp32_from_results(outs, res, blobs, chunk, n, out, rd, ws)
    q = lecb.results_to_numpy(rd)
    assert all(int(q[p]["status"]) == 0 for p in range(4))
    assert [int(q[p]["payload_bits"]) for p in range(4)] == ref["bits"]
    assert np.array_equal(out.cpu().numpy().view(np.uint32), x)
    out.zero_()
    lecb.lecb_decode_fp32(outs, [int(r[p]["bytes"]) for p in range(4)], blobs, chunk, n, out, rd, ws)
    assert all(int(v) == 0 for v in lecb.results_to_numpy(rd)["status"])
    assert np.array_equal(out.cpu().numpy().view(np.uint32), x)


def test_fp32_fixed_codebooks_and_corrupt_plane():
    """lecb_encode_fp32 with given codebooks (one per plane) and a corrupted
    third stream: that plane's status is CORRUPT, the others stay OK."""
    n, chunk = 70_000, 4096
    x = workloads.fp32_weights(n)
    planes = oracle.split_fp32(x)
    lens = [codebook_for(pl, clamp=True) for pl in planes]
    blobs = [lecb.DeviceCodebook.upload(lecb.lecb_codebook_from_lengths(ln), DEV).blob for ln in lens]
    xd = to_dev(x.view(np.int32))
    cap = lecb.lecb_encoded_bound(n, chunk)
    outs = [torch.empty(cap, dtype=torch.uint8, device=DEV) for _ in range(4)]
    res = lecb.new_results(4, DEV)
    ws = lecb.new_workspace(n, chunk, DEV)
    lecb.lecb_encode_fp32(xd, n, blobs, chunk, outs, res, ws)
    r = lecb.results_to_numpy(res)
    for p in range(4):
        want, _ = oracle.encode(planes[p], lens[p], oracle.canonical_codes(lens[p]), chunk)
        assert np.array_equal(outs[p][: int(r[p]["bytes"])].cpu().numpy(), want), p
    # a chunk-table entry past the payload: plane 2's stream is corrupt
    outs[2][0:4] = torch.tensor([255, 255, 255, 127], dtype=torch.uint8, device=DEV)
    out = torch.empty(n, dtype=torch.int32, device=DEV)
    rd = lecb.new_results(4, DEV)
    lecb.lecb_decode_fp32(outs, [int(r[p]["bytes"]) for p in range(4)], blobs, chunk, n, out, rd, ws)
    st = [int(v) for v in lecb.results_to_numpy(rd)["status"]]
    assert st[2] == lecb.LECB_ERR_CORRUPT and st[0] == st[1] == st[3] == 0


# ----------------------------------------------------------------------------- drift refresh

@pytest.mark.parametrize("tol", [0, 20_000, 10**9])
def test_adaptive_encode_over_drifting_batches(tol):
    """lecb_encode_adaptive over batches whose spread grows: the refresh
    decisions are the oracle's, every batch's stream is bit-exact to the
    oracle's with the codebook it chose, and it decodes back."""
    _say(f"adaptive encode tol={tol}")
    rng = np.random.default_rng(21)
    n, chunk = 200_003, 4096
    batches = [np.clip(np.rint(rng.normal(0, 8 + 6 * k, n)), -128, 127).astype(np.int8).view(np.uint8)
               for k in range(6)]
    hists = [oracle.histogram(b) for b in batches]
    first = oracle.package_merge_lengths(oracle.codebook_frequencies(hists[:1], 1), 16)
    want = oracle.adaptive_codebooks(hists, first, 16, tol)
    cb = lecb.lecb_codebook_from_lengths(first)
    cb.max_len = 16
    blob = lecb.new_codebook_blob(DEV)
    lecb.lecb_codebook_upload(cb, blob)
    hist = torch.zeros(256, dtype=torch.int64, device=DEV)
    out = torch.empty(lecb.lecb_encoded_bound(n, chunk), dtype=torch.uint8, device=DEV)
    res = lecb.new_results(1, DEV)
    ws = lecb.new_workspace(n, chunk, DEV)
    y = torch.empty(n, dtype=torch.uint8, device=DEV)
    rd = lecb.new_results(1, DEV)
    for b, (r_o, use_o, _, _) in zip(batches, want):
        refreshed = lecb.lecb_encode_adaptive(to_dev(b), n, chunk, 16, tol, hist, cb, blob, out, res, ws)
        assert refreshed == r_o
        assert np.array_equal(cb.lengths(), use_o)
        rr = lecb.results_to_numpy(res)[0]
        assert int(rr["status"]) == 0
        ref, _ = oracle.encode(b, use_o, oracle.canonical_codes(use_o), chunk)
        assert np.array_equal(out[: int(rr["bytes"])].cpu().numpy(), ref)
        lecb.lecb_decode_from_result(out, res, blob, chunk, n, y, rd, ws)
        assert int(lecb.results_to_numpy(rd)[0]["status"]) == 0
        assert np.array_equal(y.cpu().numpy(), b)


# ----------------------------------------------------------------------------- decode workgroup sizes

def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _big_workgroups(n, chunk, waves_per_cu_needed=16, nstreams=1, planes_per_wave=1):
    """Whether the decoder picks its big workgroups: a wave decodes 4 rows of 16
    lanes (4 / planes_per_wave row groups of 16 / G chunks), and big workgroups
    are taken when the waves of all streams give every compute unit
    `waves_per_cu_needed` of them."""
    G = min(chunk // 256, 16)
    cpt = (4 // planes_per_wave) * (16 // G)
    tasks = -(-(-(-n // chunk)) // cpt)
    return tasks * (nstreams if planes_per_wave == 1 else 1) >= _cus() * waves_per_cu_needed


def _gpu_stream_against_oracle_blocks(xd, x, ln, chunk, dcb):
    """GPU encode of x, the stream compared chunk by chunk with the oracle's
    streams of blocks of x (oracle in worker processes); returns the stream."""
    n = x.size
    out = torch.empty(lecb.lecb_encoded_bound(n, chunk), dtype=torch.uint8, device=DEV)
    res = lecb.new_results(1, DEV)
    ws = lecb.new_workspace(n, chunk, DEV)
    step = 1 << 22
    with oracle_jobs.pool() as pool:
        jobs = pool.map_async(oracle_jobs.plane_blocks, [(i, x[i:i + step], ln, chunk) for i in range(0, n, step)])
        lecb.lecb_encode(xd, n, dcb.blob, chunk, out, res, ws)
        r = lecb.results_to_numpy(res)[0]
        assert int(r["status"]) == 0
        got = out[: int(r["bytes"])].cpu().numpy()
        covered = sum(oracle_jobs.check_blocks(got, n, chunk, blocks, off) for off, blocks in jobs.get())
    assert covered == oracle.num_chunks(n, chunk)
    return out, r


@pytest.mark.parametrize("big,chunk,n", [(False, 4096, 300_007), (False, 65536, 700_001), (False, 256, 50_001),
                                         (False, 1024, 77_777), (True, 4096, None)])
def test_decode_every_workgroup_size(big, chunk, n):
    """The decoder picks 4-wave or 16-wave workgroups from the size of the job
    (no override); inputs sized so that each is chosen decode the oracle's
    stream exactly (ragged tails, chunks of 1, 4 and 16 lanes).  The big case
    decodes the GPU stream after comparing every chunk of it with the oracle."""
    if n is None:
        n = _cus() * 16 * 16384 + 4099
    assert _big_workgroups(n, chunk) == big
    _say(f"decode big={big} n={n} chunk={chunk}")
    x = _gauss(40 + chunk % 97, n, 12.0)
    ln = codebook_for(x, True)
    dcb = lecb.DeviceCodebook.upload(lecb.lecb_codebook_from_lengths(ln), DEV)
    if not big:
        ref, _ = oracle.encode(x, ln, oracle.canonical_codes(ln), chunk)
        got, r = gpu_decode(ref, dcb, chunk, n)
        assert int(r["status"]) == 0
        assert np.array_equal(got, x)
        return
    xd = to_dev(x)
    out, r = _gpu_stream_against_oracle_blocks(xd, x, ln, chunk, dcb)
    y = torch.empty(n, dtype=torch.uint8, device=DEV)
    rd = lecb.new_results(1, DEV)
    lecb.lecb_decode(out, int(r["bytes"]), dcb.blob, chunk, n, y, rd, lecb.new_workspace(n, chunk, DEV))
    assert int(lecb.results_to_numpy(rd)[0]["status"]) == 0
    assert torch.equal(y, xd)


@pytest.mark.parametrize("big", [False, True])
def test_bf16_two_plane_decode_workgroup_sizes(big):
    """Both planes decoded in one launch, as two byte planes and fused into
    16-bit words (plain and snapshot delta), at the small and the big
    workgroup size of each kernel."""
    chunk = 16384 if not big else 4096
    n = 1_000_003 if not big else _cus() * 8 * 16384 + 3
    assert _big_workgroups(n, chunk, nstreams=2) == big
    _say(f"two-plane decode big={big} n={n}")
    x = workloads.bf16_weights(n)
    hi, lo = oracle.split_bf16(x)
    lens = [codebook_for(p, False) for p in (hi, lo)]
    bh = lecb.DeviceCodebook.upload(lecb.lecb_codebook_from_lengths(lens[0]), DEV)
    bl = lecb.DeviceCodebook.upload(lecb.lecb_codebook_from_lengths(lens[1]), DEV)
    streams = []
    for p, ln, dcb in ((hi, lens[0], bh), (lo, lens[1], bl)):
        if big:
            out, r = _gpu_stream_against_oracle_blocks(to_dev(p), p, ln, chunk, dcb)
            streams.append((out, int(r["bytes"])))
        else:
            ref, _ = oracle.encode(p, ln, oracle.canonical_codes(ln), chunk)
            buf = torch.zeros(ref.size + 32, dtype=torch.uint8, device=DEV)
            buf[: ref.size] = to_dev(ref)
            streams.append((buf, ref.size))
    oh = torch.empty((n + 15) // 16 * 16, dtype=torch.uint8, device=DEV)
    ol = torch.empty_like(oh)
    res = lecb.new_results(2, DEV)
    ws = lecb.new_workspace(n, chunk, DEV)
    lecb.lecb_decode_bf16_planes(streams[0][0], streams[0][1], streams[1][0], streams[1][1], bh.blob, bl.blob,
                                 chunk, n, oh, ol, res, ws)
    r = lecb.results_to_numpy(res)
    assert int(r[0]["status"]) == 0 and int(r[1]["status"]) == 0
    assert np.array_equal(oh[:n].cpu().numpy(), hi) and np.array_equal(ol[:n].cpu().numpy(), lo)
    del oh, ol
    # the fused restores (both planes in every wave, 16-bit words out) pick
    # their own workgroup size: 12 waves when every CU gets 12 of them
    assert _big_workgroups(n, chunk, 12, planes_per_wave=2) == big
    xd = to_dev(x.view(np.int16))
    y = torch.empty(n, dtype=torch.int16, device=DEV)
    rd = lecb.new_results(2, DEV)
    lecb.lecb_decode_bf16(streams[0][0], streams[0][1], streams[1][0], streams[1][1], bh.blob, bl.blob, chunk, n,
                          y, rd, ws)
    assert all(int(v) == 0 for v in lecb.results_to_numpy(rd)["status"])
    assert torch.equal(y, xd)
    # snapshot delta: the streams are read as W0 ^ W1 with W0 drawn here
    w0 = to_dev(np.random.default_rng(77).integers(0, 1 << 16, n, dtype=np.uint16).view(np.int16))
    lecb.lecb_decode_bf16_delta(streams[0][0], streams[0][1], streams[1][0], streams[1][1], bh.blob, bl.blob,
                                chunk, n, w0, y, rd, ws)
    assert all(int(v) == 0 for v in lecb.results_to_numpy(rd)["status"])
    assert torch.equal(y, w0 ^ xd)


# ----------------------------------------------------------------------------- sizes on the device

@pytest.mark.parametrize("n,chunk", [(1, 256), (100_003, 4096), (1 << 20, 65536)])
def test_decode_from_encoder_result(n, chunk):
    """Encode then decode with the size read on the device: no host round trip."""
    _say(f"decode from result n={n} chunk={chunk}")
    x = workloads.skewed_bytes(5, n)
    ln = codebook_for(x, True)
    dcb = lecb.DeviceCodebook.upload(lecb.lecb_codebook_from_lengths(ln), DEV)
    xd = to_dev(x)
    out, res = lecb.encode_bytes(xd, dcb, chunk)
    y = torch.empty(max(16, n), dtype=torch.uint8, device=DEV)
    rd = lecb.new_results(1, DEV)
    ws = lecb.new_workspace(n, chunk, DEV)
    lecb.lecb_decode_from_result(out, res, dcb.blob, chunk, n, y, rd, ws)
    r, q = lecb.results_to_numpy(res)[0], lecb.results_to_numpy(rd)[0]
    assert int(q["status"]) == 0 and int(q["bytes"]) == int(r["bytes"])
    assert int(q["payload_bits"]) == int(r["payload_bits"])
    assert np.array_equal(y[:n].cpu().numpy(), x)


def test_decode_from_failed_encode_is_corrupt():
    """A failed encode leaves a result the decoder refuses, without a host check."""
    x = _gauss(18, 50_000, 3.0)
    ln = codebook_for(x, False)
    x[25_000] = np.uint8(np.flatnonzero(ln == 0)[0])  # a byte value with no code word
    dcb = lecb.DeviceCodebook.upload(lecb.lecb_codebook_from_lengths(ln), DEV)
    out, res = lecb.encode_bytes(to_dev(x), dcb, 4096)
    assert int(lecb.results_to_numpy(res)[0]["status"]) == lecb.LECB_ERR_UNCODED_SYMBOL
    y = torch.empty(x.size, dtype=torch.uint8, device=DEV)
    rd = lecb.new_results(1, DEV)
    ws = lecb.new_workspace(x.size, 4096, DEV)
    lecb.lecb_decode_from_result(out, res, dcb.blob, 4096, x.size, y, rd, ws)
    assert int(lecb.results_to_numpy(rd)[0]["status"]) == lecb.LECB_ERR_CORRUPT


@pytest.mark.parametrize("n,chunk", [(300_001, 16384), ((1 << 20) + 3, 65536)])
def test_bf16_decode_from_encoder_results(n, chunk):
    _say(f"bf16 decode from results n={n} chunk={chunk}")
    x = workloads.bf16_weights(n)
    xd = to_dev(x.view(np.int16))
    hist = torch.zeros(512, dtype=torch.int64, device=DEV)
    bh, bl = lecb.new_codebook_blob(DEV), lecb.new_codebook_blob(DEV)
    cap = lecb.lecb_encoded_bound(n, chunk)
    oh = torch.empty(cap, dtype=torch.uint8, device=DEV)
    ol = torch.empty(cap, dtype=torch.uint8, device=DEV)
    res = lecb.new_results(2, DEV)
    ws = lecb.new_workspace(n, chunk, DEV)
    lecb.lecb_encode_bf16_pertensor(xd, n, chunk, 16, hist, bh, bl, oh, ol, res, ws)
    y = torch.empty(n, dtype=torch.int16, device=DEV)
    rd = lecb.new_results(2, DEV)
    lecb.lecb_decode_bf16_from_results(oh, ol, res, bh, bl, chunk, n, y, rd, ws)
    q = lecb.results_to_numpy(rd)
    assert int(q[0]["status"]) == 0 and int(q[1]["status"]) == 0
    assert torch.equal(y, xd)


# ----------------------------------------------------------------------------- device-side errors

def test_uncoded_symbol_sets_status():
    x = _gauss(17, 10_000, 3.0)
    ln = codebook_for(x, False)
    x2 = x.copy()
    x2[5000] = np.uint8(np.flatnonzero(ln == 0)[0])  # a byte value with no code word
    assert ln[x2[5000]] == 0
    got, r, _ = gpu_encode(x2, ln, 4096)
    assert int(r["status"]) == lecb.LECB_ERR_UNCODED_SYMBOL


def test_capacity_overflow_sets_status():
    x = workloads.uniform_bytes(18, 50_000)
    ln = codebook_for(x, True)
    dcb = lecb.DeviceCodebook.upload(lecb.lecb_codebook_from_lengths(ln), DEV)
    small = torch.empty(lecb.lecb_header_bytes(x.size, 4096) + 64, dtype=torch.uint8, device=DEV)
    out, res = lecb.encode_bytes(to_dev(x), dcb, 4096, out=small)
    assert int(lecb.results_to_numpy(res)[0]["status"]) == lecb.LECB_ERR_CAPACITY


def test_corrupt_streams_set_status():
    x = _gauss(19, 4096 * 6 + 100, 12.0)
    ln = codebook_for(x, True)
    ref, _ = oracle.encode(x, ln, oracle.canonical_codes(ln), 4096)
    dcb = lecb.DeviceCodebook.upload(lecb.lecb_codebook_from_lengths(ln), DEV)
    nc = oracle.num_chunks(x.size, 4096)
    tb = oracle.table_bytes(x.size, 4096)
    hb = oracle.header_bytes(x.size, 4096)
    bad = {}
    t = ref.copy(); t[0:4] = 0; bad["zero end"] = t
    t = ref.copy(); e = t[:4 * nc].view("<u4").copy(); e[1], e[2] = e[2], e[1]; t[:4 * nc] = e.view(np.uint8); bad["non-monotone"] = t
    t = ref.copy(); t[4 * nc] = 1; bad["table padding"] = t
    # lane word counts: one word moved from lane 0 to lane 1 of chunk 0 (same
    # chunk total); a word given to an empty lane of the last chunk (100
    # symbols: lanes 7..15 are empty) and taken from its lane 0
    t = ref.copy(); u = t[tb:tb + 4].view("<u2").copy(); u[0] -= 1; u[1] += 1
    t[tb:tb + 4] = u.view(np.uint8); bad["word count moved"] = t
    t = ref.copy(); lw = t[tb + 2 * 16 * (nc - 1): tb + 2 * 16 * nc].view("<u2").copy(); lw[0] -= 1; lw[15] += 1
    t[tb + 2 * 16 * (nc - 1): tb + 2 * 16 * nc] = lw.view(np.uint8); bad["empty lane word"] = t
    t = ref.copy(); u = t[tb:tb + 2].view("<u2").copy(); u[0] += 1
    t[tb:tb + 2] = u.view(np.uint8); bad["word count total"] = t
    t = ref.copy(); t[hb + 40:hb + 48] ^= 0xFF; bad["payload bits"] = t
    t = ref.copy(); t[hb:hb + 4], t[hb + 4:hb + 8] = ref[hb + 4:hb + 8], ref[hb:hb + 4]; bad["words swapped"] = t
    # chunk 256 (one lane per chunk): the zero padding after the word counts
    x2 = _gauss(20, 256 * 5 + 7, 12.0)
    ref2, _ = oracle.encode(x2, ln, oracle.canonical_codes(ln), 256)
    t = ref2.copy(); t[oracle.header_bytes(x2.size, 256) - 1] = 1
    cases = [(name, t, x, 4096) for name, t in bad.items()] + [("word count padding", t, x2, 256)]
    for name, t, xx, chunk in cases:
        _say(f"corrupt case {name}")
        try:
            oracle.decode(t, ln, chunk, xx.size)
            oracle_bad = False
        except oracle.CorruptStream:
            oracle_bad = True
        y, r = gpu_decode(t, dcb, chunk, xx.size)
        # the two decoders accept and reject exactly the same streams
        assert (int(r["status"]) == lecb.LECB_ERR_CORRUPT) == oracle_bad, name
        if name not in ("payload bits", "words swapped"):
            assert oracle_bad, name
        elif not oracle_bad:
            assert np.array_equal(y, oracle.decode(t, ln, chunk, xx.size))
    # a size below the header is rejected on the host
    with pytest.raises(lecb.LecbError):
        gpu_decode(ref[: hb - 4], dcb, 4096, x.size)


# ----------------------------------------------------------------------------- tensor-level helpers

@pytest.mark.parametrize("n,chunk", [(1, 256), (70_001, 16384)])
def test_tensor_helpers_and_container(n, chunk):
    """encode / decode on uint8 tensors, and the per-tensor bf16 container:
    byte-identical to the oracle's container, decoded back exactly."""
    _say(f"tensor helpers n={n} chunk={chunk}")
    x = workloads.bf16_weights(n)
    t = to_dev(x.view(np.int16)).view(torch.bfloat16)
    buf = lecb.encode_bf16(t, chunk)
    assert np.array_equal(buf, oracle.container_bytes(oracle.encode_bf16(x, chunk)))
    y = lecb.decode_bf16(buf, DEV)
    assert np.array_equal(y.cpu().numpy().view(np.uint16), x)
    b = workloads.int8_fixed(0, n)
    ln = codebook_for(b, clamp=True)
    dcb = lecb.DeviceCodebook.upload(lecb.lecb_codebook_from_lengths(ln), DEV)
    s, res = lecb.encode(to_dev(b), dcb, chunk)
    r = lecb.results_to_numpy(res)[0]
    want, _ = oracle.encode(b, ln, oracle.canonical_codes(ln), chunk)
    assert np.array_equal(s[: int(r["bytes"])].cpu().numpy(), want)
    out, rd = lecb.decode(s, int(r["bytes"]), dcb, chunk, n)
    assert int(lecb.results_to_numpy(rd)[0]["status"]) == 0
    assert np.array_equal(out[:n].cpu().numpy(), b)
