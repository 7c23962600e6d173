"""The workloads at their full sizes, on the launch path the bench times.

Checked against the oracle element by element where it can (the offset table
of every chunk for tensors up to 2^28 elements, and sampled chunks' payload
words and unit gaps encoded one chunk at a time); everywhere else through
properties that hold at any size: exact round trip on the device, status OK,
payload bits = sum(freq * len) from the device histogram.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
import lossless_entropy_coding_byte_amd as lecb
from gpu_helpers import DEV

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[configs] {msg}", flush=True)


def _sampled_parity(buf, plane, lengths, chunk, n, picks, full_table):
    """Stream in `buf` (device) against the oracle on the chunks in `picks`."""
    nc = oracle.num_chunks(n, chunk)
    K = oracle.units_per_chunk(chunk)
    cd = oracle.canonical_codes(lengths)
    tb, hb = oracle.table_bytes(n, chunk), oracle.header_bytes(n, chunk)
    table = buf[: 4 * nc].cpu().numpy().view("<u4").astype(np.int64)
    gaps = buf[tb:tb + (nc * K + 1) // 2].cpu().numpy()
    g = np.empty(2 * gaps.size, np.uint8)
    g[0::2], g[1::2] = gaps & 15, gaps >> 4
    if full_table:
        assert np.array_equal(table, np.cumsum(oracle.chunk_word_counts(plane, lengths, chunk)))
    for c in picks:
        piece = plane[c * chunk:(c + 1) * chunk]
        one, _ = oracle.encode(piece, lengths, cd, chunk)
        s0 = int(table[c - 1]) if c else 0
        assert int(table[c]) - s0 == int(oracle.chunk_word_counts(piece, lengths, chunk)[0])
        words = buf[hb + 4 * s0: hb + 4 * int(table[c])].cpu().numpy()
        assert np.array_equal(words, one[oracle.header_bytes(piece.size, chunk):]), c
        og = one[16:16 + (K + 1) // 2]
        go = np.empty(2 * og.size, np.uint8)
        go[0::2], go[1::2] = og & 15, og >> 4
        assert np.array_equal(g[c * K:(c + 1) * K], go[:K]), c


def _picks(nc, seed):
    r = np.random.default_rng(seed)
    return sorted(set([0, 1, nc // 2, nc - 2, nc - 1] + list(r.integers(0, nc, 8))) - {-1})


def _fixed_mode(name, x, hist):
    cfg = workloads.CONFIGS[name]
    n, chunk = x.size, cfg["chunk"]
    _say(f"{name}: n={n} chunk={chunk}")
    cb = lecb.lecb_build_codebook(hist, 16, 1)
    ln = cb.lengths()
    assert np.array_equal(ln, oracle.package_merge_lengths(oracle.codebook_frequencies([hist], 1), 16))
    dcb = lecb.DeviceCodebook.upload(cb, DEV)
    xd = torch.from_numpy(x).to(DEV)
    out = torch.empty(lecb.lecb_encoded_bound(n, chunk), dtype=torch.uint8, device=DEV)
    res = lecb.new_results(1, DEV)
    ws = lecb.new_workspace(n, chunk, DEV)
    lecb.lecb_encode(xd, n, dcb.blob, chunk, out, res, ws)
    r = lecb.results_to_numpy(res)[0]
    assert int(r["status"]) == 0
    # payload bits = sum(freq * len), histogram from the device
    hd = torch.zeros(256, dtype=torch.int64, device=DEV)
    lecb.lecb_histogram(xd, hd)
    h = hd.cpu().numpy().astype(np.uint64)
    assert np.array_equal(h, oracle.histogram(x)) if n <= (1 << 28) else int(h.sum()) == n
    assert int(r["payload_bits"]) == oracle.payload_bits_identity(h, ln)
    nc = oracle.num_chunks(n, chunk)
    _sampled_parity(out, x, ln, chunk, n, _picks(nc, 7), n <= (1 << 28))
    y = torch.empty(n, dtype=torch.uint8, device=DEV)
    rd = lecb.new_results(1, DEV)
    lecb.lecb_decode(out, int(r["bytes"]), dcb.blob, chunk, n, y, rd, ws)
    assert int(lecb.results_to_numpy(rd)[0]["status"]) == 0
    assert torch.equal(y, xd)
    return r, h, ln


def _pertensor(name, x):
    cfg = workloads.CONFIGS[name]
    n, chunk = x.size, cfg["chunk"]
    _say(f"{name}: n={n} chunk={chunk}")
    xd = torch.from_numpy(x.view(np.int16)).to(DEV)
    hist = torch.zeros(512, dtype=torch.int64, device=DEV)
    bh, bl = lecb.new_codebook_blob(DEV), lecb.new_codebook_blob(DEV)
    cap = lecb.lecb_encoded_bound(n, chunk)
    oh = torch.empty(cap, dtype=torch.uint8, device=DEV)
    ol = torch.empty(cap, dtype=torch.uint8, device=DEV)
    res = lecb.new_results(2, DEV)
    ws = lecb.new_workspace(n, chunk, DEV)
    cb_hi, cb_lo = lecb.lecb_encode_bf16_pertensor(xd, n, chunk, 16, hist, bh, bl, oh, ol, res, ws)
    r = lecb.results_to_numpy(res)
    assert int(r[0]["status"]) == 0 and int(r[1]["status"]) == 0
    hi, lo = oracle.split_bf16(x)
    h = hist.cpu().numpy().astype(np.uint64)
    for plane, hp, cb, buf, rr, seed in ((hi, h[:256], cb_hi, oh, r[0], 11), (lo, h[256:], cb_lo, ol, r[1], 13)):
        assert np.array_equal(hp, oracle.histogram(plane))
        ln = cb.lengths()
        assert np.array_equal(ln, oracle.package_merge_lengths(hp, 16))
        assert int(rr["payload_bits"]) == oracle.payload_bits_identity(hp, ln)
        _sampled_parity(buf, plane, ln, chunk, n, _picks(oracle.num_chunks(n, chunk), seed), n <= (1 << 28))
    y = torch.empty(n, dtype=torch.int16, device=DEV)
    scratch = torch.empty(2 * ((n + 15) // 16 * 16), dtype=torch.uint8, device=DEV)
    rd = lecb.new_results(2, DEV)
    lecb.lecb_decode_bf16(oh, int(r[0]["bytes"]), ol, int(r[1]["bytes"]), bh, bl, chunk, n, y, scratch, rd, ws)
    rdn = lecb.results_to_numpy(rd)
    assert int(rdn[0]["status"]) == 0 and int(rdn[1]["status"]) == 0
    assert torch.equal(y, xd)
    return r


def _pertensor32(name, x):
    cfg = workloads.CONFIGS[name]
    n, chunk = x.size, cfg["chunk"]
    _say(f"{name}: n={n} chunk={chunk}")
    xd = torch.from_numpy(x.view(np.int32)).to(DEV)
    hist = torch.zeros(1024, dtype=torch.int64, device=DEV)
    blobs = [lecb.new_codebook_blob(DEV) for _ in range(4)]
    cap = lecb.lecb_encoded_bound(n, chunk)
    outs = [torch.empty(cap, dtype=torch.uint8, device=DEV) for _ in range(4)]
    res = lecb.new_results(4, DEV)
    ws = lecb.new_workspace(n, chunk, DEV)
    cbs = lecb.lecb_encode_fp32_pertensor(xd, n, chunk, 16, hist, blobs, outs, res, ws)
    r = lecb.results_to_numpy(res)
    h = hist.cpu().numpy().astype(np.uint64)
    planes = oracle.split_fp32(x)
    for p in range(4):
        assert int(r[p]["status"]) == 0
        hp = h[256 * p:256 * (p + 1)]
        assert np.array_equal(hp, oracle.histogram(planes[p]))
        ln = cbs[p].lengths()
        assert np.array_equal(ln, oracle.package_merge_lengths(hp, 16))
        assert int(r[p]["payload_bits"]) == oracle.payload_bits_identity(hp, ln)
        _sampled_parity(outs[p], planes[p], ln, chunk, n, _picks(oracle.num_chunks(n, chunk), 21 + p), True)
    y = torch.empty(n, dtype=torch.int32, device=DEV)
    scratch = torch.empty(4 * ((n + 15) // 16 * 16), dtype=torch.uint8, device=DEV)
    rd = lecb.new_results(4, DEV)
    lecb.lecb_decode_fp32_from_results(outs, res, blobs, chunk, n, y, scratch, rd, ws)
    assert all(int(v) == 0 for v in lecb.results_to_numpy(rd)["status"])
    assert torch.equal(y, xd)
    return r


def test_config_int8_fixed():
    x = workloads.int8_fixed(0)
    hist = np.sum([oracle.histogram(workloads.int8_fixed(k)) for k in (1, 2, 3, 4)], axis=0, dtype=np.uint64)
    _fixed_mode("int8_fixed", x, hist)


def test_config_int8_fixed_batched():
    """64 independent 1 Mi eval batches coded as one call (the bench's batched
    supplement): the fixed-mode checks at 64 Mi, plus the chunk payloads of a
    sampled batch equal the oracle's stream of that batch alone."""
    n1 = workloads.CONFIGS["int8_fixed"]["n"]
    chunk = workloads.CONFIGS["int8_fixed"]["chunk"]
    x = np.concatenate([workloads.int8_fixed_batch(b, n1) for b in range(64)])
    warm = [oracle.histogram(workloads.int8_fixed(r, n1)) for r in (1, 2, 3, 4)]
    hist = np.sum(warm, axis=0, dtype=np.uint64)
    r, _, ln = _fixed_mode("int8_fixed", x, hist)
    # batch 37 alone through the library and through the oracle
    b = 37
    one = workloads.int8_fixed_batch(b, n1)
    assert np.array_equal(one, x[b * n1:(b + 1) * n1])
    ref, _ = oracle.encode(one, ln, oracle.canonical_codes(ln), chunk)
    cb = lecb.lecb_build_codebook(hist, 16, 1)
    assert np.array_equal(cb.lengths(), ln)
    dcb = lecb.DeviceCodebook.upload(cb, DEV)
    xd = torch.from_numpy(x).to(DEV)
    out = torch.empty(lecb.lecb_encoded_bound(x.size, chunk), dtype=torch.uint8, device=DEV)
    res = lecb.new_results(1, DEV)
    lecb.lecb_encode(xd, x.size, dcb.blob, chunk, out, res, lecb.new_workspace(x.size, chunk, DEV))
    nc, cpb = oracle.num_chunks(x.size, chunk), n1 // chunk
    hb = oracle.header_bytes(x.size, chunk)
    table = out[: 4 * nc].cpu().numpy().view("<u4").astype(np.int64)
    s0, s1 = int(table[b * cpb - 1]), int(table[(b + 1) * cpb - 1])
    words = out[hb + 4 * s0: hb + 4 * s1].cpu().numpy()
    assert np.array_equal(words, ref[oracle.header_bytes(n1, chunk):])
    rt = ref[: 4 * cpb].view("<u4").astype(np.int64)
    assert np.array_equal(table[b * cpb:(b + 1) * cpb] - s0, rt)
    # unit gaps: K nibbles per chunk, K even, so a batch's gaps are whole bytes
    K = oracle.units_per_chunk(chunk)
    tb = oracle.table_bytes(x.size, chunk)
    g = out[tb + b * cpb * K // 2: tb + (b + 1) * cpb * K // 2].cpu().numpy()
    tb1 = oracle.table_bytes(n1, chunk)
    assert np.array_equal(g, ref[tb1: tb1 + cpb * K // 2])


def test_config_bf16_weights():
    _pertensor("bf16_weights", workloads.bf16_weights())


def test_config_int8_acts():
    x = workloads.int8_acts(0)
    hist = np.sum([oracle.histogram(workloads.int8_acts(k)) for k in (1, 2, 3, 4)], axis=0, dtype=np.uint64)
    _fixed_mode("int8_acts", x, hist)


@pytest.mark.timeout(600)
def test_config_bf16_delta():
    _pertensor("bf16_delta", workloads.bf16_delta())


@pytest.mark.timeout(900)
def test_config_int8_drift():
    n = workloads.CONFIGS["int8_drift"]["n"]
    B = workloads.BLOCK
    x = np.empty(n, dtype=np.uint8)
    for k in range(n // B):
        x[k * B:(k + 1) * B] = workloads.int8_drift_batch(k, B)
    hist = oracle.histogram(x[:B])  # one codebook from batch 0, every byte coded
    r, h, ln = _fixed_mode("int8_drift", x, hist)
    # the stream expands where the data drift away from batch 0's code
    assert int(r["payload_bits"]) > 0


def test_config_int4_packed():
    """4-bit weights two per byte, coded as packed pairs with a fixed codebook
    from warm-up batches; the pair code of the tensor is never longer than the
    best 16-symbol code of its 4-bit values (oracle)."""
    from oracle import subbyte

    x = workloads.int4_packed(0)
    hist = np.sum([oracle.histogram(workloads.int4_packed(k)) for k in (1, 2, 3, 4)], axis=0, dtype=np.uint64)
    r, h, ln = _fixed_mode("int4_packed", x, hist)
    assert oracle.per_batch_optimal_bits(h, 16) <= subbyte.nibble_code_bits(x, 8)


def test_config_fp32_weights():
    _pertensor32("fp32_weights", workloads.fp32_weights())
