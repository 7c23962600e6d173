"""The workloads at their full sizes, on the launch path the bench times, with
EVERY chunk compared against the oracle.

* int8_fixed, int8_acts, int4_packed, the batched 64 x 1 Mi int8 call,
  bf16_weights and fp32_weights: the whole GPU stream of every plane equals
  the oracle's stream of the whole tensor (one oracle call per plane);
* bf16_delta (512 Mi elements) and int8_drift (4 GiB): the stream is compared
  block by block -- each block of 2^24 symbols (whole chunks) is encoded by
  the oracle alone and must equal the GPU stream's offset-table entries
  (shifted by the block's first payload word), lane word counts and payload
  words of those chunks; the blocks cover every chunk;
* histograms equal the oracle's (np.bincount, summed over blocks for the
  long inputs); code lengths equal the oracle's package-merge lengths;
  payload bits equal the oracle's; GPU decode restores the input exactly.

The oracle runs in worker processes (``oracle_jobs``) while the GPU works.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle_jobs
import workloads
import lossless_entropy_coding_byte_amd as lecb
from gpu_helpers import DEV

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[configs] {msg}", flush=True)


def _host(buf, nbytes):
    return buf[:nbytes].cpu().numpy()


def _fixed_mode(name, x, hist, pool, extra=None):
    """Fixed-codebook encode + decode of x at full size; the whole stream
    against the oracle's (its encode runs in a worker meanwhile)."""
    cfg = workloads.CONFIGS[name]
    n, chunk = x.size, cfg["chunk"]
    _say(f"{name}: n={n} chunk={chunk}")
    ln = oracle.package_merge_lengths(oracle.codebook_frequencies([hist], 1), 16)
    job = pool.apply_async(oracle_jobs.encode, ((x, ln, chunk),))
    cb = lecb.lecb_build_codebook(hist, 16, 1)
    assert np.array_equal(cb.lengths(), ln)
    dcb = lecb.DeviceCodebook.upload(cb, DEV)
    xd = torch.from_numpy(x).to(DEV)
    out = torch.empty(lecb.lecb_encoded_bound(n, chunk), dtype=torch.uint8, device=DEV)
    res = lecb.new_results(1, DEV)
    ws = lecb.new_workspace(n, chunk, DEV)
    lecb.lecb_encode(xd, n, dcb.blob, chunk, out, res, ws)
    r = lecb.results_to_numpy(res)[0]
    assert int(r["status"]) == 0
    hd = torch.zeros(256, dtype=torch.int64, device=DEV)
    lecb.lecb_histogram(xd, hd)
    h = hd.cpu().numpy().astype(np.uint64)
    assert np.array_equal(h, oracle.histogram(x))
    y = torch.empty(n, dtype=torch.uint8, device=DEV)
    rd = lecb.new_results(1, DEV)
    lecb.lecb_decode(out, int(r["bytes"]), dcb.blob, chunk, n, y, rd, ws)
    assert int(lecb.results_to_numpy(rd)[0]["status"]) == 0
    assert torch.equal(y, xd)
    got = _host(out, int(r["bytes"]))
    ref, bits = job.get()
    assert int(r["payload_bits"]) == bits == oracle.payload_bits_identity(h, ln)
    assert np.array_equal(got, ref), f"{name}: stream differs from the oracle's"
    _say(f"{name}: whole stream ({got.size} bytes) equals the oracle's")
    return r, h, ln


def _pertensor(name, x, pool):
    cfg = workloads.CONFIGS[name]
    n, chunk = x.size, cfg["chunk"]
    _say(f"{name}: n={n} chunk={chunk}")
    hi, lo = oracle.split_bf16(x)
    lens = [oracle.package_merge_lengths(oracle.histogram(p), 16) for p in (hi, lo)]
    jobs = [pool.apply_async(oracle_jobs.encode, ((p, ln, chunk),)) for p, ln in zip((hi, lo), lens)]
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
    h = hist.cpu().numpy().astype(np.uint64)
    y = torch.empty(n, dtype=torch.int16, device=DEV)
    rd = lecb.new_results(2, DEV)
    lecb.lecb_decode_bf16(oh, int(r[0]["bytes"]), ol, int(r[1]["bytes"]), bh, bl, chunk, n, y, rd, ws)
    rdn = lecb.results_to_numpy(rd)
    assert int(rdn[0]["status"]) == 0 and int(rdn[1]["status"]) == 0
    assert torch.equal(y, xd)
    for plane, hp, cb, buf, rr, ln, job in ((hi, h[:256], cb_hi, oh, r[0], lens[0], jobs[0]),
                                           (lo, h[256:], cb_lo, ol, r[1], lens[1], jobs[1])):
        assert np.array_equal(hp, oracle.histogram(plane))
        assert np.array_equal(cb.lengths(), ln)
        ref, bits = job.get()
        assert int(rr["payload_bits"]) == bits
        assert np.array_equal(_host(buf, int(rr["bytes"])), ref), f"{name}: plane stream differs"
    _say(f"{name}: both plane streams equal the oracle's")
    return r


def test_config_int8_fixed():
    x = workloads.int8_fixed(0)
    hist = np.sum([oracle.histogram(workloads.int8_fixed(k)) for k in (1, 2, 3, 4)], axis=0, dtype=np.uint64)
    with oracle_jobs.pool() as pool:
        _fixed_mode("int8_fixed", x, hist, pool)


def test_config_int8_fixed_batched():
    """64 independent 1 Mi eval batches coded as one call (the bench's batched
    supplement): the whole 64 Mi stream equals the oracle's, and the chunk
    run of a sampled batch equals the oracle's stream of that batch alone."""
    n1 = workloads.CONFIGS["int8_fixed"]["n"]
    chunk = workloads.CONFIGS["int8_fixed"]["chunk"]
    x = np.concatenate([workloads.int8_fixed_batch(b, n1) for b in range(64)])
    warm = [oracle.histogram(workloads.int8_fixed(r, n1)) for r in (1, 2, 3, 4)]
    hist = np.sum(warm, axis=0, dtype=np.uint64)
    with oracle_jobs.pool() as pool:
        b = 37
        one = workloads.int8_fixed_batch(b, n1)
        assert np.array_equal(one, x[b * n1:(b + 1) * n1])
        ln = oracle.package_merge_lengths(oracle.codebook_frequencies([hist], 1), 16)
        alone = pool.apply_async(oracle_jobs.encode, ((one, ln, chunk),))
        cb = lecb.lecb_build_codebook(hist, 16, 1)
        dcb = lecb.DeviceCodebook.upload(cb, DEV)
        xd = torch.from_numpy(x).to(DEV)
        out = torch.empty(lecb.lecb_encoded_bound(x.size, chunk), dtype=torch.uint8, device=DEV)
        res = lecb.new_results(1, DEV)
        lecb.lecb_encode(xd, x.size, dcb.blob, chunk, out, res, lecb.new_workspace(x.size, chunk, DEV))
        r = lecb.results_to_numpy(res)[0]
        assert int(r["status"]) == 0
        got = _host(out, int(r["bytes"]))
        oracle_jobs.compare_chunk_run(got, x.size, chunk, b * n1 // chunk, alone.get()[0], n1)
        _fixed_mode("int8_fixed", x, hist, pool)


def test_config_bf16_weights():
    with oracle_jobs.pool() as pool:
        _pertensor("bf16_weights", workloads.bf16_weights(), pool)


def test_config_int8_acts():
    x = workloads.int8_acts(0)
    hist = np.sum([oracle.histogram(workloads.int8_acts(k)) for k in (1, 2, 3, 4)], axis=0, dtype=np.uint64)
    with oracle_jobs.pool() as pool:
        _fixed_mode("int8_acts", x, hist, pool)


@pytest.mark.timeout(600)
def test_encode_uneven_ranges_whole_stream():
    """An int8 input of 2^27 + 12345 symbols at chunk 4096: 8193 tasks, more
    than twice the pack launch's waves on a 256-CU GPU, so the count launch
    splits every pack range into sub-ranges, and 8193 tasks over a power of
    two of ranges make the ranges (and sub-ranges) of unequal length.  The
    whole stream equals the oracle's; decode restores the input."""
    n, chunk = (1 << 27) + 12345, 4096
    x = workloads.q8(np.random.default_rng([7, 41]).normal(0, 20.0, n))
    _say(f"uneven ranges: n={n} chunk={chunk}")
    hist = oracle.histogram(x)
    ln = oracle.package_merge_lengths(oracle.codebook_frequencies([hist], 1), 16)
    with oracle_jobs.pool() as pool:
        job = pool.apply_async(oracle_jobs.encode, ((x, ln, chunk),))
        dcb = lecb.DeviceCodebook.upload(lecb.lecb_codebook_from_lengths(ln), DEV)
        xd = torch.from_numpy(x).to(DEV)
        out = torch.empty(lecb.lecb_encoded_bound(n, chunk), dtype=torch.uint8, device=DEV)
        res = lecb.new_results(1, DEV)
        ws = lecb.new_workspace(n, chunk, DEV)
        lecb.lecb_encode(xd, n, dcb.blob, chunk, out, res, ws)
        r = lecb.results_to_numpy(res)[0]
        assert int(r["status"]) == 0
        y = torch.empty(n, dtype=torch.uint8, device=DEV)
        rd = lecb.new_results(1, DEV)
        lecb.lecb_decode(out, int(r["bytes"]), dcb.blob, chunk, n, y, rd, ws)
        assert int(lecb.results_to_numpy(rd)[0]["status"]) == 0
        assert torch.equal(y, xd)
        got = _host(out, int(r["bytes"]))
        ref, bits = job.get()
    assert int(r["payload_bits"]) == bits
    assert np.array_equal(got, ref), "uneven ranges: stream differs from the oracle's"
    _say(f"uneven ranges: whole stream ({got.size} bytes) equals the oracle's")


def test_config_int4_packed():
    """4-bit weights two per byte, coded as packed pairs with a fixed codebook
    from warm-up batches; the pair code of the tensor is never longer than the
    best 16-symbol code of its 4-bit values (oracle)."""
    from oracle import subbyte

    x = workloads.int4_packed(0)
    hist = np.sum([oracle.histogram(workloads.int4_packed(k)) for k in (1, 2, 3, 4)], axis=0, dtype=np.uint64)
    with oracle_jobs.pool() as pool:
        r, h, ln = _fixed_mode("int4_packed", x, hist, pool)
    assert oracle.per_batch_optimal_bits(h, 16) <= subbyte.nibble_code_bits(x, 8)


def test_config_fp32_weights():
    name = "fp32_weights"
    x = workloads.fp32_weights()
    cfg = workloads.CONFIGS[name]
    n, chunk = x.size, cfg["chunk"]
    _say(f"{name}: n={n} chunk={chunk}")
    planes = oracle.split_fp32(x)
    lens = [oracle.package_merge_lengths(oracle.histogram(p), 16) for p in planes]
    with oracle_jobs.pool() as pool:
        jobs = [pool.apply_async(oracle_jobs.encode, ((p, ln, chunk),)) for p, ln in zip(planes, lens)]
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
        y = torch.empty(n, dtype=torch.int32, device=DEV)
        rd = lecb.new_results(4, DEV)
        lecb.lecb_decode_fp32_from_results(outs, res, blobs, chunk, n, y, rd, ws)
        assert all(int(v) == 0 for v in lecb.results_to_numpy(rd)["status"])
        assert torch.equal(y, xd)
        for p in range(4):
            assert int(r[p]["status"]) == 0
            hp = h[256 * p:256 * (p + 1)]
            assert np.array_equal(hp, oracle.histogram(planes[p]))
            assert np.array_equal(cbs[p].lengths(), lens[p])
            ref, bits = jobs[p].get()
            assert int(r[p]["payload_bits"]) == bits
            assert np.array_equal(_host(outs[p], int(r[p]["bytes"])), ref), f"plane {p} differs"
    _say(f"{name}: all four plane streams equal the oracle's")


@pytest.mark.timeout(900)
def test_config_bf16_delta():
    """512 Mi-element snapshot delta: per-tensor codebooks, both planes compared
    block by block; the fused path (W0, W1 -> streams -> W1) gives the same
    streams at full size and restores W1."""
    name = "bf16_delta"
    cfg = workloads.CONFIGS[name]
    n, chunk = cfg["n"], cfg["chunk"]
    B = workloads.BLOCK
    _say(f"{name}: n={n} chunk={chunk}")
    w0 = np.empty(n, np.uint16)
    w1 = np.empty(n, np.uint16)
    with oracle_jobs.pool() as pool:
        for j, a, b in pool.imap_unordered(oracle_jobs.delta_snapshots, range(n // B)):
            w0[j * B:(j + 1) * B] = a
            w1[j * B:(j + 1) * B] = b
        d = w0 ^ w1
        hi, lo = oracle.split_bf16(d)
        lens = [oracle.package_merge_lengths(oracle.histogram(p), 16) for p in (hi, lo)]
        jobs = [pool.apply_async(oracle_jobs.plane_blocks, ((off, p[off:off + B], ln, chunk),))
                for p, ln in zip((hi, lo), lens) for off in range(0, n, B)]
        xd = torch.from_numpy(d.view(np.int16)).to(DEV)
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
        assert np.array_equal(cb_hi.lengths(), lens[0]) and np.array_equal(cb_lo.lengths(), lens[1])
        h = hist.cpu().numpy().astype(np.uint64)
        assert np.array_equal(h[:256], oracle.histogram(hi)) and np.array_equal(h[256:], oracle.histogram(lo))
        y = torch.empty(n, dtype=torch.int16, device=DEV)
        rd = lecb.new_results(2, DEV)
        lecb.lecb_decode_bf16(oh, int(r[0]["bytes"]), ol, int(r[1]["bytes"]), bh, bl, chunk, n, y, rd,
                              ws)
        assert all(int(v) == 0 for v in lecb.results_to_numpy(rd)["status"])
        assert torch.equal(y, xd)
        del y
        # the fused path from the two snapshots: identical streams, W1 restored
        w0d = torch.from_numpy(w0.view(np.int16)).to(DEV)
        w1d = torch.from_numpy(w1.view(np.int16)).to(DEV)
        fh = torch.empty(cap, dtype=torch.uint8, device=DEV)
        fl = torch.empty(cap, dtype=torch.uint8, device=DEV)
        fres = lecb.new_results(2, DEV)
        lecb.lecb_encode_bf16_delta_pertensor(w0d, w1d, n, chunk, 16, hist, bh, bl, fh, fl, fres, ws)
        fr = lecb.results_to_numpy(fres)
        for k, (a, b) in enumerate(((oh, fh), (ol, fl))):
            nb = int(r[k]["bytes"])
            assert int(fr[k]["bytes"]) == nb and int(fr[k]["status"]) == 0
            assert torch.equal(a[:nb], b[:nb]), "fused snapshot stream differs from the delta stream"
        w1o = torch.empty_like(w1d)
        lecb.lecb_decode_bf16_delta(fh, int(fr[0]["bytes"]), fl, int(fr[1]["bytes"]), bh, bl, chunk, n, w0d, w1o, rd, ws)
        assert all(int(v) == 0 for v in lecb.results_to_numpy(rd)["status"])
        assert torch.equal(w1o, w1d)
        del w0d, w1d, w1o, fh, fl
        streams = [_host(oh, int(r[0]["bytes"])), _host(ol, int(r[1]["bytes"]))]
        covered = [0, 0]
        bits = [0, 0]
        for idx, job in enumerate(jobs):
            k = idx // (n // B)
            off, blocks = job.get()
            covered[k] += oracle_jobs.check_blocks(streams[k], n, chunk, blocks, off)
        nc = oracle.num_chunks(n, chunk)
        assert covered == [nc, nc]
        for k, (plane, ln) in enumerate(zip((hi, lo), lens)):
            assert int(r[k]["payload_bits"]) == oracle.payload_bits_identity(oracle.histogram(plane), ln)
    _say(f"{name}: every chunk of both planes equals the oracle's")


@pytest.mark.timeout(900)
def test_config_int8_drift():
    """4 GiB drift stream in one call with batch 0's fixed codebook; every
    chunk compared with the oracle block by block."""
    name = "int8_drift"
    cfg = workloads.CONFIGS[name]
    n, chunk = cfg["n"], cfg["chunk"]
    B = workloads.BLOCK
    _say(f"{name}: n={n} chunk={chunk}")
    hist0 = oracle.histogram(workloads.int8_drift_batch(0, B))
    ln = oracle.package_merge_lengths(oracle.codebook_frequencies([hist0], 1), 16)
    x = np.empty(n, dtype=np.uint8)
    h = np.zeros(256, np.uint64)
    refs = {}
    with oracle_jobs.pool() as pool:
        for k, xb, hb, blocks in pool.imap_unordered(oracle_jobs.drift_batch, [(k, ln, chunk) for k in range(n // B)]):
            x[k * B:(k + 1) * B] = xb
            h += hb
            refs[k] = blocks
    _say(f"{name}: inputs and oracle blocks ready")
    cb = lecb.lecb_build_codebook(hist0, 16, 1)
    assert np.array_equal(cb.lengths(), ln)
    dcb = lecb.DeviceCodebook.upload(cb, DEV)
    xd = torch.from_numpy(x).to(DEV)
    out = torch.empty(lecb.lecb_encoded_bound(n, chunk), dtype=torch.uint8, device=DEV)
    res = lecb.new_results(1, DEV)
    ws = lecb.new_workspace(n, chunk, DEV)
    lecb.lecb_encode(xd, n, dcb.blob, chunk, out, res, ws)
    r = lecb.results_to_numpy(res)[0]
    assert int(r["status"]) == 0
    hd = torch.zeros(256, dtype=torch.int64, device=DEV)
    lecb.lecb_histogram(xd, hd)
    assert np.array_equal(hd.cpu().numpy().astype(np.uint64), h)
    assert int(r["payload_bits"]) == oracle.payload_bits_identity(h, ln)
    y = torch.empty(n, dtype=torch.uint8, device=DEV)
    rd = lecb.new_results(1, DEV)
    lecb.lecb_decode(out, int(r["bytes"]), dcb.blob, chunk, n, y, rd, ws)
    assert int(lecb.results_to_numpy(rd)[0]["status"]) == 0
    assert torch.equal(y, xd)
    del y, xd
    got = _host(out, int(r["bytes"]))
    del out
    covered = sum(oracle_jobs.check_blocks(got, n, chunk, refs[k], k * B) for k in range(n // B))
    assert covered == oracle.num_chunks(n, chunk)
    _say(f"{name}: every chunk ({covered}) equals the oracle's")
