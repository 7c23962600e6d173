#!/usr/bin/env python3
"""Throughput bench of the Huffman byte codec on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

One step = one pass of the whole coding path over one synthetic tensor, with
inputs resident in HBM:

* fixed codebook (default ``int8_drift``: 64 batches of 64 Mi int8 symbols,
  sigma 10 -> 40, coded as one 4 GiB call with batch 0's codebook, chunk
  4096; also ``int8_fixed``, ``int8_acts``, ``int4_packed``): encode +
  decode with a codebook built once beforehand (untimed, as in single-stage
  coding);
* per-tensor bf16 (``bf16_weights``: 64 Mi bf16 elements, chunk 16384;
  ``bf16_delta``): plane histograms -> codebooks built on the device ->
  encode both byte planes -> decode both planes (stream sizes read on the
  device) -> restore the 16-bit words;
* per-tensor fp32 (``fp32_weights``): the same with four byte planes.

Prints ONE JSON line.  Every timed step follows a 1 GiB device write (outside
its HIP events), so no step finds its input or streams in the 256 MB
Infinity Cache; ``value`` = uncompressed bytes / median step time (GB/s,
1e9), and the per-kernel times behind encode / decode rates and the roofline
of the dominant kernel are medians of the same steps.  The same steps run back
to back are reported beside them as ``warm_cache``.  The CPU oracle baseline
runs on worker processes over all host cores, started before the GPU is
touched (median of three runs when a run takes under a minute).  The timed
outputs are checked on the device before anything is reported (exact round
trip, statuses, payload bits = sum of count x code length, a well-formed chunk
table); the element-by-element parity against the oracle at the same sizes
and launch configuration is in the GPU tests.
"""

from __future__ import annotations

import argparse
import json
import multiprocessing as mp
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

DEVICE_LABELS = ("histogram", "codebook_build", "encode_pair", "decode_pair")
HOST_LABELS = ("histogram+codebooks", "encode_pair", "decode_pair")
METRIC = "encode / decode GB/s of uncompressed input on 1 MI355X; % of HBM peak; ratio"
HBM_PEAK_GBPS = 8000.0


# ============================================================================ CPU oracle baseline
# Runs in spawned worker processes that import numpy + the oracle only.

def _cpu_worker(args):
    import oracle

    kind, data, lengths, chunk = args
    t0 = time.perf_counter()
    if kind == "bytes":
        ln = lengths[0]
        s, _ = oracle.encode(data, ln, oracle.canonical_codes(ln), chunk)
        t1 = time.perf_counter()
        y = oracle.decode(s, ln, chunk, data.size)
        t2 = time.perf_counter()
        assert np.array_equal(y, data)
    else:
        planes = oracle.split_bf16(data) if kind == "bf16" else oracle.split_fp32(data)
        ss = []
        for plane, ln in zip(planes, lengths):
            ss.append(oracle.encode(plane, ln, oracle.canonical_codes(ln), chunk)[0])
        t1 = time.perf_counter()
        ys = [oracle.decode(s, ln, chunk, data.size) for s, ln in zip(ss, lengths)]
        t2 = time.perf_counter()
        merged = oracle.merge_bf16(*ys) if kind == "bf16" else oracle.merge_fp32(ys)
        assert np.array_equal(merged, data)
    return t1 - t0, t2 - t1


def _cpu_sample(cfg: dict, x: np.ndarray, sample_elems: int) -> tuple:
    """The bounded sample the oracle codes: the first sample_elems elements, or
    for the drift stream the same number taken as equal runs of whole chunks
    from the start of every batch (so every sigma is represented)."""
    chunk = cfg["chunk"]
    if cfg.get("batches") and sample_elems < x.size:
        B = x.size // cfg["batches"]
        per = max(chunk, sample_elems // cfg["batches"] // chunk * chunk)
        pieces = [x[k * B:k * B + per] for k in range(cfg["batches"])]
        return pieces, (f"{per} symbols from the start of each of the {cfg['batches']} batches "
                        f"({per * cfg['batches']} symbols in all)")
    return [x[:sample_elems]], f"first {min(sample_elems, x.size)} elements of the same tensor"


def cpu_baseline(cfg: dict, x: np.ndarray, hist, sample_elems: int, pool, cores: int) -> dict:
    """Oracle encode + decode of a bounded sample, split over chunk ranges across all host cores."""
    import oracle

    chunk = cfg["chunk"]
    pieces, what = _cpu_sample(cfg, x, sample_elems)
    t0 = time.perf_counter()
    if cfg["kind"] == "u8":
        # fixed codebook, built once from the warm-up statistics (not timed)
        lengths = [oracle.package_merge_lengths(oracle.codebook_frequencies([hist], 1), 16)]
        t_build = 0.0
    else:
        # per-tensor mode: the histograms and codebooks are part of the encode
        sample = pieces[0]
        planes = oracle.split_bf16(sample) if cfg["kind"] == "bf16" else oracle.split_fp32(sample)
        lengths = [oracle.package_merge_lengths(oracle.histogram(p), 16) for p in planes]
        t_build = time.perf_counter() - t0
    kind = "bytes" if cfg["kind"] == "u8" else cfg["kind"]
    total = sum(p.size for p in pieces)
    per = -(-total // cores)
    per = -(-per // chunk) * chunk
    jobs = []
    for piece in pieces:
        for i in range(0, piece.size, per):
            jobs.append((kind, piece[i:i + per], lengths, chunk))
    runs = []
    for _ in range(3):
        t0 = time.perf_counter()
        times = pool.map(_cpu_worker, jobs)
        wall = time.perf_counter() - t0
        # wall-clock of the whole map (every worker encodes, then decodes its
        # jobs); split into encode and decode by the workers' summed phase times
        se, sd = sum(t[0] for t in times), sum(t[1] for t in times)
        runs.append((wall + t_build, (wall * se / (se + sd)) + t_build, wall * sd / (se + sd)))
        if wall > 60:
            break
    nbytes = total * x.itemsize
    used = min(cores, len(jobs))
    i = int(np.argsort([r[0] for r in runs])[len(runs) // 2])
    tot, enc, dec = runs[i]
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": round(nbytes / tot / 1e9, 4),
        "unit": "GB/s",
        "cores": used,
        "kind": "oracle",
        "sample": f"{what} ({nbytes} bytes), {len(jobs)} jobs over chunk ranges on {used} worker processes",
        "encode_GBps": round(nbytes / enc / 1e9, 4),
        "decode_GBps": round(nbytes / dec / 1e9, 4),
        "runs": len(runs),
        "statistic": "median of the runs" if len(runs) > 1 else "one run (over a minute)",
        "wall_s": round(runs[i][0], 2),
        "cpu_model": cpu_model,
    }


# ============================================================================ inputs

def _drift_batch(args):
    k, batch = args
    return k, workloads.int8_drift_batch(k, batch)


def make_input(name: str, scale: float, pool, cache_dir=None):
    cfg = dict(workloads.CONFIGS[name])
    cfg["name"] = name
    n = int(cfg["n"] * scale)
    n = max(cfg["chunk"], n // cfg["chunk"] * cfg["chunk"]) if scale < 1 else cfg["n"]
    cfg["n"] = n
    lengths = None
    if name == "int8_fixed":
        x = workloads.int8_fixed(0, n)
        warm = [np.bincount(workloads.int8_fixed(r, n), minlength=256) for r in (1, 2, 3, 4)]
        hist = np.sum(warm, axis=0).astype(np.uint64)
    elif name == "int8_acts":
        rows = n // 2048
        x = workloads.int8_acts(0, rows)
        warm = [np.bincount(workloads.int8_acts(r, rows), minlength=256) for r in (1, 2, 3, 4)]
        hist = np.sum(warm, axis=0).astype(np.uint64)
    elif name == "int4_packed":
        # 4-bit weights, two per byte: the byte (an ordered pair of 4-bit values) is the symbol
        x = workloads.int4_packed(0, n)
        warm = [np.bincount(workloads.int4_packed(r, n), minlength=256) for r in (1, 2, 3, 4)]
        hist = np.sum(warm, axis=0).astype(np.uint64)
    elif name == "int8_drift":
        batch = min(workloads.BLOCK, n)
        cfg["batches"] = n // batch
        t0 = time.perf_counter()
        cached = os.path.join(cache_dir, f"int8_drift_{cfg['batches']}x{batch}.npy") if cache_dir else None
        if cached and os.path.exists(cached):
            x = np.load(cached)
        else:
            x = np.empty(cfg["batches"] * batch, dtype=np.uint8)
            jobs = [(k, batch) for k in range(cfg["batches"])]
            # the 64 batches are drawn in the worker processes (same recipe,
            # same seeds), or here one after the other when there are none
            for k, xb in (pool.imap_unordered(_drift_batch, jobs) if pool else map(_drift_batch, jobs)):
                x[k * batch:(k + 1) * batch] = xb
            if cached:
                os.makedirs(cache_dir, exist_ok=True)
                np.save(cached, x)
        cfg["generate_s"] = round(time.perf_counter() - t0, 2)
        cfg["n"] = n = x.size
        # one fixed codebook from batch 0, every byte coded
        hist = np.bincount(x[:batch], minlength=256).astype(np.uint64)
    elif name == "bf16_weights":
        x = workloads.bf16_weights(n)
        hist = None
    elif name == "fp32_weights":
        x = workloads.fp32_weights(n)
        hist = None
    elif name == "bf16_delta":
        # the delta is coded; the snapshots feed the fused leg (W0, W1 -> streams -> W1)
        x, cfg["w0"], cfg["w1"] = workloads.bf16_delta(n, return_snapshots=True)
        hist = None
    else:
        raise SystemExit(f"unknown config {name}")
    return cfg, x, hist


# ============================================================================ GPU runs

class Timer:
    """HIP events on the launch stream, one list of (start, stop) per label."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def start(self, label):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.setdefault(label, []).append([e, None])

    def stop(self, label):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs[label][-1][1] = e

    def chain(self, labels):
        """Record events at the boundaries of consecutive launches: returns a
        function to call after each one (label i spans boundary i to i + 1)."""
        first = self.torch.cuda.Event(enable_timing=True)
        first.record()
        state = {"prev": first, "i": 0}

        def mark():
            e = self.torch.cuda.Event(enable_timing=True)
            e.record()
            self.pairs.setdefault(labels[state["i"]], []).append([state["prev"], e])
            state["prev"] = e
            state["i"] += 1

        return mark

    def mean_ms(self, label, skip=0):
        ps = self.pairs.get(label, [])[skip:]
        return float(np.mean([a.elapsed_time(b) for a, b in ps])) if ps else 0.0


def run_gpu(cfg, x, hist, steps, warmup, lengths_out):
    import torch
    import lossless_entropy_coding_byte_amd as lecb

    dev = "cuda:0"
    torch.cuda.set_device(0)
    chunk, n = cfg["chunk"], cfg["n"]
    T = Timer(torch)
    info = {}
    if cfg["kind"] == "bf16":
        xd = torch.from_numpy(x.view(np.int16)).to(dev)
        hist_d = torch.zeros(512, dtype=torch.int64, device=dev)
        blob_hi, blob_lo = lecb.new_codebook_blob(dev), lecb.new_codebook_blob(dev)
        cap = lecb.lecb_encoded_bound(n, chunk)
        out_hi = torch.empty(cap, dtype=torch.uint8, device=dev)
        out_lo = torch.empty(cap, dtype=torch.uint8, device=dev)
        res = lecb.new_results(2, dev)
        res_dec = lecb.new_results(2, dev)
        ws = lecb.new_workspace(n, chunk, dev)
        y = torch.empty(n, dtype=torch.int16, device=dev)
        state = {}

        def step_device(tm):
            # the per-tensor path kernel by kernel -- what
            # lecb_encode_bf16_pertensor_nosync and lecb_decode_bf16_from_results
            # enqueue -- with events on the launch stream between the kernels:
            # histograms -> codebooks built on the device -> two-plane encode ->
            # two-plane decode that writes the 16-bit words (stream sizes read on
            # the device).  No host synchronisation anywhere in the step.
            mark = tm.chain(DEVICE_LABELS)
            lecb.lecb_histogram_bf16(xd, hist_d[:256], hist_d[256:])
            mark()
            lecb.lecb_build_codebook_device(hist_d, [blob_hi, blob_lo])
            mark()
            tail(mark)

        def step_host(tm):
            # the same with the codebooks built on the host: histograms -> read
            # back -> package-merge -> upload (what lecb_encode_bf16_pertensor does)
            mark = tm.chain(HOST_LABELS)
            lecb.lecb_pertensor_codebooks(xd, n, 16, hist_d, [blob_hi, blob_lo])
            mark()
            tail(mark)

        def tail(mark):
            lecb.lecb_encode_bf16(xd, n, blob_hi, blob_lo, chunk, out_hi, out_lo, res, ws)
            mark()
            lecb.lecb_decode_bf16_from_results(out_hi, out_lo, res, blob_hi, blob_lo, chunk, n, y, res_dec, ws)
            mark()

        def codebooks():
            state.update(cb_hi=lecb.lecb_codebook_download(blob_hi), cb_lo=lecb.lecb_codebook_download(blob_lo))

        nbytes = 2 * n
    elif cfg["kind"] == "fp32":
        xd = torch.from_numpy(x.view(np.int32)).to(dev)
        hist_d = torch.zeros(1024, dtype=torch.int64, device=dev)
        blobs = [lecb.new_codebook_blob(dev) for _ in range(4)]
        cap = lecb.lecb_encoded_bound(n, chunk)
        outs = [torch.empty(cap, dtype=torch.uint8, device=dev) for _ in range(4)]
        res = lecb.new_results(4, dev)
        res_dec = lecb.new_results(4, dev)
        ws = lecb.new_workspace(n, chunk, dev)
        y = torch.empty(n, dtype=torch.int32, device=dev)
        state = {}

        def step_device(tm):
            # kernel by kernel, as lecb_encode_fp32_pertensor_nosync and
            # lecb_decode_fp32_from_results enqueue it: histograms -> four
            # codebooks built on the device -> two two-plane encodes -> one
            # four-plane decode that writes the elements (sizes read on the device)
            mark = tm.chain(DEVICE_LABELS)
            lecb.lecb_histogram_fp32(xd, hist_d)
            mark()
            lecb.lecb_build_codebook_device(hist_d, blobs)
            mark()
            tail(mark)

        def step_host(tm):
            mark = tm.chain(HOST_LABELS)
            lecb.lecb_pertensor_codebooks(xd, n, 16, hist_d, blobs)
            mark()
            tail(mark)

        def tail(mark):
            lecb.lecb_encode_fp32(xd, n, blobs, chunk, outs, res, ws)
            mark()
            lecb.lecb_decode_fp32_from_results(outs, res, blobs, chunk, n, y, res_dec, ws)
            mark()

        def codebooks():
            state.update(cbs=[lecb.lecb_codebook_download(b) for b in blobs])

        nbytes = 4 * n
    else:
        xd = torch.from_numpy(x).to(dev)
        cb = lecb.lecb_build_codebook(hist, 16, 1)
        dcb = lecb.DeviceCodebook.upload(cb, dev)
        cap = lecb.lecb_encoded_bound(n, chunk)
        out = torch.empty(cap, dtype=torch.uint8, device=dev)
        res = lecb.new_results(1, dev)
        res_dec = lecb.new_results(1, dev)
        ws = lecb.new_workspace(n, chunk, dev)
        y = torch.empty(n, dtype=torch.uint8, device=dev)
        state = {"cb": cb}

        def step_device(tm):
            tm.start("encode")
            lecb.lecb_encode(xd, n, dcb.blob, chunk, out, res, ws)
            tm.stop("encode")
            tm.start("decode")
            lecb.lecb_decode_from_result(out, res, dcb.blob, chunk, n, y, res_dec, ws)
            tm.stop("decode")

        step_host = None

        def codebooks():
            pass

        nbytes = n

    # per-tensor mode has two codebook paths: built on the device (timed,
    # no host synchronisation in the step) and built on the host (histogram
    # read-back; timed afterwards for the report)
    variants = {"device": step_device}
    if step_host is not None:
        variants["host"] = step_host
    chosen = "device"
    step = lambda: variants[chosen](T)  # noqa: E731
    flush = torch.empty(1 << 28, dtype=torch.int32, device=dev)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # Timed steps, cold cache: the 256 MB Infinity Cache would hold the smaller
    # workloads' inputs and streams between steps, so every step follows a
    # 1 GiB device write, outside the step's events.  HIP events on the launch
    # stream bracket each step and each kernel; the median step is the figure.
    Tc = Timer(torch)
    cold_pairs = []
    t0 = time.perf_counter()
    for i in range(steps):
        flush.fill_(i)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        variants[chosen](Tc)
        e1.record()
        cold_pairs.append((e0, e1))
    torch.cuda.synchronize()
    cold_wall = time.perf_counter() - t0
    cold_ms = [a.elapsed_time(b) for a, b in cold_pairs]
    cold_kernels = {lb: float(np.median([a.elapsed_time(b) for a, b in ps])) for lb, ps in Tc.pairs.items()}
    del flush
    # Warm cache, labelled as such: the same K steps back to back.
    T.pairs.clear()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    warm_wall = time.perf_counter() - t0
    warm = {
        "what": "the same steps back to back, inputs and streams left in the caches (not the headline)",
        "ms_per_step": round(warm_wall / steps * 1e3, 4),
        "kernels_ms_mean": {lb: round(T.mean_ms(lb), 4) for lb in T.pairs},
    }
    warm["GBps"] = None  # filled in by main() (needs the byte count)
    other_ms = None
    if len(variants) > 1:
        other = [v for v in variants if v != chosen][0]
        # the other path ends with the same streams (both build the same codebooks)
        for _ in range(warmup):
            variants[other](Timer(torch))
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(steps):
            variants[other](Timer(torch))
        torch.cuda.synchronize()
        other_ms = {other: round((time.perf_counter() - t1) / steps * 1e3, 4)}
    codebooks()

    # ---------------- checks of the timed outputs, on the device and through the
    # library only (the element-by-element parity against the oracle at these
    # sizes and in this launch configuration is in the GPU tests)
    rd = lecb.results_to_numpy(res_dec)
    r = lecb.results_to_numpy(res)
    parity = {"round_trip": bool(torch.equal(y.view(-1)[: n], xd.view(-1)[: n])),
              "device_status": [int(v) for v in list(r["status"]) + list(rd["status"])]}
    if cfg["kind"] == "fp32":
        h4 = torch.zeros(1024, dtype=torch.int64, device=dev)
        lecb.lecb_histogram_fp32(xd, h4)
        h4n = h4.cpu().numpy().astype(np.uint64)
        hists = [h4n[256 * k:256 * (k + 1)] for k in range(4)]
        names = ["byte3", "byte2", "byte1", "byte0"]
        streams = [(outs[k], r[k], state["cbs"][k]) for k in range(4)]
        sizes = [int(r[k]["bytes"]) for k in range(4)]
        container = sum(sizes)
    elif cfg["kind"] == "bf16":
        hh = torch.zeros(256, dtype=torch.int64, device=dev)
        hl = torch.zeros(256, dtype=torch.int64, device=dev)
        lecb.lecb_histogram_bf16(xd, hh, hl)
        hists = [hh.cpu().numpy().astype(np.uint64), hl.cpu().numpy().astype(np.uint64)]
        names = ["hi", "lo"]
        streams = [(out_hi, r[0], state["cb_hi"]), (out_lo, r[1], state["cb_lo"])]
        sizes = [int(r[0]["bytes"]), int(r[1]["bytes"])]
        container = 560 + (sizes[0] + 15) // 16 * 16 + sizes[1]
    else:
        hx = torch.zeros(256, dtype=torch.int64, device=dev)
        lecb.lecb_histogram(xd, hx)
        hists = [hx.cpu().numpy().astype(np.uint64)]
        names = ["bytes"]
        streams = [(out, r[0], state["cb"])]
        sizes = [int(r[0]["bytes"])]
        container = sizes[0]
    lengths_out.extend([cbx.lengths() for _, _, cbx in streams])
    # payload bits = sum over bytes of count x code length, and a well-formed
    # chunk table: strictly increasing word ends, the last one at the stream end
    nc = lecb.lecb_num_chunks(n, chunk)
    hb = lecb.lecb_header_bytes(n, chunk)
    ident, table_ok = True, True
    for (buf, rr, cbx), h in zip(streams, hists):
        ident &= lecb.lecb_stream_stats(h, cbx.lengths(), 16)["payload_bits"] == int(rr["payload_bits"])
        table = buf[: 4 * nc].cpu().numpy().view("<u4").astype(np.int64)
        table_ok &= bool(np.all(np.diff(np.concatenate([[0], table])) > 0))
        table_ok &= hb + 4 * int(table[-1]) == int(rr["bytes"])
    parity["payload_bits_identity"] = bool(ident)
    parity["chunk_table_well_formed"] = bool(table_ok)

    # ---------------- fused snapshot leg: encode from (W0, W1), decode to W1;
    # the delta is never written (its streams are the ones timed above)
    fused = None
    if cfg.get("w0") is not None:
        w0d = torch.from_numpy(cfg["w0"].view(np.int16)).to(dev)
        w1d = torch.from_numpy(cfg["w1"].view(np.int16)).to(dev)
        w1_out = torch.empty_like(w1d)

        def fused_step():
            T.start("fused_encode")
            lecb.lecb_encode_bf16_delta_pertensor_nosync(w0d, w1d, n, chunk, 16, hist_d, blob_hi, blob_lo,
                                                         out_hi, out_lo, res, ws)
            T.stop("fused_encode")
            T.start("fused_decode")
            lecb.lecb_decode_bf16_delta_from_results(out_hi, out_lo, res, blob_hi, blob_lo, chunk, n, w0d,
                                                     w1_out, res_dec, ws)
            T.stop("fused_decode")

        fused_step()
        torch.cuda.synchronize()
        T.pairs.pop("fused_encode", None)
        T.pairs.pop("fused_decode", None)
        reps = max(3, min(steps, 10))
        t0 = time.perf_counter()
        for _ in range(reps):
            fused_step()
        torch.cuda.synchronize()
        fw = (time.perf_counter() - t0) / reps
        fe, fd = T.mean_ms("fused_encode"), T.mean_ms("fused_decode")
        T.pairs.pop("fused_encode", None)
        T.pairs.pop("fused_decode", None)
        rr, rq = lecb.results_to_numpy(res), lecb.results_to_numpy(res_dec)
        same = [int(v["bytes"]) for v in rr] == sizes
        fused = {
            "what": "W0, W1 -> delta streams -> W1 (XOR fused into the histogram, the encode and the decode's restore)",
            "step_ms": round(fw * 1e3, 4), "encode_ms": round(fe, 4), "decode_ms": round(fd, 4),
            "GBps_snapshot": round(2 * n / fw / 1e9, 2),
            "round_trip": bool(torch.equal(w1_out, w1d)),
            "streams_equal_delta_streams": bool(same),
            "status": [int(v) for v in list(rr["status"]) + list(rq["status"])],
        }
        parity["fused_delta_ok"] = fused["round_trip"] and same and not any(fused["status"])
        del w0d, w1d, w1_out

    # ---------------- timings (cold-cache medians)
    ms_step = float(np.median(cold_ms))
    kernels = {label: v for label, v in cold_kernels.items() if label not in ("encode", "decode")}
    if cfg["kind"] in ("bf16", "fp32"):
        enc_ms = sum(kernels[lb] for lb in kernels if lb in ("histogram", "codebook_build", "histogram+codebooks",
                                                              "encode_pair"))
        dec_ms = kernels["decode_pair"]
    else:
        enc_ms, dec_ms = cold_kernels["encode"], cold_kernels["decode"]
    cold = {
        "flush_bytes_before_each_step": 1 << 30,
        "ms_per_step_median": round(ms_step, 4),
        "ms_per_step_min": round(float(np.min(cold_ms)), 4),
        "wall_s_of_the_timed_steps_with_flushes": round(cold_wall, 4),
        "kernels_ms_median": {lb: round(v, 4) for lb, v in cold_kernels.items()},
    }
    # ---------------- size accounting per stream (histogram kernel + host stats)
    accounting = []
    for name, h, ln in zip(names, hists, lengths_out):
        st = lecb.lecb_stream_stats(h, ln, 16)
        accounting.append({
            "stream": name,
            "bits_per_symbol": round(st["payload_bits"] / st["n"], 5),
            "entropy_bits": round(st["shannon_bits"] / st["n"], 5),
            "gap_vs_shannon": round(st["payload_bits"] / max(st["shannon_bits"], 1e-9) - 1, 5),
            "gap_vs_per_batch_optimal": round(st["payload_bits"] / max(st["optimal_bits"], 1) - 1, 5),
        })
    subbyte = None
    if cfg["name"] == "int4_packed":
        # the other 4-bit reading, for comparison: every 4-bit value its own
        # symbol, optimal 16-symbol code of at most 8 bits on this tensor
        xb = x.view(np.uint8)
        hn = (np.bincount(xb & 15, minlength=256) + np.bincount(xb >> 4, minlength=256)).astype(np.uint64)
        cbn = lecb.lecb_build_codebook(hn, 8, 0)
        stn = lecb.lecb_stream_stats(hn, cbn.lengths(), 8)
        subbyte = {
            "values": int(2 * n),
            "bits_per_value_pairs": round(int(r[0]["payload_bits"]) / (2 * n), 5),
            "bits_per_value_16_symbol_code": round(stn["payload_bits"] / (2 * n), 5),
            "entropy_bits_per_value": round(stn["shannon_bits"] / (2 * n), 5),
        }
    batches = None
    if cfg.get("batches"):
        # drift stream: each batch against its own optimal code and entropy
        B = n // cfg["batches"]
        hb_ = torch.zeros(256, dtype=torch.int64, device=dev)
        rows = []
        for k in range(cfg["batches"]):
            lecb.lecb_histogram(xd[k * B:(k + 1) * B], hb_)
            st = lecb.lecb_stream_stats(hb_.cpu().numpy().astype(np.uint64), lengths_out[0], 16)
            rows.append((st["payload_bits"], st["optimal_bits"], st["shannon_bits"]))
        rows = np.array(rows, dtype=np.float64)
        ratio = 8.0 * B / rows[:, 0]
        gap_opt = rows[:, 0] / rows[:, 1] - 1
        gap_h = rows[:, 0] / rows[:, 2] - 1
        batches = {
            "count": int(cfg["batches"]), "symbols_each": int(B),
            "ratio_first_last": [round(float(ratio[0]), 4), round(float(ratio[-1]), 4)],
            "ratio_min_max": [round(float(ratio.min()), 4), round(float(ratio.max()), 4)],
            "gap_vs_per_batch_optimal_first_last": [round(float(gap_opt[0]), 5), round(float(gap_opt[-1]), 5)],
            "gap_vs_per_batch_optimal_max": round(float(gap_opt.max()), 5),
            "gap_vs_shannon_first_last": [round(float(gap_h[0]), 5), round(float(gap_h[-1]), 5)],
            "per_batch_ratio": [round(float(v), 4) for v in ratio],
        }
        # the same batches through the refresh rule (lecb_encode_adaptive,
        # tolerance 1 %): histogram, host decision, rebuild when needed, encode
        tol = 10_000
        cb_a = lecb.lecb_codebook_from_lengths(lengths_out[0])
        cb_a.max_len = 16
        blob_a = lecb.new_codebook_blob(dev)
        lecb.lecb_codebook_upload(cb_a, blob_a)
        hist_a = torch.zeros(256, dtype=torch.int64, device=dev)
        out_a = torch.empty(lecb.lecb_encoded_bound(B, chunk), dtype=torch.uint8, device=dev)
        res_a = lecb.new_results(1, dev)
        ws_a = lecb.new_workspace(B, chunk, dev)
        refreshes, bits_a, status_a = 0, 0, 0
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(cfg["batches"]):
            refreshes += lecb.lecb_encode_adaptive(xd[k * B:(k + 1) * B], B, chunk, 16, tol, hist_a, cb_a,
                                                   blob_a, out_a, res_a, ws_a)
            ra = lecb.results_to_numpy(res_a)[0]
            bits_a += int(ra["payload_bits"])
            status_a |= int(ra["status"])
        t_a = time.perf_counter() - t0
        batches["adaptive"] = {
            "rule": "refresh when the batch costs more than tol over its best fixed codebook",
            "tol_ppm": tol, "refreshes": int(refreshes), "status": status_a,
            "payload_ratio": round(8.0 * B * cfg["batches"] / bits_a, 4),
            "payload_ratio_fixed": round(8.0 * B * cfg["batches"] / float(rows[:, 0].sum()), 4),
            "payload_vs_fixed": round(bits_a / float(rows[:, 0].sum()) - 1, 5),
            "payload_vs_per_batch_optimal": round(bits_a / float(rows[:, 1].sum()) - 1, 5),
            "encode_GBps_with_decisions": round(B * cfg["batches"] / t_a / 1e9, 2),
        }
    batched = None
    if cfg["name"] == "int8_fixed" and n == workloads.CONFIGS["int8_fixed"]["n"]:
        # supplement, not the headline: one 1 Mi call is launch-latency bound,
        # so 64 independent eval batches (2^20 % chunk == 0: batch boundaries
        # are chunk boundaries) go through one encode and one decode call with
        # the same fixed codebook
        nb = 64
        xb = np.concatenate([workloads.int8_fixed_batch(b, n) for b in range(nb)])
        xbd = torch.from_numpy(xb).to(dev)
        N = xb.size
        out_b = torch.empty(lecb.lecb_encoded_bound(N, chunk), dtype=torch.uint8, device=dev)
        res_b, resd_b = lecb.new_results(1, dev), lecb.new_results(1, dev)
        ws_b = lecb.new_workspace(N, chunk, dev)
        y_b = torch.empty(N, dtype=torch.uint8, device=dev)
        Tb = Timer(torch)

        def batched_step():
            Tb.start("encode")
            lecb.lecb_encode(xbd, N, dcb.blob, chunk, out_b, res_b, ws_b)
            Tb.stop("encode")
            Tb.start("decode")
            lecb.lecb_decode_from_result(out_b, res_b, dcb.blob, chunk, N, y_b, resd_b, ws_b)
            Tb.stop("decode")

        for _ in range(warmup):
            batched_step()
        torch.cuda.synchronize()
        Tb.pairs.clear()
        t0 = time.perf_counter()
        for _ in range(steps):
            batched_step()
        torch.cuda.synchronize()
        wb = (time.perf_counter() - t0) / steps
        eb, db = Tb.mean_ms("encode"), Tb.mean_ms("decode")
        rb, rdb = lecb.results_to_numpy(res_b)[0], lecb.results_to_numpy(resd_b)[0]
        batched = {
            "what": "supplement: 64 independent 1 Mi eval batches coded by one call each way (not the headline)",
            "elements": int(N), "ms_per_step": round(wb * 1e3, 4),
            "value_GBps": round(N / wb / 1e9, 2),
            "encode_GBps": round(N / (eb * 1e-3) / 1e9, 2), "decode_GBps": round(N / (db * 1e-3) / 1e9, 2),
            "encode_frac_of_hbm": round((N + int(rb["bytes"])) / (eb * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "decode_frac_of_hbm": round((N + int(rb["bytes"])) / (db * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "ratio": round(N / int(rb["bytes"]), 4),
            "round_trip": bool(torch.equal(y_b, xbd)),
            "status": [int(rb["status"]), int(rdb["status"])],
        }
        parity["batched_ok"] = batched["round_trip"] and not any(batched["status"])
        del xbd, out_b, ws_b, y_b
    info.update(
        batched=batched,
        fused=fused,
        batches=batches,
        subbyte=subbyte,
        codebook_path=chosen if cfg["kind"] in ("bf16", "fp32") else None,
        cold=cold,
        warm=warm,
        other_ms=other_ms,
        accounting=accounting,
        nbytes=nbytes, ms_step=ms_step, enc_ms=enc_ms, dec_ms=dec_ms, kernels=kernels,
        sizes=sizes, container=container, parity=parity,
        payload_bits=[int(v["payload_bits"]) for v in r],
    )
    return info


KERNEL_SOURCES = {"encode": "kernels_encode.hip", "encode_pair": "kernels_encode.hip",
                  "decode": "kernels_decode.hip", "decode_pair": "kernels_decode.hip",
                  "histogram": "kernels_misc.hip"}


# headers every kernel source includes (a change there changes the kernels too)
KERNEL_HEADERS = ("lanes.hpp", "lecb_internal.hpp")


def source_sha(label):
    """SHA-256 over the kernel's source file and the shared headers, in that order."""
    import hashlib

    h = hashlib.sha256()
    for name in (KERNEL_SOURCES[label],) + KERNEL_HEADERS:
        with open(os.path.join(ROOT, "lossless_entropy_coding_byte_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, label):
    """HBM bytes per launch of `label` from profiles/traffic.json (rocprofv3
    FETCH_SIZE / WRITE_SIZE runs scaled by the copy-kernel calibration), or
    None when there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload, {}).get(label)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != source_sha(label):
        return None
    return rec.get("traffic_bytes")


def roofline(cfg, info):
    """Dominant kernel's achieved algorithmic GB/s against the 8 TB/s HBM peak."""
    n = cfg["n"]
    k = info["kernels"]
    if cfg["kind"] == "bf16":
        s_hi, s_lo = info["sizes"]
        algo = {
            # the pair encode reads the 16-bit words once and writes both streams
            "encode_pair": 2 * n + s_hi + s_lo,
            # the two-plane decode reads both streams and writes the 16-bit words
            "decode_pair": s_hi + s_lo + 2 * n,
            "histogram": 2 * n,
        }
    elif cfg["kind"] == "fp32":
        # encode: two launch pairs (bytes 3, 2 and bytes 1, 0); decode: one
        # four-plane launch; the algorithmic bytes are those of the whole
        # four-plane operation
        S = sum(info["sizes"])
        algo = {"encode_pair": 4 * n + S, "decode_pair": S + 4 * n, "histogram": 4 * n}
    else:
        s = info["sizes"][0]
        algo = {"encode": n + s, "decode": s + n}
        k = {"encode": info["enc_ms"], "decode": info["dec_ms"]}
    dom = max((lbl for lbl in k if lbl in algo), key=lambda lbl: k[lbl])
    ach = algo[dom] / (k[dom] * 1e-3) / 1e9
    per_kernel = {lbl: {"ms": round(k[lbl], 4), "GBps": round(algo[lbl] / (k[lbl] * 1e-3) / 1e9, 1),
                        "frac": round(algo[lbl] / (k[lbl] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
                  for lbl in k if lbl in algo and k[lbl] > 0}
    if k.get("codebook_build"):
        # one workgroup per plane, latency-bound: time only
        per_kernel["codebook_build"] = {"ms": round(k["codebook_build"], 4)}
    return {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(cfg["name"], dom),
            "algorithmic_bytes_per_launch": int(algo[dom])}, per_kernel


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="int8_drift", choices=list(workloads.CONFIGS))
    ap.add_argument("--scale", type=float, default=1.0, help="fraction of the config's size (tests)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workers", action="store_true",
                    help="no worker processes (inputs drawn in this process, no CPU baseline): for profilers")
    ap.add_argument("--inputs-cache", default=None, metavar="DIR",
                    help="keep the drawn 4 GiB drift stream in DIR as .npy and reuse it on later runs")
    ap.add_argument("--cpu-sample", type=int, default=1 << 26,
                    help="elements the oracle baseline codes (spread over the batches of the drift stream)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 3 device-to-device copies of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch

        src = torch.ones(args.calibrate_copy << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_mib": args.calibrate_copy, "copies": 3}))
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the codec shards by whole chunks; see the multi-GPU notes of the design)", file=sys.stderr)
        sys.exit(2)

    # Worker processes first: they start before this process touches the GPU,
    # draw the long inputs in parallel and run the CPU oracle baseline.  Under
    # a profiler that sets up the GPU before the program starts there must be
    # no worker processes (--no-workers: inputs drawn here, no baseline).
    cores = len(os.sched_getaffinity(0))
    cpu = None
    if args.no_workers:
        cfg, x, hist = make_input(args.config, args.scale, None, args.inputs_cache)
    else:
        with mp.get_context("spawn").Pool(cores) as pool:
            cfg, x, hist = make_input(args.config, args.scale, pool, args.inputs_cache)
            if not args.no_cpu_baseline:
                cpu = cpu_baseline(cfg, x, hist, min(args.cpu_sample, x.size), pool, cores)

    lengths = []
    info = run_gpu(cfg, x, hist, args.steps, args.warmup, lengths)
    roof, per_kernel = roofline(cfg, info)
    nbytes = info["nbytes"]
    value = nbytes / (info["ms_step"] * 1e-3) / 1e9
    enc_gbps = nbytes / (info["enc_ms"] * 1e-3) / 1e9
    dec_gbps = nbytes / (info["dec_ms"] * 1e-3) / 1e9
    ok = (info["parity"]["round_trip"] and info["parity"]["payload_bits_identity"]
          and info["parity"]["chunk_table_well_formed"]
          and not any(info["parity"]["device_status"]) and info["parity"].get("fused_delta_ok", True)
          and info["parity"].get("batched_ok", True))
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(info["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": args.config, "elements": cfg["n"], "element_bytes": x.itemsize,
                   "chunk": cfg["chunk"], "mode": cfg["mode"], "max_len": 16,
                   **({"batches": cfg["batches"], "generate_s": cfg.get("generate_s")} if cfg.get("batches") else {})},
        "encode_GBps": round(enc_gbps, 2),
        "decode_GBps": round(dec_gbps, 2),
        "encode_ms": round(info["enc_ms"], 4),
        "decode_ms": round(info["dec_ms"], 4),
        "ratio": round(nbytes / info["container"], 4),
        "bits_per_symbol": [round(b / cfg["n"], 4) for b in info["payload_bits"]],
        "accounting": info["accounting"],
        "batches": info["batches"],
        "batched_1mi": info["batched"],
        "fused_delta": info["fused"],
        "int4": info["subbyte"],
        "pertensor_codebooks": info["codebook_path"],
        "timing": "cold cache: a 1 GiB device write before every timed step (outside its events); "
                  "value, ms_per_step, encode/decode and roofline are medians of those steps",
        "cold_cache": dict(info["cold"], GBps_median=round(value, 2)),
        "warm_cache": dict(info["warm"], GBps=round(nbytes / (info["warm"]["ms_per_step"] * 1e-3) / 1e9, 2)),
        "strict_frac_of_hbm": {"encode": round(enc_gbps / HBM_PEAK_GBPS, 4), "decode": round(dec_gbps / HBM_PEAK_GBPS, 4)},
        "pertensor_other_codebooks_ms_per_step": info["other_ms"],
        "kernels": per_kernel,
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity": info["parity"],
        "parity_ok": bool(ok),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
