"""The host runtime (codebook builder, refresh rule, size accounting, sizes,
container header) built for the CPU with the host compiler under
AddressSanitizer and UndefinedBehaviorSanitizer, driven through
``host_runtime_check.cpp``: every answer must equal the oracle's and the
sanitizers must stay silent.  CPU only; skipped where the host compiler or its
sanitizer runtimes are missing."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lossless_entropy_coding_byte_amd", "csrc")
ERR_NO_SYMBOLS = -4
ERR_INVALID_ARG = -1


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("host_san") / "host_runtime_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-Wall", "-Wextra", "-Werror", f"-I{ROOT}/include", f"-I{CSRC}",
           os.path.join(CSRC, "codebook.cpp"), os.path.join(CSRC, "host.cpp"),
           os.path.join(ROOT, "tests", "host_runtime_check.cpp"), "-o", exe]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0 and "cannot find" in p.stderr and "asan" in p.stderr:
        pytest.skip("sanitizer runtime not installed")
    assert p.returncode == 0, p.stderr
    return exe


def _run(exe, lines):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    p = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, env=env,
                       timeout=300)
    assert p.returncode == 0, p.stdout[-2000:] + p.stderr[-4000:]
    assert "runtime error" not in p.stderr and "AddressSanitizer" not in p.stderr, p.stderr[-4000:]
    out = p.stdout.splitlines()
    assert out[0] == "edges ok", out[:5]
    assert len(out) == len(lines) + 1
    return [l.split() for l in out[1:]]


def _nums(a):
    return " ".join(str(int(v)) for v in np.asarray(a).ravel())


def _hist(rng, kind):
    h = np.zeros(256, np.uint64)
    m = int(rng.integers(1, 257))
    syms = rng.choice(256, m, replace=False)
    if kind == 0:
        h[syms] = rng.integers(1, 8, m)                     # ties everywhere
    elif kind == 1:
        h[syms] = rng.integers(1, 1 << 40, m)               # wide weights
    elif kind == 2:
        h[syms] = 1 << rng.integers(0, 48, m)               # power-of-two ties, deep trees
    else:
        h[syms] = np.maximum(1, (rng.pareto(0.7, m) * 3).astype(np.int64))
    return h


def test_codebook_builder_and_canonical_codes(checker):
    rng = np.random.default_rng(2024)
    cases, lines = [], []
    for t in range(600):
        h = _hist(rng, t % 4)
        m = int((h > 0).sum())
        min_freq = 1 if t % 5 == 0 else 0
        need = 8 if min_freq else max(1, int(np.ceil(np.log2(max(m, 2)))))
        L = int(rng.integers(max(1, need - 1), 17))            # sometimes one bit too few
        cases.append((h, L, min_freq, m if not min_freq else 256))
        lines.append(f"build {L} {min_freq} {_nums(h)}")
    for (h, L, min_freq, m_eff), ans in zip(cases, _run(checker, lines)):
        rc = int(ans[0])
        if m_eff > (1 << L):
            assert rc == ERR_NO_SYMBOLS
            continue
        assert rc == 0
        ref = oracle.package_merge_lengths(oracle.codebook_frequencies([h], min_freq), L)
        got_len = np.array(ans[1:257], dtype=np.int64)
        got_code = np.array(ans[257:513], dtype=np.int64)
        assert np.array_equal(got_len, ref)
        codes = oracle.canonical_codes(ref)
        assert np.array_equal(got_code[ref > 0], codes[ref > 0])


def test_lengths_to_codes_and_their_rejections(checker):
    rng = np.random.default_rng(7)
    vecs = []
    for t in range(200):
        h = _hist(rng, t % 4)
        ln = oracle.package_merge_lengths(h, 16).astype(np.int64)
        if t % 4 == 1:
            ln[int(rng.integers(256))] = 17                   # longer than any code word may be
        elif t % 4 == 2:
            longer = np.flatnonzero(ln > 1)
            if longer.size:
                ln[longer[int(rng.integers(longer.size))]] -= 1   # a complete code made over-full
        vecs.append(ln)
    answers = _run(checker, [f"lens {_nums(v)}" for v in vecs])
    for ln, ans in zip(vecs, answers):
        ok = int(ln.max()) <= 16 and oracle.kraft_sum_scaled(ln, 16) <= (1 << 16)
        assert (int(ans[0]) == 0) == ok, ln
        if ok:
            codes = oracle.canonical_codes(ln)
            got = np.array(ans[1:], dtype=np.int64)
            assert np.array_equal(got[ln > 0], codes[ln > 0])
        else:
            assert int(ans[0]) == ERR_INVALID_ARG


def test_refresh_rule(checker):
    rng = np.random.default_rng(11)
    cases, lines = [], []
    for t in range(300):
        h = _hist(rng, t % 4)
        cur = oracle.package_merge_lengths(oracle.codebook_frequencies([_hist(rng, (t + 1) % 4)], 1), 16)
        if t % 7 == 0:
            cur = oracle.package_merge_lengths(_hist(rng, 0), 16)     # may leave bytes of h uncoded
        tol = int(rng.choice([0, 100, 10_000, 1_000_000]))
        cases.append((h, cur, tol))
        lines.append(f"drift 16 {tol} {_nums(h)} {_nums(cur)}")
    for (h, cur, tol), ans in zip(cases, _run(checker, lines)):
        refresh, use, bits_cur, bits_opt = oracle.drift_check(h, cur, 16, tol)
        assert int(ans[0]) == 0
        assert int(ans[1]) == int(refresh)
        assert int(ans[2]) == (bits_cur if bits_cur is not None else (1 << 64) - 1)
        assert int(ans[3]) == bits_opt
        assert np.array_equal(np.array(ans[4:], dtype=np.int64), use)


def test_size_accounting(checker):
    rng = np.random.default_rng(5)
    cases, lines = [], []
    for t in range(200):
        h = _hist(rng, t % 4)
        ln = oracle.package_merge_lengths(_hist(rng, (t + 2) % 4), 16)
        cases.append((h, ln))
        lines.append(f"stats 16 {_nums(h)} {_nums(ln)}")
    for (h, ln), ans in zip(cases, _run(checker, lines)):
        assert int(ans[0]) == 0
        hi = [int(v) for v in h]
        assert int(ans[1]) == sum(hi)
        assert int(ans[2]) == oracle.payload_bits_identity(h, ln)
        assert int(ans[3]) == oracle.per_batch_optimal_bits(h, 16)
        assert int(ans[4]) == sum(f for f, l in zip(hi, ln) if l == 0)
        n = float(sum(hi))
        assert float(ans[5]) == pytest.approx(n * oracle.entropy_bits(h), rel=1e-12, abs=1e-9)


def test_sizes(checker):
    cases = [(n, chunk, L) for n in (0, 1, 15, 16, 17, 255, 256, 4095, 4096, 4097, 123457, 1 << 20, 1 << 24)
             for chunk in (256, 512, 1024, 4096, 65536) for L in (1, 9, 16)]
    cases += [(100, 300, 16), (100, 128, 16), (100, 4096, 0), (100, 4096, 17)]
    big = [(1 << 40, 65536, 16), ((1 << 44) + 4096, 4096, 12)]
    lines = [f"sizes {n} {c} {L}" for n, c, L in cases + big]
    answers = _run(checker, lines)
    for (n, chunk, L), ans in zip(cases, answers):
        valid = chunk in (256, 512, 1024, 4096, 65536)
        nc = oracle.num_chunks(n, chunk) if valid else 0
        assert int(ans[0]) == nc
        assert int(ans[1]) == (oracle.header_bytes(n, chunk) if nc else 0)
        assert int(ans[2]) == (oracle.encoded_bound(n, chunk, L) if nc and 1 <= L <= 16 else 0)
        part = -(-(64 + 8 * (nc + 4)) // 256) * 256
        assert int(ans[3]) == (2 * part + 256 if valid else 0)
    for (n, chunk, L), ans in zip(big, answers[len(cases):]):
        # whole chunks: every lane holds chunk / G symbols
        G = min(chunk // 256, 16)
        nc = -(-n // chunk)
        assert n % chunk == 0
        header = -(-4 * nc // 16) * 16 + -(-2 * nc * G // 16) * 16
        words = nc * G * (-(-(chunk // G) * L // 32))
        assert int(ans[0]) == nc and int(ans[1]) == header
        assert int(ans[2]) == -(-(header + 4 * words) // 16) * 16


def test_container_header(checker):
    rng = np.random.default_rng(9)
    cases, lines = [], []
    for t in range(50):
        lh = oracle.package_merge_lengths(_hist(rng, t % 4), 16)
        ll = oracle.package_merge_lengths(_hist(rng, (t + 1) % 4), 16)
        n = int(rng.integers(0, 1 << 40))
        chunk = int(1 << rng.integers(8, 17))
        bh, bl = int(rng.integers(0, 4096)), int(rng.integers(0, 4096))
        cases.append((n, chunk, lh, ll, bh, bl))
        lines.append(f"box {n} {chunk} 16 {bh} {bl} {_nums(lh)} {_nums(ll)}")
    for (n, chunk, lh, ll, bh, bl), ans in zip(cases, _run(checker, lines)):
        assert int(ans[0]) == 0
        enc = {"n": n, "chunk": chunk, "max_len": 16, "len_hi": lh, "len_lo": ll,
               "stream_hi": np.zeros(bh, np.uint8), "stream_lo": np.zeros(bl, np.uint8)}
        ref = oracle.container_bytes(enc)[:560]
        assert np.array_equal(np.frombuffer(bytes.fromhex(ans[1]), np.uint8), ref)
        assert tuple(int(v) for v in ans[2:8]) == (0, n, chunk, 16, bh, bl)
        assert np.array_equal(np.array(ans[8:264], dtype=np.int64), lh)
        assert np.array_equal(np.array(ans[264:520], dtype=np.int64), ll)
