"""Build liblecb.so (HIP kernels for gfx950 + host runtime) in-tree with hipcc.

Run as ``python -m lossless_entropy_coding_byte_amd.build``; every call
recompiles.  Output: ``lossless_entropy_coding_byte_amd/liblecb.so``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblecb.so")
ARCH = "gfx950"

SOURCES = ["kernels_misc.hip", "kernels_codebook.hip", "kernels_encode.hip", "kernels_decode.hip", "codebook.cpp",
           "host.cpp", "api.cpp", "noalloc.hip"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# Device code: gfx950 only; packed-FP32 instruction selection disabled.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


# The compiler's per-kernel resource report (function name, then its figures).
RESOURCE_REPORT = ["-Rpass-analysis=kernel-resource-usage"]
_FN = re.compile(r"remark: Function Name: (\S+)")
_SCRATCH = re.compile(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)")


def scratch_users(report: str) -> list[tuple[str, int]]:
    """Kernels of a resource report that use scratch (register spills or a
    stack): (name, bytes per lane)."""
    users, fn = [], None
    for line in report.splitlines():
        m = _FN.search(line)
        if m:
            fn = m.group(1)
            continue
        m = _SCRATCH.search(line)
        if m and int(m.group(1)) > 0:
            users.append((fn, int(m.group(1))))
    return users


def _compile(src: str, obj: str) -> tuple[str, int, str]:
    path = os.path.join(CSRC, src)
    hip = src.endswith(".hip")
    lang = ["-x", "hip"] if hip else []
    cmd = [hipcc()] + COMMON + DEVICE + lang + (RESOURCE_REPORT if hip else []) + ["-c", path, "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    out = p.stdout + p.stderr
    rc = p.returncode
    if rc == 0 and hip:
        # no kernel may spill registers or use a stack: every variant keeps its
        # state in registers and LDS (spilled variants of the 16-wave decode
        # gave wrong results)
        users = scratch_users(out)
        if users:
            rc = 1
            out += "\nkernels using scratch memory: " + ", ".join(f"{n} ({b} bytes/lane)" for n, b in users)
    return src, rc, "\n".join(l for l in out.splitlines() if "remark:" not in l and not l.startswith("   "))


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="lecb_build_") as tmp:
        objs = [os.path.join(tmp, s + ".o") for s in SOURCES]
        with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
            results = list(ex.map(_compile, SOURCES, objs))
        failed = False
        for src, rc, out in results:
            noisy = [l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip()]
            if rc != 0 or (verbose and noisy):
                print(f"--- {src} (rc={rc})\n" + "\n".join(noisy), file=sys.stderr)
            failed |= rc != 0
        if failed:
            raise RuntimeError("HIP library build failed")
        tmp_lib = LIB + ".tmp"
        cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp_lib] + objs
        p = subprocess.run(cmd, capture_output=True, text=True)
        if p.returncode != 0:
            raise RuntimeError("link failed:\n" + p.stdout + p.stderr)
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
