"""Build liblecb.so (HIP kernels for gfx950 + host runtime) in-tree with hipcc.

Run as ``python -m lossless_entropy_coding_byte_amd.build``; every call
recompiles.  Output: ``lossless_entropy_coding_byte_amd/liblecb.so``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
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
           "api.cpp", "noalloc.hip"]

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


def _compile(src: str, obj: str) -> tuple[str, int, str]:
    path = os.path.join(CSRC, src)
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc()] + COMMON + DEVICE + lang + ["-c", path, "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    return src, p.returncode, p.stdout + p.stderr


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
