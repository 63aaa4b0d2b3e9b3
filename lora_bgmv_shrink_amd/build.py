"""Build liblora_mi355x.so in-tree with hipcc for gfx950.

    python -m lora_bgmv_shrink_amd.build

Every HIP translation unit is compiled with packed-fp32 instructions
disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "liblora_mi355x.so"
# LORA_MI355X_LIB names another build of the library to load (the host-code
# sanitizer run's instrumented copy); the default is the in-tree build
LIB_PATH = os.environ.get("LORA_MI355X_LIB") or os.path.join(HERE, LIB_NAME)
SOURCES = ["api.hip", "segments.hip", "bgmv.hip", "mfma.hip", "decode.hip", "merge.hip", "cache.hip", "rows.hip", "sched.cpp"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def _compile(src: str, verbose: bool, build_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = False, out: str = None, build_dir: str = None, extra=(), workers: int = 0) -> str:
    """Compile every source and link the library (default: in-tree).  ``extra``
    flags go to every compile and the link (the sanitizer run passes
    ``-Xarch_host -fsanitize=...``: host code only)."""
    out = out or os.path.join(HERE, LIB_NAME)
    bdir = build_dir or BUILD_DIR
    os.makedirs(bdir, exist_ok=True)

    def one(src):
        return _compile(src, verbose, bdir, extra)

    with cf.ThreadPoolExecutor(max_workers=workers or len(SOURCES)) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
