"""CPU sanitizer runs (no GPU): the fp64 oracle under gcc's AddressSanitizer
and UndefinedBehaviorSanitizer, and the library's host code (the slot
cache in host-only mode, the admission scheduler, argument checks) built
with clang's sanitizers on the host side only, each through its own CPU
tests in a child process.  A report fails the child (halt on error)."""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(tests, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    with tempfile.TemporaryDirectory() as logs:
        # reports go to files: pytest's capture of fd 2 would lose them when the child halts
        env["ASAN_OPTIONS"] = f"detect_leaks=0:halt_on_error=1:verify_asan_link_order=0:log_path={logs}/asan"
        env["UBSAN_OPTIONS"] = f"halt_on_error=1:print_stacktrace=1:log_path={logs}/ubsan"
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                            *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
        reports = "".join(open(f).read()[:3000] for f in glob.glob(os.path.join(logs, "*")))
    tail = (r.stdout + r.stderr)[-2000:]
    assert not reports, reports
    assert r.returncode == 0, tail
    return tail


def test_oracle_under_asan_ubsan():
    import oracle
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.exists(libasan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    with tempfile.TemporaryDirectory() as d:
        lib = oracle.build(out=os.path.join(d, "liboracle_san.so"),
                           extra=("-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                                  "-fno-sanitize-recover=undefined"))
        out = _run(["tests/test_oracle_pins.py", "tests/test_cache_policy.py::test_model_matches_hand_walk"],
                   {"LORA_ORACLE_LIB": lib, "LD_PRELOAD": libasan})
        print(out[-300:])


def test_library_host_code_under_asan_ubsan():
    from lora_bgmv_shrink_amd import build as hb
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rt:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    with tempfile.TemporaryDirectory() as d:
        san = ("-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer")
        lib = hb.build(out=os.path.join(d, "liblora_san.so"), build_dir=os.path.join(d, "obj"), extra=san, workers=4)
        out = _run(["tests/test_cache_policy.py", "tests/test_admission.py", "tests/test_abi.py"],
                   {"LORA_MI355X_LIB": lib, "LD_PRELOAD": rt[0]})
        print(out[-300:])
