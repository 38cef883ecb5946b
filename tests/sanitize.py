#!/usr/bin/env python3
"""CPU sanitizer runs (no GPU needed).

1. The C-ABI tests (tests/test_abi.py) against a build of libmlap.so whose host code
   (argument checks, planning, workspace carving, the entry points) is instrumented with
   AddressSanitizer; the ASan runtime is preloaded into the test process.
2. The oracle's pins (tests/test_oracle_pins.py) against a build of liboracle.so under
   UndefinedBehaviorSanitizer, every finding fatal.

Both builds go to a temporary folder; the in-tree libraries are not touched.

    python tests/sanitize.py [--only asan|ubsan] [--keep DIR]
"""
import argparse
import glob
import os
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so") +
                  glob.glob("/opt/rocm/llvm/lib/clang/*/lib/x86_64-unknown-linux-gnu/libclang_rt.asan.so"))
    if not hits:
        raise SystemExit("no AddressSanitizer runtime under /opt/rocm/llvm")
    return hits[-1]


def pytest(args, env):
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *args]
    print("+", " ".join(cmd), flush=True)
    return subprocess.call(cmd, cwd=ROOT, env=env)


def run_asan(d):
    from mla_prolog_amd import build as mbuild

    lib = mbuild.build(out=os.path.join(d, "libmlap_asan.so"), asan=True)
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = asan_runtime() + (" " + pre if pre else "")  # the runtime must come first
    # the interpreter and torch are not instrumented: their allocations are not ours to report
    env["ASAN_OPTIONS"] = "detect_leaks=0:alloc_dealloc_mismatch=0:halt_on_error=1:abort_on_error=0"
    env["MLAP_LIBRARY"] = lib
    return pytest(["tests/test_abi.py"], env)


def run_ubsan(d):
    import oracle

    lib = oracle.build(out=os.path.join(d, "liboracle_ubsan.so"), ubsan=True)
    env = dict(os.environ)
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["MLAP_ORACLE_LIBRARY"] = lib
    return pytest(["tests/test_oracle_pins.py"], env)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--only", choices=("asan", "ubsan"))
    ap.add_argument("--keep", help="build into this folder and keep it")
    a = ap.parse_args()
    with tempfile.TemporaryDirectory(prefix="mlap_sanitize_") as tmpd:
        d = a.keep or tmpd
        os.makedirs(d, exist_ok=True)
        rc = 0
        if a.only in (None, "ubsan"):
            rc |= run_ubsan(d)
        if a.only in (None, "asan"):
            rc |= run_asan(d)
    print("sanitizer runs:", "ok" if rc == 0 else "FAILED", flush=True)
    return 1 if rc else 0


if __name__ == "__main__":
    sys.exit(main())
