"""Build ``libmlap.so`` (gfx950 only) in-tree with hipcc.

The library is the C ABI declared in ``include/mlap.h``; the Python binding in
this package loads it with ctypes. Device code is compiled for gfx950 and
nothing else.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmlap.so")
# The debug build: the same library with the kernels' bounds checks compiled in (MLAP_DEBUG;
# mlap_debug_flags reads them). The parity tests run it at ragged batch sizes.
DEBUG_LIB = os.path.join(HERE, "libmlap_debug.so")
SOURCES = ["gemm_kernels.hip", "gemm_big_bf16.hip", "gemm_big_i8.hip", "gemm_big_fp8.hip", "gemm_nt.hip",
           "row_kernels.hip", "mlap_host.hip"]
HEADERS = ["common.hpp", "gemm.hpp", "gemm_big.hpp", "gemm_big_launch.hpp", "gemm_inst.hpp", "launch.hpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3", "-std=c++17", "-fPIC",
    # IEEE semantics where the method fixes the arithmetic: no FMA contraction of the
    # RoPE / RMSNorm steps, correctly rounded fp32 divide and sqrt.
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed-fp32 VALU ops in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
    "-I" + os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    return r.returncode, "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)


# AddressSanitizer on the host half only (argument checks, planning, the C ABI); the
# device code is built as usual. The library then needs the ASan runtime preloaded.
ASAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, out: str = LIB, asan: bool = False, debug: bool = False) -> str:
    """Compile every source to an object in parallel (one hipcc per translation unit), then
    link the shared library `out`; the objects go to a temporary folder. With `asan`, the
    host code is instrumented with AddressSanitizer (ASAN_HOST); with `debug`, the kernels'
    bounds checks are compiled in (-DMLAP_DEBUG)."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    with tempfile.TemporaryDirectory(prefix="mlap_build_") as tmpd:
        objs, cmds = [], []
        for src in SOURCES:
            obj = os.path.join(tmpd, src.replace(".hip", ".o"))
            objs.append(obj)
            cmds.append([HIPCC, *FLAGS, *(ASAN_HOST if asan else []), *(["-DMLAP_DEBUG"] if debug else []),
                         "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        jobs = min(len(cmds), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(_run, cmds))
        for (rc, log), src in zip(results, SOURCES):
            if rc != 0:
                raise RuntimeError("hipcc failed on %s:\n%s" % (src, log))
            if verbose and log.strip():
                print(log)
        tmp = out + ".tmp%d" % os.getpid()
        rc, log = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                        *(ASAN_HOST[:2] + ["-shared-libsan"] if asan else []), *objs, "-o", tmp])
        if rc != 0:
            raise RuntimeError("link failed:\n" + log)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build(verbose="-v" in sys.argv, out=DEBUG_LIB, debug=True))
