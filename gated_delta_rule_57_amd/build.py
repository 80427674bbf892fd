"""Build the C-ABI KDA libraries for gfx950 with hipcc, in the package directory:
libkda.so, and libkda_debug.so (the same sources with -DKDA_DEBUG_RANGE: the chunk
kernels check the decay-factor bound and the finiteness of their operands as they run;
declared in include/kda_debug.h)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkda.so")
DEBUG_LIB = os.path.join(PKG, "libkda_debug.so")
SOURCES = ["kda_api.hip", "kda_decode.hip", "kda_prefill.hip", "kda_prefill_pipe.hip",
           "kda_scan.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libkda.so)")


def flags(debug: bool = False) -> list:
    return ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
            # packed-float32 VALU forms stay off: plain float code only
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC] + (["-DKDA_DEBUG_RANGE"] if debug else [])


def command(out: str = LIB, debug: bool = False) -> list:
    """One hipcc line that builds a library from every source (the build itself compiles
    the sources separately and in parallel, with the same flags, then links)."""
    return [hipcc(), *flags(debug), "-shared", *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


def _run(cmd, verbose):
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")


CAPI_SRC = os.path.join(ROOT, "tests", "capi", "kda_capi_main.c")
CAPI_BIN = os.path.join(ROOT, "tests", "capi", "kda_capi_check")


def build_capi_check(verbose: bool = True) -> str:
    """The plain C caller used by the tests (tests/capi), linked against libkda.so."""
    rocm = os.path.dirname(os.path.dirname(hipcc()))
    _run(["gcc", "-O2", "-std=c11", "-Wall", "-I", os.path.join(ROOT, "include"),
          "-I", os.path.join(rocm, "include"), "-D__HIP_PLATFORM_AMD__", CAPI_SRC,
          "-L", PKG, "-lkda", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
          "-Wl,-rpath,$ORIGIN/../../gated_delta_rule_57_amd",
          "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", CAPI_BIN], verbose)
    return CAPI_BIN


def build(verbose: bool = True, debug_lib: bool = True) -> str:
    """Compile every source for each library variant (in parallel), link, and move the
    libraries into place.  Returns the path of libkda.so."""
    variants = [(LIB, False)] + ([(DEBUG_LIB, True)] if debug_lib else [])
    with tempfile.TemporaryDirectory(prefix="kda_build_") as tmp:
        jobs = [(os.path.join(CSRC, src), os.path.join(tmp, f"{'d' if dbg else 'r'}_{src}.o"), dbg)
                for _, dbg in variants for src in SOURCES]
        workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
        with ThreadPoolExecutor(max_workers=workers) as pool:
            list(pool.map(lambda j: _run([hipcc(), *flags(j[2]), "-c", j[0], "-o", j[1]], verbose),
                          jobs))
        for out, dbg in variants:
            objs = [o for _, o, d in jobs if d == dbg]
            _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out + ".tmp"],
                 verbose)
            os.replace(out + ".tmp", out)
    if os.path.exists(CAPI_SRC):
        build_capi_check(verbose)
    return LIB


if __name__ == "__main__":
    build()
