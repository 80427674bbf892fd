"""The C ABI's host-side validation under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's sources are built with both sanitizers on their host code (the GPU code is
built as usual and never runs here), linked with tests/sanitize/abi_checks.cpp, and run:
every call in it must be rejected with the expected status before any launch, or be a
pure size query, so no GPU is needed.  A sanitizer report (an out-of-bounds access, a
signed overflow in the size arithmetic, an out-of-range enumeration value) ends the run
with a non-zero status.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_57_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
SOURCES = ("kda_api", "kda_decode", "kda_prefill", "kda_prefill_pipe", "kda_scan")
# sanitizers on the host code only; the GPU code keeps the library's own flags
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_abi_validation_under_sanitizers(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    common = ["-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops"]

    def compile_one(name):
        obj = str(tmp_path / f"{name}.o")
        rc, out = _run([HIPCC, "--offload-arch=gfx950", *common, *SAN, *inc, "-c",
                        os.path.join(CSRC, f"{name}.hip"), "-o", obj])
        assert rc == 0, out
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
        objs = list(pool.map(compile_one, SOURCES))
    exe = str(tmp_path / "abi_checks")
    rc, out = _run([HIPCC, "-O1", "-g", "-std=c++17", *SAN[:4], *inc, *objs, "-x", "c++",
                    os.path.join(ROOT, "tests", "sanitize", "abi_checks.cpp"), "-o", exe])
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    rc, out = _run([exe], env=env, timeout=120)
    print(out)
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
    assert rc == 0 and " 0 failures" in out, out
    shutil.rmtree(tmp_path, ignore_errors=True)
