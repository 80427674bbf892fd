"""The gfx950 code the library's sources compile to, checked on the host (no GPU).

Every kernel source is compiled to assembly with the library's own flags, and the text
is checked for:
- no packed float32 arithmetic (v_pk_add_f32, v_pk_mul_f32, v_pk_fma_f32): the build
  turns the feature off, and none is written by hand;
- no store, atomic, write-back or discard through the scalar data cache: every write
  goes through vector memory instructions;
- no scratch memory (register spills) in the kernels that the bench measures: the
  64-token prefill, the split summary pass, the pipelined 32-token prefill, the decode
  step and the speculative verify and commit, bfloat16 in and out at d = 128.
"""
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "gated_delta_rule_57_amd"))
import build  # noqa: E402  (the library's build script: its flags and sources)

HIPCC = "/opt/rocm/bin/hipcc"
KERNEL_SOURCES = [s for s in build.SOURCES if s != "kda_api.hip"]
PACKED_F32 = re.compile(r"^\s*v_pk_(add|mul|fma)_f32\b", re.M)
SCALAR_WRITE = re.compile(r"^\s*s_(store|buffer_store|scratch_store|atomic|buffer_atomic|dcache_wb|"
                          r"dcache_discard)\w*", re.M)
# kernels whose private segment must be empty (mangled-name fragments)
NO_SCRATCH = [
    "chunk_fwd_kernelIDF16bDF16bLi128ELi128ELi64ELb0E",
    "chunk_fwd_summary_kernelIDF16bLb0E",
    "chunk_pipe_kernelIDF16bLi128ELi128ELi2ELb0E",
    "decode_step_kernelIDF16bDF16bLi128ELi128ELb0E",
    "multi_token_kernelIDF16bDF16bLi128ELi128ELb0E",
    "multi_token_kernelIDF16bDF16bLi128ELi128ELb1E",
]


def _assembly(tmp, name):
    out = os.path.join(tmp, name + ".s")
    cmd = [HIPCC, *build.flags(False), "--cuda-device-only", "-S",
           os.path.join(build.CSRC, name), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    with open(out) as f:
        return f.read()


def _private_sizes(text):
    """{kernel symbol: private segment bytes} from the .amdhsa_kernel blocks."""
    sizes = {}
    for m in re.finditer(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", text, re.S):
        p = re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", m.group(2))
        sizes[m.group(1)] = int(p.group(1))
    return sizes


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not installed")
    tmp = str(tmp_path_factory.mktemp("asm"))
    with ThreadPoolExecutor(max_workers=len(KERNEL_SOURCES)) as pool:
        texts = list(pool.map(lambda n: _assembly(tmp, n), KERNEL_SOURCES))
    return dict(zip(KERNEL_SOURCES, texts))


def test_no_packed_float32_arithmetic(assembly):
    for name, text in assembly.items():
        hits = PACKED_F32.findall(text)
        assert not hits, f"{name}: {len(hits)} packed float32 instructions"


def test_no_writes_through_the_scalar_cache(assembly):
    for name, text in assembly.items():
        hits = SCALAR_WRITE.findall(text)
        assert not hits, f"{name}: scalar-cache writes {sorted(set(hits))}"


def test_measured_kernels_use_no_scratch(assembly):
    sizes = {}
    for text in assembly.values():
        sizes.update(_private_sizes(text))
    for frag in NO_SCRATCH:
        found = [k for k in sizes if frag in k]
        assert found, f"no kernel matches {frag}"
        for k in found:
            assert sizes[k] == 0, f"{k}: {sizes[k]} bytes of scratch"
