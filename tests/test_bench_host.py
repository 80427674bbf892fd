"""Host-side checks of bench.py: the algorithmic work it divides by, the one-GPU guard and
the rule that counted traffic is reported only for the kernel source it was taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_prefill_work_of_the_4x4096x32_workload():
    # per token-head: 6 d^2 for the three state products, 2 C (10/16)(3d + 2d) for the five
    # block-triangular intra-chunk products on dense 16-tiles, (2/3) C^2 for the UT solve
    assert round(bench.prefill_flops_per_token_head(128, 128)) == 152235
    # q, k, g, v (bf16) + beta read, o written: 1,282 B per token-head, plus the state twice
    per_tok = (3 * 128 + 128 + 1) * 2 + 128 * 2
    assert per_tok == 1282
    assert bench.prefill_bytes(4, 4096, 32, 128, 128) == 4 * 4096 * 32 * 1282 + 2 * 128 * 65536
    assert bench.prefill_bytes(4, 4096, 32, 128, 128) == 688914432


def test_decode_and_draft_bytes():
    # state (64 KiB fp32) read and written, one token's inputs and output per head
    assert bench.decode_bytes(256, 32, 128, 128) == 1084243968
    # verify: state read once, 4 drafts' q, k, g, v, beta read and o written
    assert bench.verify_bytes(256, 4, 32, 128, 128) == 256 * 32 * (65536 + 4 * (1026 + 256))
    # commit: state read and written once, 4 drafts' k, g, v, beta read
    assert bench.commit_bytes(256, 4, 32, 128, 128) == 256 * 32 * (131072 + 4 * 770)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_only_for_the_profiled_source(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    hdr = tmp_path / "shared.h"
    src.write_text("// one version of a kernel\n")
    hdr.write_text("// one version of a header\n")
    monkeypatch.setattr(bench, "_CSRC", str(tmp_path))
    monkeypatch.setitem(bench.KERNEL_SOURCES, "prefill", ("kernel.hip", "shared.h"))
    rec = {"prefill": {"bytes_per_launch": 123, "source_sha256_16": bench.source_hash("prefill")}}
    traffic = tmp_path / "hbm_traffic.json"
    traffic.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    assert bench.measured_traffic("prefill") == 123
    hdr.write_text("// another version of the header\n")  # a header the kernel includes
    assert bench.measured_traffic("prefill") is None
    hdr.write_text("// one version of a header\n")
    assert bench.measured_traffic("prefill") == 123
    src.write_text("// another version\n")
    assert bench.measured_traffic("prefill") is None
    assert bench.measured_traffic("decode") is None  # no record


@pytest.mark.parametrize("which", ["prefill", "prefill_chunk32", "decode", "verify", "commit"])
def test_committed_traffic_is_close_to_the_algorithmic_bytes(which):
    """Counted HBM bytes of the committed summary: no wasted re-reads (within 5%).  A summary
    taken on another version of the source is not reported by the bench; it is skipped here."""
    rec = json.load(open(bench.TRAFFIC_FILE)).get(which)
    if rec is None:
        pytest.skip(f"{which}: no counter summary committed")
    if rec["source_sha256_16"] != bench.source_hash(which):
        pytest.skip(f"{which}: counters were taken on another version of the kernel source")
    ratio = rec["bytes_per_launch"] / rec["algorithmic_bytes_per_launch"]
    assert 0.99 < ratio < 1.05, ratio
