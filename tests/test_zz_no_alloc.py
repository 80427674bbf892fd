"""kda_chunk_fwd_noalloc (the entry point for callers that cannot allocate: its segment-path
workspace is the library's own device array) against kda_chunk_fwd with a caller-allocated
workspace, through the C ABI: two calls in a row, the second with smaller inputs, each
bit for bit equal to kda_chunk_fwd's result (the same kernels run on the same inputs)."""
import pytest
import torch

import gated_delta_rule_57_amd as kda
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _pair(w):
    d = synth.device_prefill_inputs(w, DEV)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"])
    ref_o, ref_s, _ = kda.kda_chunk_fwd(*args)
    o = torch.empty_like(ref_o)
    s = torch.empty_like(ref_s)
    kda.kda_chunk_fwd_noalloc(*args, o, s)
    torch.cuda.synchronize()
    return (o, s), (ref_o, ref_s)


def test_noalloc_matches_workspace_call_twice_second_smaller():
    big = synth.PREFILL_B4_T4096.replace(B=1, T=16384 + 77, H=8)
    small = synth.PREFILL_B4_T4096.replace(B=1, T=4096 + 5, H=4, seed=9)
    for w in (big, small):
        seg = kda.kda_chunk_fwd_segment_tokens(w.B, w.T, w.H, w.dk, w.dv)
        need = kda.kda_chunk_fwd_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv)
        print(f"[noalloc] B{w.B} T{w.T} H{w.H}: segment {seg}, workspace {need} bytes",
              flush=True)
        assert seg < w.T and 0 < need <= (64 << 20)  # the segment path, so the scratch is used
        (o, s), (ref_o, ref_s) = _pair(w)
        assert torch.equal(o, ref_o) and torch.equal(s, ref_s)
        assert bool(torch.isfinite(s).all())


def test_noalloc_single_segment_needs_no_scratch():
    w = synth.PREFILL_B4_T4096.replace(B=2, T=333, H=32)
    assert kda.kda_chunk_fwd_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv) == 0
    (o, s), (ref_o, ref_s) = _pair(w)
    assert torch.equal(o, ref_o) and torch.equal(s, ref_s)
