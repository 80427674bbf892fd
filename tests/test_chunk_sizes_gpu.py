"""Chunk length as a parameter: kda_chunk_fwd with chunk = 16, 32 and 64 (the 16- and
32-token chunks run the pipelined kernel, 64 the fused 64-token one) against the float64
oracle on the same inputs, and against each other: the result does not depend on the
chunk length (the chunked form is an exact rewrite of the token recurrence, so the three
agree to within rounding)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_57_amd as kda
import oracle
import parity
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CHUNKS = (16, 32, 64)


def _ref(x, every=0):
    (o, s, ck), _ = oracle.kda_forward_heads_parallel(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                                      x["s0"], every)
    return o, s, ck


def _run(d, chunk, **kw):
    out = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], chunk=chunk, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("B,T,H,dk,dv,law,out", [
    (1, 64, 1, 128, 128, "n02", torch.float32),
    (2, 333, 3, 128, 128, "n02", torch.float32),
    (2, 333, 3, 128, 128, "n02", None),
    (1, 200, 2, 64, 64, "n02", torch.float32),
    (1, 130, 2, 128, 64, "n51", torch.float32),
    (1, 130, 2, 64, 128, "mixed", torch.float32),
    (1, 1, 2, 128, 128, "n02", torch.float32),
    (1, 17, 2, 128, 128, "n02", torch.float32),
    (1, 32, 2, 128, 128, "n51", torch.float32),
    (1, 1024 + 37, 4, 128, 128, "mixed", None),
])
def test_chunk_lengths_match_oracle_and_each_other(B, T, H, dk, dv, law, out):
    w = synth.PREFILL_B4_T4096.replace(B=B, T=T, H=H, dk=dk, dv=dv, a_law=law, seed=11 + T)
    x = synth.prefill_inputs(w)
    d = synth.to_torch(x, w.dtype, DEV)
    o_r, s_r, _ = _ref(x)
    res = {}
    for chunk in CHUNKS:
        print(f"[chunk] B{B} T{T} H{H} dk{dk} dv{dv} {law} out={out} chunk {chunk}", flush=True)
        o, s, _ = _run(d, chunk, out_dtype=out)
        parity.check(f"o, chunk {chunk}", o, o_r, 3e-3, "tokens")
        parity.check(f"final state, chunk {chunk}", s, s_r, 3e-3, "state")
        res[chunk] = (o, s)
    # chunk-length invariance: every pair agrees to within the rounding of the bf16 path
    for a, b in ((16, 32), (32, 64), (16, 64)):
        parity.check(f"o, chunk {a} vs {b}", res[a][0], res[b][0], 3e-3, "tokens")
        parity.check(f"state, chunk {a} vs {b}", res[a][1], res[b][1], 3e-3, "state")


@pytest.mark.parametrize("chunk", [16, 32])
def test_small_chunks_long_memory(chunk):
    """Decay logits ~ N(-7, 1): the state carries across the whole sequence; the
    pipelined kernel carries S, Kbar and U as hi + lo pairs."""
    w = synth.PREFILL_B4_T4096.replace(B=1, T=2048, H=4, a_law="slow")
    x = synth.prefill_inputs(w)
    d = synth.to_torch(x, w.dtype, DEV)
    o, s, _ = _run(d, chunk, out_dtype=torch.float32)
    o_r, s_r, _ = _ref(x)
    parity.check(f"o, chunk {chunk}, long memory", o, o_r, 3e-3, "tokens")
    parity.check(f"state, chunk {chunk}, long memory", s, s_r, 3e-3, "state")


@pytest.mark.parametrize("chunk", [16, 32])
def test_small_chunks_decay_floor_on_every_channel(chunk):
    """Every channel of every token on the floor (and below it, clamped): every diagonal
    tile's column factors reach e^80."""
    w = synth.PREFILL_B4_T4096.replace(B=1, T=320, H=2, init_state=True)
    x = synth.prefill_inputs(w)
    g = np.full_like(x["g"], -5.0)
    g[..., ::3] = -7.0
    x["g"] = g
    d = synth.to_torch(x, w.dtype, DEV)
    o, s, _ = _run(d, chunk, out_dtype=torch.float32)
    o_r, s_r, _ = _ref(x)
    parity.check(f"o, chunk {chunk}, floor", o, o_r, 3e-3, "tokens")
    parity.check(f"state, chunk {chunk}, floor", s, s_r, 3e-3, "state")


@pytest.mark.parametrize("chunk", [16, 32])
def test_small_chunks_checkpoints_and_segments(chunk):
    w = synth.PREFILL_B4_T4096.replace(B=2, T=640 + 7, H=2)
    x = synth.prefill_inputs(w)
    d = synth.to_torch(x, w.dtype, DEV)
    o_r, s_r, ck_r = _ref(x, 128)
    for seg in (None, 192):
        print(f"[chunk] chunk {chunk} segment {seg}", flush=True)
        o, s, ck = _run(d, chunk, out_dtype=torch.float32, checkpoint_every=128,
                        segment_tokens=seg)
        parity.check("o", o, o_r, 3e-3, "tokens")
        parity.check("final state", s, s_r, 3e-3, "state")
        parity.check("checkpoints", ck, ck_r, 3e-3, "ckpt")


@pytest.mark.parametrize("chunk", [16, 32])
def test_small_chunks_library_segments_gate_and_logits(chunk):
    """Few heads, long sequence (the library cuts segments), with the output gate; then
    raw decay logits."""
    w = synth.PREFILL_B4_T4096.replace(B=1, T=8192 + 37, H=8)
    assert kda.kda_chunk_fwd_segment_tokens(w.B, w.T, w.H, w.dk, w.dv, chunk) < w.T
    x = synth.prefill_inputs(w, with_logits=True)
    z = synth.gate_inputs(w)
    d = synth.to_torch(dict(x, z=z), w.dtype, DEV)
    o_r, s_r, _ = _ref(x)
    o, s, _ = _run(d, chunk, output_gate=d["z"])
    parity.check("gated o, library segments", o, oracle.apply_output_gate(o_r, z), 3e-3, "tokens")
    parity.check("final state", s, s_r, 3e-3, "state")
    o2, s2, _ = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["a"], d["beta"], d["s0"],
                                  chunk=chunk, gate_logits=True)
    torch.cuda.synchronize()
    g = oracle.log_decay_from_logits(x["a"])
    o2_r, s2_r, _ = _ref(dict(x, g=g))
    parity.check("o from logits", o2, o2_r, 3e-3, "tokens")
    parity.check("state from logits", s2, s2_r, 3e-3, "state")


def test_chunk_32_full_size_workload():
    """4 x 4096 tokens x 32 heads, d = 128, bfloat16, 32-token chunks: every output and
    final state against the oracle."""
    w = synth.PREFILL_B4_T4096
    x = synth.prefill_inputs(w)
    d = synth.to_torch(x, w.dtype, DEV)
    o, s, _ = _run(d, 32)
    o_r, s_r, _ = _ref(x)
    parity.check("o, chunk 32, full size", o, o_r, 3e-3, "tokens")
    parity.check("final state, chunk 32, full size", s, s_r, 3e-3, "state")


def test_small_chunks_deterministic_and_in_place():
    w = synth.PREFILL_B4_T4096.replace(B=1, T=1500, H=3)
    d = synth.to_torch(synth.prefill_inputs(w), w.dtype, DEV)
    a = _run(d, 32)
    b = _run(d, 32)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    st = d["s0"].clone()
    o3, _, _ = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], st, final_state=st,
                                 chunk=32)
    torch.cuda.synchronize()
    assert torch.equal(o3, a[0]) and torch.equal(st, a[1])
