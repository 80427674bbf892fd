"""Fused output gate: kda_chunk_fwd_output_gate and kda_recurrent_step_output_gate write
o = (S^T q) * sigmoid(z), z one gate value per token, head and value channel (the gate the
Towards-AI article on the Kimi K3 report gives K3's Gated MLA layers, with a counterpart in
KDA, section "Gated MLA and No Position Encoding (NoPE)").  Against the float64 oracle
(oracle.apply_output_gate on the oracle's o), and against the ungated call by closed forms
that hold bit for bit: sigmoid(0) = 1/2, sigmoid(+large) = 1, sigmoid(-large) = 0."""
import numpy as np
import pytest
import torch

import gated_delta_rule_57_amd as kda
import oracle
import parity
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {"f32": 1e-5, "bf16": 3e-3}


def _ref(x):
    (o, s, _), _ = oracle.kda_forward_heads_parallel(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                                     x["s0"])
    return o, s


@pytest.mark.parametrize("w,out_dtype", [
    (synth.TINY_F32.replace(T=200, init_state=True), torch.float32),
    (synth.PREFILL_B4_T4096.replace(B=2, T=333, H=3), None),
    (synth.PREFILL_B4_T4096.replace(B=2, T=333, H=3), torch.float32),
    (synth.PREFILL_B4_T4096.replace(B=1, T=200, H=3, dk=64, dv=64), None),
    (synth.PREFILL_B4_T4096.replace(B=1, T=130, H=2, dk=128, dv=64), torch.float32),
    (synth.PREFILL_B4_T4096.replace(B=1, T=130, H=2, dk=64, dv=128), None),
], ids=["f32", "bf16", "bf16_f32out", "bf16_d64", "bf16_dk128_dv64", "bf16_dk64_dv128"])
def test_prefill_gate_matches_oracle(w, out_dtype):
    x = synth.prefill_inputs(w)
    z = synth.gate_inputs(w)
    print(f"[gate] prefill {w.dtype} B{w.B} T{w.T} H{w.H} dk{w.dk} dv{w.dv} out={out_dtype}",
          flush=True)
    d = synth.to_torch(dict(x, z=z), w.dtype, DEV)
    o, s, _ = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"],
                                out_dtype=out_dtype, output_gate=d["z"])
    o0, s0, _ = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"],
                                  out_dtype=out_dtype)
    torch.cuda.synchronize()
    o_r, s_r = _ref(x)
    parity.check("gated o", o, oracle.apply_output_gate(o_r, z), TOL[w.dtype], "tokens")
    parity.check("final state", s, s_r, TOL[w.dtype], "state")
    # the gate touches the output only
    assert torch.equal(s, s0)


def test_prefill_gate_through_the_segment_path():
    """Few heads, long sequence: the library cuts segments; the gate applies in the summary
    pass (segment 0's outputs) and in the output pass alike."""
    w = synth.PREFILL_B4_T4096.replace(B=1, T=8192 + 37, H=8)
    assert kda.kda_chunk_fwd_segment_tokens(w.B, w.T, w.H, w.dk, w.dv) < w.T
    x = synth.prefill_inputs(w)
    z = synth.gate_inputs(w)
    print(f"[gate] segment path B{w.B} T{w.T} H{w.H}", flush=True)
    d = synth.to_torch(dict(x, z=z), w.dtype, DEV)
    o, s, _ = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"],
                                output_gate=d["z"])
    torch.cuda.synchronize()
    o_r, s_r = _ref(x)
    parity.check("gated o", o, oracle.apply_output_gate(o_r, z), 3e-3, "tokens")
    parity.check("final state", s, s_r, 3e-3, "state")


@pytest.mark.parametrize("out_dtype", [None, torch.float32])
def test_prefill_gate_closed_forms_bitwise(out_dtype):
    """z = 0 halves o exactly; z = +60 and +inf pass it through, z = -inf closes it; z = -60
    scales it by sigmoid(-60) = 8.8e-27 (bfloat16 z)."""
    w = synth.PREFILL_B4_T4096.replace(B=1, T=150, H=2)
    x = synth.prefill_inputs(w)
    d = synth.to_torch(x, w.dtype, DEV)
    o0, _, _ = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"],
                                 out_dtype=out_dtype)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"])
    zeros = torch.zeros_like(d["v"])
    oh, _, _ = kda.kda_chunk_fwd(*args, out_dtype=out_dtype, output_gate=zeros)
    op, _, _ = kda.kda_chunk_fwd(*args, out_dtype=out_dtype, output_gate=zeros + 60.0)
    om, _, _ = kda.kda_chunk_fwd(*args, out_dtype=out_dtype, output_gate=zeros - 60.0)
    opi, _, _ = kda.kda_chunk_fwd(*args, out_dtype=out_dtype, output_gate=zeros + float("inf"))
    omi, _, _ = kda.kda_chunk_fwd(*args, out_dtype=out_dtype, output_gate=zeros - float("inf"))
    torch.cuda.synchronize()
    assert torch.equal(op, o0) and torch.equal(opi, o0)
    assert torch.equal(oh, o0 * 0.5)
    assert bool((omi == 0).all())
    sig = 1.0 / (1.0 + np.exp(60.0))
    ratio = (om.double() / (o0.double() * sig))[o0 != 0]
    assert float((ratio - 1).abs().max()) < 1e-2  # one rounding of o in the output dtype


@pytest.mark.parametrize("dtype,dk,dv", [("f32", 64, 64), ("bf16", 128, 128), ("bf16", 64, 128),
                                         ("bf16", 128, 64)])
def test_decode_gate_matches_oracle(dtype, dk, dv):
    w = synth.DECODE_N256.replace(B=5, H=3, dk=dk, dv=dv, dtype=dtype)
    s0 = synth.initial_state(w)
    state = torch.from_numpy(s0).float().to(DEV)
    S = s0.copy()
    for step in range(3):
        x = synth.decode_step_inputs(w, step)
        z = synth.gate_inputs(w.replace(seed=w.seed + step), (w.B, w.H, w.dv))
        d = synth.to_torch(dict(x, z=z), dtype, DEV)
        o = kda.kda_recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state,
                                   out_dtype=torch.float32, output_gate=d["z"])
        o_r, S = oracle.kda_decode_step(S, x["q"], x["k"], x["v"], x["g"], x["beta"])
        torch.cuda.synchronize()
        parity.check(f"decode gated o, step {step}", o, oracle.apply_output_gate(o_r, z),
                     TOL[dtype], "step")
    parity.check("decode state", state, S, TOL[dtype], "state")


def test_gate_rejected_when_overlapping_the_output():
    w = synth.PREFILL_B4_T4096.replace(B=1, T=64, H=1)
    d = synth.to_torch(synth.prefill_inputs(w), w.dtype, DEV)
    o = torch.empty_like(d["v"])
    with pytest.raises(kda.KdaError):
        kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], o=o, output_gate=o)
