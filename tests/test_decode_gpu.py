"""kda_recurrent_step on the GPU against the float64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_57_amd as kda
import oracle
import parity
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run_steps(w, steps, seqs=None, out_dtype=None):
    """Run `steps` chained decode steps; returns the largest whole / per-head error of o over
    the steps and the whole / per-head error of the final state."""
    s0 = synth.initial_state(w)
    if seqs is not None:
        s0 = s0[seqs]
    state = torch.from_numpy(s0).float().to(DEV)
    ref = s0.copy()
    e_o = [0.0, 0.0]
    for s in range(steps):
        x = synth.decode_step_inputs(w, s, seqs)
        d = synth.to_torch(x, w.dtype, DEV)
        o = kda.kda_recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state,
                                   out_dtype=out_dtype)
        o_ref, ref = oracle.kda_decode_step(ref, x["q"], x["k"], x["v"], x["g"], x["beta"])
        torch.cuda.synchronize()
        whole, head, _ = parity.errors(o, o_ref, "step")
        e_o = [max(e_o[0], whole), max(e_o[1], head)]
    whole, head, _ = parity.errors(state, ref, "state")
    print(f"[decode]   o whole {e_o[0]:.3e} head-max {e_o[1]:.3e}; state whole {whole:.3e} "
          f"head-max {head:.3e}", flush=True)
    return e_o, (whole, head)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_small(dk, dv, dtype):
    w = synth.DECODE_N256.replace(B=3, H=5, dk=dk, dv=dv, dtype=dtype)
    print(f"[decode] dk={dk} dv={dv} {dtype}", flush=True)
    e_o, e_s = _run_steps(w, 4, out_dtype=torch.float32)
    tol = 1e-5 if dtype == "f32" else 3e-3
    assert max(*e_o, *e_s) <= tol, (e_o, e_s)


def test_decode_full_width_ten_steps_bf16_out():
    """All 8192 heads of the 256-sequence decode workload, steps 0..9, bfloat16 o."""
    w = synth.DECODE_N256
    print("[decode] N256 H32 10 steps", flush=True)
    e_o, e_s = _run_steps(w, 10)
    assert max(*e_o, *e_s) <= 3e-3, (e_o, e_s)


def test_decode_1000_chained_steps_sampled_sequences():
    """1000 chained steps on 16 of the 256 sequences (inputs drawn per step)."""
    w = synth.DECODE_N256
    print("[decode] 16 seqs x 1000 steps", flush=True)
    e_o, e_s = _run_steps(w, 1000, seqs=slice(0, 256, 16))
    assert max(*e_o, *e_s) <= 3e-3, (e_o, e_s)


def test_decode_no_write_no_decay_keeps_state_bitwise():
    w = synth.DECODE_N256.replace(B=2, H=3)
    x = synth.decode_step_inputs(w, 0)
    x["beta"][:] = 0.0
    x["g"][:] = 0.0
    d = synth.to_torch(x, w.dtype, DEV)
    s0 = torch.from_numpy(synth.initial_state(w)).float().to(DEV)
    state = s0.clone()
    kda.kda_recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state)
    torch.cuda.synchronize()
    assert torch.equal(state, s0)
