"""Raw decay logits: kda_chunk_fwd_gate_logits and kda_recurrent_step_gate_logits take the
logits a in place of g and apply g = -softplus(a) (then the floor) in their gate preparation.
Against the float64 oracle fed -softplus(a) of the same (rounded) logits."""
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


def _np(t):
    return t.double().cpu().numpy()


@pytest.mark.parametrize("w", [
    synth.TINY_F32.replace(T=200, init_state=True),
    synth.PREFILL_B4_T4096.replace(B=2, T=333, H=3),
    synth.PREFILL_B4_T4096.replace(B=1, T=1024, H=4, a_law="mixed"),
], ids=["f32", "bf16", "bf16_mixed"])
def test_prefill_from_logits_matches_oracle(w):
    x = synth.prefill_inputs(w, with_logits=True)
    a = x["a"].copy()
    a[..., 0, 0, :4] = [0.0, 30.0, -30.0, 200.0]  # closed forms and both tails (first token)
    x["a"] = synth.round_to(a, w.dtype)
    g = oracle.log_decay_from_logits(x["a"])
    (o_r, s_r, _), _ = oracle.kda_forward_heads_parallel(x["q"], x["k"], x["v"], g, x["beta"], x["s0"])
    d = synth.to_torch(x, w.dtype, DEV)
    o, s, _ = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["a"], d["beta"], d["s0"],
                                out_dtype=torch.float32, gate_logits=True)
    torch.cuda.synchronize()
    print(f"[logits] {w.name} {w.dtype} T{w.T}", flush=True)
    parity.check("o", o, o_r, TOL[w.dtype], "tokens")
    parity.check("final state", s, s_r, TOL[w.dtype], "state")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_from_logits_matches_oracle(dtype):
    d_ = 64 if dtype == "f32" else 128
    w = synth.PREFILL_B4_T4096.replace(B=8, T=6, H=4, dk=d_, dv=d_, dtype=dtype)
    x = synth.prefill_inputs(w, with_logits=True)
    d = synth.to_torch(x, dtype, DEV)
    state = d["s0"].clone()
    S = x["s0"].copy()
    for t in range(w.T):
        o = kda.kda_recurrent_step(d["q"][:, t].contiguous(), d["k"][:, t].contiguous(),
                                   d["v"][:, t].contiguous(), d["a"][:, t].contiguous(),
                                   d["beta"][:, t].contiguous(), state, out_dtype=torch.float32,
                                   gate_logits=True)
        o_r, S = oracle.kda_decode_step(S, x["q"][:, t], x["k"][:, t], x["v"][:, t],
                                        oracle.log_decay_from_logits(x["a"][:, t]), x["beta"][:, t])
        torch.cuda.synchronize()
        parity.check(f"decode o, token {t}", o, o_r, TOL[dtype], "step")
    parity.check(f"decode {dtype} state", state, S, TOL[dtype], "state")


def test_nan_logit_stays_in_its_head():
    w = synth.PREFILL_B4_T4096.replace(B=1, T=128, H=3)
    x = synth.prefill_inputs(w, with_logits=True)
    x["a"][0, 70, 1, 5] = np.nan
    d = synth.to_torch(x, w.dtype, DEV)
    o, sf, _ = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["a"], d["beta"], d["s0"],
                                 out_dtype=torch.float32, gate_logits=True)
    torch.cuda.synchronize()
    assert torch.isnan(sf[0, 1]).any() and torch.isfinite(sf[0, [0, 2]]).all()
    assert torch.isfinite(o[0, :, [0, 2]]).all() and torch.isfinite(o[0, :64, 1]).all()
