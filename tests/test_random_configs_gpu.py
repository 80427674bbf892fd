"""Seeded random combinations of the prefill's options against the float64 oracle.

Each case draws, from its own seed, one valid combination of: batch, sequence length
(ragged tails included), heads, head dimensions, input and output dtype, chunk length,
decay-logit law, initial state or none, and one of the entry points (plain, every-N
checkpoints, listed checkpoint positions, explicit segments, fused output gate, raw
decay logits).  Every output the call returns is compared with the oracle, whole
tensor, per head and per 64-token window.  The draws are fixed by the seeds, so a
failure names a reproducible case.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_57_amd as kda
import oracle
import parity
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ENTRIES = ("plain", "every", "positions", "segments", "output_gate", "gate_logits")


def _draw(seed):
    rng = np.random.default_rng(seed)
    dtype = "f32" if rng.random() < 0.2 else "bf16"
    if dtype == "f32":
        dk = dv = 64
        chunk = 64
    else:
        dk, dv = (int(x) for x in rng.choice([64, 128], 2))
        chunk = int(rng.choice([16, 32, 64]))
    B = int(rng.integers(1, 4))
    H = int(rng.integers(1, 6))
    T = int(rng.integers(1, 700))
    law = str(rng.choice(["n02", "n51", "mixed", "slow"]))
    entry = ENTRIES[int(rng.integers(len(ENTRIES)))]
    out = [None, torch.float32][int(rng.integers(2))]
    return dict(dtype=dtype, dk=dk, dv=dv, chunk=chunk, B=B, H=H, T=T, law=law, entry=entry,
                out=out, init=bool(rng.random() < 0.7), rng=rng)


@pytest.mark.parametrize("seed", range(1000, 1036))
def test_random_combination(seed):
    c = _draw(seed)
    rng = c["rng"]
    w = synth.PREFILL_B4_T4096.replace(B=c["B"], T=c["T"], H=c["H"], dk=c["dk"], dv=c["dv"],
                                       dtype=c["dtype"], a_law=c["law"], init_state=c["init"],
                                       seed=seed)
    x = synth.prefill_inputs(w, with_logits=c["entry"] == "gate_logits")
    # 5e-3 for the 64-token kernel on the long-memory law (single-bfloat16 state operands)
    tol = 1e-5 if c["dtype"] == "f32" else (5e-3 if c["law"] == "slow" and c["chunk"] == 64 else 3e-3)
    print(f"[random] seed {seed}: {c['entry']} B{c['B']} T{c['T']} H{c['H']} dk{c['dk']} "
          f"dv{c['dv']} {c['dtype']} out={c['out']} chunk {c['chunk']} {c['law']} "
          f"init={c['init']}", flush=True)
    names = ["q", "k", "v", "g", "beta", "s0"] + (["a"] if c["entry"] == "gate_logits" else [])
    d = synth.to_torch({n: x[n] for n in names}, w.dtype, DEV)
    s0 = d["s0"] if c["init"] else None
    s0_np = x["s0"] if c["init"] else None
    g_ref = x["g"]
    kw = dict(chunk=c["chunk"], out_dtype=c["out"])
    every, positions = 0, None
    z = None
    if c["entry"] == "every" and c["T"] >= c["chunk"]:
        every = c["chunk"] * int(rng.integers(1, max(2, c["T"] // c["chunk"] + 1)))
        kw["checkpoint_every"] = every
    elif c["entry"] == "positions" and c["T"] >= c["chunk"]:
        ends = np.arange(c["chunk"], c["T"] + 1, c["chunk"])
        pick = np.sort(rng.choice(ends, size=min(len(ends), int(rng.integers(1, 4))),
                                  replace=False))
        positions = pick.astype(np.int64)
    elif c["entry"] == "segments":
        kw["segment_tokens"] = c["chunk"] * int(rng.integers(1, 6))
    elif c["entry"] == "output_gate":
        z = synth.gate_inputs(w)
        kw["output_gate"] = synth.to_torch({"z": z}, w.dtype, DEV)["z"]
    if positions is not None:
        pos = torch.from_numpy(positions).to(DEV)
        o, s, ck = kda.kda_chunk_fwd_checkpoints_at(d["q"], d["k"], d["v"], d["g"], d["beta"], pos,
                                                    s0, chunk=c["chunk"], out_dtype=c["out"])
    elif c["entry"] == "gate_logits":
        o, s, ck = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["a"], d["beta"], s0,
                                     gate_logits=True, **kw)
        g_ref = oracle.log_decay_from_logits(x["a"])
    else:
        o, s, ck = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], s0, **kw)
    torch.cuda.synchronize()
    (o_r, s_r, ck_r), _ = oracle.kda_forward_heads_parallel(x["q"], x["k"], x["v"], g_ref,
                                                            x["beta"], s0_np, every)
    if z is not None:
        o_r = oracle.apply_output_gate(o_r, z)
    parity.check("o", o, o_r, tol, "tokens")
    parity.check("final state", s, s_r, tol, "state")
    if every:
        parity.check("checkpoints", ck, ck_r, tol, "ckpt")
    if positions is not None:
        # the oracle's state after each listed position: its checkpoints every chunk
        (_, _, ck_all), _ = oracle.kda_forward_heads_parallel(x["q"], x["k"], x["v"], g_ref,
                                                              x["beta"], s0_np, c["chunk"])
        want = ck_all[:, positions // c["chunk"] - 1]
        parity.check("listed checkpoints", ck, want, tol, "ckpt")
