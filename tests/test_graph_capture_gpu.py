"""Graph capture: the entry points that allocate nothing, replayed from a HIP graph.

A caller under graph capture cannot allocate; kda_chunk_fwd_noalloc (whose segment-path
workspace is the library's static device array) and kda_recurrent_step (no workspace)
are captured into one graph together with the output buffers the caller owns.  The
graph is replayed three times, with new inputs copied into the captured input buffers
by ordinary eager work between replays, and every replay's outputs are compared bit for
bit with eager calls of the same entry points on the same inputs.
"""
import pytest
import torch

import gated_delta_rule_57_amd as kda
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_noalloc_prefill_and_decode_replayed_from_a_graph():
    w = synth.PREFILL_B4_T4096.replace(B=1, T=4096 + 5, H=4)
    assert kda.kda_chunk_fwd_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv) > 0  # segment path
    wd = synth.DECODE_N256.replace(B=8, H=4)
    names = ("q", "k", "v", "g", "beta", "s0")
    pin = {n: t.clone() for n, t in synth.device_prefill_inputs(w, DEV).items()}
    dec0 = synth.device_decode_inputs(wd, 1, DEV)
    din = {n: (t[0].clone() if n != "s0" else t.clone()) for n, t in dec0.items()}
    state = din["s0"].clone()
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=pin["q"].dtype, device=DEV)
    s = torch.empty_like(pin["s0"])
    od = torch.empty((wd.B, wd.H, wd.dv), dtype=din["q"].dtype, device=DEV)

    def body():
        kda.kda_chunk_fwd_noalloc(*(pin[n] for n in names), o, s)
        kda.kda_recurrent_step(din["q"], din["k"], din["v"], din["g"], din["beta"], state, o=od)

    # eager warm-up (the first no-allocation call on a device looks up its array)
    body()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        body()
    torch.cuda.synchronize()

    for r in range(3):
        fresh = synth.device_prefill_inputs(w, DEV, seed_offset=r + 1)
        dfresh = synth.device_decode_inputs(wd, 1, DEV, seed_offset=r + 1)
        for n in names:
            pin[n].copy_(fresh[n])
        for n in ("q", "k", "v", "g", "beta"):
            din[n].copy_(dfresh[n][0])
        state.copy_(dfresh["s0"])
        torch.cuda.synchronize()
        print(f"[graph] replay {r}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        ref_o, ref_s, _ = kda.kda_chunk_fwd(*(fresh[n] for n in names))
        ref_state = dfresh["s0"].clone()
        ref_od = kda.kda_recurrent_step(dfresh["q"][0], dfresh["k"][0], dfresh["v"][0],
                                        dfresh["g"][0], dfresh["beta"][0], ref_state)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(s, ref_s), f"prefill, replay {r}"
        assert torch.equal(od, ref_od) and torch.equal(state, ref_state), f"decode, replay {r}"
