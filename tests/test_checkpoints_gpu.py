"""kda_chunk_fwd_checkpoints_at: states saved after listed token counts (a sparse subset of
fixed-size block ends, as prefix caching keeps them), against the float64 oracle; entries
that are not chunk ends inside the sequence are left untouched; a restored checkpoint
continues the sequence."""
import numpy as np
import pytest
import torch

import gated_delta_rule_57_amd as kda
import oracle
import parity
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _oracle_chunk_states(x):
    """Oracle states after every 64 tokens: [B, T // 64, H, dk, dv]; plus o."""
    (o, s, ck), _ = oracle.kda_forward_heads_parallel(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                                      x["s0"], 64)
    return o, s, ck


def _np(t):
    return t.double().cpu().numpy()


@pytest.mark.parametrize("B,T,H,positions", [
    (2, 700, 3, [128, 512, 640]),             # one segment
    (1, 4096, 4, [512, 1024, 2560, 4096]),    # the library cuts this into segments
])
def test_listed_positions_match_oracle(B, T, H, positions):
    w = synth.PREFILL_B4_T4096.replace(B=B, T=T, H=H)
    seg = kda.kda_chunk_fwd_segment_tokens(B, T, H, w.dk, w.dv)
    x = synth.prefill_inputs(w)
    d = synth.to_torch(x, w.dtype, DEV)
    pos = torch.tensor(positions, dtype=torch.int64, device=DEV)
    o, sf, ck = kda.kda_chunk_fwd_checkpoints_at(d["q"], d["k"], d["v"], d["g"], d["beta"], pos,
                                                 d["s0"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_r, s_r, ck_r = _oracle_chunk_states(x)
    want = ck_r[:, [p // 64 - 1 for p in positions]]
    print(f"[ckpt] B{B} T{T} H{H} segment {seg}", flush=True)
    parity.check("checkpoints", ck, want, 3e-3, "ckpt")
    parity.check("o", o, o_r, 3e-3, "tokens")
    if positions[-1] == T:
        assert torch.equal(ck[:, -1], sf)


def test_entries_off_chunk_ends_are_untouched():
    w = synth.PREFILL_B4_T4096.replace(B=1, T=320, H=2)
    x = synth.prefill_inputs(w)
    d = synth.to_torch(x, w.dtype, DEV)
    positions = [100, 256, 300, 4096]  # 100, 300: not chunk ends; 4096: past the end
    pos = torch.tensor(positions, dtype=torch.int64, device=DEV)
    ck = torch.full((1, len(positions), 2, w.dk, w.dv), float("nan"), device=DEV)
    kda.kda_chunk_fwd_checkpoints_at(d["q"], d["k"], d["v"], d["g"], d["beta"], pos, d["s0"],
                                     checkpoints=ck)
    torch.cuda.synchronize()
    assert torch.isnan(ck[:, [0, 2, 3]]).all()
    _, _, ck_r = _oracle_chunk_states(x)
    parity.check("checkpoint after 256 tokens", ck[:, 1], ck_r[:, 256 // 64 - 1], 3e-3, "state")


def test_restoring_a_checkpoint_continues_the_sequence():
    """Prefix-cache hit: the state saved after 512 tokens, used as the initial state of the
    remaining tokens, continues the sequence: outputs and final state match the oracle's
    uninterrupted run (and the library's own)."""
    w = synth.PREFILL_B4_T4096.replace(B=2, T=1024, H=3)
    x = synth.prefill_inputs(w)
    d = synth.to_torch(x, w.dtype, DEV)
    pos = torch.tensor([512], dtype=torch.int64, device=DEV)
    o, sf, ck = kda.kda_chunk_fwd_checkpoints_at(d["q"], d["k"], d["v"], d["g"], d["beta"], pos,
                                                 d["s0"], out_dtype=torch.float32)
    rest = {n: d[n][:, 512:].contiguous() for n in ("q", "k", "v", "g", "beta")}
    o2, s2, _ = kda.kda_chunk_fwd(rest["q"], rest["k"], rest["v"], rest["g"], rest["beta"],
                                  ck[:, 0].contiguous(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_r, s_r, _ = _oracle_chunk_states(x)
    print("[ckpt] restored at 512", flush=True)
    parity.check("o after the restore", o2, o_r[:, 512:], 3e-3, "tokens")
    parity.check("final state", s2, s_r, 3e-3, "state")
    assert oracle.rel_l2(_np(o2), _np(o[:, 512:])) <= 1e-3
