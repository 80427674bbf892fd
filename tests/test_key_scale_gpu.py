"""Keys and queries that are not unit-norm (norms up to 30) at the log-decay floor.

The chunked kernels factor each diagonal tile's decay into a row factor <= 1 and a
column factor up to e^80 (16 tokens at the -5 floor), which the orkas.ai "Kimi K3
architecture" blog ("A lower bound that deleted a GPU code path") shows fits bfloat16.
With |k| up to 30 the column operand reaches 30 e^80 and the masked (upper) entries of
a diagonal tile's product overflow float32; the kernels must discard them by select,
and the kept entries must keep their relative precision.  Every chunk length, both
kernels, against the float64 oracle.
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


def _case(dtype, law, floor_every_channel, T=333, H=4, d=128, seed=5):
    w = synth.PREFILL_B4_T4096.replace(B=1, T=T, H=H, dk=d, dv=d, dtype=dtype, a_law=law,
                                       seed=seed, init_state=True)
    x = synth.scale_keys(synth.prefill_inputs(w), w)
    if floor_every_channel:
        g = np.full_like(x["g"], -5.0)
        g[..., ::3] = -7.0  # below the floor: clamped to it
        x["g"] = g
    kn = np.linalg.norm(x["k"], axis=-1)
    assert kn.max() > 25.0 and kn.min() < 1.5
    assert np.all(x["beta"] * kn ** 2 < 2.0)
    return w, x


@pytest.mark.parametrize("chunk", [64, 32, 16])
@pytest.mark.parametrize("floor", [True, False])
def test_large_keys_bf16(chunk, floor):
    w, x = _case("bf16", "n02", floor)
    d = synth.to_torch(x, w.dtype, DEV)
    print(f"[keys] bf16 chunk {chunk} floor={floor}", flush=True)
    o, s, _ = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"],
                                chunk=chunk, out_dtype=torch.float32)
    torch.cuda.synchronize()
    (o_r, s_r, _), _ = oracle.kda_forward_heads_parallel(x["q"], x["k"], x["v"], x["g"],
                                                         x["beta"], x["s0"], 0)
    assert np.isfinite(o.cpu().numpy()).all() and np.isfinite(s.cpu().numpy()).all()
    parity.check(f"o, large keys, chunk {chunk}", o, o_r, 3e-3, "tokens")
    parity.check(f"state, large keys, chunk {chunk}", s, s_r, 3e-3, "state")


@pytest.mark.parametrize("floor", [True, False])
def test_large_keys_f32(floor):
    """float32 inputs (the library's float32 path takes d_k = d_v = 64)."""
    w, x = _case("f32", "n02", floor, d=64)
    d = synth.to_torch(x, w.dtype, DEV)
    print(f"[keys] f32 floor={floor}", flush=True)
    o, s, _ = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"])
    torch.cuda.synchronize()
    (o_r, s_r, _), _ = oracle.kda_forward_heads_parallel(x["q"], x["k"], x["v"], x["g"],
                                                         x["beta"], x["s0"], 0)
    parity.check("o, large keys, f32", o, o_r, 1e-5, "tokens")
    parity.check("state, large keys, f32", s, s_r, 1e-5, "state")
