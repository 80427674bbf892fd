"""Identities of the GPU path that need no oracle: state hand-off, aliasing, determinism,
the clamp, padding, decode-versus-prefill agreement."""
import numpy as np
import pytest
import torch

import gated_delta_rule_57_amd as kda
import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(w):
    return synth.to_torch(synth.prefill_inputs(w), w.dtype, DEV)


def _fwd(d, s0="s0", **kw):
    return kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                             d[s0] if isinstance(s0, str) else s0, **kw)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_at_chunk_boundary_matches_monolithic(dtype):
    w = synth.PREFILL_B4_T4096.replace(B=2, T=448, H=3, dtype=dtype,
                                       dk=64 if dtype == "f32" else 128,
                                       dv=64 if dtype == "f32" else 128)
    d = _inputs(w)
    one = 1 << 40  # one segment: the single pass of the chunk kernel
    o, sf, _ = _fwd(d, segment_tokens=one)
    cut = 192
    first = {n: d[n][:, :cut].contiguous() for n in ("q", "k", "v", "g", "beta")}
    rest = {n: d[n][:, cut:].contiguous() for n in ("q", "k", "v", "g", "beta")}
    o1, s1, _ = _fwd(dict(first, s0=d["s0"]), segment_tokens=one)
    o2, s2, _ = _fwd(dict(rest, s0=s1), segment_tokens=one)
    torch.cuda.synchronize()
    # same arithmetic per chunk, so the hand-off is exact
    assert torch.equal(torch.cat([o1, o2], 1), o) and torch.equal(s2, sf)


def test_in_place_state_update_and_determinism():
    w = synth.PREFILL_B4_T4096.replace(B=2, T=300, H=4)
    d = _inputs(w)
    o_a, s_a, _ = _fwd(d)
    o_b, s_b, _ = _fwd(d)
    st = d["s0"].clone()
    o_c, s_c, _ = _fwd(d, s0=st, final_state=st)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(s_a, s_b)  # run-to-run bitwise
    assert s_c.data_ptr() == st.data_ptr()
    assert torch.equal(o_c, o_a) and torch.equal(st, s_a)


def test_clamp_below_floor_is_bitwise_the_floor():
    w = synth.PREFILL_B4_T4096.replace(B=1, T=256, H=2)
    x = synth.prefill_inputs(w)
    lo = dict(x)
    lo["g"] = x["g"].copy()
    lo["g"][..., ::3] = -5.0
    far = dict(lo)
    far["g"] = lo["g"].copy()
    far["g"][..., ::3] = -7.0
    far["g"][..., 1::7] = 0.0
    lo["g"][..., 1::7] = 0.0
    far["g"][..., 1::7] = 3.0  # above zero: clamped to zero
    a = _fwd(synth.to_torch(lo, w.dtype, DEV))
    b = _fwd(synth.to_torch(far, w.dtype, DEV))
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_padding_with_no_op_tokens_is_neutral():
    w = synth.PREFILL_B4_T4096.replace(B=1, T=130, H=2)
    x = synth.prefill_inputs(w)
    pad = 62
    y = {}
    for n in ("q", "k", "v", "g", "beta"):
        z = np.zeros((x[n].shape[0], pad) + x[n].shape[2:])
        if n in ("q", "k", "v"):
            z = np.random.default_rng(0).standard_normal(z.shape)
        y[n] = np.concatenate([x[n], z], axis=1)
    y["s0"] = x["s0"]
    a = _fwd(synth.to_torch(x, w.dtype, DEV), segment_tokens=1 << 40)
    b = _fwd(synth.to_torch(y, w.dtype, DEV), segment_tokens=1 << 40)
    torch.cuda.synchronize()
    assert torch.allclose(a[1], b[1], rtol=0, atol=1e-6 * float(a[1].abs().max()))
    assert torch.equal(a[0], b[0][:, :130])


def test_nan_in_decay_stays_in_its_head():
    w = synth.PREFILL_B4_T4096.replace(B=1, T=128, H=3)
    x = synth.prefill_inputs(w)
    x["g"][0, 70, 1, 5] = np.nan
    o, sf, _ = _fwd(synth.to_torch(x, w.dtype, DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isnan(sf[0, 1]).any() and torch.isfinite(sf[0, [0, 2]]).all()
    assert torch.isfinite(o[0, :, [0, 2]]).all() and torch.isfinite(o[0, :64, 1]).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_steps_equal_prefill(dtype):
    d_ = 64 if dtype == "f32" else 128
    w = synth.PREFILL_B4_T4096.replace(B=2, T=40, H=2, dtype=dtype, dk=d_, dv=d_)
    x = synth.prefill_inputs(w)
    d = synth.to_torch(x, w.dtype, DEV)
    o, sf, _ = _fwd(d, out_dtype=torch.float32)
    st = d["s0"].clone()
    outs = []
    for t in range(w.T):
        outs.append(kda.kda_recurrent_step(d["q"][:, t].contiguous(), d["k"][:, t].contiguous(),
                                           d["v"][:, t].contiguous(), d["g"][:, t].contiguous(),
                                           d["beta"][:, t].contiguous(), st,
                                           out_dtype=torch.float32))
    torch.cuda.synchronize()
    od = torch.stack(outs, 1)
    tol = 1e-5 if dtype == "f32" else 3e-3
    assert oracle.rel_l2(od.double().cpu().numpy(), o.double().cpu().numpy()) <= tol
    assert oracle.rel_l2(st.double().cpu().numpy(), sf.double().cpu().numpy()) <= tol
