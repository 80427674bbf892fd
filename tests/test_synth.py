"""The seeded input generators: laws, determinism, prefix consistency, exact dtypes."""
import numpy as np
import pytest
import torch

import synth


def test_prefix_is_consistent_with_full_sequence():
    w = synth.TINY_F32.replace(T=300)
    full = synth.prefill_inputs(w)
    pre = synth.prefill_inputs(w, t_end=100)
    for n in ("q", "k", "v", "g", "beta"):
        assert np.array_equal(full[n][:, :100], pre[n])
    assert np.array_equal(full["s0"], pre["s0"])


def test_block_boundaries_regenerate(monkeypatch):
    monkeypatch.setattr(synth, "BLOCK_T", 64)
    w = synth.TINY_F32.replace(T=200)
    full = synth.prefill_inputs(w)
    pre = synth.prefill_inputs(w, t_end=130)
    assert np.array_equal(full["k"][:, :130], pre["k"])


@pytest.mark.parametrize("w", [synth.TINY_F32, synth.PREFILL_B4_T4096.replace(B=1, T=128, H=2),
                               synth.DECAY_FLOOR_T65536.replace(T=128, H=2),
                               synth.MILLION_TOKEN.replace(T=128, H=2)], ids=lambda w: w.name)
def test_laws(w):
    x = synth.prefill_inputs(w)
    tol = 1e-6 if w.dtype == "f32" else 1e-2
    assert np.allclose(np.linalg.norm(x["q"], axis=-1), 1.0, atol=tol)
    assert np.allclose(np.linalg.norm(x["k"], axis=-1), 1.0, atol=tol)
    assert np.all(x["g"] >= -5.0) and np.all(x["g"] < 0.0)
    assert np.all(x["beta"] > 0.0) and np.all(x["beta"] < 1.0)
    if w.a_law == "n51":
        assert np.mean(x["g"] == -5.0) > 0.3
    if w.a_law == "mixed":
        half = w.dk // 2
        assert np.mean(x["g"][..., half:] == -5.0) > 0.3
        assert np.mean(x["g"][..., :half] == -5.0) < 0.05
    if w.init_state:
        assert 0.015 < np.std(x["s0"]) < 0.025
    else:
        assert not np.any(x["s0"])
    # values are exactly representable in the storage dtype
    td = synth.torch_dtype(w.dtype)
    for n in ("q", "k", "v", "g", "beta"):
        t = torch.from_numpy(x[n])
        assert torch.equal(t.to(td).to(torch.float64), t)


def test_decode_steps_are_seeded_per_step():
    w = synth.DECODE_N256.replace(B=4, H=2)
    a = synth.decode_step_inputs(w, 5)
    b = synth.decode_step_inputs(w, 5)
    c = synth.decode_step_inputs(w, 6)
    assert np.array_equal(a["q"], b["q"]) and not np.array_equal(a["q"], c["q"])
    sub = synth.decode_step_inputs(w, 5, seqs=slice(1, 3))
    assert np.array_equal(sub["v"], a["v"][1:3])


def test_device_generator_laws_on_cpu():
    w = synth.DECAY_FLOOR_T65536.replace(T=256, H=2)
    d = synth.device_prefill_inputs(w, "cpu")
    assert d["q"].dtype == torch.bfloat16 and d["s0"].dtype == torch.float32
    g = d["g"].float()
    assert bool((g >= -5).all()) and bool((g < 0).all())
    assert float((g == -5).float().mean()) > 0.3


def test_scale_keys_recipe():
    """Large-key inputs: norms in [1, 30], beta |k|^2 < 2, storage-dtype values, seeded,
    v, g and the initial state untouched."""
    w = synth.PREFILL_B4_T4096.replace(B=1, T=200, H=3, dk=64, dv=64, init_state=True)
    x = synth.prefill_inputs(w)
    a = synth.scale_keys(x, w)
    b = synth.scale_keys(x, w)
    for n in ("q", "k", "beta"):
        assert np.array_equal(a[n], b[n])
        assert np.array_equal(synth.round_to(a[n], w.dtype), a[n])
    for n in ("v", "g", "s0"):
        assert a[n] is x[n]
    for n in ("q", "k"):
        norms = np.linalg.norm(a[n], axis=-1)
        assert norms.min() > 0.97 and norms.max() < 30.5
        assert (norms > 15).mean() > 0.15 and (norms < 3).mean() > 0.15
    bk = a["beta"] * np.sum(a["k"] ** 2, axis=-1)
    assert bk.max() < 2.0 and bk.min() >= 0.0 and bk.mean() > 0.5
