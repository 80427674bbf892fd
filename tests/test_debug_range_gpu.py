"""The range-check build (libkda_debug.so, include/kda_debug.h) on the GPU.

The chunk kernels of that build check, as they run, what the -5 log-decay floor
guarantees (orkas.ai blog "Kimi K3 architecture", section "A lower bound that deleted a
GPU code path"): a diagonal tile's row factor 2^L in [0, 1] and column factor 2^-L in
[1, e^80], every product operand finite and inside the bfloat16 range, every kept A / P
tile entry and every state value finite.  Here: no violation on the decay-floor workload
at full size (65,536 tokens x 32 heads, about half of all channels on the floor), with
every channel on the floor at every chunk length (segment path included), with keys of
norm up to 30, and on the float32 path; and, as negative controls, keys of norm 1e5 at
the floor (column operands beyond the bfloat16 range) and a NaN log-decay (NaN factors)
do raise their bits.  Results of the checked runs also match the oracle and the release
library.
"""
import ctypes

import numpy as np
import pytest
import torch

import gated_delta_rule_57_amd as kda
import oracle
import parity
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
FACTOR, OPERAND, TILE, STATE = 1, 2, 4, 8


@pytest.fixture(scope="module")
def dlib():
    lib = kda.load_library(kda.DEBUG_LIB_PATH)
    lib.kda_debug_range_flags.restype = ctypes.c_int
    lib.kda_debug_range_flags.argtypes = [ctypes.POINTER(ctypes.c_uint), ctypes.c_int]
    return lib


def _flags(lib, clear=True) -> int:
    f = ctypes.c_uint(0xFFFFFFFF)
    assert lib.kda_debug_range_flags(ctypes.byref(f), 1 if clear else 0) == 0
    return f.value


def _fwd(lib, d, chunk, out_dtype=torch.float32):
    """kda_chunk_fwd of library `lib` (the library picks the segmentation)."""
    B, T, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    o = torch.empty((B, T, H, dv), dtype=out_dtype, device=DEV)
    sf = torch.empty_like(d["s0"])
    cin, cout = kda._dtype_code(d["q"].dtype), kda._dtype_code(out_dtype)
    nws = lib.kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, cin)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=DEV)
    st = lib.kda_chunk_fwd(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(),
                           d["g"].data_ptr(), d["beta"].data_ptr(), d["s0"].data_ptr(),
                           o.data_ptr(), sf.data_ptr(), None, 0, B, T, H, dk, dv, chunk, cin,
                           cout, ws.data_ptr() if nws else None, nws,
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0, kda.status_str(st)
    torch.cuda.synchronize()
    return o, sf


def _floor(x):
    g = np.full_like(x["g"], -5.0)
    g[..., ::3] = -7.0  # below the floor: clamped to it
    return dict(x, g=g)


def test_flag_word_reads_and_clears(dlib):
    _flags(dlib)
    assert _flags(dlib) == 0


@pytest.mark.parametrize("chunk", [64, 32, 16])
def test_every_channel_on_the_floor(dlib, chunk):
    """Every channel of every token at (or below) the floor, few heads and 2,085 tokens:
    the library cuts segments, so summaries from the identity run too."""
    w = synth.PREFILL_B4_T4096.replace(B=1, T=2048 + 37, H=4, init_state=True)
    assert kda.kda_chunk_fwd_segment_tokens(w.B, w.T, w.H, w.dk, w.dv, chunk) < w.T
    x = _floor(synth.prefill_inputs(w))
    d = synth.to_torch(x, w.dtype, DEV)
    _flags(dlib)
    print(f"[range] floor, chunk {chunk}", flush=True)
    o, s = _fwd(dlib, d, chunk)
    assert _flags(dlib) == 0
    (o_r, s_r, _), _ = oracle.kda_forward_heads_parallel(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                                         x["s0"], 0)
    parity.check(f"o, floor, chunk {chunk}, checked build", o, o_r, 3e-3, "tokens")
    parity.check(f"state, floor, chunk {chunk}, checked build", s, s_r, 3e-3, "state")
    # the checks add no arithmetic: the release library agrees to within rounding (the
    # compiler schedules the two builds differently, so the bits may differ)
    o2, s2, _ = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], chunk=chunk,
                                  out_dtype=torch.float32)
    torch.cuda.synchronize()
    e_o = oracle.rel_l2(o.cpu().double().numpy(), o2.cpu().double().numpy())
    e_s = oracle.rel_l2(s.cpu().double().numpy(), s2.cpu().double().numpy())
    print(f"[range] checked vs release build, chunk {chunk}: o {e_o:.2e} state {e_s:.2e}", flush=True)
    assert e_o <= 1e-3 and e_s <= 1e-3


def test_decay_floor_workload_full_size(dlib):
    """65,536 tokens x 32 heads, decay logits ~ N(5, 1): about half of all channels on the
    floor, 16-token sums reaching -80; the library's segment path."""
    w = synth.DECAY_FLOOR_T65536
    d = synth.device_prefill_inputs(w, DEV)
    _flags(dlib)
    print("[range] decay-floor workload, 65,536 x 32", flush=True)
    o, s = _fwd(dlib, d, 64, out_dtype=torch.bfloat16)
    assert _flags(dlib) == 0
    assert bool(torch.isfinite(s).all())


@pytest.mark.parametrize("chunk", [64, 32])
def test_large_keys_at_the_floor(dlib, chunk):
    w = synth.PREFILL_B4_T4096.replace(B=1, T=333, H=4, init_state=True, seed=5)
    x = _floor(synth.scale_keys(synth.prefill_inputs(w), w))
    d = synth.to_torch(x, w.dtype, DEV)
    _flags(dlib)
    _fwd(dlib, d, chunk)
    assert _flags(dlib) == 0


def test_float32_path_on_the_floor(dlib):
    w = synth.TINY_F32.replace(T=300, H=3, init_state=True)
    x = _floor(synth.prefill_inputs(w))
    d = synth.to_torch(x, w.dtype, DEV)
    _flags(dlib)
    o, s = _fwd(dlib, d, 64)
    assert _flags(dlib) == 0
    (o_r, s_r, _), _ = oracle.kda_forward_heads_parallel(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                                         x["s0"], 0)
    parity.check("o, float32, floor, checked build", o, o_r, 1e-5, "tokens")


@pytest.mark.parametrize("chunk", [64, 32])
def test_keys_beyond_the_bound_raise_the_operand_bit(dlib, chunk):
    """Negative control: keys of norm 1e5 at the floor make column operands of about
    1e5 / sqrt(128) x e^80 > 3.4e38, beyond the bfloat16 range."""
    w = synth.PREFILL_B4_T4096.replace(B=1, T=64, H=1, init_state=True)
    x = _floor(synth.prefill_inputs(w))
    x["k"] = synth.round_to(x["k"] * 1e5, w.dtype)
    d = synth.to_torch(x, w.dtype, DEV)
    _flags(dlib)
    _fwd(dlib, d, chunk)
    f = _flags(dlib)
    print(f"[range] keys of norm 1e5, chunk {chunk}: flags {f:#x}", flush=True)
    assert f & OPERAND


@pytest.mark.parametrize("chunk", [64, 32])
def test_nan_log_decay_raises_the_factor_bit(dlib, chunk):
    """Negative control: a NaN log-decay propagates (as the method requires) into that
    channel's decay factors, which the check reports."""
    w = synth.PREFILL_B4_T4096.replace(B=1, T=64, H=1, init_state=True)
    x = synth.prefill_inputs(w)
    x["g"][0, 5, 0, 3] = np.nan
    d = synth.to_torch(x, w.dtype, DEV)
    _flags(dlib)
    _fwd(dlib, d, chunk)
    f = _flags(dlib)
    print(f"[range] NaN log-decay, chunk {chunk}: flags {f:#x}", flush=True)
    assert f & FACTOR
