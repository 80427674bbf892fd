"""Seeded synthetic inputs for Kimi Delta Attention (KDA) workloads.

This module is shared by the CPU oracle, the GPU parity tests and the bench.
It only draws random numbers and rounds them to the storage dtype; it holds
none of the KDA arithmetic (no decay, no delta update, no chunking).

Input recipe (one per workload, all tensors token-major ``[B, T, H, D]``):

* q, k ~ N(0, 1), then each head vector is scaled to unit L2 norm;
* v ~ N(0, 1);
* beta = sigmoid(x) with x ~ N(0, 1), one scalar per (token, head);
* g = max(-softplus(a), -5) per channel, with the decay logit ``a`` drawn
  from N(0, 2) (variance 2), N(5, 1), or a per-channel mix of the two.
  The negative-softplus parametrisation of the decay logits is the one the
  Towards-AI article on Kimi K3 describes in its "Kimi Delta Attention"
  section; the -5 floor is the one the orkas.ai "Kimi K3 architecture" blog
  gives in "A lower bound that deleted a GPU code path".
* initial state S0 ~ N(0, 0.02^2) per element, or zeros.

Floating-point inputs are drawn in float64, normalised in float64, then
rounded to the storage dtype (round-to-nearest-even, torch semantics).  The
float64 arrays returned alongside hold exactly the rounded values, so the
oracle sees bit-for-bit what the GPU receives.

Token blocks: the T axis is drawn in blocks of ``BLOCK_T`` tokens, block
``j`` from ``SeedSequence([seed, j])``.  Any prefix (or block) of a long
sequence can therefore be regenerated alone, and a prefix of a workload is
identical to the same tokens of the full workload.  The initial state comes
from ``SeedSequence([seed, STATE_STREAM])``.

Decode workloads draw the inputs of step ``s`` from ``SeedSequence([seed,
DECODE_STREAM, s])``.

Output-gate inputs (the gate projection z, one value per token, head and value
channel) are z ~ N(0, 1), from ``SeedSequence([seed, GATE_STREAM])``.

Large-key inputs (``scale_keys``): each (token, head) query and key vector is
rescaled to a norm drawn log-uniformly from [1, max_norm], and beta is redrawn as
u * 1.9 / |k|^2 with u ~ U(0, 1), which keeps beta |k|^2 < 2 (so the factor
1 - beta |k|^2 of the delta update along k stays inside (-1, 1)).  Draws come from
``SeedSequence([seed, KEY_SCALE_STREAM])``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BLOCK_T = 65536
STATE_STREAM = 0x7FFF_0001
DECODE_STREAM = 0x7FFF_0002
GATE_STREAM = 0x7FFF_0003
KEY_SCALE_STREAM = 0x7FFF_0004

_SQRT2 = math.sqrt(2.0)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic KDA workload (shapes, dtype and the decay-logit law)."""

    name: str
    kind: str  # "prefill" or "decode"
    B: int  # batch (prefill) or independent sequences N (decode)
    T: int  # tokens (prefill) or chained steps (decode)
    H: int
    dk: int
    dv: int
    chunk: int
    dtype: str  # "f32" or "bf16": storage dtype of q, k, v, g, beta
    a_law: str  # "n02" = N(0, 2), "n51" = N(5, 1), "mixed" = half/half, "slow" = N(-7, 1)
    init_state: bool
    seed: int

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads the KDA path is measured and checked on.
TINY_F32 = Workload("tiny_fp32_b1_t256_h2_d64", "prefill", 1, 256, 2, 64, 64, 64,
                    "f32", "n02", False, 0)
PREFILL_B4_T4096 = Workload("prefill_bf16_b4_t4096_h32_d128", "prefill", 4, 4096, 32, 128,
                            128, 64, "bf16", "n02", True, 1)
DECAY_FLOOR_T65536 = Workload("decay_floor_bf16_b1_t65536_h32_d128", "prefill", 1, 65536, 32,
                              128, 128, 64, "bf16", "n51", True, 2)
DECODE_N256 = Workload("decode_bf16_n256_h32_d128_1000steps", "decode", 256, 1000, 32, 128,
                       128, 1, "bf16", "n02", True, 3)
MILLION_TOKEN = Workload("million_token_bf16_b1_t1048576_h16_d128", "prefill", 1, 1 << 20,
                         16, 128, 128, 64, "bf16", "mixed", True, 4)

WORKLOADS = {w.name: w for w in (TINY_F32, PREFILL_B4_T4096, DECAY_FLOOR_T65536, DECODE_N256,
                                 MILLION_TOKEN)}


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 ``x`` to ``dtype`` ("f32"/"bf16"/"f64"); return float64 values."""
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        import torch

        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
        return t.to(torch.bfloat16).to(torch.float64).numpy()
    raise ValueError(f"unknown dtype {dtype!r}")


def _softplus(a: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, a)


def _unit(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _decay_logits(rng: np.random.Generator, shape, a_law: str) -> np.ndarray:
    if a_law == "n02":
        return rng.normal(0.0, _SQRT2, shape)
    if a_law == "n51":
        return rng.normal(5.0, 1.0, shape)
    if a_law == "slow":
        # long memory (g ~ -1e-3 per token): a state carries across thousands of
        # tokens, so long-range hand-offs are exercised, not erased by the decay
        return rng.normal(-7.0, 1.0, shape)
    if a_law == "mixed":
        d = shape[-1]
        a = rng.normal(0.0, _SQRT2, shape)
        hi = rng.normal(5.0, 1.0, shape)
        a[..., d // 2:] = hi[..., d // 2:]
        return a
    raise ValueError(f"unknown decay-logit law {a_law!r}")


def _draw_block(rng, B, t, H, dk, dv, a_law):
    q = _unit(rng.standard_normal((B, t, H, dk)))
    k = _unit(rng.standard_normal((B, t, H, dk)))
    v = rng.standard_normal((B, t, H, dv))
    beta = _sigmoid(rng.standard_normal((B, t, H)))
    a = _decay_logits(rng, (B, t, H, dk), a_law)
    g = np.maximum(-_softplus(a), -5.0)
    return q, k, v, g, beta, a


def initial_state(w: Workload, heads: Optional[slice] = None) -> np.ndarray:
    """Initial state [B, H, dk, dv] as float64 holding float32-rounded values."""
    shape = (w.B, w.H, w.dk, w.dv)
    if not w.init_state:
        s0 = np.zeros(shape)
    else:
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, STATE_STREAM])))
        s0 = round_to(rng.normal(0.0, 0.02, shape), "f32")
    return s0 if heads is None else s0[:, heads]


def prefill_inputs(w: Workload, t_end: Optional[int] = None, with_logits: bool = False):
    """Inputs of a prefill workload for tokens [0, t_end).

    Returns a dict of float64 arrays (exactly the storage-dtype values):
    q, k [B,t,H,dk]; v [B,t,H,dv]; g [B,t,H,dk]; beta [B,t,H]; s0 [B,H,dk,dv];
    with ``with_logits`` also the raw decay logits a [B,t,H,dk] that g was made
    from (rounded to the storage dtype on their own).
    """
    assert w.kind == "prefill"
    t_end = w.T if t_end is None else min(t_end, w.T)
    parts = []
    for blk in range((t_end + BLOCK_T - 1) // BLOCK_T):
        t0 = blk * BLOCK_T
        tb = min(BLOCK_T, w.T - t0)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, blk])))
        arrs = _draw_block(rng, w.B, tb, w.H, w.dk, w.dv, w.a_law)
        keep = min(tb, t_end - t0)
        parts.append([x[:, :keep] for x in arrs])
    names = ("q", "k", "v", "g", "beta") + (("a",) if with_logits else ())
    out = {n: round_to(np.concatenate([p[i] for p in parts], axis=1), w.dtype)
           for i, n in enumerate(names)}
    out["s0"] = initial_state(w)
    return out


def scale_keys(x: dict, w: Workload, max_norm: float = 30.0) -> dict:
    """A copy of prefill inputs ``x`` (from ``prefill_inputs(w)``) with q and k of
    norms log-uniform in [1, max_norm] per (token, head) and beta = u 1.9 / |k|^2,
    u ~ U(0, 1), all rounded to the storage dtype; float64 arrays."""
    shape = x["beta"].shape
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, KEY_SCALE_STREAM])))
    lo, hi = 0.0, math.log(max_norm)
    nq = np.exp(rng.uniform(lo, hi, shape))[..., None]
    nk = np.exp(rng.uniform(lo, hi, shape))[..., None]
    u = rng.uniform(0.0, 1.0, shape)
    out = dict(x)
    out["q"] = round_to(x["q"] / np.linalg.norm(x["q"], axis=-1, keepdims=True) * nq, w.dtype)
    k = round_to(x["k"] / np.linalg.norm(x["k"], axis=-1, keepdims=True) * nk, w.dtype)
    out["k"] = k
    out["beta"] = round_to(u * 1.9 / np.sum(k * k, axis=-1), w.dtype)
    return out


def gate_inputs(w: Workload, shape=None) -> np.ndarray:
    """Output-gate projection z ~ N(0, 1) with the shape of o ([B, T, H, dv] for a
    prefill workload, or `shape`), rounded to the storage dtype; float64."""
    if shape is None:
        shape = (w.B, w.T, w.H, w.dv)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, GATE_STREAM])))
    return round_to(rng.standard_normal(shape), w.dtype)


def decode_step_inputs(w: Workload, step: int, seqs: Optional[slice] = None):
    """Inputs of decode step ``step`` for all N sequences (or the slice ``seqs``).

    q, k, g [N,H,dk]; v [N,H,dv]; beta [N,H], float64 holding storage-dtype values.
    """
    assert w.kind == "decode"
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, DECODE_STREAM,
                                                                      step])))
    q, k, v, g, beta, _ = _draw_block(rng, w.B, 1, w.H, w.dk, w.dv, w.a_law)
    out = {}
    for n, x in zip(("q", "k", "v", "g", "beta"), (q, k, v, g, beta)):
        x = x[:, 0]
        if seqs is not None:
            x = x[seqs]
        out[n] = round_to(x, w.dtype)
    return out


def torch_dtype(dtype: str):
    import torch

    return {"f32": torch.float32, "bf16": torch.bfloat16, "f64": torch.float64}[dtype]


def to_torch(arrs: dict, dtype: str, device="cpu") -> dict:
    """Copy the float64 arrays of an input dict into torch tensors of ``dtype``.

    The initial state ``s0`` is always float32 (the state dtype).
    """
    import torch

    out = {}
    for n, x in arrs.items():
        dt = torch.float32 if n == "s0" else torch_dtype(dtype)
        out[n] = torch.from_numpy(np.ascontiguousarray(x)).to(dt).to(device).contiguous()
    return out


def device_prefill_inputs(w: Workload, device, seed_offset: int = 0):
    """Fill device tensors with a workload's distributions using torch's device RNG.

    Used where the host generator would be too slow for the volume (timing runs,
    full-length runs checked only through sampled or property-based comparisons).
    Same laws as :func:`prefill_inputs`; a different random stream.
    """
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(1_000_003 * (w.seed + 1) + seed_offset)
    dt = torch_dtype(w.dtype)
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv

    def unit(shape):
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        x = x / x.norm(dim=-1, keepdim=True)
        return x.to(dt)

    q = unit((B, T, H, dk))
    k = unit((B, T, H, dk))
    v = torch.randn((B, T, H, dv), generator=gen, device=device, dtype=torch.float32).to(dt)
    beta = torch.sigmoid(torch.randn((B, T, H), generator=gen, device=device)).to(dt)
    a = torch.randn((B, T, H, dk), generator=gen, device=device, dtype=torch.float32)
    if w.a_law == "n02":
        a.mul_(_SQRT2)
    elif w.a_law == "n51":
        a.add_(5.0)
    elif w.a_law == "slow":
        a.sub_(7.0)
    else:
        a[..., : dk // 2].mul_(_SQRT2)
        a[..., dk // 2:].add_(5.0)
    g = torch.clamp(-torch.nn.functional.softplus(a), min=-5.0).to(dt)
    del a
    if w.init_state:
        s0 = 0.02 * torch.randn((B, H, dk, dv), generator=gen, device=device, dtype=torch.float32)
    else:
        s0 = torch.zeros((B, H, dk, dv), device=device, dtype=torch.float32)
    return {"q": q, "k": k, "v": v, "g": g, "beta": beta, "s0": s0}


def device_decode_inputs(w: Workload, steps: int, device, seed_offset: int = 0):
    """Per-step decode inputs for ``steps`` chained steps, drawn on the device.

    q, k, g [steps,N,H,dk]; v [steps,N,H,dv]; beta [steps,N,H]; s0 [N,H,dk,dv] f32.
    """
    import torch

    ww = w.replace(kind="prefill", B=steps, T=w.B)
    d = device_prefill_inputs(ww, device, seed_offset)
    # prefill layout [B=steps, T=N, H, D] is exactly the decode layout [steps, N, H, D]
    if w.init_state:
        gen = torch.Generator(device=device)
        gen.manual_seed(2_000_003 * (w.seed + 1) + seed_offset)
        d["s0"] = 0.02 * torch.randn((w.B, w.H, w.dk, w.dv), generator=gen, device=device)
    else:
        d["s0"] = torch.zeros((w.B, w.H, w.dk, w.dv), device=device)
    return d


def device_one_hot_inputs(w: Workload, device, seed_offset: int = 0, memory_tokens: int = 4096):
    """A prefill workload's shapes and laws with one-hot keys and queries, on the device.

    Keys: k_t = e_{c_t} with c_t uniform over channels 0 .. dk-3 for every token
    and head, except that inside the first ``memory_tokens`` tokens every 64th
    token's key is channel dk-2 instead.  Channels dk-2 and dk-1 get log-decay 0
    (no decay): dk-2 is written early and then held for the rest of the sequence,
    dk-1 is never written.  Queries: q_t = e_{r_h}, one read channel r_h per head,
    uniform over 0 .. dk-3.  v, beta, the other channels' log-decays and the
    initial state follow the workload's laws.  One-hot vectors are exact in every
    storage dtype.

    Returns the tensors of :func:`device_prefill_inputs` plus ``chan`` [B,T,H]
    (int64, the key channel of each token) and ``read`` [H] (int64).
    """
    import torch

    d = device_prefill_inputs(w, device, seed_offset)
    gen = torch.Generator(device=device)
    gen.manual_seed(3_000_017 * (w.seed + 1) + seed_offset)
    B, T, H, dk = w.B, w.T, w.H, w.dk
    dt = torch_dtype(w.dtype)
    chan = torch.randint(0, dk - 2, (B, T, H), generator=gen, device=device)
    chan[:, : min(memory_tokens, T) : 64] = dk - 2
    read = torch.randint(0, dk - 2, (H,), generator=gen, device=device)
    k = torch.zeros((B, T, H, dk), dtype=dt, device=device)
    k.scatter_(-1, chan.unsqueeze(-1), 1.0)
    q = torch.zeros((B, T, H, dk), dtype=dt, device=device)
    q.scatter_(-1, read.view(1, 1, H, 1).expand(B, T, H, 1), 1.0)
    d["g"][..., dk - 2:] = 0.0
    d.update(q=q, k=k, chan=chan, read=read)
    return d
