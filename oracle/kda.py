"""Float64 token-by-token KDA recurrence (the oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).  Every array here is
float64; callers pass the exact values the GPU receives.
"""
from __future__ import annotations

import os
from typing import Optional

import numpy as np

# orkas.ai "Kimi K3 architecture" blog, "A lower bound that deleted a GPU code
# path": each step may forget down to ~0.67% of a channel and no further;
# exp(-5) = 0.674%, and 16 steps at the floor give the (-80, 0) tile range.
LOG_DECAY_FLOOR = -5.0


def clamp_log_decay(g: np.ndarray) -> np.ndarray:
    """g' = min(max(g, -5), 0), elementwise; NaN stays NaN (np.maximum keeps it)."""
    return np.minimum(np.maximum(np.asarray(g, dtype=np.float64), LOG_DECAY_FLOOR), 0.0)


def log_decay_from_logits(a: np.ndarray) -> np.ndarray:
    """g = -softplus(a) = -log(1 + e^a): the negative-softplus map from decay logits to
    log-decays (Towards-AI article on the Kimi K3 report, section "Kimi Delta Attention
    (KDA)").  Computed as -logaddexp(0, a) in float64, which is exact to rounding for
    every finite a; NaN stays NaN.  The floor is applied afterwards by the recurrence."""
    with np.errstate(invalid="ignore"):  # NaN in, NaN out
        return -np.logaddexp(0.0, np.asarray(a, dtype=np.float64))


def _step(S, q, k, v, g, beta):
    """One token for a stack of states.

    S [..., dk, dv]; q, k, g [..., dk]; v [..., dv]; beta [...].  Returns (S', o).
    """
    S = np.exp(clamp_log_decay(g))[..., :, None] * S
    w = np.einsum("...cj,...c->...j", S, k)
    S = S + beta[..., None, None] * k[..., :, None] * (v - w)[..., None, :]
    o = np.einsum("...cj,...c->...j", S, q)
    return S, o


def kda_decode_step(state, q, k, v, g, beta):
    """Single recurrent step: state [N,H,dk,dv] -> (o [N,H,dv], new state)."""
    S, o = _step(np.asarray(state, np.float64), np.asarray(q, np.float64),
                 np.asarray(k, np.float64), np.asarray(v, np.float64),
                 np.asarray(g, np.float64), np.asarray(beta, np.float64))
    return o, S


def kda_forward(q, k, v, g, beta, s0=None, checkpoint_every: int = 0):
    """Full-sequence KDA, one token at a time.

    q, k, g: [B,T,H,dk]; v: [B,T,H,dv]; beta: [B,T,H]; s0: [B,H,dk,dv] or None.
    Returns (o [B,T,H,dv], final state [B,H,dk,dv], checkpoints) where
    checkpoints is [B, T // every, H, dk, dv] (the state after tokens
    every*(j+1)) or None when checkpoint_every == 0.
    """
    q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if s0 is None else np.array(s0, dtype=np.float64)
    o = np.empty((B, T, H, dv))
    ck = None
    if checkpoint_every:
        ck = np.empty((B, T // checkpoint_every, H, dk, dv))
    for t in range(T):
        S, o[:, t] = _step(S, q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t])
        if checkpoint_every and (t + 1) % checkpoint_every == 0:
            ck[:, (t + 1) // checkpoint_every - 1] = S
    return o, S, ck


_SHARED = None  # inputs handed to forked workers without pickling


def _one_head(idx):
    q, k, v, g, beta, s0, every = _SHARED
    b, h = divmod(idx, q.shape[2])
    o, S, ck = kda_forward(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1],
                           v[b:b + 1, :, h:h + 1], g[b:b + 1, :, h:h + 1],
                           beta[b:b + 1, :, h:h + 1], s0[b:b + 1, h:h + 1], every)
    return o[0, :, 0], S[0, 0], None if ck is None else ck[0, :, 0]


def kda_forward_heads_parallel(q, k, v, g, beta, s0=None, checkpoint_every: int = 0,
                               processes: Optional[int] = None):
    """kda_forward with the independent (b, h) sequences spread over processes.

    Identical arithmetic per head; only the scheduling differs.  Returns the
    same triple as :func:`kda_forward` and the number of processes used.
    """
    global _SHARED
    q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if s0 is None:
        s0 = np.zeros((B, H, dk, dv))
    n_jobs = B * H
    if processes is None:
        processes = min(16, len(os.sched_getaffinity(0)))
    processes = max(1, min(processes, n_jobs))
    _SHARED = (q, k, v, g, beta, np.asarray(s0, np.float64), checkpoint_every)
    try:
        if processes == 1:
            res = [_one_head(i) for i in range(n_jobs)]
        else:
            import multiprocessing as mp

            with mp.get_context("fork").Pool(processes) as pool:
                res = pool.map(_one_head, range(n_jobs), chunksize=1)
    finally:
        _SHARED = None
    o = np.empty((B, T, H, dv))
    S = np.empty((B, H, dk, dv))
    ck = np.empty((B, T // checkpoint_every, H, dk, dv)) if checkpoint_every else None
    for idx, (oh, Sh, ckh) in enumerate(res):
        b, h = divmod(idx, H)
        o[b, :, h] = oh
        S[b, h] = Sh
        if ck is not None:
            ck[b, :, h] = ckh
    return (o, S, ck), processes


def rel_l2(x, ref) -> float:
    """||x - ref||_2 / ||ref||_2 in float64 over the whole array."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    return float(num / den) if den > 0 else float(num)


def one_hot_key_rows(rows0, g, hit, beta, v):
    """Rows of the KDA state when every key is a one-hot vector (closed form).

    With k_t = e_{c_t}, S^T k_t is row c_t of the decayed state, so the delta
    update touches that row alone: every row c is an independent gated moving
    average,

        S[c] <- exp(g'_{t,c}) S[c]                       (decay, g' clamped as above)
        S[c] <- (1 - beta_t) S[c] + beta_t v_t           (only when c == c_t)

    and a one-hot query e_r reads o_t = S_t[r].  Follows from the recurrence in
    the package docstring; pinned against :func:`kda_forward` in the tests.

    rows0 [R, dv] entry rows; g [T, R] their log-decays; hit [T, R] bool (the
    token's key is that row's channel); beta [T, R]; v [T, R, dv] the value vector
    of each row's head.  Returns (trajectory [T, R, dv] = rows after each token,
    final rows [R, dv]), float64.
    """
    x = np.array(rows0, dtype=np.float64)
    keep = np.exp(clamp_log_decay(g))
    hb = np.where(np.asarray(hit, bool), np.asarray(beta, np.float64), 0.0)
    v = np.asarray(v, np.float64)
    traj = np.empty((keep.shape[0],) + x.shape)
    for t in range(keep.shape[0]):
        x = ((1.0 - hb[t]) * keep[t])[:, None] * x + hb[t][:, None] * v[t]
        traj[t] = x
    return traj, x
