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


def _head_task(args):
    """One (b, h) sequence: args = (q, k, v, g, beta, s0, every) for that head alone,
    [T, d] arrays and a [dk, dv] state.  Runs in a worker process."""
    q, k, v, g, beta, s0, every = args
    o, S, ck = kda_forward(q[None, :, None], k[None, :, None], v[None, :, None],
                           g[None, :, None], beta[None, :, None], s0[None, None], every)
    return o[0, :, 0], S[0, 0], None if ck is None else ck[0, :, 0]


_DEFAULT_POOL = None  # a head_pool() set by the caller, used when none is passed


def oracle_processes() -> int:
    """Worker count for the oracle's process pool: $ORACLE_PROCESSES if set, else up to
    16 of the cores this process may run on."""
    env = os.environ.get("ORACLE_PROCESSES")
    if env:
        return max(1, int(env))
    return min(16, len(os.sched_getaffinity(0)))


def head_pool(processes: Optional[int] = None):
    """A process pool for :func:`kda_forward_heads_parallel`.

    Workers are started with the "spawn" method: each is a fresh interpreter that
    imports numpy and this module only, and receives every head's inputs as its own
    arrays.  Make the pool before the calling process touches a GPU: a forked copy of
    a process that holds GPU runtime state can crash at exit, and a process that holds
    it should start no new programs at all.
    """
    import multiprocessing as mp

    return mp.get_context("spawn").Pool(max(1, processes or oracle_processes()))


def set_default_pool(pool) -> None:
    """Use `pool` (from :func:`head_pool`, or None) when a call passes none."""
    global _DEFAULT_POOL
    _DEFAULT_POOL = pool


def kda_forward_heads_parallel(q, k, v, g, beta, s0=None, checkpoint_every: int = 0,
                               processes: Optional[int] = None, pool=None):
    """kda_forward with the independent (b, h) sequences spread over processes.

    Identical arithmetic per head; only the scheduling differs.  Each head's inputs
    are sent to a worker as their own arrays (streamed, one task at a time).  The
    workers are `pool` if given; else, with `processes` None, the default pool
    (:func:`set_default_pool`) if one is set; else a pool of its own when
    `processes` > 1 asks for one; else this process.  Returns the same triple as :func:`kda_forward` and the number of
    processes used.
    """
    q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    s0 = np.zeros((B, H, dk, dv)) if s0 is None else np.asarray(s0, np.float64)
    n_jobs = B * H
    if pool is None and processes is None:
        pool = _DEFAULT_POOL
    own = pool is None and processes is not None and processes > 1 and n_jobs > 1
    if own:
        pool = head_pool(min(processes, n_jobs))
    used = 1 if pool is None else min(pool._processes, n_jobs)

    def tasks():
        for idx in range(n_jobs):
            b, h = divmod(idx, H)
            yield (np.ascontiguousarray(q[b, :, h]), np.ascontiguousarray(k[b, :, h]),
                   np.ascontiguousarray(v[b, :, h]), np.ascontiguousarray(g[b, :, h]),
                   np.ascontiguousarray(beta[b, :, h]), s0[b, h], checkpoint_every)

    try:
        if pool is None or n_jobs == 1:
            res = [_head_task(t) for t in tasks()]
            used = 1
        else:
            res = list(pool.imap(_head_task, tasks(), chunksize=1))
    finally:
        if own:
            pool.terminate()
            pool.join()
    o = np.empty((B, T, H, dv))
    S = np.empty((B, H, dk, dv))
    ck = np.empty((B, T // checkpoint_every, H, dk, dv)) if checkpoint_every else None
    for idx, (oh, Sh, ckh) in enumerate(res):
        b, h = divmod(idx, H)
        o[b, :, h] = oh
        S[b, h] = Sh
        if ck is not None:
            ck[b, :, h] = ckh
    return (o, S, ck), used


def rel_l2(x, ref) -> float:
    """Relative L2 error ||x - ref||_2 / ||ref||_2 in float64 over the whole array
    (the square root of the summed squared differences over the square root of the
    summed squared reference values); ||x - ref||_2 itself when ref is all zeros."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    return float(num / den) if den > 0 else float(num)


def rel_l2_groups(x, ref, group_axes) -> np.ndarray:
    """Relative L2 error of every slice: for each index over `group_axes` (say the
    batch and head axes of a [B, T, H, D] output), ||x - ref||_2 / ||ref||_2 over the
    remaining axes, as :func:`rel_l2` defines it for one array.  Returns an array
    shaped like the group axes."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    group_axes = tuple(a % x.ndim for a in group_axes)
    other = tuple(a for a in range(x.ndim) if a not in group_axes)
    num = np.sqrt(np.sum((x - ref) ** 2, axis=other))
    den = np.sqrt(np.sum(ref ** 2, axis=other))
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def rel_l2_chunks(x, ref, chunk: int, t_axis: int = 1, group_axes=(0, 2)) -> np.ndarray:
    """Relative L2 error of every run of `chunk` consecutive tokens along `t_axis`
    (the last run may be shorter), separately for each index over `group_axes` and
    over all remaining axes, as :func:`rel_l2` defines it.  For a [B, T, H, D] output
    with the defaults the result is [B, ceil(T / chunk), H]."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    t_axis = t_axis % x.ndim
    group_axes = tuple(a % x.ndim for a in group_axes)
    other = tuple(a for a in range(x.ndim) if a not in group_axes and a != t_axis)
    d2 = np.sum((x - ref) ** 2, axis=other, keepdims=True)
    r2 = np.sum(ref ** 2, axis=other, keepdims=True)
    starts = np.arange(0, x.shape[t_axis], chunk)
    num = np.sqrt(np.add.reduceat(d2, starts, axis=t_axis))
    den = np.sqrt(np.add.reduceat(r2, starts, axis=t_axis))
    out = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    return np.squeeze(out, axis=other)


def apply_output_gate(o, z):
    """KDA's output gate: o * sigmoid(z), elementwise, sigmoid(z) = 1 / (1 + e^-z).

    z has o's shape: one gate value per token, head and value channel, projected from
    the token's input by the caller, so each token chooses which output channels pass.
    The Towards-AI article on the Kimi K3 report gives K3's Gated MLA layers such a gate
    and says KDA has a counterpart (section "Gated MLA and No Position Encoding
    (NoPE)").  The logistic form of the gate is the reading taken where the page names
    no function.  Float64; computed as e^z / (1 + e^z) for z < 0 so that neither
    branch overflows; NaN stays NaN."""
    o = np.asarray(o, np.float64)
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore", under="ignore", invalid="ignore"):
        ez = np.exp(-np.abs(z))
        sig = np.where(z >= 0, 1.0 / (1.0 + ez), ez / (1.0 + ez))
        sig = np.where(np.isnan(z), np.nan, sig)
    return o * sig


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
