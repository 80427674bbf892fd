"""Comparison of GPU results with the float64 oracle, shared by the GPU tests.

Three figures per tensor, each a relative L2 error as oracle.rel_l2 defines it:
  whole     over the whole tensor (the figure the method's tolerance is stated for:
            1e-5 on the float32 path, 3e-3 for bfloat16 inputs);
  per head  the largest over the (batch row, head) slices;
  per chunk for token tensors, the largest over runs of 64 tokens of one head (the
            last run of a ragged tail included).
The whole-tensor figure alone can hide a few wrong token-heads in a large tensor (one
wrong token-head of the 4 x 4096 x 32-head workload moves it by only ~1.4e-3); the
maxima cannot.  Per head the bound is the whole-tensor tolerance.  A 64-token chunk of
one head holds 64 x d_v values (8192 at d_v = 128, 2048 at d_v = 32... fewer on a
ragged tail), so its error scatters more around the whole-tensor figure; its bound
is twice the tolerance, still far below what one wrong token does to a chunk (its
share of the chunk's norm, about 1 / sqrt(64) = 0.125).
"""
import numpy as np

import oracle

CHUNK = 64


def _np(x):
    if hasattr(x, "detach"):
        return x.detach().double().cpu().numpy()
    return np.asarray(x, np.float64)


def errors(got, ref, kind: str):
    """(whole, per-head max, per-chunk max or None) for a tensor of the given kind:
    "tokens" [B, T, H, D]; "state" [B, H, dk, dv]; "ckpt" [B, n, H, dk, dv];
    "step" [N, H, D] (one decode token); "draft" [N, K, H, D]."""
    got, ref = _np(got), _np(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    whole = oracle.rel_l2(got, ref)
    if got.size == 0:
        return whole, 0.0, None
    if kind == "tokens":
        head = oracle.rel_l2_groups(got, ref, (0, 2)).max()
        chunk = oracle.rel_l2_chunks(got, ref, CHUNK, t_axis=1, group_axes=(0, 2)).max()
        return whole, float(head), float(chunk)
    if kind == "state":
        return whole, float(oracle.rel_l2_groups(got, ref, (0, 1)).max()), None
    if kind == "ckpt":
        return whole, float(oracle.rel_l2_groups(got, ref, (0, 1, 2)).max()), None
    if kind == "step":
        return whole, float(oracle.rel_l2_groups(got, ref, (0, 1)).max()), None
    if kind == "draft":
        return whole, float(oracle.rel_l2_groups(got, ref, (0, 2)).max()), None
    raise ValueError(kind)


def check(label: str, got, ref, tol: float, kind: str = "tokens", head_tol=None,
          chunk_tol=None):
    """Assert the three figures against tol, head_tol (default tol) and chunk_tol (default
    2 tol); print them first, so that a failing run still shows every figure.  Returns
    the whole-tensor figure."""
    whole, head, chunk = errors(got, ref, kind)
    head_tol = tol if head_tol is None else head_tol
    chunk_tol = 2 * tol if chunk_tol is None else chunk_tol
    extra = "" if chunk is None else f" chunk-max {chunk:.3e}"
    print(f"[parity] {label}: whole {whole:.3e} head-max {head:.3e}{extra} (tol {tol:.0e})",
          flush=True)
    assert whole <= tol, (label, "whole", whole, tol)
    assert head <= head_tol, (label, "per head", head, head_tol)
    if chunk is not None:
        assert chunk <= chunk_tol, (label, "per chunk", chunk, chunk_tol)
    return whole
