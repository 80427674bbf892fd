"""Kimi Delta Attention (KDA) on AMD MI355X: Python binding of the C-ABI library libkda.so.

The binding only marshals arguments (device pointers, sizes, dtypes, the
current HIP stream) into the entry points declared in include/kda.h; every
step of the computation runs in the library's gfx950 kernels.  There is no
fallback: if libkda.so is missing or a GPU is absent, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")
# the range-check build of the same sources (include/kda_debug.h); for tests
DEBUG_LIB_PATH = os.path.join(_PKG, "libkda_debug.so")

KDA_F32, KDA_BF16 = 0, 1
STATUS = {0: "KDA_OK", -1: "KDA_ERR_NULL", -2: "KDA_ERR_SHAPE", -3: "KDA_ERR_DTYPE",
          -4: "KDA_ERR_ALIGN", -5: "KDA_ERR_WORKSPACE", -6: "KDA_ERR_ALIAS", -7: "KDA_ERR_HIP"}
EXPORTS = ("kda_status_str", "kda_chunk_fwd_workspace_bytes", "kda_chunk_fwd",
           "kda_chunk_fwd_segmented", "kda_chunk_fwd_segmented_workspace_bytes",
           "kda_chunk_fwd_segment_tokens", "kda_chunk_fwd_checkpoints_at", "kda_recurrent_step",
           "kda_recurrent_verify", "kda_recurrent_commit", "kda_chunk_fwd_gate_logits",
           "kda_recurrent_step_gate_logits", "kda_chunk_fwd_output_gate",
           "kda_recurrent_step_output_gate", "kda_chunk_fwd_noalloc")

_lib = None


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)}")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkda.so and declare the C signatures (no GPU needed to load)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with gated_delta_rule_57_amd.build")
    lib = ctypes.CDLL(path)
    vp, i64, c_int, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.kda_status_str.restype = ctypes.c_char_p
    lib.kda_status_str.argtypes = [c_int]
    lib.kda_chunk_fwd_workspace_bytes.restype = sz
    lib.kda_chunk_fwd_workspace_bytes.argtypes = [i64, i64, i64, c_int, c_int, c_int, c_int]
    lib.kda_chunk_fwd.restype = c_int
    lib.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, c_int,
                                  c_int, c_int, c_int, c_int, vp, sz, vp]
    lib.kda_chunk_fwd_segmented.restype = c_int
    lib.kda_chunk_fwd_segmented.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                            c_int, c_int, c_int, c_int, c_int, i64, vp, sz, vp]
    lib.kda_chunk_fwd_segmented_workspace_bytes.restype = sz
    lib.kda_chunk_fwd_segmented_workspace_bytes.argtypes = [i64, i64, i64, c_int, c_int, c_int,
                                                            c_int, i64]
    lib.kda_chunk_fwd_segment_tokens.restype = i64
    lib.kda_chunk_fwd_segment_tokens.argtypes = [i64, i64, i64, c_int, c_int, c_int, c_int]
    lib.kda_recurrent_step.restype = c_int
    lib.kda_recurrent_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, c_int, c_int, c_int,
                                       c_int, vp]
    lib.kda_chunk_fwd_checkpoints_at.restype = c_int
    lib.kda_chunk_fwd_checkpoints_at.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64,
                                                 i64, i64, c_int, c_int, c_int, c_int, c_int, vp,
                                                 sz, vp]
    lib.kda_chunk_fwd_gate_logits.restype = c_int
    lib.kda_chunk_fwd_gate_logits.argtypes = list(lib.kda_chunk_fwd.argtypes)
    lib.kda_recurrent_step_gate_logits.restype = c_int
    lib.kda_recurrent_step_gate_logits.argtypes = list(lib.kda_recurrent_step.argtypes)
    lib.kda_chunk_fwd_output_gate.restype = c_int
    lib.kda_chunk_fwd_output_gate.argtypes = [vp] * 6 + list(lib.kda_chunk_fwd.argtypes[5:])
    lib.kda_recurrent_step_output_gate.restype = c_int
    lib.kda_recurrent_step_output_gate.argtypes = [vp] * 6 + list(lib.kda_recurrent_step.argtypes[5:])
    lib.kda_chunk_fwd_noalloc.restype = c_int
    lib.kda_chunk_fwd_noalloc.argtypes = list(lib.kda_chunk_fwd.argtypes[:18]) + [vp]
    lib.kda_recurrent_verify.restype = c_int
    lib.kda_recurrent_verify.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, c_int, c_int,
                                         c_int, c_int, vp]
    lib.kda_recurrent_commit.restype = c_int
    lib.kda_recurrent_commit.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, c_int, c_int, c_int,
                                         vp]
    if path == LIB_PATH:
        _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().kda_status_str(int(status)).decode()


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return KDA_BF16
    if dt == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported dtype {dt}; KDA takes float32 or bfloat16")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("KDA tensors must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("KDA tensors must be contiguous")
    return t.data_ptr()


def _expect(t, name: str, shape, dtype, device) -> None:
    """Raise ValueError unless tensor t has exactly this shape, dtype and device.  The C
    ABI sees only pointers, so a tensor of the wrong size would be read or written out
    of bounds on the GPU; every tensor is checked here before anything is launched."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(int(s) for s in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device} (the device of q)")


def _token_inputs(q, k, v, g, beta, name_g="g"):
    """Shapes of [B, T, H, .] token inputs (q first), checked against each other."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-D tensor [B, T, H, dk]")
    if not isinstance(v, torch.Tensor) or v.dim() != 4:
        raise ValueError("v must be a 4-D tensor [B, T, H, dv]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    _expect(k, "k", (B, T, H, dk), dt, dev)
    _expect(v, "v", (B, T, H, dv), dt, dev)
    _expect(g, name_g, (B, T, H, dk), dt, dev)
    _expect(beta, "beta", (B, T, H), dt, dev)
    return B, T, H, dk, dv


def _workspace_bytes(workspace, device) -> int:
    if workspace is None:
        return 0
    if not isinstance(workspace, torch.Tensor) or workspace.device != device:
        raise ValueError(f"workspace must be a tensor on {device}")
    return workspace.numel() * workspace.element_size()


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def kda_chunk_fwd_workspace_bytes(B: int, T: int, H: int, dk: int, dv: int, chunk: int = 64,
                                  in_dtype: torch.dtype = torch.bfloat16) -> int:
    return int(load_library().kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk,
                                                            _dtype_code(in_dtype)))


def kda_chunk_fwd_segmented_workspace_bytes(B: int, T: int, H: int, dk: int, dv: int,
                                            segment_tokens: int, chunk: int = 64,
                                            in_dtype: torch.dtype = torch.bfloat16) -> int:
    return int(load_library().kda_chunk_fwd_segmented_workspace_bytes(
        B, T, H, dk, dv, chunk, _dtype_code(in_dtype), segment_tokens))


def kda_chunk_fwd_segment_tokens(B: int, T: int, H: int, dk: int, dv: int, chunk: int = 64,
                                 in_dtype: torch.dtype = torch.bfloat16) -> int:
    """Segment length kda_chunk_fwd picks for these sizes (>= T: one segment)."""
    return int(load_library().kda_chunk_fwd_segment_tokens(B, T, H, dk, dv, chunk,
                                                           _dtype_code(in_dtype)))


def kda_chunk_fwd(q, k, v, g, beta, initial_state=None, *, out_dtype=None, o=None,
                  final_state=None, want_final_state=True, checkpoint_every: int = 0,
                  checkpoints=None, chunk: int = 64, workspace=None, stream=None,
                  segment_tokens: Optional[int] = None, gate_logits: bool = False,
                  output_gate=None):
    """Chunked KDA forward.  Shapes as in include/kda.h; returns (o, final_state, checkpoints).

    q, k, g [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H] (all one dtype); initial_state
    [B,H,dk,dv] float32 or None.  Outputs are allocated when not given; pass
    final_state=initial_state for an in-place state update.  ``segment_tokens``
    None calls kda_chunk_fwd (the library picks the segmentation); an integer
    calls kda_chunk_fwd_segmented with that segment length.  A workspace of the
    size the library asks for is allocated when not given.  ``gate_logits=True``
    passes raw decay logits in ``g`` (kda_chunk_fwd_gate_logits; log-decay = -softplus).
    ``output_gate`` [B,T,H,dv] (q's dtype) calls kda_chunk_fwd_output_gate: o = (S^T q) *
    sigmoid(output_gate).
    """
    B, T, H, dk, dv = _token_inputs(q, k, v, g, beta)
    in_dt, dev = q.dtype, q.device
    out_dt = (o.dtype if o is not None else in_dt) if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dt, device=dev)
    _expect(o, "o", (B, T, H, dv), out_dt, dev)
    if initial_state is not None:
        _expect(initial_state, "initial_state", (B, H, dk, dv), torch.float32, dev)
    if final_state is None and want_final_state:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if final_state is not None:
        _expect(final_state, "final_state", (B, H, dk, dv), torch.float32, dev)
    if checkpoint_every and checkpoints is None:
        checkpoints = torch.empty((B, T // checkpoint_every, H, dk, dv), dtype=torch.float32,
                                  device=dev)
    if checkpoints is not None:
        if not checkpoint_every:
            raise ValueError("checkpoints given with checkpoint_every = 0")
        _expect(checkpoints, "checkpoints", (B, T // checkpoint_every, H, dk, dv),
                torch.float32, dev)
    if segment_tokens is None:
        need = kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, in_dt)
    else:
        need = kda_chunk_fwd_segmented_workspace_bytes(B, T, H, dk, dv, segment_tokens, chunk,
                                                       in_dt)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = _workspace_bytes(workspace, dev)
    lib = load_library()
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(o),
            _ptr(final_state), _ptr(checkpoints), int(checkpoint_every), B, T, H, dk, dv, chunk,
            _dtype_code(in_dt), _dtype_code(o.dtype))
    tail = (_ptr(workspace), ws_bytes, _stream(stream))
    if output_gate is not None:
        _expect(output_gate, "output_gate", (B, T, H, dv), in_dt, dev)
        if gate_logits or segment_tokens is not None:
            raise ValueError("output_gate takes log-decays and the library's segmentation")
        st = lib.kda_chunk_fwd_output_gate(*args[:5], _ptr(output_gate), *args[5:], *tail)
        where = "kda_chunk_fwd_output_gate"
    elif gate_logits:
        if segment_tokens is not None:
            raise ValueError("gate_logits takes the library's segmentation")
        st, where = lib.kda_chunk_fwd_gate_logits(*args, *tail), "kda_chunk_fwd_gate_logits"
    elif segment_tokens is None:
        st, where = lib.kda_chunk_fwd(*args, *tail), "kda_chunk_fwd"
    else:
        st = lib.kda_chunk_fwd_segmented(*args, int(segment_tokens), *tail)
        where = "kda_chunk_fwd_segmented"
    if st != 0:
        raise KdaError(st, where)
    return o, final_state, checkpoints


def kda_recurrent_step(q, k, v, g, beta, state, *, out_dtype=None, o=None, stream=None,
                       gate_logits: bool = False, output_gate=None):
    """One decode step; ``state`` [N,H,dk,dv] float32 is updated in place.  Returns o [N,H,dv].
    ``gate_logits=True`` passes raw decay logits in ``g``; ``output_gate`` [N,H,dv] gives
    o = (S^T q) * sigmoid(output_gate)."""
    if not isinstance(q, torch.Tensor) or q.dim() != 3 or not isinstance(v, torch.Tensor) \
            or v.dim() != 3:
        raise ValueError("q and v must be 3-D tensors [N, H, d]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    _expect(k, "k", (N, H, dk), dt, dev)
    _expect(v, "v", (N, H, dv), dt, dev)
    _expect(g, "g", (N, H, dk), dt, dev)
    _expect(beta, "beta", (N, H), dt, dev)
    _expect(state, "state", (N, H, dk, dv), torch.float32, dev)
    out_dt = (o.dtype if o is not None else dt) if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((N, H, dv), dtype=out_dt, device=dev)
    _expect(o, "o", (N, H, dv), out_dt, dev)
    lib = load_library()
    tail = (_ptr(state), _ptr(o), N, H, dk, dv, _dtype_code(q.dtype), _dtype_code(o.dtype),
            _stream(stream))
    if output_gate is not None:
        _expect(output_gate, "output_gate", (N, H, dv), dt, dev)
        if gate_logits:
            raise ValueError("output_gate takes log-decays")
        st = lib.kda_recurrent_step_output_gate(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                                _ptr(output_gate), *tail)
    else:
        fn = lib.kda_recurrent_step_gate_logits if gate_logits else lib.kda_recurrent_step
        st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), *tail)
    if st != 0:
        raise KdaError(st, "kda_recurrent_step")
    return o


def kda_recurrent_verify(q, k, v, g, beta, state, *, out_dtype=None, o=None, stream=None):
    """Outputs of K draft tokens per sequence from the committed ``state`` (only read).

    q, k, g [N,K,H,dk]; v [N,K,H,dv]; beta [N,K,H]; state [N,H,dk,dv] float32.
    Returns o [N,K,H,dv]."""
    N, K, H, dk, dv = _token_inputs(q, k, v, g, beta)
    dev = q.device
    _expect(state, "state", (N, H, dk, dv), torch.float32, dev)
    out_dt = (o.dtype if o is not None else q.dtype) if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((N, K, H, dv), dtype=out_dt, device=dev)
    _expect(o, "o", (N, K, H, dv), out_dt, dev)
    st = load_library().kda_recurrent_verify(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                             _ptr(state), _ptr(o), N, K, H, dk, dv,
                                             _dtype_code(q.dtype), _dtype_code(o.dtype),
                                             _stream(stream))
    if st != 0:
        raise KdaError(st, "kda_recurrent_verify")
    return o


def kda_recurrent_commit(k, v, g, beta, accept, state, *, stream=None):
    """Advance ``state`` [N,H,dk,dv] in place by accept[n] (int32, on the GPU) draft tokens."""
    if not isinstance(k, torch.Tensor) or k.dim() != 4 or not isinstance(v, torch.Tensor) \
            or v.dim() != 4:
        raise ValueError("k and v must be 4-D tensors [N, K, H, d]")
    N, K, H, dk = k.shape
    dv = v.shape[-1]
    dt, dev = k.dtype, k.device
    _expect(v, "v", (N, K, H, dv), dt, dev)
    _expect(g, "g", (N, K, H, dk), dt, dev)
    _expect(beta, "beta", (N, K, H), dt, dev)
    _expect(accept, "accept", (N,), torch.int32, dev)
    _expect(state, "state", (N, H, dk, dv), torch.float32, dev)
    st = load_library().kda_recurrent_commit(_ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(accept),
                                             _ptr(state), N, K, H, dk, dv, _dtype_code(k.dtype),
                                             _stream(stream))
    if st != 0:
        raise KdaError(st, "kda_recurrent_commit")
    return state


def kda_chunk_fwd_checkpoints_at(q, k, v, g, beta, positions, initial_state=None, *,
                                 out_dtype=None, o=None, final_state=None, checkpoints=None,
                                 chunk: int = 64, workspace=None, stream=None):
    """Chunked forward saving the state after each of ``positions`` tokens (int64 on the GPU,
    increasing multiples of ``chunk``).  Returns (o, final_state, checkpoints [B,P,H,dk,dv])."""
    B, T, H, dk, dv = _token_inputs(q, k, v, g, beta)
    dev = q.device
    if not isinstance(positions, torch.Tensor) or positions.dim() != 1:
        raise ValueError("positions must be a 1-D tensor")
    P = positions.numel()
    _expect(positions, "positions", (P,), torch.int64, dev)
    if initial_state is not None:
        _expect(initial_state, "initial_state", (B, H, dk, dv), torch.float32, dev)
    out_dt = (o.dtype if o is not None else q.dtype) if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dt, device=dev)
    _expect(o, "o", (B, T, H, dv), out_dt, dev)
    if final_state is None:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _expect(final_state, "final_state", (B, H, dk, dv), torch.float32, dev)
    if checkpoints is None:
        checkpoints = torch.empty((B, P, H, dk, dv), dtype=torch.float32, device=dev)
    _expect(checkpoints, "checkpoints", (B, P, H, dk, dv), torch.float32, dev)
    need = kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, q.dtype)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = _workspace_bytes(workspace, dev)
    st = load_library().kda_chunk_fwd_checkpoints_at(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(o),
        _ptr(final_state), _ptr(checkpoints), _ptr(positions), P, B, T, H, dk, dv, chunk,
        _dtype_code(q.dtype), _dtype_code(o.dtype), _ptr(workspace), ws_bytes, _stream(stream))
    if st != 0:
        raise KdaError(st, "kda_chunk_fwd_checkpoints_at")
    return o, final_state, checkpoints


def kda_chunk_fwd_noalloc(q, k, v, g, beta, initial_state, o, final_state=None, *,
                          checkpoint_every: int = 0, checkpoints=None, chunk: int = 64,
                          stream=None):
    """kda_chunk_fwd_noalloc: the chunked forward with the library's own device scratch as
    the segment path's workspace.  Every output buffer is the caller's (nothing is
    allocated here or in the library).  Returns (o, final_state, checkpoints)."""
    B, T, H, dk, dv = _token_inputs(q, k, v, g, beta)
    dev = q.device
    _expect(o, "o", (B, T, H, dv), o.dtype if isinstance(o, torch.Tensor) else None, dev)
    if initial_state is not None:
        _expect(initial_state, "initial_state", (B, H, dk, dv), torch.float32, dev)
    if final_state is not None:
        _expect(final_state, "final_state", (B, H, dk, dv), torch.float32, dev)
    if checkpoints is not None or checkpoint_every:
        if not checkpoint_every or checkpoints is None:
            raise ValueError("checkpoints and checkpoint_every go together")
        _expect(checkpoints, "checkpoints", (B, T // checkpoint_every, H, dk, dv),
                torch.float32, dev)
    st = load_library().kda_chunk_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(o),
        _ptr(final_state), _ptr(checkpoints), int(checkpoint_every), B, T, H, dk, dv, chunk,
        _dtype_code(q.dtype), _dtype_code(o.dtype), _stream(stream))
    if st != 0:
        raise KdaError(st, "kda_chunk_fwd_noalloc")
    return o, final_state, checkpoints
