"""The C ABI: the library loads, exports every declared entry point, and rejects bad
arguments with a status code before anything is launched (no GPU needed)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_57_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "kda.h")).read()
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        pytest.skip("libkda.so not built")
    return kda.load_library()


def test_every_declared_symbol_is_exported(lib):
    declared = _declared()
    assert set(declared) == set(kda.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code, name in kda.STATUS.items():
        assert lib.kda_status_str(code).decode().startswith(name)
    assert lib.kda_status_str(99).decode() == "KDA_ERR_UNKNOWN"


def test_workspace_sizes(lib):
    bf = kda.KDA_BF16
    # 128 heads fill the GPU: one segment, no workspace
    assert lib.kda_chunk_fwd_segment_tokens(4, 4096, 32, 128, 128, 64, bf) >= 4096
    assert lib.kda_chunk_fwd_workspace_bytes(4, 4096, 32, 128, 128, 64, bf) == 0
    # few heads, long sequences: several segments, workspace = entry + zero-start states
    # [B, nseg, H, dk, dv] and transitions [B, nseg, H, dk, dk], float32
    for B, T, H, dk, dv in [(1, 65536, 32, 128, 128), (1, 1 << 20, 16, 128, 128),
                            (1, 32768, 8, 64, 128)]:
        seg = lib.kda_chunk_fwd_segment_tokens(B, T, H, dk, dv, 64, bf)
        assert 0 < seg < T and seg % 64 == 0
        nseg = -(-T // seg)
        want = 4 * B * nseg * H * dk * (2 * dv + dk)
        got = lib.kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, 64, bf)
        assert want <= got < want + 3 * 256
        assert got == lib.kda_chunk_fwd_segmented_workspace_bytes(B, T, H, dk, dv, 64, bf, seg)
    # explicit segment lengths
    assert lib.kda_chunk_fwd_segmented_workspace_bytes(1, 256, 2, 64, 64, 64, kda.KDA_F32, 256) == 0
    assert lib.kda_chunk_fwd_segmented_workspace_bytes(1, 256, 2, 64, 64, 64, kda.KDA_F32,
                                                       64) == 4 * 4 * 2 * 64 * 192
    assert lib.kda_chunk_fwd_segmented_workspace_bytes(1, 256, 2, 64, 64, 64, kda.KDA_F32, 100) == 0
    # unsupported sizes
    assert lib.kda_chunk_fwd_segment_tokens(1, 256, 2, 96, 64, 64, bf) == 0
    assert lib.kda_chunk_fwd_workspace_bytes(1, 256, 2, 96, 64, 64, bf) == 0


FAKE = 1 << 20  # aligned, never dereferenced: every call below fails validation first


def _fwd(lib, **kw):
    a = dict(q=FAKE, k=2 * FAKE, v=3 * FAKE, g=4 * FAKE, beta=5 * FAKE, s0=None, o=None,
             sf=None, ck=None, every=0, B=1, T=64, H=1, dk=128, dv=128, chunk=64,
             din=kda.KDA_BF16, dout=kda.KDA_BF16)
    a.update(kw)
    return lib.kda_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["o"], a["sf"],
                             a["ck"], a["every"], a["B"], a["T"], a["H"], a["dk"], a["dv"],
                             a["chunk"], a["din"], a["dout"], None, 0, None)


def test_chunk_fwd_rejects_before_launch(lib):
    o = 64 * FAKE
    assert _fwd(lib) == -1  # o missing
    assert _fwd(lib, o=o, q=None) == -1
    assert _fwd(lib, o=o, every=64) == -1  # checkpoints missing
    assert _fwd(lib, o=o, din=7) == -3
    assert _fwd(lib, o=o, dk=96) == -2
    assert _fwd(lib, o=o, dv=256) == -2
    assert _fwd(lib, o=o, chunk=48) == -2
    assert _fwd(lib, o=o, chunk=128) == -2
    # 16- and 32-token chunks take bfloat16 inputs only
    assert _fwd(lib, o=o, chunk=32, din=kda.KDA_F32, dk=64, dv=64) == -2
    assert _fwd(lib, o=o, chunk=16, din=kda.KDA_F32, dk=64, dv=64) == -2
    assert _fwd(lib, o=o, chunk=32, every=48, ck=96 * FAKE) == -2  # not a multiple of the chunk
    assert _fwd(lib, o=o, T=0) == -2
    assert _fwd(lib, o=o, din=kda.KDA_F32, dk=128) == -2
    assert _fwd(lib, o=o, ck=96 * FAKE, every=100) == -2
    assert _fwd(lib, o=o + 4) == -4
    assert _fwd(lib, o=2 * FAKE + 64) == -6  # o inside k
    assert _fwd(lib, o=o, sf=o + 128) == -6  # final state overlaps o
    assert _fwd(lib, o=o, s0=80 * FAKE, sf=80 * FAKE + 16) == -6  # partial state overlap
    # per-chunk row offsets are 32-bit: 64 rows x H x 128 channels x 4 bytes must fit
    assert _fwd(lib, o=o, H=131072) == -2
    assert _fwd(lib, o=o, H=262144, dk=64, dv=64) == -2
    assert lib.kda_chunk_fwd_workspace_bytes(1, 64, 131072, 128, 128, 64, kda.KDA_BF16) == 0
    assert lib.kda_chunk_fwd_segment_tokens(1, 64, 131072, 128, 128, 64, kda.KDA_BF16) == 0


def _seg(lib, seg, ws=None, ws_bytes=0, **kw):
    a = dict(q=FAKE, k=2 * FAKE, v=3 * FAKE, g=4 * FAKE, beta=5 * FAKE, s0=None, o=64 * FAKE,
             sf=None, ck=None, every=0, B=1, T=256, H=1, dk=128, dv=128, chunk=64,
             din=kda.KDA_BF16, dout=kda.KDA_BF16)
    a.update(kw)
    return lib.kda_chunk_fwd_segmented(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["o"],
                                       a["sf"], a["ck"], a["every"], a["B"], a["T"], a["H"],
                                       a["dk"], a["dv"], a["chunk"], a["din"], a["dout"], seg, ws,
                                       ws_bytes, None)


def test_segmented_rejects_before_launch(lib):
    need = lib.kda_chunk_fwd_segmented_workspace_bytes(1, 256, 1, 128, 128, 64, kda.KDA_BF16, 64)
    assert need > 0
    ws = 128 * FAKE
    assert _seg(lib, 0, ws, need) == -2
    assert _seg(lib, 100, ws, need) == -2
    assert _seg(lib, 64) == -5  # no workspace
    assert _seg(lib, 64, ws, need - 1) == -5
    assert _seg(lib, 64, ws + 8, need) == -4
    assert _seg(lib, 64, 64 * FAKE + 256, need) == -6  # workspace inside o
    assert _seg(lib, 64, 2 * FAKE, need) == -6  # workspace inside k
    assert _seg(lib, 64, ws, need, q=None) == -1


def _step(lib, **kw):
    a = dict(q=FAKE, k=2 * FAKE, v=3 * FAKE, g=4 * FAKE, beta=5 * FAKE, st=6 * FAKE, o=None,
             N=1, H=1, dk=128, dv=128, din=kda.KDA_BF16, dout=kda.KDA_BF16)
    a.update(kw)
    return lib.kda_recurrent_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["st"], a["o"],
                                  a["N"], a["H"], a["dk"], a["dv"], a["din"], a["dout"], None)


def test_recurrent_step_rejects_before_launch(lib):
    o = 64 * FAKE
    assert _step(lib) == -1
    assert _step(lib, o=o, st=None) == -1
    assert _step(lib, o=o, dout=3) == -3
    assert _step(lib, o=o, dk=32) == -2
    assert _step(lib, o=o, N=0) == -2
    assert _step(lib, o=o, N=1 << 31, H=2) == -2
    assert _step(lib, o=o + 2) == -4
    assert _step(lib, o=6 * FAKE + 256) == -6  # o inside the state
    assert _step(lib, o=o, st=3 * FAKE) == -6  # state overlaps v


def test_verify_and_commit_reject_before_launch(lib):
    def verify(**kw):
        a = dict(q=FAKE, k=2 * FAKE, v=3 * FAKE, g=4 * FAKE, beta=5 * FAKE, st=6 * FAKE,
                 o=64 * FAKE, N=2, K=4, H=2, dk=128, dv=128, din=kda.KDA_BF16, dout=kda.KDA_BF16)
        a.update(kw)
        return lib.kda_recurrent_verify(a["q"], a["k"], a["v"], a["g"], a["beta"], a["st"], a["o"],
                                        a["N"], a["K"], a["H"], a["dk"], a["dv"], a["din"],
                                        a["dout"], None)

    def commit(**kw):
        a = dict(k=2 * FAKE, v=3 * FAKE, g=4 * FAKE, beta=5 * FAKE, acc=7 * FAKE, st=6 * FAKE,
                 N=2, K=4, H=2, dk=128, dv=128, din=kda.KDA_BF16)
        a.update(kw)
        return lib.kda_recurrent_commit(a["k"], a["v"], a["g"], a["beta"], a["acc"], a["st"],
                                        a["N"], a["K"], a["H"], a["dk"], a["dv"], a["din"], None)

    assert verify(q=None) == -1
    assert verify(o=None) == -1
    assert verify(dout=5) == -3
    assert verify(K=0) == -2
    assert verify(dk=32) == -2
    assert verify(o=64 * FAKE + 8) == -4
    assert verify(o=6 * FAKE + 64) == -6  # o inside the state
    assert commit(acc=None) == -1
    assert commit(st=None) == -1
    assert commit(din=9) == -3
    assert commit(N=0) == -2
    assert commit(acc=7 * FAKE + 4) == -4
    assert commit(st=3 * FAKE) == -6  # state overlaps v


def test_checkpoints_at_rejects_before_launch(lib):
    def call(**kw):
        a = dict(q=FAKE, k=2 * FAKE, v=3 * FAKE, g=4 * FAKE, beta=5 * FAKE, o=64 * FAKE,
                 ck=96 * FAKE, pos=8 * FAKE, n=2, B=1, T=256, H=1, dk=128, dv=128)
        a.update(kw)
        return lib.kda_chunk_fwd_checkpoints_at(a["q"], a["k"], a["v"], a["g"], a["beta"], None,
                                                a["o"], None, a["ck"], a["pos"], a["n"], a["B"],
                                                a["T"], a["H"], a["dk"], a["dv"], 64, kda.KDA_BF16,
                                                kda.KDA_BF16, None, 0, None)

    assert call(n=0) == -2
    assert call(n=-3) == -2
    assert call(pos=None) == -1
    assert call(ck=None) == -1
    assert call(pos=8 * FAKE + 4) == -4
    assert call(ck=64 * FAKE + 128) == -6  # checkpoints overlap o


def test_binding_rejects_host_tensors():
    import torch

    x = torch.zeros(1, 1, 128)
    with pytest.raises((ValueError, RuntimeError)):
        kda.kda_recurrent_step(x, x, x, x, torch.zeros(1, 1), torch.zeros(1, 1, 128, 128))


def test_binding_checks_every_tensor_before_launch():
    """The binding checks shapes, dtypes and devices of every tensor (the C ABI sees only
    pointers); each bad call raises before any pointer reaches the library."""
    import torch

    def t(*shape, dtype=torch.bfloat16):
        return torch.zeros(*shape, dtype=dtype)

    B, T, H, d = 1, 8, 2, 64
    q, k, v, g, beta = t(B, T, H, d), t(B, T, H, d), t(B, T, H, d), t(B, T, H, d), t(B, T, H)
    bad = [
        dict(k=t(B, T, H, d + 1)),                       # k of another size
        dict(k=t(B, T, H, d, dtype=torch.float32)),       # k of another dtype
        dict(g=t(B, T + 1, H, d)),
        dict(beta=t(B, T, H, 1)),
        dict(v=t(B, T, H + 1, d)),
        dict(initial_state=t(B, H, d, d)),                # state must be float32
        dict(initial_state=t(B, H, d, d - 1, dtype=torch.float32)),
        dict(o=t(B, T, H, d - 1)),
        dict(final_state=t(B, H, d, d, dtype=torch.float32)[:, :1]),
        dict(checkpoints=t(B, 1, H, d, d, dtype=torch.float32)),  # given without every
        dict(workspace=[0] * 16),
    ]
    for kw in bad:
        args = dict(q=q, k=k, v=v, g=g, beta=beta)
        args.update({n: kw[n] for n in ("k", "v", "g", "beta") if n in kw})
        rest = {n: x for n, x in kw.items() if n not in ("k", "v", "g", "beta")}
        with pytest.raises((ValueError, TypeError)):
            kda.kda_chunk_fwd(args["q"], args["k"], args["v"], args["g"], args["beta"], **rest)
    st = t(B, H, d, d, dtype=torch.float32)
    q1, v1, b1 = t(B, H, d), t(B, H, d), t(B, H)
    for kw in [dict(k=t(B, H, d + 1)), dict(beta=t(B, H, 2)), dict(state=t(B, H, d, d)),
               dict(state=t(B, H + 1, d, d, dtype=torch.float32)), dict(o=t(B, H, d - 1))]:
        a = dict(q=q1, k=q1, v=v1, g=q1, beta=b1, state=st)
        a.update(kw)
        o = a.pop("o", None)
        with pytest.raises((ValueError, TypeError)):
            kda.kda_recurrent_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state"], o=o)
    acc = torch.zeros(B, dtype=torch.int64)  # must be int32
    with pytest.raises((ValueError, TypeError)):
        kda.kda_recurrent_commit(k, v, g, beta, acc, st)
    with pytest.raises((ValueError, TypeError)):
        kda.kda_recurrent_verify(q, k, v, g, beta, t(B, H, d, d, dtype=torch.float32)[:, :1])
    with pytest.raises((ValueError, TypeError)):
        kda.kda_chunk_fwd_checkpoints_at(q, k, v, g, beta, torch.zeros(2, dtype=torch.int32))


def test_output_gate_entry_points_reject_before_launch(lib):
    bf = kda.KDA_BF16
    o = 64 * FAKE

    def fwd(gate, o=o, **kw):
        a = dict(B=1, T=64, H=1, dk=128, dv=128)
        a.update(kw)
        return lib.kda_chunk_fwd_output_gate(FAKE, 2 * FAKE, 3 * FAKE, 4 * FAKE, 5 * FAKE, gate,
                                             None, o, None, None, 0, a["B"], a["T"], a["H"],
                                             a["dk"], a["dv"], 64, bf, bf, None, 0, None)

    assert fwd(None) == -1
    assert fwd(7 * FAKE + 8) == -4
    assert fwd(o + 64) == -6          # gate inside o
    assert fwd(7 * FAKE, o=7 * FAKE + 256) == -6
    assert fwd(7 * FAKE, dk=96) == -2

    def step(gate, o=o):
        return lib.kda_recurrent_step_output_gate(FAKE, 2 * FAKE, 3 * FAKE, 4 * FAKE, 5 * FAKE,
                                                  gate, 6 * FAKE, o, 1, 1, 128, 128, bf, bf, None)

    assert step(None) == -1
    assert step(7 * FAKE + 4) == -4
    assert step(o) == -6
    assert step(6 * FAKE + 16) == -6  # gate inside the state


def test_noalloc_rejects_before_launch(lib):
    bf = kda.KDA_BF16

    def call(**kw):
        a = dict(q=FAKE, o=64 * FAKE, B=1, T=64, H=1, dk=128, dv=128, chunk=64)
        a.update(kw)
        return lib.kda_chunk_fwd_noalloc(a["q"], 2 * FAKE, 3 * FAKE, 4 * FAKE, 5 * FAKE, None,
                                         a["o"], None, None, 0, a["B"], a["T"], a["H"], a["dk"],
                                         a["dv"], a["chunk"], bf, bf, None)

    assert call(q=None) == -1
    assert call(dk=96) == -2
    assert call(chunk=48) == -2
    assert call(o=2 * FAKE) == -6
    # a size that takes the segment path: the other arguments are checked before the
    # library's scratch is looked up (no GPU call is made on the way to these errors)
    assert lib.kda_chunk_fwd_workspace_bytes(1, 65536, 32, 128, 128, 64, bf) > 0
    assert call(q=None, T=65536, H=32) == -1
    assert call(o=64 * FAKE + 4, T=65536, H=32) == -4


def test_debug_library_exports_and_rejects_null():
    """libkda_debug.so (the range-check build) exports every entry point of kda.h and the
    flag reader of kda_debug.h, which rejects a NULL output before any GPU call."""
    if not os.path.exists(kda.DEBUG_LIB_PATH):
        pytest.skip("libkda_debug.so not built")
    lib = kda.load_library(kda.DEBUG_LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    src = open(os.path.join(ROOT, "include", "kda_debug.h")).read()
    for name in sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", src))):
        assert hasattr(lib, name), name
    lib.kda_debug_range_flags.restype = ctypes.c_int
    lib.kda_debug_range_flags.argtypes = [ctypes.c_void_p, ctypes.c_int]
    assert lib.kda_debug_range_flags(None, 0) == -1  # KDA_ERR_NULL
    # the release library has no debug entry point
    assert not hasattr(kda.load_library(), "kda_debug_range_flags")
