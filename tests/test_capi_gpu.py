"""The C ABI from a plain C program (tests/capi/kda_capi_main.c, built by the library's
build): a prefill through kda_chunk_fwd with a workspace the program allocates itself,
then one kda_recurrent_step on the final states, no Python or torch in the calling
process.  Its float32 outputs are compared with the float64 oracle."""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import parity
import synth
from gated_delta_rule_57_amd import build as kda_build

pytestmark = pytest.mark.gpu


def _bf16_bytes(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).view(torch.int16).numpy().tobytes()


@pytest.mark.parametrize("B,T,H,chunk", [(2, 333, 3, 64), (1, 4096 + 9, 4, 64), (1, 200, 2, 32)])
def test_plain_c_caller(tmp_path, B, T, H, chunk):
    if not os.path.exists(kda_build.CAPI_BIN):
        pytest.skip("tests/capi/kda_capi_check not built")
    w = synth.PREFILL_B4_T4096.replace(B=B, T=T, H=H, init_state=True, seed=31 + T)
    x = synth.prefill_inputs(w)
    for n in ("q", "k", "v", "g", "beta"):
        (tmp_path / f"{n}.bin").write_bytes(_bf16_bytes(x[n]))
    (tmp_path / "s0.bin").write_bytes(np.ascontiguousarray(x["s0"], np.float32).tobytes())
    r = subprocess.run([kda_build.CAPI_BIN, str(tmp_path), str(B), str(T), str(H), str(w.dk),
                        str(w.dv), str(chunk)], capture_output=True, text=True, timeout=120)
    print(r.stdout + r.stderr, flush=True)
    assert r.returncode == 0
    o = np.fromfile(tmp_path / "o.bin", np.float32).reshape(B, T, H, w.dv)
    s = np.fromfile(tmp_path / "s.bin", np.float32).reshape(B, H, w.dk, w.dv)
    od = np.fromfile(tmp_path / "od.bin", np.float32).reshape(B, H, w.dv)
    sd = np.fromfile(tmp_path / "sd.bin", np.float32).reshape(B, H, w.dk, w.dv)
    (o_r, s_r, _), _ = oracle.kda_forward_heads_parallel(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                                         x["s0"], 0)
    # the decode step from the state the C program's prefill produced (the prefill's own
    # error is checked above; a single token's output per head is too small a sample to
    # carry it as well)
    last = {n: x[n][:, T - 1] for n in ("q", "k", "v", "g", "beta")}
    od_r, sd_r = oracle.kda_decode_step(s.astype(np.float64), last["q"], last["k"], last["v"],
                                        last["g"], last["beta"])
    parity.check("o from C", o, o_r, 3e-3, "tokens")
    parity.check("state from C", s, s_r, 3e-3, "state")
    # the step itself is float32 arithmetic on exact bfloat16 inputs
    parity.check("decode o from C", od, od_r, 1e-5, "step")
    parity.check("decode state from C", sd, sd_r, 1e-5, "state")
