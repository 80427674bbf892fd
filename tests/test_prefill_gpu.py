"""kda_chunk_fwd on the GPU against the float64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_57_amd as kda
import oracle
import parity
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {"f32": 1e-5, "bf16": 3e-3}


def _gpu(w, x, out_dtype=None, every=0):
    d = synth.to_torch(x, w.dtype, DEV)
    o, sf, ck = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"],
                                  out_dtype=out_dtype, checkpoint_every=every)
    torch.cuda.synchronize()
    return (o.double().cpu().numpy(), sf.double().cpu().numpy(),
            None if ck is None else ck.double().cpu().numpy())


def _ref(x, every=0):
    (o, s, ck), _ = oracle.kda_forward_heads_parallel(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                                      x["s0"], every)
    return o, s, ck


def _check(w, out_dtype=None, every=0, tol=None, x=None):
    x = synth.prefill_inputs(w) if x is None else x
    print(f"[prefill] {w.name} B{w.B} T{w.T} H{w.H} dk{w.dk} dv{w.dv} {w.dtype} "
          f"out={out_dtype}", flush=True)
    o, s, ck = _gpu(w, x, out_dtype, every)
    o_r, s_r, ck_r = _ref(x, every)
    tol = TOL[w.dtype] if tol is None else tol
    e_o = parity.check("o", o, o_r, tol, "tokens")
    e_s = parity.check("final state", s, s_r, tol, "state")
    if every:
        parity.check("checkpoints", ck, ck_r, tol, "ckpt")
    return e_o, e_s


def test_tiny_fp32_workload():
    _check(synth.TINY_F32)


def test_tiny_fp32_ragged_tail_and_fp32_out():
    _check(synth.TINY_F32.replace(T=200, init_state=True), out_dtype=torch.float32)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_bf16_small_shapes(dk, dv):
    w = synth.PREFILL_B4_T4096.replace(B=2, T=200, H=3, dk=dk, dv=dv)
    _check(w, out_dtype=torch.float32)


@pytest.mark.parametrize("law", ["n02", "n51", "mixed"])
def test_bf16_laws_bf16_out(law):
    w = synth.PREFILL_B4_T4096.replace(B=1, T=1024 + 37, H=4, a_law=law)
    _check(w)


def test_bf16_long_memory_fp32_out():
    """Decay logits ~ N(-7, 1) (long memory, outside the pages' workloads).  The rounding
    of the single-bfloat16 operands accumulates; a float64 model of the chunked algorithm
    with the kernel's roundings predicts about 3.2e-3 at 4096 tokens, so the bound here
    is 5e-3."""
    w = synth.PREFILL_B4_T4096.replace(B=1, T=4096, H=4, a_law="slow")
    _check(w, out_dtype=torch.float32, tol=5e-3)


def test_checkpoints_match_oracle():
    w = synth.PREFILL_B4_T4096.replace(B=2, T=640, H=2)
    _check(w, out_dtype=torch.float32, every=128)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decay_floor_on_every_channel(dtype):
    """Log-decay -5 on every channel of every token (and -7, clamped to it, on a third of
    them): every 16-token sub-tile's cumulative log-decay reaches -80, so every diagonal
    tile carries column factors up to e^80 ~ 5.5e34, the largest the floor allows."""
    w = (synth.TINY_F32 if dtype == "f32" else synth.PREFILL_B4_T4096).replace(
        B=1, T=320, H=2, init_state=True)
    x = synth.prefill_inputs(w)
    g = np.full_like(x["g"], -5.0)
    g[..., ::3] = -7.0
    x["g"] = g
    _check(w, out_dtype=torch.float32, x=x)


def test_tiny_t_below_one_chunk():
    _check(synth.PREFILL_B4_T4096.replace(B=1, T=1, H=2))
    _check(synth.TINY_F32.replace(T=17))


# ------------------------------------------------------------------ full-size workloads


def test_prefill_workload_full_size():
    """4 x 4096 tokens, 32 heads, d = 128, bfloat16: every output and final state."""
    _check(synth.PREFILL_B4_T4096)


def test_decay_floor_workload_full_size():
    """65,536 tokens x 32 heads with decay logits ~ N(5, 1): most channels sit on the floor."""
    _check(synth.DECAY_FLOOR_T65536)


def test_million_token_prefix_checkpoint():
    """1,048,576 tokens x 16 heads (inputs drawn on the device); the state after token
    65,536 (a checkpoint) and o over that prefix against the oracle run on the prefix."""
    w = synth.MILLION_TOKEN
    d = synth.device_prefill_inputs(w, DEV)
    P = 65536
    o, sf, ck = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"],
                                  checkpoint_every=P)
    torch.cuda.synchronize()
    assert ck.shape[1] == w.T // P
    x = {n: d[n][:, :P].double().cpu().numpy() for n in ("q", "k", "v", "g", "beta")}
    s0 = d["s0"].double().cpu().numpy()
    o_r, s_r, _ = _ref(dict(x, s0=s0))
    print(f"[prefill] 1M tokens, prefix {P}", flush=True)
    parity.check("o over the prefix", o[:, :P], o_r, 3e-3, "tokens")
    parity.check("checkpoint after the prefix", ck[:, 0], s_r, 3e-3, "state")
    assert bool(torch.isfinite(sf).all()) and bool(torch.isfinite(o.float()).all())
    # the last checkpoint is the final state
    assert torch.equal(ck[:, -1], sf)


def test_million_token_one_hot_keys_full_length():
    """1,048,576 tokens x 16 heads with one-hot keys and queries (the rest as the
    million-token workload): every state row is then an independent gated moving
    average (oracle.one_hot_key_rows), so outputs and final states can be checked
    over the whole length, across every segment the library cuts.  Tracked per
    head: the read row (all outputs), a row written in the first 4096 tokens and
    never decayed (carried across all segments), and a row never written and never
    decayed (must come out as the initial state, bit for bit)."""
    w = synth.MILLION_TOKEN
    print(f"[prefill] one-hot keys B{w.B} T{w.T} H{w.H} d{w.dk}", flush=True)
    d = synth.device_one_hot_inputs(w, DEV)
    o, sf, _ = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(sf).all()) and bool(torch.isfinite(o.float()).all())
    dk = w.dk
    heads = [0, 5, 10, 15]
    read = d["read"].cpu().tolist()
    rows = [(h, c) for h in heads for c in (read[h], dk - 2, dk - 1)]
    hh = torch.tensor([h for h, _ in rows], device=DEV)
    cc = torch.tensor([c for _, c in rows], device=DEV)
    g_rows = d["g"][0][:, hh, cc].double().cpu().numpy()
    hit = (d["chan"][0][:, hh] == cc).cpu().numpy()
    beta = d["beta"][0][:, hh].double().cpu().numpy()
    rows0 = d["s0"][0, hh, cc].double().cpu().numpy()
    v_h = d["v"][0][:, heads].float().cpu().numpy()             # [T, 4, dv]
    o_h = o[0][:, heads].float().cpu().numpy()                  # [T, 4, dv]
    head_of_row = [heads.index(h) for h, _ in rows]
    read_rows = [3 * i for i in range(len(heads))]               # trajectory rows read by q
    x, num, den = rows0, 0.0, 0.0
    for t0 in range(0, w.T, synth.BLOCK_T):
        t1 = min(w.T, t0 + synth.BLOCK_T)
        traj, x = oracle.one_hot_key_rows(x, g_rows[t0:t1], hit[t0:t1], beta[t0:t1],
                                          v_h[t0:t1][:, head_of_row])
        ref = traj[:, read_rows]
        num += float(np.sum((o_h[t0:t1] - ref) ** 2))
        den += float(np.sum(ref ** 2))
    e_o = (num / den) ** 0.5
    got = sf[0, hh, cc].double().cpu().numpy()
    e_s = oracle.rel_l2(got, x)
    print(f"[prefill]   one-hot full length: o (tracked heads) {e_o:.3e} "
          f"state rows {e_s:.3e}", flush=True)
    assert e_o <= 3e-3 and e_s <= 3e-3
    # the never-written, never-decayed row of every head is the initial state exactly
    assert torch.equal(sf[0, :, dk - 1], d["s0"][0, :, dk - 1])


def _random_cases(n=10, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = "f32" if i % 4 == 0 else "bf16"
        dk, dv = (64, 64) if dtype == "f32" else [(128, 128), (64, 64), (64, 128), (128, 64)][i % 4]
        cases.append((dtype, int(rng.integers(1, 4)), int(rng.integers(1, 700)),
                      int(rng.integers(1, 6)), dk, dv, bool(rng.integers(0, 2)),
                      ["n02", "n51", "mixed", "slow"][int(rng.integers(0, 4))]))
    return cases


@pytest.mark.parametrize("dtype,B,T,H,dk,dv,init,law", _random_cases())
def test_seeded_irregular_shapes(dtype, B, T, H, dk, dv, init, law):
    """Seeded irregular sizes (T from 1 to 699, ragged tails, one to five heads, one to
    three batch rows, every supported head-dimension pair, with and without an initial
    state, every decay law) against the oracle, float32 outputs."""
    base = synth.TINY_F32 if dtype == "f32" else synth.PREFILL_B4_T4096
    w = base.replace(B=B, T=T, H=H, dk=dk, dv=dv, init_state=init, a_law=law, seed=7 + T)
    _check(w, out_dtype=torch.float32, tol=5e-3 if (law == "slow" and dtype == "bf16") else None)
