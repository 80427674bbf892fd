"""Throughput of the KDA hot path on one MI355X, printed as one JSON line.

A step is one kda_chunk_fwd (chunked prefill, 64-token chunks) over the 4 x 4096-token,
32-head, d = 128 bfloat16 workload with a float32 initial state, inputs resident in HBM.
The same run also times that workload in 32-token chunks (the pipelined kernel) and
through the output-gate, raw-logit and listed-checkpoint entry points,
kda_recurrent_step on the 256-sequence decode workload
(1000 chained steps), speculative verify / commit, the two few-head long-sequence
prefill workloads (65,536 tokens x 32 heads, 1,048,576 tokens x 16 heads), and the
float64 CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s + % bf16 MFMA peak; decode-step HBM GB/s (% peak)"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2516.6


def prefill_flops_per_token_head(dk: int, dv: int, C: int = 64) -> float:
    """State products + block-triangular intra-chunk products (dense 16-tiles) + UT solve."""
    return 6 * dk * dv + 2 * C * (10 / 16) * (3 * dk + 2 * dv) + (2 / 3) * C * C


def prefill_bytes(B, T, H, dk, dv, in_bytes=2, out_bytes=2) -> float:
    """q, k, g, v, beta read once; o written once; state read and written once."""
    per_tok = (3 * dk + dv + 1) * in_bytes + dv * out_bytes
    return B * T * H * per_tok + 2 * B * H * dk * dv * 4


def decode_bytes(N, H, dk, dv, in_bytes=2, out_bytes=2) -> float:
    per_head = 2 * dk * dv * 4 + (3 * dk + dv + 1) * in_bytes + dv * out_bytes
    return N * H * per_head


def verify_bytes(N, K, H, dk, dv, in_bytes=2, out_bytes=2) -> float:
    """State read once; K draft tokens' q, k, g, v, beta read; K outputs written."""
    return N * H * (dk * dv * 4 + K * ((3 * dk + dv + 1) * in_bytes + dv * out_bytes))


def commit_bytes(N, K, H, dk, dv, in_bytes=2) -> float:
    """State read and written once; K tokens' k, g, v, beta read (all accepted)."""
    return N * H * (2 * dk * dv * 4 + K * ((2 * dk + dv + 1) * in_bytes))


_CSRC = os.path.join(ROOT, "gated_delta_rule_57_amd", "csrc")
# the sources each kernel is compiled from (its own file and the shared headers)
_SHARED = ("kda_device.h", "kda_internal.h")
KERNEL_SOURCES = {
    "prefill": ("kda_prefill.hip", "kda_prefill_body.inc") + _SHARED,
    "prefill_chunk32": ("kda_prefill_pipe.hip",) + _SHARED,
    "decode": ("kda_decode.hip",) + _SHARED,
    "verify": ("kda_decode.hip",) + _SHARED,
    "commit": ("kda_decode.hip",) + _SHARED,
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
COPY_CALIBRATION_BYTES = 1 << 30


def source_hash(which: str) -> str:
    """sha256 (first 16 hex digits) over the sources of one kernel, in order."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[which]:
        h.update(open(os.path.join(_CSRC, name), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(which: str):
    """HBM bytes per launch from the committed counter summary, or None when that
    summary was taken on a different version of the kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))[which]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256_16") != source_hash(which):
        return None
    return rec.get("bytes_per_launch")


def copy_calibration(torch, reps: int = 3):
    """A plain device-to-device copy of known size, for scaling the HBM byte counters."""
    n = COPY_CALIBRATION_BYTES // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    print(json.dumps({"copy_calibration": {"bytes_read": COPY_CALIBRATION_BYTES,
                                           "bytes_written": COPY_CALIBRATION_BYTES,
                                           "ms": ms,
                                           "GBps": 2 * COPY_CALIBRATION_BYTES / ms / 1e6}}))


def time_prefill(kda, torch, w, steps, warmup, chunk=64, cold=True):
    import synth

    d = synth.device_prefill_inputs(w, "cuda")
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=d["q"].dtype, device="cuda")
    sf = torch.empty_like(d["s0"])

    def step():
        kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], o=o,
                          final_state=sf, chunk=chunk)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    assert bool(torch.isfinite(o.float()).all()), "non-finite prefill output"
    if not cold:
        return ms, None, None
    # the same launch with the last-level cache (256 MB MALL) flushed before each one by a
    # 512 MiB write, each launch timed on its own
    # (control: the same single-launch timing without the flush)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold, single = [], []
    for i in range(10):
        for flush, out in ((True, cold), (False, single)):
            if flush:
                scratch.fill_(i)
            e0.record()
            step()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1))
    del scratch
    return ms, sum(cold) / len(cold), sum(single) / len(single)


def time_variants(kda, torch, w, steps, warmup):
    """The headline workload through the NEXT entry points, each timed like the headline
    (warm-up, then `steps` back-to-back launches with HIP events on the current stream):
    the fused output gate (one more [B,T,H,dv] input), raw decay logits (the same bytes,
    -softplus in the gate step), and states saved at every 512th token (a prefix cache's
    sparse block ends; 8 states per head written)."""
    import synth

    d = synth.device_prefill_inputs(w, "cuda")
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=d["q"].dtype, device="cuda")
    sf = torch.empty_like(d["s0"])
    z = torch.randn((w.B, w.T, w.H, w.dv), device="cuda").to(d["q"].dtype)
    pos = torch.arange(512, w.T + 1, 512, dtype=torch.int64, device="cuda")
    ck = torch.empty((w.B, pos.numel(), w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    base = prefill_bytes(w.B, w.T, w.H, w.dk, w.dv)
    legs = {
        "output_gate": (lambda: kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                                  d["s0"], o=o, final_state=sf, output_gate=z),
                        base + w.B * w.T * w.H * w.dv * 2),
        "gate_logits": (lambda: kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                                  d["s0"], o=o, final_state=sf, gate_logits=True),
                        base),
        "checkpoints_every_512": (lambda: kda.kda_chunk_fwd_checkpoints_at(
            d["q"], d["k"], d["v"], d["g"], d["beta"], pos, d["s0"], o=o, final_state=sf,
            checkpoints=ck), base + ck.numel() * 4),
    }
    out = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for name, (fn, nbytes) in legs.items():
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms_per_step": ms, "tokens_per_s": w.B * w.T / (ms * 1e-3),
                     "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                                  "algorithmic_bytes_per_launch": nbytes}}
    assert bool(torch.isfinite(sf).all()), "non-finite state in the variant legs"
    return out


def time_decode(kda, torch, w, steps, warmup):
    import synth

    d = synth.device_decode_inputs(w, steps, "cuda")
    state = d["s0"].clone()
    o = torch.empty((w.B, w.H, w.dv), dtype=d["q"].dtype, device="cuda")

    def step(s):
        kda.kda_recurrent_step(d["q"][s], d["k"][s], d["v"][s], d["g"][s], d["beta"][s], state,
                               o=o)

    for s in range(warmup):
        step(s % steps)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(steps):
        step(s)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / steps
    assert bool(torch.isfinite(state).all()), "non-finite decode state"
    return us


def time_speculative(kda, torch, w, K, reps):
    """One verify of K draft tokens per sequence and one commit of all of them, timed apart
    with HIP events on the current stream (mean over `reps` launches of each)."""
    import synth

    d = synth.device_prefill_inputs(w.replace(T=K), "cuda")  # [N, K, H, .] draft inputs
    state = d["s0"].clone()
    o = torch.empty((w.B, K, w.H, w.dv), dtype=d["q"].dtype, device="cuda")
    accept = torch.full((w.B,), K, dtype=torch.int32, device="cuda")

    def verify():
        kda.kda_recurrent_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], state, o=o)

    def commit():
        kda.kda_recurrent_commit(d["k"], d["v"], d["g"], d["beta"], accept, state)

    out = {}
    for name, fn in (("verify", verify), ("commit", commit)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name] = e0.elapsed_time(e1) * 1000.0 / reps
    assert bool(torch.isfinite(state).all()), "non-finite state after commits"
    return out


def time_long_prefill(kda, torch, w, reps: int = 3):
    """kda_chunk_fwd on a few-head long-sequence workload with the library's own segment choice:
    one warm call, then `reps` calls timed together with HIP events on the current stream."""
    import synth

    d = synth.device_prefill_inputs(w, "cuda")
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=d["q"].dtype, device="cuda")
    sf = torch.empty_like(d["s0"])
    ws_bytes = kda.kda_chunk_fwd_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def call():
        kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], o=o,
                          final_state=sf, workspace=ws)

    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    assert bool(torch.isfinite(sf).all()), "non-finite final state"
    seg = kda.kda_chunk_fwd_segment_tokens(w.B, w.T, w.H, w.dk, w.dv)
    del d, o, sf, ws
    torch.cuda.empty_cache()
    nbytes = prefill_bytes(w.B, w.T, w.H, w.dk, w.dv)
    flops = prefill_flops_per_token_head(w.dk, w.dv) * w.B * w.T * w.H
    gbs, tflops = nbytes / (ms * 1e-3) / 1e9, flops / (ms * 1e-3) / 1e12
    return {"workload": w.name, "ms_per_call": ms, "calls_timed": reps,
            "tokens_per_s": w.B * w.T / (ms * 1e-3), "segments": -(-w.T // seg),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_call": nbytes},
            "mfma": {"achieved": tflops, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / BF16_MFMA_PEAK_TFLOPS}}


def cpu_baseline(w, sample_batches: int):
    """The float64 oracle on `sample_batches` sequences of the workload's shape and laws (all
    heads), host-drawn.  Returns the baseline record and the sample (inputs and the oracle's
    outputs), which the GPU leg later runs through kda_chunk_fwd for the line's parity figures.

    Runs before this process touches the GPU: the oracle's worker pool is spawned here
    (started and warmed before the timed call, which then measures the oracle alone)."""
    import oracle
    import synth

    nb = max(1, min(sample_batches, w.B))
    x = synth.prefill_inputs(w.replace(B=nb))
    args = [x[n] for n in ("q", "k", "v", "g", "beta")]
    with oracle.head_pool() as pool:
        tiny = {n: v[:1, :8] for n, v in x.items() if n != "s0"}
        oracle.kda_forward_heads_parallel(*[tiny[n] for n in ("q", "k", "v", "g", "beta")],
                                          x["s0"][:1], pool=pool)  # workers up and importing
        t = time.perf_counter()
        (o_ref, s_ref, _), procs = oracle.kda_forward_heads_parallel(*args, x["s0"], pool=pool)
        dt = time.perf_counter() - t
    tokens = nb * w.T
    # one process on a smaller sample (two heads of one sequence), scaled to all heads
    h1 = min(2, w.H)
    x1 = {n: v[:1, :, :h1] for n, v in x.items() if n != "s0"}
    t = time.perf_counter()
    oracle.kda_forward_heads_parallel(*[x1[n] for n in ("q", "k", "v", "g", "beta")],
                                      x["s0"][:1, :h1], processes=1)
    dt1 = time.perf_counter() - t
    rec = {"value": tokens / dt, "unit": "tokens/s", "cores": procs, "kind": "oracle",
           "sample": f"{nb} sequences x {w.T} tokens x {w.H} heads of the workload's shape and "
                     f"laws, host-drawn ({tokens * w.H} token-heads, {dt:.1f} s wall on {procs} "
                     "processes)",
           "single_core": {"value": w.T * h1 / w.H / dt1, "unit": "tokens/s",
                           "sample": f"1 sequence x {w.T} tokens x {h1} heads on one process "
                                     f"({dt1:.2f} s), scaled to {w.H} heads"}}
    return rec, {"x": x, "o": o_ref, "s": s_ref}


def parity_of_sample(kda, torch, w, sample, tol=3e-3):
    """The CPU leg's sample through kda_chunk_fwd (bf16 output, as timed) against the
    oracle's outputs: relative L2 over each tensor, its maximum over (b, h), and for o its
    maximum over 64-token windows of each head."""
    import numpy as np
    import synth

    x = sample["x"]
    d = synth.to_torch(x, w.dtype, "cuda")
    o, s, _ = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"])
    torch.cuda.synchronize()
    o = o.float().cpu().double().numpy()
    s = s.cpu().double().numpy()

    def rel(a, b, axes):
        num = np.sqrt(np.sum((a - b) ** 2, axis=axes))
        den = np.sqrt(np.sum(b ** 2, axis=axes))
        return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)

    o_ref, s_ref = sample["o"], sample["s"]
    B, T, H, _ = o.shape
    nw = T // 64
    ow = rel(o[:, :nw * 64].reshape(B, nw, 64, H, -1), o_ref[:, :nw * 64].reshape(B, nw, 64, H, -1),
             (2, 4))
    out = {"sample": f"the CPU leg's {B} x {T} x {H} sample, bf16 output", "tol": tol,
           "o_rel_l2": float(rel(o, o_ref, None)), "o_head_max": float(rel(o, o_ref, (1, 3)).max()),
           "o_window_max": float(ow.max()), "state_rel_l2": float(rel(s, s_ref, None)),
           "state_head_max": float(rel(s, s_ref, (2, 3)).max())}
    out["pass"] = bool(max(out["o_rel_l2"], out["o_head_max"], out["state_rel_l2"],
                           out["state_head_max"]) <= tol and out["o_window_max"] <= 2 * tol)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the two few-head long-sequence prefill workloads")
    ap.add_argument("--draft", type=int, default=4, help="draft tokens per speculative verify")
    ap.add_argument("--cpu-sample-batches", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the KDA path here has "
              "no multi-GPU leg", file=sys.stderr)
        sys.exit(2)

    import synth

    w = synth.PREFILL_B4_T4096
    # the CPU leg first: its worker processes are started before anything here touches
    # the GPU
    cpu = sample = None
    if not args.no_cpu_baseline and not args.copy_calibration:
        cpu, sample = cpu_baseline(w, args.cpu_sample_batches)

    import torch

    if args.copy_calibration:
        copy_calibration(torch)
        return

    import gated_delta_rule_57_amd as kda

    # Python's cyclic garbage collector is paused while kernels are timed: a full
    # collection stalls the launching thread for tens of milliseconds (a 31 ms idle gap
    # between two back-to-back launches of a 0.1 ms kernel in one kernel trace), which
    # is host noise, not time spent in the library
    gc.collect()
    gc.disable()
    ms, ms_cold, ms_single = time_prefill(kda, torch, w, args.steps, args.warmup)
    toks = w.B * w.T
    flops = prefill_flops_per_token_head(w.dk, w.dv) * toks * w.H
    nbytes = prefill_bytes(w.B, w.T, w.H, w.dk, w.dv)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": toks / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "dk": w.dk, "dv": w.dv,
                   "chunk": w.chunk, "inputs": "bf16", "state": "f32", "output": "bf16",
                   "decay_logits": "N(0,2)"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic("prefill"),
                     "kernel": "chunk_fwd_kernel<bf16,bf16,128,128,64>",
                     "algorithmic_bytes_per_launch": nbytes},
        "mfma": {"achieved": tflops, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": tflops / BF16_MFMA_PEAK_TFLOPS, "algorithmic_flops_per_launch": flops},
        "cold_cache": {"ms_per_step": ms_cold, "launches": 10,
                       "ms_per_step_unflushed": ms_single,
                       "note": "each launch timed alone after a 512 MiB write that flushes the "
                               "256 MB MALL; unflushed: the same single-launch timing without it"},
    }
    # the same workload in 32-token chunks (the pipelined kernel); not the headline
    ms32, _, _ = time_prefill(kda, torch, w, args.steps, args.warmup, chunk=32, cold=False)
    gbs32, tf32 = nbytes / (ms32 * 1e-3) / 1e9, flops / (ms32 * 1e-3) / 1e12
    line["prefill_chunk_32"] = {
        "workload": w.name, "chunk": 32, "ms_per_step": ms32, "tokens_per_s": toks / (ms32 * 1e-3),
        "roofline": {"bound": "hbm", "achieved": gbs32, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs32 / HBM_PEAK_GBS, "traffic": measured_traffic("prefill_chunk32"),
                     "kernel": "chunk_pipe_kernel<bf16,128,128,2>",
                     "algorithmic_bytes_per_launch": nbytes},
        "mfma": {"achieved": tf32, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": tf32 / BF16_MFMA_PEAK_TFLOPS}}
    line["variants"] = time_variants(kda, torch, w, args.steps, args.warmup)
    if not args.no_decode:
        wd = synth.DECODE_N256
        us = time_decode(kda, torch, wd, args.decode_steps, 10)
        db = decode_bytes(wd.B, wd.H, wd.dk, wd.dv)
        dgbs = db / (us * 1e-6) / 1e9
        line["decode"] = {"workload": wd.name, "us_per_step": us, "steps_timed": args.decode_steps,
                          "roofline": {"bound": "hbm", "achieved": dgbs, "peak": HBM_PEAK_GBS,
                                       "unit": "GB/s", "frac": dgbs / HBM_PEAK_GBS,
                                       "traffic": measured_traffic("decode"),
                                       "kernel": "decode_step_kernel<bf16,bf16,128,128>",
                                       "algorithmic_bytes_per_launch": db}}
        K = args.draft
        us = time_speculative(kda, torch, wd, K, 200)
        vb, cb = verify_bytes(wd.B, K, wd.H, wd.dk, wd.dv), commit_bytes(wd.B, K, wd.H, wd.dk, wd.dv)
        vgbs, cgbs = vb / (us["verify"] * 1e-6) / 1e9, cb / (us["commit"] * 1e-6) / 1e9
        line["speculative"] = {
            "workload": f"draft_bf16_n{wd.B}_h{wd.H}_d{wd.dk}_k{K}",
            "us_per_verify": us["verify"], "us_per_commit": us["commit"],
            "draft_tokens_per_s": wd.B * K / (us["verify"] * 1e-6),
            "verify_roofline": {"bound": "hbm", "achieved": vgbs, "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": vgbs / HBM_PEAK_GBS,
                                "traffic": measured_traffic("verify"),
                                "kernel": "multi_token_kernel<bf16,bf16,128,128,verify>",
                                "algorithmic_bytes_per_launch": vb},
            "commit_roofline": {"bound": "hbm", "achieved": cgbs, "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": cgbs / HBM_PEAK_GBS,
                                "traffic": measured_traffic("commit"),
                                "kernel": "multi_token_kernel<bf16,bf16,128,128,commit>",
                                "algorithmic_bytes_per_launch": cb}}
    if not args.no_long:
        line["long_prefill"] = [time_long_prefill(kda, torch, wl)
                                for wl in (synth.DECAY_FLOOR_T65536, synth.MILLION_TOKEN)]
    gc.enable()
    if cpu is not None:
        line["cpu_baseline"] = cpu
        line["parity"] = parity_of_sample(kda, torch, w, sample)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
