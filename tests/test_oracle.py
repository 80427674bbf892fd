"""Pins for the float64 CPU oracle: nothing here calls the oracle to check itself.

Each pin reaches the KDA result through different arithmetic or a different
source: hand-derived worked examples, the constants the pages print, dense
products of the per-token transition matrices, closed forms, invariants and
the segment composition law.  A mutation test at the end plants plausible
mistakes in copies of the oracle's step and checks that the pins catch them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import kda as okda

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _single_head(fn, q, k, v, g, beta, s0, every=0):
    """Run a batched [B,T,H,...] oracle on one head given as [T, ...] arrays."""
    o, S, ck = fn(q[None, :, None], k[None, :, None], v[None, :, None], g[None, :, None],
                  beta[None, :, None], s0[None, None], every)
    return o[0, :, 0], S[0, 0], None if ck is None else ck[0, :, 0]


def _rand_head(rng, T, dk, dv, g_lo=-5.0, unit_k=True):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, dv))
    g = rng.uniform(g_lo, 0.0, (T, dk))
    beta = rng.uniform(0.0, 1.0, T)
    s0 = rng.standard_normal((dk, dv))
    return q, k, v, g, beta, s0


def brute_force(q, k, v, g, beta, s0):
    """S_t from explicit products of M_t = (I - b_t k_t k_t^T) Diag(exp g_t), g in [-5, 0]."""
    T, dk = q.shape
    M = [(np.eye(dk) - beta[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(g[t])) for t in range(T)]
    outs, S_t = [], None
    for t in range(T):
        prod = np.eye(dk)
        for s in range(t, -1, -1):
            prod = prod @ M[s]
        S_t = prod @ s0
        for s in range(t + 1):
            tail = np.eye(dk)
            for r in range(t, s, -1):
                tail = tail @ M[r]
            S_t = S_t + tail @ (beta[s] * np.outer(k[s], v[s]))
        outs.append(S_t.T @ q[t])
    return np.array(outs), S_t


# ---------------------------------------------------------------- pages + golden


def test_pages_printed_constants():
    c = json.load(open(os.path.join(GOLDEN, "pages_constants.json")))
    sig = c["printed_sig_figs"]

    def rounds_to(x, printed):
        e = math.floor(math.log10(abs(printed)))
        return round(x / 10 ** e, sig - 1) == round(printed / 10 ** e, sig - 1)

    floor = oracle.LOG_DECAY_FLOOR
    assert rounds_to(math.exp(floor), c["min_retained_fraction_per_step"])
    tile_lo = c["tile_tokens"] * floor
    assert tile_lo == c["tile_cum_log_decay_lower"]
    assert rounds_to(math.exp(-tile_lo), c["tile_reciprocal_bound"])
    import torch

    bf16_max = float(torch.finfo(torch.bfloat16).max)
    assert rounds_to(bf16_max, c["bf16_max_approx"])
    assert math.exp(-tile_lo) < bf16_max
    # the oracle's clamp holds the floor exactly
    assert oracle.clamp_log_decay(np.array([-1e9]))[0] == floor


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "worked_examples.json")))
                         ["cases"], ids=lambda c: c["name"])
def test_worked_examples(case):
    a = {n: np.array(case[n], dtype=np.float64) for n in ("q", "k", "v", "g", "beta", "s0")}
    o, S, _ = _single_head(oracle.kda_forward, a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"])
    np.testing.assert_allclose(o, np.array(case["o"], float), rtol=0, atol=case["tol"] * 10)
    np.testing.assert_allclose(S, np.array(case["final_state"], float), rtol=0,
                               atol=case["tol"] * 10)


# ---------------------------------------------------------------- brute force


@pytest.mark.parametrize("T,dk,dv,seed", [(1, 3, 3, 0), (2, 4, 3, 1), (5, 3, 5, 2), (8, 6, 4, 3),
                                          (8, 4, 4, 4)])
def test_brute_force_products(T, dk, dv, seed):
    rng = np.random.default_rng(seed)
    q, k, v, g, beta, s0 = _rand_head(rng, T, dk, dv, unit_k=(seed % 2 == 0))
    o, S, _ = _single_head(oracle.kda_forward, q, k, v, g, beta, s0)
    o_bf, S_bf = brute_force(q, k, v, g, beta, s0)
    assert oracle.rel_l2(o, o_bf) < 1e-12
    assert oracle.rel_l2(S, S_bf) < 1e-12


def test_brute_force_at_the_floor():
    rng = np.random.default_rng(7)
    q, k, v, g, beta, s0 = _rand_head(rng, 8, 4, 4)
    g[:] = -5.0
    o, S, _ = _single_head(oracle.kda_forward, q, k, v, g, beta, s0)
    o_bf, S_bf = brute_force(q, k, v, g, beta, s0)
    assert oracle.rel_l2(o, o_bf) < 1e-12 and oracle.rel_l2(S, S_bf) < 1e-12


# ---------------------------------------------------------------- invariants


def test_invariant_no_write_no_decay_keeps_state_bitwise():
    rng = np.random.default_rng(11)
    q, k, v, _, _, s0 = _rand_head(rng, 6, 5, 7)
    g = np.zeros((6, 5))
    beta = np.zeros(6)
    o, S, _ = _single_head(oracle.kda_forward, q, k, v, g, beta, s0)
    assert np.array_equal(S, s0)
    np.testing.assert_allclose(o, q @ s0, rtol=1e-14, atol=1e-14)


def test_invariant_unit_key_full_write_retrieves_value():
    rng = np.random.default_rng(12)
    T, dk, dv = 10, 6, 5
    q, k, v, g, _, s0 = _rand_head(rng, T, dk, dv, unit_k=True)
    beta = np.ones(T)
    _, _, ck = _single_head(oracle.kda_forward, q, k, v, g, beta, s0, every=1)
    for t in range(T):
        np.testing.assert_allclose(ck[t].T @ k[t], v[t], rtol=0, atol=1e-13)


# ---------------------------------------------------------------- closed forms


def test_closed_form_no_write_is_pure_decay():
    rng = np.random.default_rng(13)
    T, dk, dv = 12, 4, 3
    q, k, v, _, _, s0 = _rand_head(rng, T, dk, dv)
    g = rng.uniform(-9.0, 2.0, (T, dk))  # outside [-5, 0] on purpose: the clamp applies
    beta = np.zeros(T)
    o, S, _ = _single_head(oracle.kda_forward, q, k, v, g, beta, s0)
    gc = np.clip(g, -5.0, 0.0)
    G = np.cumsum(gc, axis=0)
    for t in range(T):
        np.testing.assert_allclose(o[t], s0.T @ (np.exp(G[t]) * q[t]), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S, np.exp(G[-1])[:, None] * s0, rtol=1e-12, atol=1e-14)


def test_closed_form_one_hot_keys_are_gated_emas():
    rng = np.random.default_rng(14)
    T, dk, dv = 40, 5, 3
    chan = rng.integers(0, dk, T)
    k = np.eye(dk)[chan]
    read = rng.integers(0, dk, T)
    q = np.eye(dk)[read]
    v = rng.standard_normal((T, dv))
    g = rng.uniform(-5.0, 0.0, (T, dk))
    beta = rng.uniform(0.0, 1.0, T)
    s0 = rng.standard_normal((dk, dv))
    o, S, _ = _single_head(oracle.kda_forward, q, k, v, g, beta, s0)
    rows = [list(s0[c]) for c in range(dk)]
    for t in range(T):
        for c in range(dk):
            keep = math.exp(g[t, c])
            for j in range(dv):
                x = keep * rows[c][j]
                if c == chan[t]:
                    x = (1.0 - beta[t]) * x + beta[t] * v[t, j]
                rows[c][j] = x
        for j in range(dv):
            assert abs(o[t, j] - rows[read[t]][j]) < 1e-12
    np.testing.assert_allclose(S, np.array(rows), rtol=0, atol=1e-12)


def test_one_hot_row_closed_form_follows_the_hand_loop():
    """oracle.one_hot_key_rows (the closed form used at the million-token length)
    against a plain scalar loop of the gated moving averages, written out here, with
    log-decays below the floor and above zero (both clamped) and rows never hit."""
    rng = np.random.default_rng(16)
    T, dk, dv = 60, 6, 3
    chan = rng.integers(0, dk - 1, T)            # the last channel is never hit
    g = rng.uniform(-7.0, 0.5, (T, dk))
    g[:, 2] = 0.0                                # a channel that never decays
    beta = rng.uniform(0.0, 1.0, T)
    v = rng.standard_normal((T, dv))
    s0 = rng.standard_normal((dk, dv))
    rows = [list(s0[c]) for c in range(dk)]
    want = np.empty((T, dk, dv))
    for t in range(T):
        for c in range(dk):
            keep = math.exp(min(max(g[t, c], -5.0), 0.0))
            for j in range(dv):
                x = keep * rows[c][j]
                if c == chan[t]:
                    x = x + beta[t] * (v[t, j] - x)
                rows[c][j] = x
                want[t, c, j] = x
    hit = chan[:, None] == np.arange(dk)[None, :]
    traj, fin = oracle.one_hot_key_rows(s0, g, hit, np.repeat(beta[:, None], dk, 1),
                                        np.repeat(v[:, None], dk, 1))
    np.testing.assert_allclose(traj, want, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(fin, want[-1], rtol=1e-13, atol=1e-15)
    # the row that is never hit only decays
    np.testing.assert_allclose(fin[dk - 1], s0[dk - 1] * np.prod(np.exp(np.clip(g[:, dk - 1],
                                                                             -5.0, 0.0))),
                               rtol=1e-12)
    # the undecayed channel: its row is a plain beta-weighted average, unchanged between hits
    last = np.nonzero(chan == 2)[0]
    if len(last):
        assert np.array_equal(fin[2], traj[last[-1], 2])


def test_clamp_is_idempotent_and_nan_propagates():
    rng = np.random.default_rng(15)
    q, k, v, g, beta, s0 = _rand_head(rng, 5, 4, 4)
    g_lo = g.copy()
    g_lo[:, 0] = -5.0
    g_far = g.copy()
    g_far[:, 0] = -7.25
    g_far[:, 1] = np.maximum(g_far[:, 1], 0.0) + 1.5  # above the ceiling
    g_lo[:, 1] = 0.0
    a = _single_head(oracle.kda_forward, q, k, v, g_lo, beta, s0)
    b = _single_head(oracle.kda_forward, q, k, v, g_far, beta, s0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    g_nan = g.copy()
    g_nan[2, 3] = np.nan
    o, S, _ = _single_head(oracle.kda_forward, q, k, v, g_nan, beta, s0)
    assert np.all(np.isfinite(o[:2])) and np.isnan(o[2:]).any() and np.isnan(S).any()


# ---------------------------------------------------------------- segment law


def test_segment_composition_transition_plus_zero_start():
    """orkas.ai blog, "The cost is paid in the serving stack": a segment's effect is a
    cumulative transition applied to the entering state plus the state the segment
    produces from zero; the two compose across segments."""
    rng = np.random.default_rng(16)
    T, dk, dv = 9, 5, 4
    q, k, v, g, beta, s_in = _rand_head(rng, T, dk, dv)
    _, Phi, _ = _single_head(oracle.kda_forward, q, k, np.zeros((T, dk)), g, beta, np.eye(dk))
    _, Z, _ = _single_head(oracle.kda_forward, q, k, v, g, beta, np.zeros((dk, dv)))
    _, S, _ = _single_head(oracle.kda_forward, q, k, v, g, beta, s_in)
    np.testing.assert_allclose(S, Phi @ s_in + Z, rtol=1e-12, atol=1e-13)
    # two segments: the pairs compose by (P2 P1, P2 Z1 + Z2)
    t1 = 4
    _, P1, _ = _single_head(oracle.kda_forward, q[:t1], k[:t1], np.zeros((t1, dk)), g[:t1],
                            beta[:t1], np.eye(dk))
    _, Z1, _ = _single_head(oracle.kda_forward, q[:t1], k[:t1], v[:t1], g[:t1], beta[:t1],
                            np.zeros((dk, dv)))
    _, P2, _ = _single_head(oracle.kda_forward, q[t1:], k[t1:], np.zeros((T - t1, dk)), g[t1:],
                            beta[t1:], np.eye(dk))
    _, Z2, _ = _single_head(oracle.kda_forward, q[t1:], k[t1:], v[t1:], g[t1:], beta[t1:],
                            np.zeros((dk, dv)))
    np.testing.assert_allclose(P2 @ P1, Phi, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(P2 @ Z1 + Z2, Z, rtol=1e-12, atol=1e-13)


def test_split_sequence_handoff_is_bitwise():
    rng = np.random.default_rng(17)
    q, k, v, g, beta, s0 = _rand_head(rng, 11, 4, 6)
    o, S, _ = _single_head(oracle.kda_forward, q, k, v, g, beta, s0)
    o1, S1, _ = _single_head(oracle.kda_forward, q[:6], k[:6], v[:6], g[:6], beta[:6], s0)
    o2, S2, _ = _single_head(oracle.kda_forward, q[6:], k[6:], v[6:], g[6:], beta[6:], S1)
    assert np.array_equal(np.concatenate([o1, o2]), o) and np.array_equal(S2, S)


def test_decode_step_is_one_token_of_forward():
    rng = np.random.default_rng(18)
    q, k, v, g, beta, s0 = _rand_head(rng, 3, 4, 5)
    o, S, _ = _single_head(oracle.kda_forward, q, k, v, g, beta, s0)
    st = s0[None, None]
    for t in range(3):
        ot, st = oracle.kda_decode_step(st, q[t][None, None], k[t][None, None],
                                        v[t][None, None], g[t][None, None],
                                        np.array([[beta[t]]]))
        assert np.array_equal(ot[0, 0], o[t])
    assert np.array_equal(st[0, 0], S)


def test_heads_parallel_matches_batched():
    rng = np.random.default_rng(19)
    B, T, H, dk, dv = 2, 7, 3, 4, 5
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    g = rng.uniform(-5, 0, (B, T, H, dk))
    beta = rng.uniform(0, 1, (B, T, H))
    s0 = rng.standard_normal((B, H, dk, dv))
    ref = oracle.kda_forward(q, k, v, g, beta, s0, 7)
    (o, S, ck), n = oracle.kda_forward_heads_parallel(q, k, v, g, beta, s0, 7, processes=2)
    assert n == 2
    assert np.array_equal(o, ref[0]) and np.array_equal(S, ref[1]) and np.array_equal(ck, ref[2])


# ---------------------------------------------------------------- mutation check


def _mut_read_before_write(S, q, k, v, g, beta):
    S = np.exp(okda.clamp_log_decay(g))[..., :, None] * S
    o = np.einsum("...cj,...c->...j", S, q)
    w = np.einsum("...cj,...c->...j", S, k)
    return S + beta[..., None, None] * k[..., :, None] * (v - w)[..., None, :], o


def _mut_decay_after_write(S, q, k, v, g, beta):
    w = np.einsum("...cj,...c->...j", S, k)
    S = S + beta[..., None, None] * k[..., :, None] * (v - w)[..., None, :]
    S = np.exp(okda.clamp_log_decay(g))[..., :, None] * S
    return S, np.einsum("...cj,...c->...j", S, q)


def _mut_transposed_read(S, q, k, v, g, beta):
    S = np.exp(okda.clamp_log_decay(g))[..., :, None] * S
    w = np.einsum("...jc,...c->...j", S, k)
    S = S + beta[..., None, None] * k[..., :, None] * (v - w)[..., None, :]
    return S, np.einsum("...cj,...c->...j", S, q)


def _mut_sign(S, q, k, v, g, beta):
    S = np.exp(okda.clamp_log_decay(g))[..., :, None] * S
    w = np.einsum("...cj,...c->...j", S, k)
    S = S + beta[..., None, None] * k[..., :, None] * (w - v)[..., None, :]
    return S, np.einsum("...cj,...c->...j", S, q)


def _mut_floor(S, q, k, v, g, beta):
    S = np.exp(np.minimum(np.maximum(g, -8.0), 0.0))[..., :, None] * S
    w = np.einsum("...cj,...c->...j", S, k)
    S = S + beta[..., None, None] * k[..., :, None] * (v - w)[..., None, :]
    return S, np.einsum("...cj,...c->...j", S, q)


def _mut_decay_on_values(S, q, k, v, g, beta):
    S = S * np.exp(okda.clamp_log_decay(g))[..., None, :]
    w = np.einsum("...cj,...c->...j", S, k)
    S = S + beta[..., None, None] * k[..., :, None] * (v - w)[..., None, :]
    return S, np.einsum("...cj,...c->...j", S, q)


@pytest.mark.parametrize("mutant", [_mut_read_before_write, _mut_decay_after_write,
                                    _mut_transposed_read, _mut_sign, _mut_floor,
                                    _mut_decay_on_values], ids=lambda f: f.__name__)
def test_pins_reject_planted_mistakes(mutant, monkeypatch):
    """Each mistake planted in the oracle's step must fail at least one pin (a shape
    error on non-square states counts as caught)."""
    monkeypatch.setattr(okda, "_step", mutant)
    failures = 0
    for case in json.load(open(os.path.join(GOLDEN, "worked_examples.json")))["cases"]:
        try:
            test_worked_examples(case)
        except (AssertionError, ValueError):
            failures += 1
    for args in [(5, 3, 5, 2), (8, 4, 4, 4)]:
        try:
            test_brute_force_products(*args)
        except (AssertionError, ValueError):
            failures += 1
    try:
        test_clamp_is_idempotent_and_nan_propagates()
        test_closed_form_no_write_is_pure_decay()
    except (AssertionError, ValueError):
        failures += 1
    assert failures > 0, f"{mutant.__name__} passed every pin"


# ------------------------------------------------------------- raw decay logits
def test_negative_softplus_closed_forms():
    """Towards-AI article, "Kimi Delta Attention (KDA)": decay logits map to log-decays by
    negative softplus.  Pinned by closed forms, not by re-evaluating the same formula."""
    f = oracle.log_decay_from_logits
    assert f(0.0) == pytest.approx(-np.log(2.0), abs=1e-16)
    # softplus(log(e - 1)) = log(e) = 1
    assert f(np.log(np.e - 1.0)) == pytest.approx(-1.0, abs=1e-15)
    # softplus(log(3)) = log(4)
    assert f(np.log(3.0)) == pytest.approx(-2.0 * np.log(2.0), abs=1e-15)
    # tails: softplus(a) = a + e^-a + O(e^-2a) for large a, e^a - e^2a/2 for very negative a
    assert f(40.0) == pytest.approx(-(40.0 + np.exp(-40.0)), rel=1e-15)
    assert f(-40.0) == pytest.approx(-np.exp(-40.0), rel=1e-12)
    assert np.isnan(f(np.nan)) and f(np.inf) == -np.inf and f(-np.inf) == 0.0
    # the derivative of softplus is the logistic function
    a, h = np.linspace(-8.0, 8.0, 33), 1e-6
    assert np.allclose((f(a - h) - f(a + h)) / (2 * h), 1.0 / (1.0 + np.exp(-a)), atol=1e-8)
    # strictly decreasing and below zero; the -5 floor is reached at a = log(e^5 - 1)
    g = f(np.linspace(-20.0, 20.0, 401))
    assert np.all(np.diff(g) < 0) and np.all(g < 0)
    assert oracle.clamp_log_decay(f(np.log(np.expm1(5.0)))) == pytest.approx(-5.0, abs=1e-14)
