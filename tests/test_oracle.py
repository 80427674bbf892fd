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
    # a pool of its own, the session's default pool, and in-process
    for kw in ({"processes": 2}, {}, {"processes": 1}):
        (o, S, ck), n = oracle.kda_forward_heads_parallel(q, k, v, g, beta, s0, 7, **kw)
        assert n == kw.get("processes", n)
        assert np.array_equal(o, ref[0]) and np.array_equal(S, ref[1])
        assert np.array_equal(ck, ref[2])


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


# ------------------------------------------------------------- comparators
# Every parity claim is a value of these functions, so they are pinned by hand values
# and by copies with plausible mistakes planted in them, not by re-evaluating them.


def _rel_no_sqrt(x, ref):
    x, ref = np.asarray(x, float), np.asarray(ref, float)
    return float(np.sum((x - ref) ** 2) / np.sum(ref ** 2))


def _rel_wrong_denominator(x, ref):
    x, ref = np.asarray(x, float), np.asarray(ref, float)
    return float(np.linalg.norm(x - ref) / np.linalg.norm(x))


def _rel_max_abs(x, ref):
    x, ref = np.asarray(x, float), np.asarray(ref, float)
    return float(np.max(np.abs(x - ref)) / np.linalg.norm(ref))


def _rel_l1(x, ref):
    x, ref = np.asarray(x, float), np.asarray(ref, float)
    return float(np.sum(np.abs(x - ref)) / np.sum(np.abs(ref)))


# (x, ref, value worked out by hand)
REL_L2_HAND = [
    # x - ref = [1, 2, -2]: norm 3; ||ref|| = 4
    ([1.0, 2.0, 2.0], [0.0, 0.0, 4.0], 0.75),
    # x - ref = [3, -1]: norm sqrt(10); ||ref|| = 5
    ([3.0, 4.0], [0.0, 5.0], math.sqrt(10.0) / 5.0),
    # equal arrays, in any shape
    ([[1.5, -2.0], [0.25, 8.0]], [[1.5, -2.0], [0.25, 8.0]], 0.0),
    # zero in place of ref: the whole of ref is missing
    ([0.0, 0.0, 0.0, 0.0], [1.0, -1.0, 1.0, -1.0], 1.0),
    # 2x ref: off by ref itself
    ([2.0, -6.0], [1.0, -3.0], 1.0),
    # ref all zeros: the plain norm of x (documented special case)
    ([3.0, 4.0], [0.0, 0.0], 5.0),
]


@pytest.mark.parametrize("x,ref,want", REL_L2_HAND)
def test_rel_l2_hand_values(x, ref, want):
    assert oracle.rel_l2(np.array(x), np.array(ref)) == pytest.approx(want, rel=1e-15, abs=1e-300)


@pytest.mark.parametrize("mistake", [_rel_no_sqrt, _rel_wrong_denominator, _rel_max_abs, _rel_l1],
                         ids=lambda f: f.__name__)
def test_rel_l2_hand_values_reject_planted_mistakes(mistake):
    """Each plausible mistake in the comparator misses at least one hand value."""
    wrong = 0
    for x, ref, want in REL_L2_HAND[:2]:
        with np.errstate(all="ignore"):
            got = mistake(np.array(x), np.array(ref))
        wrong += abs(got - want) > 1e-9
    assert wrong > 0


def test_rel_l2_groups_hand_values():
    # two heads (axis 2) of a [1, 2, 2, 2] output: head 0 exact, head 1 off by [1, 2, -2] / 4
    ref = np.zeros((1, 2, 2, 2))
    ref[0, :, 0] = [[1.0, 2.0], [3.0, 4.0]]
    ref[0, :, 1] = [[0.0, 0.0], [0.0, 4.0]]
    x = ref.copy()
    x[0, :, 1] = [[1.0, 2.0], [0.0, 2.0]]
    per = oracle.rel_l2_groups(x, ref, (0, 2))
    assert per.shape == (1, 2)
    assert per[0, 0] == 0.0 and per[0, 1] == pytest.approx(0.75, rel=1e-15)
    # the whole-tensor value mixes both heads: sqrt(9 / (30 + 16))
    assert oracle.rel_l2(x, ref) == pytest.approx(3.0 / math.sqrt(46.0), rel=1e-15)
    # states [B, H, dk, dv]: one value per (b, h)
    s_ref = np.ones((2, 3, 2, 2))
    s = s_ref.copy()
    s[1, 2, 0, 0] = 3.0  # off by 2 in one of four unit entries: 2 / 2
    per_s = oracle.rel_l2_groups(s, s_ref, (0, 1))
    assert per_s.shape == (2, 3) and per_s[1, 2] == pytest.approx(1.0) and per_s.sum() == per_s[1, 2]


def test_rel_l2_chunks_hand_values():
    # one head, T = 5 tokens, D = 1, chunks of 2: token runs [0, 1], [2, 3], [4]
    ref = np.array([3.0, 4.0, 1.0, 0.0, 2.0]).reshape(1, 5, 1, 1)
    x = np.array([3.0, 4.0, 1.0, 1.0, 1.0]).reshape(1, 5, 1, 1)
    per = oracle.rel_l2_chunks(x, ref, 2)
    assert per.shape == (1, 3, 1)
    assert per[0, 0, 0] == 0.0
    assert per[0, 1, 0] == pytest.approx(1.0)        # |[0, 1]| / |[1, 0]|
    assert per[0, 2, 0] == pytest.approx(0.5)        # the one-token tail: 1 / 2
    # chunks of the whole length reduce to the per-head value
    assert oracle.rel_l2_chunks(x, ref, 5)[0, 0, 0] == pytest.approx(
        oracle.rel_l2_groups(x, ref, (0, 2))[0, 0])


def test_one_wrong_token_head_hides_in_the_whole_tensor_but_not_per_head_or_chunk():
    """Why the parity helpers assert maxima too: at the 4 x 4096 x 32-head size, one
    token-head gone completely wrong moves the whole-tensor error by only about 1.4e-3,
    under the 3e-3 bound; the per-head and per-chunk maxima see it at once."""
    rng = np.random.default_rng(5)
    ref = rng.standard_normal((2, 256, 8, 16))
    x = ref * (1.0 + 1e-4 * rng.standard_normal(ref.shape))
    x[1, 200, 3] = rng.standard_normal(16)  # one token of one head replaced
    assert oracle.rel_l2(x, ref) < 3e-2
    assert oracle.rel_l2_groups(x, ref, (0, 2)).max() > 5e-2
    per_chunk = oracle.rel_l2_chunks(x, ref, 64)
    assert per_chunk.max() > 1e-1 and np.argwhere(per_chunk > 1e-2).tolist() == [[1, 3, 3]]


# ------------------------------------------------------------- output gate


def test_output_gate_closed_forms():
    """o * sigmoid(z): pinned by values of the logistic function that need no evaluation
    of it (z = 0, z = log 3, the tails, the symmetry sigma(z) + sigma(-z) = 1)."""
    f = oracle.apply_output_gate
    o = np.array([2.0, -4.0, 8.0, 1.0])
    assert np.array_equal(f(o, np.zeros(4)), o / 2.0)
    # sigma(log 3) = 3 / 4, sigma(-log 3) = 1 / 4
    assert f(o, np.full(4, np.log(3.0))) == pytest.approx(0.75 * o, rel=1e-15)
    assert f(o, np.full(4, -np.log(3.0))) == pytest.approx(0.25 * o, rel=1e-15)
    # saturation: +inf passes o through, -inf closes the gate; no overflow on the way
    with np.errstate(all="raise"):
        assert np.array_equal(f(o, np.full(4, np.inf)), o)
        assert np.array_equal(f(o, np.full(4, -np.inf)), 0.0 * o)
        assert np.array_equal(f(o, np.full(4, 800.0)), o)
        assert np.all(f(o, np.full(4, -800.0)) == 0.0)
    z = np.linspace(-30.0, 30.0, 121)
    one = np.ones_like(z)
    assert np.allclose(f(one, z) + f(one, -z), 1.0, rtol=0, atol=1e-15)
    # its derivative at 0 is 1/4; monotone; gates each element by its own z
    h = 1e-6
    assert (f(1.0, h) - f(1.0, -h)) / (2 * h) == pytest.approx(0.25, rel=1e-8)
    assert np.all(np.diff(f(one, z)) > 0)
    assert np.array_equal(f(o, np.array([np.inf, -np.inf, 0.0, np.inf])), [2.0, -0.0, 4.0, 1.0])
    assert np.isnan(f(o, np.array([np.nan, 0, 0, 0]))[0])
