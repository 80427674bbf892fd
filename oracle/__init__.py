"""CPU oracle for Kimi Delta Attention (KDA): plain, slow, float64.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the tests, the smoke check of the package entry point and the CPU
baseline leg of the bench use it.  It shares no code with the HIP library.

What it computes (per batch row b and head h, tokens t = 0..T-1):

    g'_t = min(max(g_t, -5), 0)                     (per channel, NaN kept)
    S    <- Diag(exp(g'_t)) S                       (decay each key row)
    w    =  S^T k_t
    S    <- S + beta_t k_t (v_t - w)^T              (delta rule)
    o_t  =  S^T q_t

which is S_t = (I - beta_t k_t k_t^T) Diag(exp g'_t) S_{t-1} + beta_t k_t v_t^T,
o_t = S_t^T q_t.  S is d_k x d_v.  Sources:

* the update family - the delta rule of DeltaNet, the scalar forget gate of
  Gated DeltaNet, and KDA's per-channel (diagonal) gate - is the lineage the
  Towards-AI article on Kimi K3 walks through in "Kimi Delta Attention (KDA)"
  (its formulas did not survive extraction; the form above is the standard
  one for that lineage, decay applied before the delta correction, output
  read from the updated state);
* the floor of -5 on the log-decay, i.e. at least ~0.67% of each channel kept
  per step, is from the orkas.ai "Kimi K3 architecture" blog, section "A lower
  bound that deleted a GPU code path"; the upper clamp at 0 follows from the
  same section describing the decay as a product of factors below one.

Parity pins (tests/test_oracle.py): brute-force products of the dense
per-token transition matrices, the beta = 0 / g = 0 and beta = 1 retrieval
invariants, the beta = 0 closed form, one-hot-key gated EMAs, the segment
composition law of the blog's "The cost is paid in the serving stack"
section, and hand-derived worked examples under tests/golden/.
"""
from .kda import (  # noqa: F401
    log_decay_from_logits,
    LOG_DECAY_FLOOR,
    clamp_log_decay,
    kda_decode_step,
    kda_forward,
    kda_forward_heads_parallel,
    head_pool,
    set_default_pool,
    oracle_processes,
    apply_output_gate,
    rel_l2_groups,
    rel_l2_chunks,
    one_hot_key_rows,
    rel_l2,
)
