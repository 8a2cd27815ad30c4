"""Parameter and multiply accounting for MoE layers.

TEST INFRASTRUCTURE ONLY.  These are the bookkeeping identities the pages state
in words and print numbers for; the tests check them against those numbers.

* total vs active parameters: total = E x per-expert FFN size (+ shared parts),
  active = k x per-expert FFN size (+ shared parts)
  [LLM-T11 §Active vs total parameters; ITM-14 §The computation].
* a SwiGLU expert has three d x d_ff matrices (gate W1, up W3, down W2)
  [LLM-T11 §Modern MoE variants, parameter-count listing]; a plain MLP expert
  has two [LLM-T11 §The mathematics].
* per-token expert multiplies scale with k, not E
  [LLM-T11 §The mathematics; NNV-15 §Mixture-of-experts routing, live].
* the transformer parameter calculator of LLM-T11 §Modern MoE variants:
  attention 4 d^2, two LayerNorms 4 d, E experts, router E d, per layer,
  times the layer count; LLM-T11 Exercise 2 adds 2 * vocab * d embeddings.
"""

from __future__ import annotations


def n_matrices(act):
    return 3 if act == "swiglu" else 2


def expert_params(d, d_ff, act="swiglu"):
    """Weights in one expert FFN (no biases)."""
    return n_matrices(act) * d * d_ff


def expert_multiplies_per_token(d, d_ff, k, act="relu", num_shared=0, d_ff_shared=0):
    """Multiplies the experts perform for one token: each of the k selected
    experts multiplies every one of its weights once; shared SwiGLU experts
    run for every token."""
    return k * expert_params(d, d_ff, act) + num_shared * 3 * d * d_ff_shared


def moe_layer_params(E, k, d, d_ff, act="swiglu", num_shared=0, d_ff_shared=0,
                     router=True):
    """(total, active) parameters of one MoE FFN layer (router included)."""
    r = E * d if router else 0
    sh = num_shared * 3 * d * d_ff_shared
    total = E * expert_params(d, d_ff, act) + sh + r
    active = k * expert_params(d, d_ff, act) + sh + r
    return total, active


def transformer_params(num_experts, k, d_model, d_ffn=None, num_layers=32,
                       vocab_size=None):
    """(total, active) for a whole MoE transformer, the way the LLM-T11
    calculator counts: per layer 4 d^2 attention + 4 d LayerNorm + E (or k)
    SwiGLU experts of 3 d d_ffn + E d router; times num_layers; plus
    2 * vocab * d embeddings when vocab_size is given (Exercise 2)."""
    if d_ffn is None:
        d_ffn = 4 * d_model
    attn = 4 * d_model * d_model
    ln = 4 * d_model
    ffn = 3 * d_model * d_ffn
    router = num_experts * d_model
    layer_total = attn + ln + num_experts * ffn + router
    layer_active = attn + ln + k * ffn + router
    total = num_layers * layer_total
    active = num_layers * layer_active
    if vocab_size is not None:
        total += 2 * vocab_size * d_model
        active += 2 * vocab_size * d_model
    return total, active


def sparsity(k, E):
    """Fraction of routed-expert parameters a token touches: k / E."""
    return k / E
