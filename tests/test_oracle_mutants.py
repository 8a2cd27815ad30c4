"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one.  Each mutant replaces one oracle function for the duration of
one test; the battery below must then fail somewhere."""

import math

import numpy as np
import pytest

from oracle import moe_oracle as O
import tests.test_oracle_pins as P


def _battery():
    P.test_oracle_matches_brute_force("swiglu", "softmax_topk", 0.5, True)
    P.test_oracle_matches_brute_force("gelu", "sigmoid_topk", 0.5, True)
    P.test_oracle_matches_brute_force("relu", "softmax_full", 1.0, False)
    P.test_single_expert_is_dense_mlp("gelu")
    P.test_single_expert_is_dense_mlp("swiglu")
    P.test_k_equals_E_is_full_softmax_mixture("relu")
    P.test_topk_tie_break_lower_index_and_signed_zero()
    P.test_topk_equals_torch_topk_for_distinct_scores()
    P.test_gates_sum_to_one_and_top1_gate_is_one()
    P.test_selection_bias_changes_choice_not_gates()
    P.test_hand_worked_two_expert_layer()
    P.test_hand_worked_swiglu_and_gelu()
    P.test_shared_expert_added_with_weight_one()
    P.test_capacity_formula_values()
    P.test_drop_count_closed_form_and_monotone()
    P.test_permutation_is_stable_bijection()
    P.test_partial_drop_not_renormalised()


_orig = {n: getattr(O, n) for n in (
    "sigmoid", "ordered_topk", "gate_values", "capacity", "permute",
    "expert_ffn", "combine", "router_logits", "selection_keys", "gelu")}


def m_sigmoid_sign(z):
    return 1.0 / (1.0 + np.exp(np.asarray(z, dtype=np.float64)))


def m_topk_high_index(q, k):
    T, E = q.shape
    idx = np.broadcast_to(np.arange(E), (T, E))
    return np.lexsort((-idx, -q), axis=-1)[:, :k]


def m_topk_ascending(q, k):
    return _orig["ordered_topk"](-np.asarray(q), k)


def m_gates_full_softmax(s, topk_idx, gating):
    if gating == "softmax_topk":
        return _orig["gate_values"](s, topk_idx, "softmax_full")
    return _orig["gate_values"](s, topk_idx, gating)


def m_gates_from_keys_with_bias(s, topk_idx, gating):
    # gates taken from the biased key instead of the raw affinity
    return _orig["gate_values"](np.asarray(s) + 0.25, topk_idx, "sigmoid_topk") \
        if gating == "sigmoid_topk" else _orig["gate_values"](s, topk_idx, gating)


def m_capacity_ceil(rho, k, T, E):
    if rho <= 0:
        return None
    return int(math.ceil(rho * k * T / E))


def m_permute_keep_last(topk_idx, E, C):
    T, k = topk_idx.shape
    rev = topk_idx[::-1]
    p = _orig["permute"](rev, E, C)
    # map back: slot positions of reversed order
    sp = p.slot_pos.reshape(T, k)[::-1].reshape(-1)
    return O.Permutation(p.counts, p.offsets, p.perm_src, sp, p.num_dropped)


def m_expert_w1_transposed(xr, w1, w2, w3=None, act="swiglu"):
    w1 = np.asarray(w1)
    if w1.shape[0] == w1.shape[1]:
        w1 = w1.T
    else:
        w1 = w1.reshape(w1.shape[1], w1.shape[0]).T.copy()  # garbled layout
    return _orig["expert_ffn"](xr, w1, w2, w3, act)


def m_combine_no_shared(x, topk_idx, gates, kept_mask, w1, w2, w3, act, shared=None, rows=None):
    return _orig["combine"](x, topk_idx, gates, kept_mask, w1, w2, w3, act, None, rows)


def m_combine_renormalise(x, topk_idx, gates, kept_mask, w1, w2, w3, act, shared=None, rows=None):
    g = np.asarray(gates, dtype=np.float64) * np.asarray(kept_mask)
    z = g.sum(-1, keepdims=True)
    g = np.where(z > 0, g / np.where(z > 0, z, 1), 0)
    return _orig["combine"](x, topk_idx, g, kept_mask, w1, w2, w3, act, shared, rows)


def m_router_no_offset(x, w_router, logit_offset=None):
    return _orig["router_logits"](x, w_router, None)


def m_keys_ignore_bias(s, gating, select_bias=None):
    return _orig["selection_keys"](s, gating, None)


def m_gelu_tanh(z):
    return 0.5 * z * (1 + np.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))


MUTANTS = {
    "sigmoid_sign": ("sigmoid", m_sigmoid_sign),
    "topk_ties_to_high_index": ("ordered_topk", m_topk_high_index),
    "topk_smallest": ("ordered_topk", m_topk_ascending),
    "softmax_over_all_experts": ("gate_values", m_gates_full_softmax),
    "gate_uses_biased_affinity": ("gate_values", m_gates_from_keys_with_bias),
    "capacity_ceil": ("capacity", m_capacity_ceil),
    "capacity_keeps_last_tokens": ("permute", m_permute_keep_last),
    "w1_transposed": ("expert_ffn", m_expert_w1_transposed),
    "shared_expert_dropped": ("combine", m_combine_no_shared),
    "partial_drop_renormalised": ("combine", m_combine_renormalise),
    "logit_offset_dropped": ("router_logits", m_router_no_offset),
    "selection_bias_ignored": ("selection_keys", m_keys_ignore_bias),
    "gelu_tanh_form": ("gelu", m_gelu_tanh),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    with pytest.raises(Exception):
        _battery()


def test_battery_passes_unmutated():
    _battery()
