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
    P.test_balance_loss_is_alpha_at_uniform_routing()
    P.test_balance_loss_is_alpha_n_at_collapse()
    P.test_balance_loss_lower_for_balanced_than_collapsed_routing()
    P.test_routing_stats_invariants_and_brute_force()
    P.test_bias_update_hand_worked()
    P.test_slot_priority_matches_brute_force()
    P.test_slot_priority_hand_worked()
    P.test_slot_priority_invariants()


_orig = {n: getattr(O, n) for n in (
    "sigmoid", "ordered_topk", "gate_values", "capacity", "permute",
    "expert_ffn", "combine", "router_logits", "selection_keys", "gelu",
    "routing_stats", "softmax_probs", "priority_order")}


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


def m_stats_no_n(logits, counts, **kw):
    r = _orig["routing_stats"](logits, counts, **kw)
    r["loss"] /= np.asarray(logits).shape[1]
    return r


def m_stats_bias_sign(logits, counts, **kw):
    kw = dict(kw)
    kw["gamma"] = -kw.get("gamma", 0.0)
    return _orig["routing_stats"](logits, counts, **kw)


def m_stats_bias_ge(logits, counts, **kw):
    # "at or above the mean" counted as overloaded
    r = _orig["routing_stats"](logits, counts, **kw)
    if r["bias"] is not None:
        T, E = np.asarray(logits).shape
        at = np.asarray(counts) * E == T * kw.get("k", 1)
        r["bias"] = np.where(at, r["bias"] - kw.get("gamma", 0.0), r["bias"])
    return r


def m_stats_f_over_assignments(logits, counts, **kw):
    r = _orig["routing_stats"](logits, counts, **kw)
    k = kw.get("k", 1)
    r["f"] = r["f"] / k
    r["loss"] = r["loss"] / k
    return r


def m_stats_drop_rate_over_tokens(logits, counts, **kw):
    r = _orig["routing_stats"](logits, counts, **kw)
    r["drop_rate"] = r["drop_rate"] * kw.get("k", 1)
    return r


def m_probs_kept_only(s):
    # probabilities of the top-2 experts only, renormalised (the gates, not
    # the router's full distribution)
    s = np.asarray(s, dtype=np.float64)
    keep = np.zeros_like(s, dtype=bool)
    top = np.argsort(-s, axis=-1, kind="stable")[:, :2]
    np.put_along_axis(keep, top, True, axis=-1)
    z = np.where(keep, np.exp(s - s.max(axis=-1, keepdims=True)), 0.0)
    return z / z.sum(axis=-1, keepdims=True)


def m_priority_ignored(T, k, priority="token"):
    return _orig["priority_order"](T, k, "token")


def m_priority_slot_tokens_reversed(T, k, priority="token"):
    if priority == "slot":
        return [t * k + j for j in range(k) for t in reversed(range(T))]
    return _orig["priority_order"](T, k, priority)


MUTANTS = {
    "slot_priority_ignored": ("priority_order", m_priority_ignored),
    "slot_priority_tokens_reversed": ("priority_order", m_priority_slot_tokens_reversed),
    "balance_loss_without_n": ("routing_stats", m_stats_no_n),
    "bias_update_sign_flipped": ("routing_stats", m_stats_bias_sign),
    "bias_moves_at_mean_load": ("routing_stats", m_stats_bias_ge),
    "load_fraction_over_assignments": ("routing_stats", m_stats_f_over_assignments),
    "drop_rate_over_tokens": ("routing_stats", m_stats_drop_rate_over_tokens),
    "router_probs_from_kept_experts": ("softmax_probs", m_probs_kept_only),
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
