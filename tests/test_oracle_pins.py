"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself:
* a pure-Python brute force with explicit index loops (tiny shapes);
* torch float64 library routines where the layer reduces to them (a dense
  MLP when E = 1, k = 1; the full softmax mixture when k = E);
* closed forms and invariants the pages state (gates sum to 1, top-1 gate is
  1, a token gets k distinct experts, drop count, bijection, monotone drops);
* numbers the pages print (tests/golden/page_numbers.json).
"""

import itertools
import json
import math
import os
import zlib

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import softmax as sp_softmax

from oracle import accounting, brute
from oracle import moe_oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


def rand_layer(rng, T, d, E, d_ff, act, shared=0, d_ff_s=4):
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d)) / math.sqrt(d)
    w1 = rng.standard_normal((E, d_ff, d)) / math.sqrt(d)
    w3 = rng.standard_normal((E, d_ff, d)) / math.sqrt(d) if act == "swiglu" else None
    w2 = rng.standard_normal((E, d, d_ff)) / math.sqrt(d_ff)
    sh = None
    if shared:
        sh = (rng.standard_normal((shared, d_ff_s, d)) / math.sqrt(d),
              rng.standard_normal((shared, d_ff_s, d)) / math.sqrt(d),
              rng.standard_normal((shared, d, d_ff_s)) / math.sqrt(d_ff_s))
    return x, wr, w1, w2, w3, sh


def tolist(a):
    return None if a is None else np.asarray(a).tolist()


# --------------------------------------------------------------------------
# brute force vs oracle on tiny shapes, every combination of options
# --------------------------------------------------------------------------
COMBOS = list(itertools.product(
    ["relu", "gelu", "swiglu"],
    ["softmax_topk", "sigmoid_topk", "softmax_full"],
    [0.0, 0.5, 1.0],          # capacity factor
    [False, True],            # offset / bias / shared on
))


@pytest.mark.parametrize("act,gating,rho,extras", COMBOS)
def test_oracle_matches_brute_force(act, gating, rho, extras):
    rng = np.random.default_rng(zlib.crc32(repr((act, gating, rho, extras)).encode()))
    T, d, E, d_ff = 9, 6, 5, 7
    for k in (1, 2, E):
        x, wr, w1, w2, w3, sh = rand_layer(rng, T, d, E, d_ff, act,
                                           shared=2 if extras else 0)
        off = rng.standard_normal(E) if extras else None
        bias = 0.3 * rng.standard_normal(E) if extras else None
        ref = O.forward(x, wr, w1, w2, w3, k=k, act=act, gating=gating,
                        capacity_factor=rho, logit_offset=off, select_bias=bias,
                        shared=sh)
        y, idx, g, kept = brute.forward(
            tolist(x), tolist(wr), tolist(w1), tolist(w2), tolist(w3), k=k,
            act=act, gating=gating, capacity_factor=rho, logit_offset=tolist(off),
            select_bias=tolist(bias),
            shared=None if sh is None else tuple(tolist(a) for a in sh))
        assert (ref.topk_idx == np.array(idx)).all()
        np.testing.assert_allclose(ref.gates, np.array(g), rtol=0, atol=1e-13)
        assert ((ref.perm.slot_pos.reshape(T, k) >= 0) == np.array(kept)).all()
        np.testing.assert_allclose(ref.y, np.array(y), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# special cases that reduce to library routines
# --------------------------------------------------------------------------
@pytest.mark.parametrize("act", ["relu", "gelu", "swiglu"])
def test_single_expert_is_dense_mlp(act):
    """E = 1, k = 1: the MoE layer is the dense FFN it replaces [LLM-T11 §The
    mathematics; LLM-T11 calculator with num_experts=1, k=1]."""
    rng = np.random.default_rng(1)
    T, d, d_ff = 11, 8, 12
    x, wr, w1, w2, w3, _ = rand_layer(rng, T, d, 1, d_ff, act)
    ref = O.forward(x, wr, w1, w2, w3, k=1, act=act)
    xt = torch.from_numpy(x)
    z = F.linear(xt, torch.from_numpy(w1[0]))
    if act == "relu":
        h = F.relu(z)
    elif act == "gelu":
        h = F.gelu(z, approximate="none")
    else:
        h = F.silu(z) * F.linear(xt, torch.from_numpy(w3[0]))
    y = F.linear(h, torch.from_numpy(w2[0])).numpy()
    assert (ref.gates == 1.0).all()
    np.testing.assert_allclose(ref.y, y, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("act", ["relu", "swiglu"])
def test_k_equals_E_is_full_softmax_mixture(act):
    """k = E with softmax over the kept scores is the dense softmax mixture."""
    rng = np.random.default_rng(2)
    T, d, E, d_ff = 10, 6, 4, 5
    x, wr, w1, w2, w3, _ = rand_layer(rng, T, d, E, d_ff, act)
    ref = O.forward(x, wr, w1, w2, w3, k=E, act=act)
    p = sp_softmax(x @ wr.T, axis=-1)
    y = np.zeros((T, d))
    xt = torch.from_numpy(x)
    for e in range(E):
        z = F.linear(xt, torch.from_numpy(w1[e]))
        h = F.relu(z) if act == "relu" else F.silu(z) * F.linear(xt, torch.from_numpy(w3[e]))
        y += p[:, e:e + 1] * F.linear(h, torch.from_numpy(w2[e])).numpy()
    np.testing.assert_allclose(ref.y, y, rtol=1e-12, atol=1e-13)
    # the slot order is the descending-score order
    np.testing.assert_allclose(np.take_along_axis(p, ref.topk_idx, -1), ref.gates, atol=1e-14)
    assert (np.diff(np.take_along_axis(x @ wr.T, ref.topk_idx, -1), axis=-1) <= 0).all()


def test_topk_equals_torch_topk_for_distinct_scores():
    rng = np.random.default_rng(3)
    s = rng.standard_normal((200, 37))
    for k in (1, 2, 8, 37):
        ref = O.ordered_topk(s, k)
        tv, ti = torch.topk(torch.from_numpy(s), k, dim=-1, largest=True, sorted=True)
        assert (ref == ti.numpy()).all()


def test_topk_tie_break_lower_index_and_signed_zero():
    q = np.array([[1.0, 3.0, 3.0, 2.0, 3.0],
                  [0.0, -0.0, 0.0, -1.0, -0.0],
                  [-0.0, 0.0, -2.0, -2.0, -3.0]])
    assert O.ordered_topk(q, 3).tolist() == [[1, 2, 4], [0, 1, 2], [0, 1, 2]]
    assert O.ordered_topk(q, 5)[2].tolist() == [0, 1, 2, 3, 4]
    b = brute.topk_by_selection(q[0].tolist(), 3)
    assert b == [1, 2, 4]


def test_softmax_full_gate_is_full_softmax_probability():
    rng = np.random.default_rng(4)
    s = rng.standard_normal((50, 8)) * 2
    idx = O.ordered_topk(s, 1)
    g = O.gate_values(s, idx, "softmax_full")
    p = sp_softmax(s, axis=-1)
    np.testing.assert_allclose(g[:, 0], p.max(axis=-1), rtol=1e-14)


# --------------------------------------------------------------------------
# closed forms and invariants stated on the pages
# --------------------------------------------------------------------------
def test_gates_sum_to_one_and_top1_gate_is_one():
    """Gates over the kept experts form a distribution [LLM-T11 §The routing
    decision; LLM-T11 Exercise 1]; with one kept expert the gate is 1."""
    rng = np.random.default_rng(5)
    s = rng.standard_normal((300, 16)) * 3
    for gating in ("softmax_topk", "sigmoid_topk"):
        for k in (1, 2, 4, 16):
            idx = O.ordered_topk(O.selection_keys(s, gating), k)
            g = O.gate_values(s, idx, gating)
            np.testing.assert_allclose(g.sum(-1), 1.0, atol=1e-14)
            assert (g > 0).all()
            if k == 1:
                assert (g == 1.0).all()
            # every token lands on exactly k distinct experts
            assert all(len(set(r)) == k for r in idx.tolist())


def test_selection_bias_changes_choice_not_gates():
    """The balancing bias takes part in choosing experts only; the gates use
    the original affinity [ITM-14 §Auxiliary-loss-free balancing; §Check
    yourself]."""
    s = np.array([[2.0, 1.0, 0.0, -1.0]])
    b = np.array([0.0, 0.0, 0.0, 5.0])           # forces expert 3 in
    q = O.selection_keys(s, "sigmoid_topk", b)
    idx = O.ordered_topk(q, 2)
    assert idx.tolist() == [[3, 0]]
    g = O.gate_values(s, idx, "sigmoid_topk")
    sig = lambda v: 1 / (1 + math.exp(-v))
    exp = [sig(-1.0) / (sig(-1.0) + sig(2.0)), sig(2.0) / (sig(-1.0) + sig(2.0))]
    np.testing.assert_allclose(g[0], exp, rtol=1e-15)
    # without bias: experts 0, 1
    assert O.ordered_topk(O.selection_keys(s, "sigmoid_topk"), 2).tolist() == [[0, 1]]


def test_hand_worked_two_expert_layer():
    """A layer small enough to evaluate by hand (d = 2, d_ff = 3, E = 2, k = 1,
    ReLU).  x = (1, 2).  W_r = [[1, 0], [0, 1]] -> s = (1, 2) -> expert 1, g = 1.
    W1[1] = [[1, 0], [0, 1], [1, -1]] -> W1 x = (1, 2, -1) -> relu (1, 2, 0).
    W2[1] = [[1, 1, 1], [2, 0, 5]] -> y = (3, 2).  Transposing either weight
    matrix breaks the shapes or the result."""
    x = np.array([[1.0, 2.0]])
    wr = np.array([[1.0, 0.0], [0.0, 1.0]])
    w1 = np.zeros((2, 3, 2)); w2 = np.zeros((2, 2, 3))
    w1[1] = [[1, 0], [0, 1], [1, -1]]
    w2[1] = [[1, 1, 1], [2, 0, 5]]
    r = O.forward(x, wr, w1, w2, None, k=1, act="relu")
    assert r.topk_idx.tolist() == [[1]]
    assert r.y.tolist() == [[3.0, 2.0]]
    # same layer with top-2 softmax: gates e^1/(e^1+e^2), e^2/(e^1+e^2);
    # expert 0 has zero weights so y = g_1 * (3, 2)
    r2 = O.forward(x, wr, w1, w2, None, k=2, act="relu")
    g1 = math.exp(2) / (math.exp(1) + math.exp(2))
    assert r2.topk_idx.tolist() == [[1, 0]]
    np.testing.assert_allclose(r2.y, [[3 * g1, 2 * g1]], rtol=1e-15)


def test_hand_worked_swiglu_and_gelu():
    """SwiGLU: W2 (silu(W1 x) * W3 x); GeLU: W2 gelu(W1 x) (erf form)."""
    x = np.array([[1.0, -1.0]])
    w1 = np.array([[[1.0, 0.0]]])   # z = 1
    w3 = np.array([[[0.0, -2.0]]])  # u = 2
    w2 = np.array([[[1.0], [-1.0]]])
    r = O.expert_ffn(x, w1[0], w2[0], w3[0], "swiglu")
    silu1 = 1.0 / (1.0 + math.exp(-1.0))
    np.testing.assert_allclose(r, [[2 * silu1, -2 * silu1]], rtol=1e-15)
    r = O.expert_ffn(x, w1[0], w2[0], None, "gelu")
    g = 0.5 * (1 + math.erf(1 / math.sqrt(2)))
    np.testing.assert_allclose(r, [[g, -g]], rtol=1e-15)
    assert abs(F.gelu(torch.tensor(1.0, dtype=torch.float64)).item() - g) < 1e-15


@pytest.mark.parametrize("act", ["relu", "swiglu"])
def test_identical_experts_make_routing_irrelevant(act):
    """If every expert has the same weights and nothing is dropped, the gates
    sum to 1 so y = Expert(x) whatever the router does."""
    rng = np.random.default_rng(6)
    T, d, E, d_ff = 20, 6, 6, 9
    x, wr, w1, w2, w3, _ = rand_layer(rng, T, d, E, d_ff, act)
    w1[:] = w1[0]; w2[:] = w2[0]
    if w3 is not None:
        w3[:] = w3[0]
    dense = O.expert_ffn(x, w1[0], w2[0], None if w3 is None else w3[0], act)
    for gating in ("softmax_topk", "sigmoid_topk"):
        for k in (1, 3, 6):
            r = O.forward(x, wr, w1, w2, w3, k=k, act=act, gating=gating,
                          select_bias=rng.standard_normal(E))
            np.testing.assert_allclose(r.y, dense, rtol=1e-12, atol=1e-13)


def test_shared_expert_added_with_weight_one():
    rng = np.random.default_rng(7)
    T, d, E, d_ff = 12, 6, 4, 5
    x, wr, w1, w2, w3, sh = rand_layer(rng, T, d, E, d_ff, "swiglu", shared=2, d_ff_s=3)
    a = O.forward(x, wr, w1, w2, w3, k=2, act="swiglu", shared=sh)
    b = O.forward(x, wr, w1, w2, w3, k=2, act="swiglu")
    xt = torch.from_numpy(x)
    extra = 0
    for s in range(2):
        h = F.silu(F.linear(xt, torch.from_numpy(sh[0][s]))) * F.linear(xt, torch.from_numpy(sh[1][s]))
        extra = extra + F.linear(h, torch.from_numpy(sh[2][s])).numpy()
    np.testing.assert_allclose(a.y - b.y, extra, rtol=1e-11, atol=1e-13)


# --------------------------------------------------------------------------
# capacity and permutation
# --------------------------------------------------------------------------
def test_capacity_formula_values():
    # (T / N) x capacity factor [ITM-14 §Auxiliary loss]; truncated [LLM-T11 Ex. 4]
    assert O.capacity(1.25, 1, 8192, 8) == 1280          # 8192/8 * 1.25
    assert O.capacity(1.0, 1, 100, 3) == 33              # floor(33.33)
    assert O.capacity(2.0, 2, 10, 4) == 10               # k slots per token
    assert O.capacity(0.0, 2, 10, 4) is None
    assert O.capacity(-1.0, 2, 10, 4) is None
    assert O.capacity(1e-9, 1, 10, 4) == 0


def test_drop_count_closed_form_and_monotone():
    """drops = sum_e max(0, count_e - C) [LLM-T11 Exercise 4]; the drop rate
    does not increase with the capacity factor [LLM-T11 §Expert capacity and
    dropped tokens]; rho >= E/k keeps everything."""
    rng = np.random.default_rng(8)
    T, E = 997, 8
    logits = rng.standard_normal((T, E)) + np.linspace(0, 2, E)[None, :]
    idx = O.ordered_topk(logits, 1)
    counts = np.bincount(idx[:, 0], minlength=E)
    last = None
    for rho in np.arange(0.5, 2.01, 0.25):
        C = O.capacity(rho, 1, T, E)
        p = O.permute(idx, E, C)
        assert p.num_dropped == sum(max(0, c - C) for c in counts)
        assert (p.counts == counts).all()
        if last is not None:
            assert p.num_dropped <= last
        last = p.num_dropped
    p = O.permute(idx, E, O.capacity(E / 1, 1, T, E))
    assert p.num_dropped == 0


def test_permutation_is_stable_bijection():
    rng = np.random.default_rng(9)
    T, E, k = 333, 7, 3
    q = rng.standard_normal((T, E))
    idx = O.ordered_topk(q, k)
    for C in (None, 0, 50, 120, 10**6):
        p = O.permute(idx, E, C)
        kept = p.slot_pos >= 0
        n = int(kept.sum())
        assert p.offsets[-1] == n and p.offsets[0] == 0
        assert (np.diff(p.offsets) >= 0).all()
        assert p.counts.sum() == T * k
        assert p.num_dropped == T * k - n
        # bijection between kept slots and rows [0, n)
        assert sorted(p.slot_pos[kept].tolist()) == list(range(n))
        assert (p.perm_src[p.slot_pos[kept]] == np.nonzero(kept)[0]).all()
        assert (p.perm_src[n:] == -1).all()
        # stable: expert ascending, then token ascending
        src = p.perm_src[:n]
        e_of = idx.reshape(-1)[src]
        assert (np.diff(e_of) >= 0).all()
        for e in range(E):
            rows = src[e_of == e]
            assert (np.diff(rows) > 0).all()
            # the kept ones are the earliest tokens
            all_e = np.nonzero(idx.reshape(-1) == e)[0]
            assert rows.tolist() == all_e[:len(rows)].tolist()
        if C == 0:
            assert n == 0


def test_all_dropped_gives_zero_or_shared():
    rng = np.random.default_rng(10)
    T, d, E, d_ff = 8, 4, 4, 5
    x, wr, w1, w2, w3, sh = rand_layer(rng, T, d, E, d_ff, "swiglu", shared=1, d_ff_s=3)
    r = O.forward(x, wr, w1, w2, w3, k=2, act="swiglu", capacity_factor=1e-6)
    assert r.capacity == 0 and (r.y == 0).all() and r.perm.num_dropped == T * 2
    r = O.forward(x, wr, w1, w2, w3, k=2, act="swiglu", capacity_factor=1e-6, shared=sh)
    np.testing.assert_allclose(r.y, O.expert_ffn(x, sh[0][0], sh[2][0], sh[1][0], "swiglu"), rtol=1e-14)


def test_partial_drop_not_renormalised():
    """A token that keeps 1 of its 2 slots gets g_kept * Expert(x), not the
    renormalised Expert(x)."""
    x = np.array([[1.0, 0.0], [1.0, 0.0]])
    wr = np.array([[2.0, 0.0], [1.0, 0.0], [0.0, 0.0]])  # both tokens: experts 0 then 1
    w1 = np.stack([np.eye(2)] * 3); w2 = np.stack([np.eye(2) * (e + 1) for e in range(3)])
    r = O.forward(x, wr, w1, w2, None, k=2, act="relu", capacity_factor=1.5)
    # C = floor(1.5 * 2 * 2 / 3) = 2 -> nothing dropped
    assert r.capacity == 2 and r.perm.num_dropped == 0
    r = O.forward(x, wr, w1, w2, None, k=2, act="relu", capacity_factor=0.75)
    # C = floor(0.75*2*2/3) = 1 -> token 1 loses both slots; token 0 keeps both
    assert r.capacity == 1 and r.perm.num_dropped == 2
    assert (r.y[1] == 0).all()
    g0 = math.exp(2) / (math.exp(2) + math.exp(1))
    np.testing.assert_allclose(r.y[0], [g0 * 1 + (1 - g0) * 2, 0.0], rtol=1e-14)


# --------------------------------------------------------------------------
# routing from float32 scores (the precision the GPU decides in)
# --------------------------------------------------------------------------
def test_route_from_logits_agrees_with_float64_route_except_near_ties():
    rng = np.random.default_rng(11)
    T, d, E = 400, 32, 16
    x = rng.standard_normal((T, d)); wr = rng.standard_normal((E, d)) / math.sqrt(d)
    b = 0.3 * rng.standard_normal(E)
    s64 = O.router_logits(x, wr)
    for gating, bias in (("softmax_topk", None), ("sigmoid_topk", b), ("softmax_full", None)):
        r = O.route_from_logits(s64.astype(np.float32), k=4, gating=gating, select_bias=bias)
        idx64 = O.ordered_topk(O.selection_keys(s64, gating, bias), 4)
        ok = ~r["near_tie"]
        assert (r["topk_idx"][ok] == idx64[ok]).all()
        np.testing.assert_allclose(r["gates"], O.gate_values(s64, r["topk_idx"], gating), atol=1e-6)


def test_near_tie_listing():
    keys = np.array([[1.0, 1.0 + 5e-7, 0.0], [3.0, 2.0, 1.0], [3.0, 2.0, 2.0 - 1e-7]])
    assert O.near_tie_tokens(keys, 1).tolist() == [True, False, False]
    assert O.near_tie_tokens(keys, 2).tolist() == [True, False, True]


# --------------------------------------------------------------------------
# the pages' printed numbers
# --------------------------------------------------------------------------
def test_multiply_counts_match_the_page_by_counting():
    """Run the brute force on the 64->256->64 toy shape with 8 experts and
    count the multiplies the experts actually perform."""
    rng = np.random.default_rng(12)
    d, d_ff, E = 64, 256, 8
    x, wr, w1, w2, _, _ = rand_layer(rng, 1, d, E, d_ff, "relu")
    assert d * d_ff * 2 == GOLD["toy_mlp_weights"]["value"]
    for k, key in ((2, "toy_multiplies_top2"), (8, "toy_multiplies_all_fire")):
        c = brute.MulCounter()
        brute.forward(tolist(x), tolist(wr), tolist(w1), tolist(w2), None, k=k,
                      act="gelu", counter=c)
        assert c.n == GOLD[key]["value"]
        assert accounting.expert_multiplies_per_token(d, d_ff, k, "gelu") == GOLD[key]["value"]


def test_parameter_accounting_matches_the_pages():
    dims = GOLD["mixtral_dims"]["value"]
    d, f, L, E, k = dims["d_model"], dims["d_ffn"], dims["num_layers"], dims["num_experts"], dims["top_k"]
    per_expert_all_layers = L * accounting.expert_params(d, f, "swiglu")
    assert round(per_expert_all_layers / 1e9, 1) == GOLD["mixtral_expert_params_B"]["value"]
    # idle experts per token: (E - k) of them, ~ 5.6B x 6
    idle = (E - k) * per_expert_all_layers
    assert abs(idle / 1e9 - GOLD["mixtral_idle_params_B"]["value"]) / 33.6 < 0.01
    # total - active = (E - k) per-expert FFN sizes, whatever the shared parts
    tot, act = accounting.transformer_params(E, k, d, f, L)
    assert tot - act == idle
    # 16-bit weights of a 46.7B-parameter model ~ 94 GB
    gb = GOLD["mixtral_total_B"]["value"] * 1e9 * 2 / 1e9
    assert abs(gb - GOLD["mixtral_weight_GB_16bit"]["value"]) < 1.0
    assert round(100 * accounting.sparsity(2, 8)) == GOLD["mixtral_sparsity_pct"]["value"]
    assert round(100 * accounting.sparsity(2, 64), 1) == GOLD["top2_of_64_pct"]["value"]
    assert round(100 * 37 / 671, 1) == GOLD["deepseek_v3_active_pct"]["value"]
    # layer-level accounting: total vs active for the toy
    t, a = accounting.moe_layer_params(8, 2, 64, 256, "relu", router=False)
    assert (t, a) == (GOLD["toy_multiplies_all_fire"]["value"], GOLD["toy_multiplies_top2"]["value"])


# ------------------------------------------------------------------ O9 stats
# Balance signals [ITM-14 §Auxiliary loss; LLM-T11 §The auxiliary loss;
# ITM-14 §Auxiliary-loss-free balancing; LLM-T11 Exercise 4].

def test_balance_loss_is_alpha_at_uniform_routing():
    # equal scores and equal loads: f = P = 1/N, so alpha N sum f P = alpha
    # (the factor N makes the minimum 1 whatever N is [ITM-14 §Check yourself])
    for E in (2, 4, 8, 64):
        T = 3 * E
        s = np.full((T, E), 0.25)
        counts = np.full(E, T // E)
        r = O.routing_stats(s, counts, k=1, alpha=0.01)
        assert np.allclose(r["f"], 1.0 / E, rtol=0, atol=1e-15)
        assert np.allclose(r["P"], 1.0 / E, rtol=0, atol=1e-15)
        assert abs(r["loss"] - 0.01) < 1e-15


def test_balance_loss_is_alpha_n_at_collapse():
    # every token to expert 0 with probability 1: f = P = e_0, loss = alpha N
    for E in (2, 8, 128):
        T = 10
        s = np.full((T, E), -60.0)
        s[:, 0] = 60.0
        counts = np.zeros(E, dtype=np.int64)
        counts[0] = T
        r = O.routing_stats(s, counts, k=1, alpha=0.01)
        assert r["P"][0] == 1.0
        assert abs(r["loss"] - 0.01 * E) < 1e-12


def test_balance_loss_lower_for_balanced_than_collapsed_routing():
    # the comparison the pages make [LLM-T11 §The auxiliary loss; LLM-T11
    # Exercise 3]: probabilities drawn from a flat and from a peaked
    # Dirichlet, each token sent to its most probable expert; log-probabilities
    # are scores whose softmax is exactly those probabilities
    rng = np.random.default_rng(0)
    E, T = 4, 100
    out = []
    for conc in ([5.0] * E, [10.0, 0.1, 0.1, 0.1]):
        p = rng.dirichlet(conc, size=T)
        s = np.log(np.maximum(p, 1e-300))
        assign = np.argmax(p, axis=-1)
        counts = np.bincount(assign, minlength=E)
        r = O.routing_stats(s, counts, k=1, alpha=0.01)
        assert np.allclose(r["P"], p.mean(axis=0), rtol=1e-12, atol=1e-15)
        out.append(r["loss"])
    assert out[0] < out[1]


def test_routing_stats_invariants_and_brute_force():
    rng = np.random.default_rng(5)
    for T, E, k in ((1, 3, 1), (5, 4, 2), (9, 6, 3), (12, 5, 5), (7, 8, 2)):
        s = rng.normal(0.0, 2.0, size=(T, E))
        idx = O.ordered_topk(s, k)
        counts = np.bincount(idx.ravel(), minlength=E)
        bias = rng.normal(0.0, 0.1, size=E)
        dropped = int(rng.integers(0, T * k + 1))
        r = O.routing_stats(s, counts, k=k, num_dropped=dropped, alpha=0.02,
                            select_bias=bias, gamma=1e-3)
        assert abs(r["f"].sum() - k) < 1e-12          # each token counted k times
        assert abs(r["P"].sum() - 1.0) < 1e-12        # probabilities
        assert 0.0 <= r["loss"] <= 0.02 * E * k + 1e-12
        f, P, loss, rate, nb = brute.routing_stats(s.tolist(), counts.tolist(), k, dropped,
                                                   0.02, bias.tolist(), 1e-3)
        assert np.allclose(r["f"], f, rtol=0, atol=1e-15)
        assert np.allclose(r["P"], P, rtol=1e-12, atol=1e-15)
        assert abs(r["loss"] - loss) <= 1e-12 * max(1.0, loss)
        assert r["drop_rate"] == rate
        assert np.array_equal(r["bias"], np.array(nb))
        # relabelling the experts permutes f and P and keeps the loss
        perm = rng.permutation(E)
        r2 = O.routing_stats(s[:, perm], counts[perm], k=k, alpha=0.02)
        assert np.allclose(r2["P"], r["P"][perm], rtol=1e-12, atol=1e-15)
        assert abs(r2["loss"] - r["loss"]) <= 1e-12 * max(1.0, r["loss"])


def test_bias_update_hand_worked():
    # T = 6 tokens, k = 2, E = 4: mean load T k / E = 3 assignments per expert;
    # overloaded experts move down by gamma, underloaded up, the one at the
    # mean stays [ITM-14 §Auxiliary-loss-free balancing]
    s = np.zeros((6, 4))
    r = O.routing_stats(s, np.array([5, 3, 1, 3]), k=2, select_bias=np.array([0.5, 0.0, -0.25, 1.0]),
                        gamma=0.125)
    assert r["bias"].tolist() == [0.375, 0.0, -0.125, 1.0]
    # drop rate: 3 of the 12 assignments dropped [LLM-T11 Exercise 4]
    assert O.routing_stats(s, np.array([5, 3, 1, 3]), k=2, num_dropped=3)["drop_rate"] == 0.25


# ------------------------------------------------ slot-major capacity priority
# A NEXT routing variant: every token's first choice claims capacity before
# any second choice (GShard-style priority).  The pages name capacity and
# drops [LLM-T11 §Expert capacity and dropped tokens] but not this order.

def test_slot_priority_matches_brute_force():
    rng = np.random.default_rng(77)
    T, d, E, d_ff = 10, 6, 4, 5
    for k in (2, 3):
        for rho in (0.5, 0.8, 1.0):
            x, wr, w1, w2, w3, sh = rand_layer(rng, T, d, E, d_ff, "relu", shared=0)
            ref = O.forward(x, wr, w1, w2, w3, k=k, act="relu", capacity_factor=rho,
                            capacity_priority="slot")
            y, idx, g, kept = brute.forward(tolist(x), tolist(wr), tolist(w1), tolist(w2),
                                            None, k=k, act="relu", capacity_factor=rho,
                                            capacity_priority="slot")
            assert ((ref.perm.slot_pos.reshape(T, k) >= 0) == np.array(kept)).all()
            np.testing.assert_allclose(ref.y, np.array(y), rtol=0, atol=1e-12)


def test_slot_priority_hand_worked():
    # E = 2, C = 2; token 0 prefers expert 1, tokens 1 and 2 prefer expert 0.
    # Token order keeps (t0: both, t1: both) and drops all of token 2;
    # slot-major keeps every first choice and drops the second choices of
    # tokens 0 and 2.
    idx = np.array([[1, 0], [0, 1], [0, 1]])
    tok = O.permute(idx, 2, 2, "token")
    slot = O.permute(idx, 2, 2, "slot")
    assert (tok.slot_pos.reshape(3, 2) >= 0).tolist() == [[True, True], [True, True], [False, False]]
    assert (slot.slot_pos.reshape(3, 2) >= 0).tolist() == [[True, False], [True, True], [True, False]]
    # same counts and drops, rows of each expert in priority order
    assert tok.counts.tolist() == slot.counts.tolist() == [3, 3]
    assert tok.num_dropped == slot.num_dropped == 2
    assert slot.perm_src.tolist()[:4] == [2, 4, 0, 3]    # e0: t1.j0, t2.j0; e1: t0.j0, t1.j1


def test_slot_priority_invariants():
    rng = np.random.default_rng(3)
    for _ in range(30):
        T, E = int(rng.integers(1, 40)), int(rng.integers(2, 9))
        k = int(rng.integers(1, E + 1))
        idx = O.ordered_topk(rng.normal(size=(T, E)), k)
        C = int(rng.integers(0, T + 1))
        tok, slot = O.permute(idx, E, C, "token"), O.permute(idx, E, C, "slot")
        # kept per expert is min(count, C) either way
        assert (tok.offsets == slot.offsets).all() and tok.num_dropped == slot.num_dropped
        if k == 1:   # one slot per token: the two orders coincide
            assert (tok.slot_pos == slot.slot_pos).all() and (tok.perm_src == slot.perm_src).all()
        # an expert with at most C first choices keeps all of them
        first = np.bincount(idx[:, 0], minlength=E)
        ok = first[idx[:, 0]] <= C
        assert (slot.slot_pos.reshape(T, k)[ok, 0] >= 0).all()
