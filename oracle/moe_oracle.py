"""numpy float64 oracle for the sparse MoE layer forward pass.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain, slow and meant to
be checked by eye against the pages: every step is one numbered function below,
written in the order the method computes it, with no fusion, blocking or
reordering.  Floating-point arithmetic is float64 unless a routing decision is
being reproduced at the GPU's precision (``route_from_logits``), where the
pages' own precision rule -- the router runs in FP32 -- decides.

Steps (sources in the package docstring):

 O1 ``router_logits``   s = W_r x (+ optional per-expert logit offset)
      [ITM-14 §The computation, equation block; LLM-T11 §The mathematics;
       LM-33 §The Router (linear layer without bias)]
 O2 ``selection_keys``  affinity a = s (softmax gating) or sigmoid(s)
      (sigmoid gating); selection key q = a + b, with b a selection-only bias
      [ITM-14 §The computation ("renormalized sigmoids");
       ITM-14 §Auxiliary-loss-free balancing; ITM-14 §Check yourself]
 O3 ``ordered_topk``    the k experts with the largest keys, in descending key
      order; equal keys go to the lower expert index
      [LLM-T11 §The routing decision; LLM-T11 Exercise 1; LM-33 §The Router]
 O4 ``gate_values``     softmax over the k kept scores (default), renormalised
      sigmoids over the kept experts, or the full-softmax probability of each
      kept expert (the Switch variant)
      [LLM-T11 §The routing decision; LLM-T11 §Top-1 vs top-2;
       ITM-14 §The computation]
 O5 ``capacity``        C = floor(rho * k * T / E), unlimited when rho <= 0
      [LLM-T11 §Expert capacity and dropped tokens; LLM-T11 Exercise 4;
       ITM-14 §Auxiliary loss]
 O6 ``permute``         per-expert counts, kept = min(count, C), stable order
      (expert ascending, then token ascending -- or, with slot-major
      priority, slot then token), drop mask, drop count
      [LLM-T11 Exercise 4; LM-33 §Simple MoE Layer Implementation]
 O7 ``expert_ffn``      ReLU / GeLU(erf) MLP or SwiGLU gated MLP, no biases
      [LLM-T11 §The mathematics; LLM-T11 §Modern MoE variants (SwiGLU
       parameter count); ITM-14 §The computation ("gated MLP")]
 O8 ``combine``         y_t = sum over kept slots of g * Expert(x_t), plus every
      shared expert with weight 1; dropped slots add 0, gates are not
      renormalised, so a fully dropped token gets y = 0 (its residual carries
      it)  [ITM-14 §The computation; LLM-T11 §Expert capacity and dropped
      tokens; ITM-14 §Fine-grained and shared experts]
 O9 ``routing_stats``   balance signals of a batch: load fractions f, mean
      router probabilities P, the balance loss alpha N sum f P, the drop rate,
      and the loss-free bias update  [ITM-14 §Auxiliary loss;
      LLM-T11 §The auxiliary loss; LLM-T11 Exercise 4;
      ITM-14 §Auxiliary-loss-free balancing]

Readings of points the pages leave open are listed in the repository's design
notes; each is restated at the function that takes it.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np
from scipy.special import erf as _erf

GATINGS = ("softmax_topk", "sigmoid_topk", "softmax_full")
ACTS = ("relu", "gelu", "swiglu")
NEAR_TIE_EPS = 1e-6


# ----------------------------------------------------------------------------
# O1  router scores
# ----------------------------------------------------------------------------
def router_logits(x, w_router, logit_offset=None):
    """s[t, e] = sum_i x[t, i] * W_r[e, i]  (+ o[e]).

    W_r has one row per expert and no bias [ITM-14 §The computation;
    LM-33 §The Router].  The optional offset o is an input of the synthetic
    workloads (skewed routers); it is added to the score and so takes part in
    both selection and gates.  Evaluated in float64 from the exact input values.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_router, dtype=np.float64)
    s = x @ w.T
    if logit_offset is not None:
        s = s + np.asarray(logit_offset, dtype=np.float64)[None, :]
    return s


def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


# ----------------------------------------------------------------------------
# O2  selection keys
# ----------------------------------------------------------------------------
def selection_keys(s, gating, select_bias=None):
    """Key used to choose experts: q = a + b.

    a = s for the softmax gatings, a = sigmoid(s) for sigmoid gating
    [ITM-14 §The computation].  b is the per-expert balancing bias that takes
    part in choosing experts only; the gate values are computed from s alone
    [ITM-14 §Auxiliary-loss-free balancing; ITM-14 §Check yourself].
    Reading: b is added to the affinity that the gate uses (sigmoid(s) under
    sigmoid gating), as the auxiliary-loss-free section describes.
    """
    if gating not in GATINGS:
        raise ValueError(gating)
    s = np.asarray(s, dtype=np.float64)
    a = sigmoid(s) if gating == "sigmoid_topk" else s
    if select_bias is not None:
        a = a + np.asarray(select_bias, dtype=np.float64)[None, :]
    return a


# ----------------------------------------------------------------------------
# O3  ordered top-k
# ----------------------------------------------------------------------------
def ordered_topk(q, k):
    """Indices of the k largest keys per row, largest first.

    [LLM-T11 §The routing decision: pick the indices of the k largest;
    LLM-T11 Exercise 1 sorts descending].  Equal keys go to the lower expert
    index (reading: the pages' sorts leave ties open).  -0.0 and +0.0 are equal.
    Implemented as a full stable sort on (-q, index) -- a library primitive.
    """
    q = np.asarray(q)
    T, E = q.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, -q), axis=-1)  # primary -q, secondary index
    return order[:, :k].astype(np.int64)


# ----------------------------------------------------------------------------
# O4  gate values
# ----------------------------------------------------------------------------
def gate_values(s, topk_idx, gating):
    """Gate g_j for each kept slot j (float64).

    softmax_topk: softmax over the kept scores only, max-subtracted
        [LLM-T11 §The routing decision; LLM-T11 §The mathematics, softmax].
    sigmoid_topk: sigmoid(s_j) / sum over kept of sigmoid(s)
        [ITM-14 §The computation; ITM-14 §Auxiliary-loss-free balancing].
    softmax_full: the full-softmax probability of the kept expert (the Switch
        variant of top-1) [LLM-T11 §Top-1 vs top-2].
    """
    s = np.asarray(s, dtype=np.float64)
    kept = np.take_along_axis(s, topk_idx, axis=-1)
    if gating == "softmax_topk":
        m = kept.max(axis=-1, keepdims=True)
        e = np.exp(kept - m)
        return e / e.sum(axis=-1, keepdims=True)
    if gating == "sigmoid_topk":
        a = sigmoid(kept)
        return a / a.sum(axis=-1, keepdims=True)
    if gating == "softmax_full":
        m = s.max(axis=-1, keepdims=True)
        return np.exp(kept - m) / np.exp(s - m).sum(axis=-1, keepdims=True)
    raise ValueError(gating)


# ----------------------------------------------------------------------------
# O5  capacity
# ----------------------------------------------------------------------------
def capacity(capacity_factor, k, T, E):
    """C = floor(((rho * k) * T) / E) in IEEE double; None = unlimited (rho <= 0).

    The pages: tokens per batch over experts, times the capacity factor
    [ITM-14 §Auxiliary loss], truncated to an integer [LLM-T11 Exercise 4].
    Reading: with k slots per token the fair share is k*T/E; at k = 1 this is
    the pages' formula.  ``capacity_factor`` should be the float32 value the
    library receives (pass ``float(np.float32(rho))``).
    """
    rho = float(capacity_factor)
    if rho <= 0.0:
        return None
    return int(math.floor(((rho * k) * T) / E))


# ----------------------------------------------------------------------------
# O6  permutation
# ----------------------------------------------------------------------------
@dataclass
class Permutation:
    counts: np.ndarray        # [E]   assignments per expert before capacity
    offsets: np.ndarray       # [E+1] exclusive scan of kept counts
    perm_src: np.ndarray      # [T*k] flat slot t*k+j at each permuted row; -1 past the kept rows
    slot_pos: np.ndarray      # [T*k] permuted row of each slot; -1 = dropped
    num_dropped: int


PRIORITIES = ("token", "slot")


def priority_order(T, k, priority="token"):
    """The order in which slots claim expert capacity: token-major (every slot
    of token 0, then of token 1, ...) or slot-major (every token's first
    choice, then every token's second choice, ...; GShard-style priority, a
    NEXT routing variant), as flat slot indices t*k + j."""
    if priority == "slot":
        return [t * k + j for j in range(k) for t in range(T)]
    return list(range(T * k))


def permute(topk_idx, E, C, priority="token"):
    """Group kept slots by expert.

    A slot is kept iff fewer than C slots that come before it in the priority
    order were already sent to the same expert (reading: "the excess is
    dropped" [LLM-T11 §Expert capacity and dropped tokens] keeps the first C;
    the default order is ascending token).  Rows of expert e are its kept
    slots in that same order, and experts follow in ascending order.
    num_dropped = sum_e max(0, count_e - C) [LLM-T11 Exercise 4].
    """
    topk_idx = np.asarray(topk_idx)
    T, k = topk_idx.shape
    flat = topk_idx.reshape(-1)
    counts = np.zeros(E, dtype=np.int64)
    rank = np.zeros(T * k, dtype=np.int64)
    for a in priority_order(T, k, priority):
        e = int(flat[a])
        rank[a] = counts[e]
        counts[e] += 1
    kept = counts.copy() if C is None else np.minimum(counts, C)
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + kept[e]
    slot_pos = np.full(T * k, -1, dtype=np.int64)
    perm_src = np.full(T * k, -1, dtype=np.int64)
    for a in range(T * k):
        e = int(flat[a])
        if rank[a] < kept[e]:
            p = offsets[e] + rank[a]
            slot_pos[a] = p
            perm_src[p] = a
    num_dropped = int((counts - kept).sum())
    return Permutation(counts, offsets, perm_src, slot_pos, num_dropped)


# ----------------------------------------------------------------------------
# O7  experts
# ----------------------------------------------------------------------------
def gelu(z):
    """GeLU, exact erf form 0.5 z (1 + erf(z / sqrt 2)) (reading: the pages say
    only "GeLU" [LLM-T11 §The mathematics])."""
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def silu(z):
    """z * sigmoid(z), the gate nonlinearity of SwiGLU."""
    return z * sigmoid(z)


def expert_ffn(xr, w1, w2, w3=None, act="swiglu"):
    """One expert applied to rows xr [n, d], float64, no biases.

    W1 [d_ff, d] and W2 [d, d_ff] are used as x @ W1^T then @ W2^T, the
    layout of the pages' expert weight arrays [LLM-T11 §The mathematics,
    numpy forward pass].  SwiGLU: W1 is the gate, W3 the up and W2 the down
    projection [LLM-T11 §Modern MoE variants, parameter count]:
    W2 (silu(W1 x) * (W3 x)).  ReLU: W2 max(W1 x, 0).  GeLU: W2 gelu(W1 x).
    """
    xr = np.asarray(xr, dtype=np.float64)
    w1 = np.asarray(w1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    z = xr @ w1.T
    if act == "relu":
        h = np.maximum(z, 0.0)
    elif act == "gelu":
        h = gelu(z)
    elif act == "swiglu":
        u = xr @ np.asarray(w3, dtype=np.float64).T
        h = silu(z) * u
    else:
        raise ValueError(act)
    return h @ w2.T


# ----------------------------------------------------------------------------
# O8  gate-weighted combination
# ----------------------------------------------------------------------------
def combine(x, topk_idx, gates, kept_mask, w1, w2, w3, act,
            shared: Optional[Sequence] = None, rows: Optional[np.ndarray] = None):
    """y_t = sum_{kept j} g_tj Expert_{S_tj}(x_t) + sum_s Shared_s(x_t).

    Loops over experts: each expert runs once on the rows routed to it
    [LM-33 §Simple MoE Layer Implementation]; experts that receive no row are
    never evaluated [LLM-T11 §The routing decision].  Shared experts are SwiGLU,
    run on every token with weight 1 [ITM-14 §Fine-grained and shared experts].
    ``w1``/``w2``/``w3`` and the shared weights are indexed per expert
    (``w1[e]``), so an expert can be materialised in float64 one at a time.
    ``rows`` optionally restricts the output to a subset of tokens.
    """
    x = np.asarray(x, dtype=np.float64)
    if rows is None:
        rows = np.arange(x.shape[0])
    rows = np.asarray(rows)
    xs = x[rows]
    idx = np.asarray(topk_idx)[rows]
    g = np.asarray(gates, dtype=np.float64)[rows]
    km = np.asarray(kept_mask, dtype=bool)[rows]
    y = np.zeros_like(xs)
    experts = np.unique(idx[km]) if km.any() else np.array([], dtype=np.int64)
    for e in experts:
        sel_t, sel_j = np.nonzero((idx == e) & km)
        out = expert_ffn(xs[sel_t], w1[e], w2[e], None if w3 is None else w3[e], act)
        # a token's k slots name distinct experts, so each (t) appears once here
        y[sel_t] += g[sel_t, sel_j][:, None] * out
    if shared is not None:
        ws1, ws3, ws2 = shared
        for si in range(len(ws1)):
            y += expert_ffn(xs, ws1[si], ws2[si], ws3[si], "swiglu")
    return y


# ----------------------------------------------------------------------------
# The whole layer
# ----------------------------------------------------------------------------
@dataclass
class Result:
    logits: np.ndarray
    keys: np.ndarray
    topk_idx: np.ndarray
    gates: np.ndarray
    capacity: Optional[int]
    perm: Permutation
    y: np.ndarray
    extra: dict = field(default_factory=dict)


def forward(x, w_router, w1, w2, w3=None, *, k, act, gating="softmax_topk",
            capacity_factor=0.0, logit_offset=None, select_bias=None,
            shared=None, capacity_priority="token"):
    """The forward pass O1..O8 over all T tokens, float64 throughout."""
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    E = np.asarray(w_router).shape[0]
    s = router_logits(x, w_router, logit_offset)
    q = selection_keys(s, gating, select_bias)
    idx = ordered_topk(q, k)
    g = gate_values(s, idx, gating)
    C = capacity(capacity_factor, k, T, E)
    perm = permute(idx, E, C, capacity_priority)
    kept = (perm.slot_pos >= 0).reshape(T, k)
    y = combine(x, idx, g, kept, w1, w2, w3, act, shared)
    return Result(s, q, idx, g, C, perm, y)


# ----------------------------------------------------------------------------
# Routing from given float32 router scores (the GPU's precision)
# ----------------------------------------------------------------------------
def selection_keys_f32(logits_f32, gating, select_bias=None):
    """O2 evaluated as the FP32 router does it: the affinity is rounded to
    float32 (sigmoid taken in float64, then rounded once), the bias is added in
    float32, and -0.0 becomes +0.0.  The pages require the router math in FP32
    [LLM-T11 §Training instability]."""
    s = np.asarray(logits_f32, dtype=np.float32)
    if gating == "sigmoid_topk":
        a = sigmoid(s.astype(np.float64)).astype(np.float32)
    else:
        a = s.copy()
    if select_bias is not None:
        a = (a + np.asarray(select_bias, dtype=np.float32)[None, :]).astype(np.float32)
    return (a + np.float32(0.0)).astype(np.float32)


def near_tie_tokens(keys, k, eps=NEAR_TIE_EPS):
    """Tokens whose routing is decided by a gap <= eps between adjacent keys
    among their top min(k+1, E) keys.  Such tokens are listed, not failed,
    when routing is compared bit for bit."""
    keys = np.asarray(keys, dtype=np.float64)
    E = keys.shape[1]
    m = min(k + 1, E)
    srt = -np.sort(-keys, axis=-1)[:, :m]
    if m < 2:
        return np.zeros(keys.shape[0], dtype=bool)
    gaps = srt[:, :-1] - srt[:, 1:]
    return (gaps <= eps).any(axis=-1)


def route_from_logits(logits_f32, *, k, gating, capacity_factor=0.0,
                      select_bias=None, capacity_priority="token"):
    """O2..O6 starting from given float32 scores: keys in float32, top-k,
    float64 gates, capacity and permutation.  Returns a dict."""
    s32 = np.asarray(logits_f32, dtype=np.float32)
    T, E = s32.shape
    q = selection_keys_f32(s32, gating, select_bias)
    idx = ordered_topk(q, k)
    g = gate_values(s32.astype(np.float64), idx, gating)
    C = capacity(capacity_factor, k, T, E)
    perm = permute(idx, E, C, capacity_priority)
    return dict(keys=q, topk_idx=idx, gates=g, capacity=C, perm=perm,
                near_tie=near_tie_tokens(q, k))


# ----------------------------------------------------------------------------
# O9  routing statistics and balance signals


def softmax_probs(s):
    """Router probabilities: the softmax over all E scores of each token
    (max subtracted first) [LLM-T11 §The routing decision]."""
    s = np.asarray(s, dtype=np.float64)
    z = np.exp(s - s.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def routing_stats(logits, counts, *, k, num_dropped=0, alpha=0.01,
                  select_bias=None, gamma=0.0):
    """O9 from the scores s [T, E] (with any logit offset, as O1 returns them)
    and the per-expert assignment counts before capacity (O6 ``counts``):

      f_i  = count_i / T       fraction of the batch's tokens sent to expert i
      P_i  = mean_t softmax(s_t)_i   average router probability of expert i
      loss = alpha * E * sum_i f_i P_i          [ITM-14 §Auxiliary loss]
      drop_rate = num_dropped / (T k)           [LLM-T11 Exercise 4]
      bias_i' = bias_i - gamma if count_i > T k / E (overloaded),
                bias_i + gamma if count_i < T k / E (underloaded),
                bias_i          otherwise   [ITM-14 §Auxiliary-loss-free
                balancing]

    Readings: with k > 1 a token counts once for each expert it is sent to,
    so sum f = k and N sum f P is k (not 1) under uniform routing; P is the
    full-softmax probability for every gating; the load that decides the
    bias update is the count before capacity, compared exactly (count_i * E
    against T * k).  Returns a dict."""
    s = np.asarray(logits, dtype=np.float64)
    counts = np.asarray(counts, dtype=np.int64)
    T, E = s.shape
    f = counts.astype(np.float64) / T
    P = softmax_probs(s).mean(axis=0)
    loss = alpha * E * float(np.sum(f * P))
    drop_rate = float(num_dropped) / (T * k)
    bias_new = None
    if select_bias is not None:
        b = np.asarray(select_bias, dtype=np.float64)
        load = counts * E          # compared with T * k: both exact integers
        step = np.where(load > T * k, -gamma, np.where(load < T * k, gamma, 0.0))
        bias_new = b + step
    return dict(f=f, P=P, loss=loss, drop_rate=drop_rate, bias=bias_new)
