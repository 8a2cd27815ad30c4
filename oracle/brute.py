"""Pure-Python brute force of the sparse MoE forward pass, for tiny inputs.

TEST INFRASTRUCTURE ONLY.  A second spelling of the definition with explicit
index loops (no numpy linear algebra, no sorting library): it pins the numpy
oracle in ``moe_oracle`` on tiny shapes.  It also counts the multiplies the
experts perform, so that "only the k selected experts run" is checked by
counting, against the figures the pages print for the 64->256->64 toy
[NNV-15 §Mixture-of-experts routing, live (FLOPs readout)].

Conventions follow the pages [LLM-T11 §The mathematics, numpy forward pass]:
x is [T][d], W_r is [E][d], W1/W3 are [E][d_ff][d], W2 is [E][d][d_ff];
expert e computes W2[e] . act(W1[e] . x).
"""

from __future__ import annotations

import math


class MulCounter:
    def __init__(self):
        self.n = 0


def _dot(a, b, counter=None):
    acc = 0.0
    for i in range(len(a)):
        acc += a[i] * b[i]
    if counter is not None:
        counter.n += len(a)
    return acc


def _sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def _act(z, act):
    if act == "relu":
        return z if z > 0.0 else 0.0
    if act == "gelu":
        return 0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0)))
    raise ValueError(act)


def expert(xv, w1e, w2e, w3e, act, counter=None):
    """One expert on one token: explicit sums over the pages' weight layout."""
    d_ff = len(w1e)
    h = []
    for f in range(d_ff):
        z = _dot(w1e[f], xv, counter)
        if act == "swiglu":
            u = _dot(w3e[f], xv, counter)
            h.append(z * _sig(z) * u)
        else:
            h.append(_act(z, act))
    return [_dot(w2e[i], h, counter) for i in range(len(w2e))]


def topk_by_selection(q, k):
    """k rounds of 'take the largest remaining key, lower index on ties'."""
    taken = []
    for _ in range(k):
        best = None
        for e in range(len(q)):
            if e in taken:
                continue
            if best is None or q[e] > q[best]:
                best = e
        taken.append(best)
    return taken


def forward(x, w_r, w1, w2, w3=None, *, k, act, gating="softmax_topk",
            capacity_factor=0.0, capacity_priority="token", logit_offset=None, select_bias=None,
            shared=None, counter=None):
    """Returns (y, topk_idx, gates, kept) as nested Python lists."""
    T, E = len(x), len(w_r)
    idx_all, g_all = [], []
    for t in range(T):
        s = [_dot(w_r[e], x[t]) + (logit_offset[e] if logit_offset else 0.0)
             for e in range(E)]
        a = [_sig(v) for v in s] if gating == "sigmoid_topk" else list(s)
        q = [a[e] + (select_bias[e] if select_bias else 0.0) for e in range(E)]
        sel = topk_by_selection(q, k)
        if gating == "softmax_topk":
            m = max(s[e] for e in sel)
            w = [math.exp(s[e] - m) for e in sel]
            z = sum(w)
            g = [v / z for v in w]
        elif gating == "sigmoid_topk":
            w = [_sig(s[e]) for e in sel]
            z = sum(w)
            g = [v / z for v in w]
        else:  # softmax_full
            m = max(s)
            z = sum(math.exp(v - m) for v in s)
            g = [math.exp(s[e] - m) / z for e in sel]
        idx_all.append(sel)
        g_all.append(g)
    # capacity: the first C slots per expert are kept, visiting the slots
    # token by token, or (slot-major priority) every token's first choice,
    # then every token's second choice, ...
    cap = None
    if capacity_factor > 0.0:
        cap = math.floor(capacity_factor * k * T / E)
    seen = [0] * E
    kept = [[False] * k for _ in range(T)]
    if capacity_priority == "slot":
        visits = [(t, j) for j in range(k) for t in range(T)]
    else:
        visits = [(t, j) for t in range(T) for j in range(k)]
    for t, j in visits:
        e = idx_all[t][j]
        kept[t][j] = cap is None or seen[e] < cap
        seen[e] += 1
    d = len(x[0])
    y = []
    for t in range(T):
        out = [0.0] * d
        for j in range(k):
            if not kept[t][j]:
                continue
            e = idx_all[t][j]
            o = expert(x[t], w1[e], w2[e], None if w3 is None else w3[e], act, counter)
            for i in range(d):
                out[i] += g_all[t][j] * o[i]
        if shared is not None:
            ws1, ws3, ws2 = shared
            for si in range(len(ws1)):
                o = expert(x[t], ws1[si], ws2[si], ws3[si], "swiglu", counter)
                for i in range(d):
                    out[i] += o[i]
        y.append(out)
    return y, idx_all, g_all, kept


def routing_stats(logits, counts, k, num_dropped, alpha, bias, gamma):
    """Balance signals with explicit loops [ITM-14 §Auxiliary loss;
    ITM-14 §Auxiliary-loss-free balancing; LLM-T11 Exercise 4]: f_i = count_i
    / T, P_i = average over tokens of exp(s_ti) / sum_j exp(s_tj), loss =
    alpha * E * sum f_i P_i, drop rate = dropped / (T k), and the bias moved
    by gamma against the load's side of the mean T k / E."""
    T = len(logits)
    E = len(logits[0])
    f = [counts[i] / T for i in range(E)]
    P = [0.0] * E
    for t in range(T):
        m = max(logits[t])
        den = 0.0
        for j in range(E):
            den += math.exp(logits[t][j] - m)
        for i in range(E):
            P[i] += math.exp(logits[t][i] - m) / den / T
    loss = 0.0
    for i in range(E):
        loss += f[i] * P[i]
    loss *= alpha * E
    new_bias = None
    if bias is not None:
        new_bias = []
        for i in range(E):
            if counts[i] * E > T * k:
                new_bias.append(bias[i] - gamma)
            elif counts[i] * E < T * k:
                new_bias.append(bias[i] + gamma)
            else:
                new_bias.append(bias[i])
    return f, P, loss, num_dropped / (T * k), new_bias
