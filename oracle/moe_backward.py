"""numpy float64 oracle for the backward pass of the sparse MoE layer.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain and slow: each
step below is one function, applying the chain rule to one step of the forward
definition in ``moe_oracle``, in reverse order.  float64 throughout.

What is differentiated.  The layer's output gradient dy = dLoss/dy is given;
the functions return the gradients of L = <dy, y> (plus, optionally, of the
balance loss alpha E sum_i f_i P_i) with respect to x, the router weights W_r,
the expert weights W1, W3, W2 and the shared experts' weights.

Routing is held fixed.  Top-k selection and the capacity cut are discrete:
their derivative is zero almost everywhere, and the gradient reaches the router
only through the soft gate values g that weight the expert outputs
[LLM-T11 §The routing decision, last paragraph; LLM-T11 §Training instability]
and, when the balance loss is added, through the router probabilities P; the
load fractions f are counts and carry no gradient [ITM-14 §Check yourself,
balance-loss question; ITM-14 §Auxiliary loss].

Steps (reverse order of the forward):

 B1 ``combine_backward``  y_t = sum_kept g_tj Expert_{S_tj}(x_t) + shared:
      dg_tj = <dy_t, Expert_{S_tj}(x_t)> for a kept slot, 0 for a dropped one;
      the expert's output gradient on that row is g_tj dy_t; each shared
      expert's output gradient is dy_t  [ITM-14 §The computation;
      ITM-14 §Fine-grained and shared experts]
 B2 ``expert_backward``   chain rule through W2 . act(W1 x) or
      W2 . (silu(W1 x) * (W3 x))  [LLM-T11 §The mathematics;
      LLM-T11 §Modern MoE variants]
 B3 ``gate_backward``     ds = J^T dg with J the Jacobian of the k gates with
      respect to the E scores of the token, for each gating (softmax over the
      k selected scores, renormalised sigmoids, full softmax)
      [LLM-T11 §The routing decision; LLM-T11 §Top-1 vs top-2;
       ITM-14 §The computation]
 B4 ``balance_loss_backward``  d(alpha E sum_i f_i P_i)/ds with f fixed
      [ITM-14 §Auxiliary loss; ITM-14 §Check yourself]
 B5 ``router_backward``   s = W_r x (+ o): dW_r = ds^T x, dx += ds W_r
      [ITM-14 §The computation; LM-33 §The Router]

Readings (restated where they are taken):
 * a slot dropped by the capacity cut contributes nothing to y, so dg = 0 for
   it, but its score still enters the normalisation of the other gates (the
   forward does not renormalise after drops), so it can receive a score
   gradient through them;
 * the selection bias b and the logit offset o receive no gradient: b is moved
   by the loss-free rule, not by the loss [ITM-14 §Auxiliary-loss-free
   balancing], and o is a fixed input of the synthetic workloads;
 * ReLU's derivative at exactly 0 is taken as 0.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np
from scipy.special import erf as _erf

from . import moe_oracle as O


# ----------------------------------------------------------------------------
# B2  one expert
# ----------------------------------------------------------------------------
def gelu_grad(z):
    """d/dz of z Phi(z): Phi(z) + z phi(z), the exact (erf) GeLU."""
    z = np.asarray(z, dtype=np.float64)
    cdf = 0.5 * (1.0 + _erf(z / math.sqrt(2.0)))
    pdf = np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)
    return cdf + z * pdf


def silu_grad(z):
    """d/dz of z sigmoid(z): sigmoid(z) (1 + z (1 - sigmoid(z)))."""
    sg = O.sigmoid(z)
    return sg * (1.0 + np.asarray(z, dtype=np.float64) * (1.0 - sg))


def expert_backward(xr, w1, w2, w3, act, dout):
    """Gradients of sum <dout, Expert(xr)> for one expert on rows xr [n, d].

    Forward (as ``moe_oracle.expert_ffn``): z = xr W1^T, h = act(z) or
    silu(z) * u with u = xr W3^T, out = h W2^T.  Backward, step by step:
      dW2 = dout^T h            dh = dout W2
      relu/gelu: dz = dh * act'(z)
      swiglu:    du = dh * silu(z),  dz = dh * u * silu'(z),  dW3 = du^T xr
      dW1 = dz^T xr             dxr = dz W1 (+ du W3)
    Returns (dxr, dw1, dw2, dw3) with dw3 None unless SwiGLU.
    """
    xr = np.asarray(xr, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    w1 = np.asarray(w1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    z = xr @ w1.T
    du = dw3 = None
    if act == "relu":
        h = np.maximum(z, 0.0)
    elif act == "gelu":
        h = O.gelu(z)
    elif act == "swiglu":
        w3 = np.asarray(w3, dtype=np.float64)
        u = xr @ w3.T
        h = O.silu(z) * u
    else:
        raise ValueError(act)
    dw2 = dout.T @ h
    dh = dout @ w2
    if act == "relu":
        dz = dh * (z > 0.0)
    elif act == "gelu":
        dz = dh * gelu_grad(z)
    else:
        du = dh * O.silu(z)
        dz = dh * u * silu_grad(z)
        dw3 = du.T @ xr
    dw1 = dz.T @ xr
    dxr = dz @ w1
    if du is not None:
        dxr = dxr + du @ w3
    return dxr, dw1, dw2, dw3


# ----------------------------------------------------------------------------
# B1  gate-weighted combination
# ----------------------------------------------------------------------------
def combine_backward(x, topk_idx, gates, kept_mask, w1, w2, w3, act, dy,
                     shared: Optional[Sequence] = None):
    """Backward of ``moe_oracle.combine`` over all tokens.

    For each expert, its kept rows are run forward once to get the expert
    output (needed for dg) and backward once with output gradient g * dy.
    Returns a dict: dgate [T, k] (0 on dropped slots), dx [T, d] (expert and
    shared paths only), dw1/dw2/dw3 [E, ...] (zeros for an expert with no
    kept row), and dws1/dws3/dws2 [S, ...] for the shared experts.
    """
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    idx = np.asarray(topk_idx)
    g = np.asarray(gates, dtype=np.float64)
    km = np.asarray(kept_mask, dtype=bool)
    T, d = x.shape
    k = idx.shape[1]
    E = len(w1)
    dgate = np.zeros((T, k))
    dx = np.zeros_like(x)
    first = np.asarray(w1[0])
    dw1 = np.zeros((E,) + first.shape)
    dw2 = np.zeros((E,) + np.asarray(w2[0]).shape)
    dw3 = np.zeros_like(dw1) if act == "swiglu" else None
    for e in range(E):
        sel_t, sel_j = np.nonzero((idx == e) & km)
        if sel_t.size == 0:
            continue
        xr = x[sel_t]
        we3 = None if w3 is None else w3[e]
        out = O.expert_ffn(xr, w1[e], w2[e], we3, act)
        dgate[sel_t, sel_j] = np.sum(dy[sel_t] * out, axis=1)
        dout = g[sel_t, sel_j][:, None] * dy[sel_t]
        dxr, a1, a2, a3 = expert_backward(xr, w1[e], w2[e], we3, act, dout)
        dx[sel_t] += dxr            # a token names an expert at most once
        dw1[e], dw2[e] = a1, a2
        if dw3 is not None:
            dw3[e] = a3
    out = dict(dgate=dgate, dx=dx, dw1=dw1, dw2=dw2, dw3=dw3,
               dws1=None, dws3=None, dws2=None)
    if shared is not None:
        ws1, ws3, ws2 = shared
        S = len(ws1)
        out["dws1"] = np.zeros((S,) + np.asarray(ws1[0]).shape)
        out["dws3"] = np.zeros_like(out["dws1"])
        out["dws2"] = np.zeros((S,) + np.asarray(ws2[0]).shape)
        for si in range(S):
            dxs, a1, a2, a3 = expert_backward(x, ws1[si], ws2[si], ws3[si], "swiglu", dy)
            dx += dxs
            out["dws1"][si], out["dws2"][si], out["dws3"][si] = a1, a2, a3
    return out


# ----------------------------------------------------------------------------
# B3  gates
# ----------------------------------------------------------------------------
def gate_jacobian(s, topk_idx, gating):
    """J[t, j, e] = d g_tj / d s_te for the k gates of each token.

    softmax_topk: g = softmax(s_S) over the k selected scores, so
        dg_j/ds_{S_l} = g_j (delta_jl - g_l), 0 for unselected experts.
    sigmoid_topk: g_j = sig_j / Z with sig_l = sigmoid(s_{S_l}), Z = sum sig:
        dg_j/ds_{S_l} = (delta_jl - g_j) sig_l (1 - sig_l) / Z.
    softmax_full: g_j = p_{S_j} with p = softmax(s) over all E:
        dg_j/ds_e = p_{S_j} (delta(S_j, e) - p_e).
    """
    s = np.asarray(s, dtype=np.float64)
    idx = np.asarray(topk_idx)
    T, E = s.shape
    k = idx.shape[1]
    g = O.gate_values(s, idx, gating)
    eye = np.eye(k)
    onehot = np.zeros((T, k, E))            # onehot[t, l, e] = [S_tl == e]
    np.put_along_axis(onehot, idx[:, :, None], 1.0, axis=2)
    if gating == "softmax_topk":
        jkk = g[:, :, None] * (eye[None] - g[:, None, :])           # [T, j, l]
        return np.einsum("tjl,tle->tje", jkk, onehot)
    if gating == "sigmoid_topk":
        sig = O.sigmoid(np.take_along_axis(s, idx, axis=-1))
        z = sig.sum(axis=-1)
        jkk = (eye[None] - g[:, :, None]) * (sig * (1.0 - sig))[:, None, :] / z[:, None, None]
        return np.einsum("tjl,tle->tje", jkk, onehot)
    if gating == "softmax_full":
        p = O.softmax_probs(s)
        return g[:, :, None] * (onehot - p[:, None, :])
    raise ValueError(gating)


def gate_backward(s, topk_idx, dgate, gating):
    """ds[t, e] = sum_j dgate[t, j] J[t, j, e]."""
    J = gate_jacobian(s, topk_idx, gating)
    return np.einsum("tje,tj->te", J, np.asarray(dgate, dtype=np.float64))


# ----------------------------------------------------------------------------
# B4  balance loss
# ----------------------------------------------------------------------------
def balance_loss_backward(s, counts, alpha):
    """d/ds of alpha E sum_i f_i P_i with f_i = count_i / T held fixed and
    P_i = (1/T) sum_t p_ti, p_t = softmax(s_t):
        d/ds_te = (alpha E / T) sum_i f_i p_ti (delta_ie - p_te)
                = (alpha E / T) p_te (f_e - sum_i f_i p_ti)."""
    s = np.asarray(s, dtype=np.float64)
    T, E = s.shape
    f = np.asarray(counts, dtype=np.float64) / T
    p = O.softmax_probs(s)
    return (alpha * E / T) * p * (f[None, :] - (p * f[None, :]).sum(axis=1, keepdims=True))


# ----------------------------------------------------------------------------
# B5  router
# ----------------------------------------------------------------------------
def router_backward(x, w_router, ds):
    """s = x W_r^T (+ o): dW_r = ds^T x and the input gradient ds W_r."""
    x = np.asarray(x, dtype=np.float64)
    ds = np.asarray(ds, dtype=np.float64)
    return ds.T @ x, ds @ np.asarray(w_router, dtype=np.float64)


# ----------------------------------------------------------------------------
# The whole backward pass
# ----------------------------------------------------------------------------
def backward(x, w_router, w1, w2, w3, dy, *, s, topk_idx, kept_mask, gating, act,
             shared=None, aux_alpha=0.0, counts=None):
    """B1..B5 for all T tokens given the forward's routing.

    ``s`` are the router scores (with any offset), ``topk_idx`` and
    ``kept_mask`` the selection and capacity decisions of the forward (held
    fixed); the gates are recomputed from s.  With aux_alpha != 0 the balance
    loss is added, f taken from ``counts`` (assignments per expert before
    capacity).  Returns a dict with dx, dw_router, dw1, dw2, dw3, dws1, dws3,
    dws2, dgate [T, k] and ds [T, E].
    """
    s = np.asarray(s, dtype=np.float64)
    g = O.gate_values(s, topk_idx, gating)
    r = combine_backward(x, topk_idx, g, kept_mask, w1, w2, w3, act, dy, shared)
    ds = gate_backward(s, topk_idx, r["dgate"], gating)
    if aux_alpha != 0.0:
        ds = ds + balance_loss_backward(s, counts, aux_alpha)
    dwr, dxr = router_backward(x, w_router, ds)
    r["dx"] = r["dx"] + dxr
    r["dw_router"] = dwr
    r["ds"] = ds
    return r
