"""Pins for the backward oracle (``oracle.moe_backward``), no GPU.

The backward oracle is checked against things other than itself:
* central finite differences of the (separately pinned) forward oracle and
  balance loss, along random directions, for every input and weight;
* torch.autograd (float64, CPU) of an independent torch spelling of the layer
  with the routing held fixed;
* closed forms and invariants: softmax shift invariance (score gradients sum
  to 0 per token), a top-1 gate of 1 has no score gradient, fully dropped
  tokens get no gradient, identical experts make the router gradient vanish,
  uniform load makes the balance-loss gradient vanish, linearity in dy, and a
  two-expert layer worked by hand.
"""

import itertools
import math
import zlib

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import moe_backward as BW
from oracle import moe_oracle as O

ACTS = ("relu", "gelu", "swiglu")
GATINGS = ("softmax_topk", "sigmoid_topk", "softmax_full")


def seed_of(*key):
    """A seed that does not depend on the interpreter's string hashing."""
    return zlib.crc32(repr(key).encode())


def make_layer(rng, T=7, d=6, E=5, d_ff=4, act="swiglu", shared=0, d_ff_s=3):
    p = dict(
        x=rng.standard_normal((T, d)),
        wr=rng.standard_normal((E, d)),
        w1=rng.standard_normal((E, d_ff, d)) / math.sqrt(d),
        w2=rng.standard_normal((E, d, d_ff)) / math.sqrt(d_ff),
        w3=rng.standard_normal((E, d_ff, d)) / math.sqrt(d) if act == "swiglu" else None,
    )
    if shared:
        p["ws1"] = rng.standard_normal((shared, d_ff_s, d)) / math.sqrt(d)
        p["ws3"] = rng.standard_normal((shared, d_ff_s, d)) / math.sqrt(d)
        p["ws2"] = rng.standard_normal((shared, d, d_ff_s)) / math.sqrt(d_ff_s)
    return p


def shared_of(p):
    return (p["ws1"], p["ws3"], p["ws2"]) if "ws1" in p else None


def run_forward(p, *, k, act, gating, rho, off):
    return O.forward(p["x"], p["wr"], p["w1"], p["w2"], p["w3"], k=k, act=act,
                     gating=gating, capacity_factor=rho, logit_offset=off,
                     shared=shared_of(p))


def counts_of(idx, E):
    return np.bincount(np.asarray(idx).ravel(), minlength=E)


def oracle_grads(p, dy, *, k, act, gating, rho, off, alpha):
    f = run_forward(p, k=k, act=act, gating=gating, rho=rho, off=off)
    kept = (f.perm.slot_pos >= 0).reshape(f.topk_idx.shape)
    E = p["wr"].shape[0]
    return f, BW.backward(p["x"], p["wr"], p["w1"], p["w2"], p["w3"], dy, s=f.logits,
                          topk_idx=f.topk_idx, kept_mask=kept, gating=gating, act=act,
                          shared=shared_of(p), aux_alpha=alpha,
                          counts=counts_of(f.topk_idx, E))


GRAD_NAME = dict(x="dx", wr="dw_router", w1="dw1", w2="dw2", w3="dw3",
                 ws1="dws1", ws3="dws3", ws2="dws2")


# --------------------------------------------------------------------------
# finite differences of the forward oracle
# --------------------------------------------------------------------------
FD_COMBOS = list(itertools.product(ACTS, GATINGS, [0.0, 0.6], [False, True]))


@pytest.mark.parametrize("act,gating,rho,extras", FD_COMBOS)
def test_backward_matches_finite_differences(act, gating, rho, extras):
    rng = np.random.default_rng(seed_of("fd", act, gating, rho, extras))
    E = 5
    for k in (1, 2, 3):
        p = make_layer(rng, E=E, act=act, shared=2 if extras else 0)
        off = rng.standard_normal(E) if extras else None
        alpha = 0.7 if extras else 0.0
        dy = rng.standard_normal(p["x"].shape)
        base, g = oracle_grads(p, dy, k=k, act=act, gating=gating, rho=rho, off=off,
                               alpha=alpha)
        counts = counts_of(base.topk_idx, E)

        def relu_on(q):
            return np.einsum("td,efd->tef", q["x"], q["w1"]) > 0.0

        def loss(q):
            f = run_forward(q, k=k, act=act, gating=gating, rho=rho, off=off)
            # neither the routing nor a ReLU's side may move under the perturbation
            assert np.array_equal(f.topk_idx, base.topk_idx)
            assert np.array_equal(f.perm.slot_pos, base.perm.slot_pos)
            assert act != "relu" or np.array_equal(relu_on(q), relu_on(p))
            L = float(np.sum(dy * f.y))
            if alpha:
                L += O.routing_stats(f.logits, counts, k=k, alpha=alpha)["loss"]
            return L

        h = 1e-5
        for name, val in p.items():
            if val is None:
                continue
            v = rng.standard_normal(val.shape)
            qp = dict(p, **{name: val + h * v})
            qm = dict(p, **{name: val - h * v})
            fd = (loss(qp) - loss(qm)) / (2 * h)
            an = float(np.sum(g[GRAD_NAME[name]] * v))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, k, fd, an)


# --------------------------------------------------------------------------
# torch.autograd of an independent torch spelling
# --------------------------------------------------------------------------
def torch_layer(t, idx, kept, *, act, gating, off):
    """The layer in torch float64 with the selection (idx) and the capacity
    decision (kept) given; written with torch's own softmax/sigmoid/gelu/silu."""
    x, wr = t["x"], t["wr"]
    s = x @ wr.T
    if off is not None:
        s = s + torch.as_tensor(off)
    sel = torch.gather(s, 1, idx)
    if gating == "softmax_topk":
        g = torch.softmax(sel, dim=1)
    elif gating == "sigmoid_topk":
        a = torch.sigmoid(sel)
        g = a / a.sum(dim=1, keepdim=True)
    else:
        g = torch.gather(torch.softmax(s, dim=1), 1, idx)
    y = torch.zeros_like(x)
    T, k = idx.shape
    for t_ in range(T):
        for j in range(k):
            if not kept[t_, j]:
                continue
            e = int(idx[t_, j])
            z = t["w1"][e] @ x[t_]
            if act == "relu":
                h = torch.relu(z)
            elif act == "gelu":
                h = F.gelu(z)
            else:
                h = F.silu(z) * (t["w3"][e] @ x[t_])
            y[t_] = y[t_] + g[t_, j] * (t["w2"][e] @ h)
    if "ws1" in t:
        for si in range(t["ws1"].shape[0]):
            h = F.silu(x @ t["ws1"][si].T) * (x @ t["ws3"][si].T)
            y = y + h @ t["ws2"][si].T
    return y, s


@pytest.mark.parametrize("act,gating,extras", list(itertools.product(ACTS, GATINGS, [False, True])))
def test_backward_matches_torch_autograd(act, gating, extras):
    rng = np.random.default_rng(seed_of("ag", act, gating, extras))
    E = 6
    for k, rho in ((1, 0.0), (2, 0.5), (4, 0.0), (E, 1.0)):
        p = make_layer(rng, T=9, E=E, act=act, shared=1 if extras else 0)
        off = rng.standard_normal(E) if extras else None
        alpha = 0.3 if extras else 0.0
        dy = rng.standard_normal(p["x"].shape)
        f, g = oracle_grads(p, dy, k=k, act=act, gating=gating, rho=rho, off=off, alpha=alpha)
        kept = (f.perm.slot_pos >= 0).reshape(f.topk_idx.shape)
        t = {n: torch.tensor(v, requires_grad=True) for n, v in p.items() if v is not None}
        y, s = torch_layer(t, torch.as_tensor(f.topk_idx), kept, act=act, gating=gating, off=off)
        L = (torch.as_tensor(dy) * y).sum()
        if alpha:
            fr = torch.as_tensor(counts_of(f.topk_idx, E), dtype=torch.float64) / s.shape[0]
            P = torch.softmax(s, dim=1).mean(dim=0)
            L = L + alpha * E * (fr * P).sum()
        L.backward()
        for n, tv in t.items():
            ref = tv.grad.numpy()
            got = g[GRAD_NAME[n]]
            assert np.allclose(got, ref, rtol=1e-10, atol=1e-12), (n, k, np.abs(got - ref).max())


# --------------------------------------------------------------------------
# closed forms and invariants
# --------------------------------------------------------------------------
def test_score_gradient_sums_to_zero_for_softmax_gatings():
    rng = np.random.default_rng(11)
    for gating in ("softmax_topk", "softmax_full"):
        for k in (1, 2, 5):
            p = make_layer(rng, T=12, E=7)
            dy = rng.standard_normal(p["x"].shape)
            _, g = oracle_grads(p, dy, k=k, act="swiglu", gating=gating, rho=0.5, off=None,
                                alpha=0.2)
            assert np.allclose(g["ds"].sum(axis=1), 0.0, atol=1e-13)
    # sigmoid gates are not shift invariant: the sums are not all zero
    p = make_layer(rng, T=12, E=7)
    _, g = oracle_grads(p, rng.standard_normal(p["x"].shape), k=2, act="gelu",
                        gating="sigmoid_topk", rho=0.0, off=None, alpha=0.0)
    assert np.abs(g["ds"].sum(axis=1)).max() > 1e-6


@pytest.mark.parametrize("gating", ["softmax_topk", "sigmoid_topk"])
def test_top1_gate_of_one_has_no_score_gradient(gating):
    rng = np.random.default_rng(12)
    p = make_layer(rng, T=10, E=4)
    _, g = oracle_grads(p, rng.standard_normal(p["x"].shape), k=1, act="relu",
                        gating=gating, rho=0.0, off=None, alpha=0.0)
    assert np.all(g["ds"] == 0.0) and np.all(g["dw_router"] == 0.0)
    # the full-softmax top-1 gate is a probability below 1: it has a gradient
    _, g = oracle_grads(p, rng.standard_normal(p["x"].shape), k=1, act="relu",
                        gating="softmax_full", rho=0.0, off=None, alpha=0.0)
    assert np.abs(g["dw_router"]).max() > 1e-6


def test_fully_dropped_token_gets_no_gradient():
    rng = np.random.default_rng(13)
    E, k = 4, 2
    p = make_layer(rng, T=16, E=E, act="gelu")
    p["wr"][0] += 5.0 * p["x"].mean(axis=0)   # crowd expert 0 so capacity bites
    dy = rng.standard_normal(p["x"].shape)
    f, g = oracle_grads(p, dy, k=k, act="gelu", gating="softmax_topk", rho=0.3, off=None,
                        alpha=0.0)
    kept = (f.perm.slot_pos >= 0).reshape(f.topk_idx.shape)
    gone = ~kept.any(axis=1)
    assert gone.any()
    assert np.all(g["dx"][gone] == 0.0) and np.all(g["dgate"][gone] == 0.0)
    assert np.all(g["ds"][gone] == 0.0)
    assert np.all(g["dgate"][~kept] == 0.0)


def test_identical_experts_leave_the_router_without_gradient():
    rng = np.random.default_rng(14)
    E, d, d_ff = 5, 6, 4
    p = make_layer(rng, T=11, d=d, E=E, d_ff=d_ff)
    for n in ("w1", "w2", "w3"):
        p[n] = np.broadcast_to(p[n][:1], p[n].shape).copy()
    dy = rng.standard_normal(p["x"].shape)
    for gating in ("softmax_topk", "sigmoid_topk"):
        _, g = oracle_grads(p, dy, k=3, act="swiglu", gating=gating, rho=0.0, off=None,
                            alpha=0.0)
        assert np.abs(g["dw_router"]).max() < 1e-12
        # then the layer is one dense SwiGLU MLP: dx from torch autograd of it
        xt = torch.tensor(p["x"], requires_grad=True)
        w1, w2, w3 = (torch.tensor(p[n][0]) for n in ("w1", "w2", "w3"))
        y = (F.silu(xt @ w1.T) * (xt @ w3.T)) @ w2.T
        (torch.as_tensor(dy) * y).sum().backward()
        assert np.allclose(g["dx"], xt.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_balance_loss_gradient_vanishes_at_uniform_load():
    rng = np.random.default_rng(15)
    s = rng.standard_normal((20, 4))
    assert np.abs(BW.balance_loss_backward(s, [10, 10, 10, 10], 0.5)).max() < 1e-16
    g = BW.balance_loss_backward(s, [25, 5, 5, 5], 0.5)
    # pushing the overloaded expert's score down lowers the loss
    assert np.all(g[:, 0] > 0.0)


def test_gradients_are_linear_in_dy():
    rng = np.random.default_rng(16)
    p = make_layer(rng, T=8, E=5, act="gelu", shared=1)
    a, b = 0.7, -1.9
    dy1, dy2 = rng.standard_normal(p["x"].shape), rng.standard_normal(p["x"].shape)
    kw = dict(k=2, act="gelu", gating="sigmoid_topk", rho=0.6, off=None, alpha=0.0)
    _, g1 = oracle_grads(p, dy1, **kw)
    _, g2 = oracle_grads(p, dy2, **kw)
    _, g3 = oracle_grads(p, a * dy1 + b * dy2, **kw)
    for n in ("dx", "dw_router", "dw1", "dw2", "dws1", "dws3", "dws2", "ds"):
        assert np.allclose(g3[n], a * g1[n] + b * g2[n], rtol=1e-11, atol=1e-12), n
    _, g0 = oracle_grads(p, np.zeros_like(dy1), **kw)
    for n in ("dx", "dw_router", "dw1", "dw2", "dws1"):
        assert np.all(g0[n] == 0.0), n


def test_two_expert_layer_worked_by_hand():
    # d = 1, d_ff = 1, E = k = 2, ReLU, softmax over the two scores.
    # y = g0 a0 + g1 a1 with a_e = v_e relu(u_e x), (g0, g1) = softmax(r0 x, r1 x).
    # dL/ds0 = dy g0 g1 (a0 - a1) = -dL/ds1;  dL/dr_e = x dL/ds_e;
    # dL/du_e = dy g_e v_e x [u_e x > 0];  dL/dv_e = dy g_e relu(u_e x).
    x, dy = 1.5, 0.8
    r = np.array([0.4, -0.2])
    u = np.array([2.0, -1.0])
    v = np.array([0.5, 3.0])
    s = r * x
    g0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
    g1 = 1.0 - g0
    a = v * np.maximum(u * x, 0.0)            # a1 = 0 (ReLU off)
    ds0 = dy * g0 * g1 * (a[0] - a[1])
    out = BW.backward(np.array([[x]]), r[:, None], u[:, None, None], v[:, None, None], None,
                      np.array([[dy]]), s=s[None, :], topk_idx=np.array([[0, 1]]),
                      kept_mask=np.array([[True, True]]), gating="softmax_topk", act="relu")
    assert np.allclose(out["ds"], [[ds0, -ds0]], rtol=1e-14)
    assert np.allclose(out["dw_router"][:, 0], [x * ds0, -x * ds0], rtol=1e-14)
    assert np.allclose(out["dw1"][:, 0, 0], [dy * g0 * v[0] * x, 0.0], rtol=1e-14)
    assert np.allclose(out["dw2"][:, 0, 0], [dy * g0 * u[0] * x, 0.0], rtol=1e-14)
    dx = dy * g0 * v[0] * u[0] + (ds0 * r[0] - ds0 * r[1])
    assert np.allclose(out["dx"], [[dx]], rtol=1e-14)
