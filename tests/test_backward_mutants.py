"""Plant plausible mistakes in the backward oracle (on the CPU) and check that
the pins in test_backward_pins catch every one.  Each mutant replaces one
function of ``oracle.moe_backward`` for the duration of one test."""

import numpy as np
import pytest

from oracle import moe_backward as BW
from oracle import moe_oracle as O
import tests.test_backward_pins as P


def _battery():
    for act in ("relu", "gelu", "swiglu"):
        for gating in ("softmax_topk", "sigmoid_topk", "softmax_full"):
            P.test_backward_matches_torch_autograd(act, gating, True)
    P.test_backward_matches_finite_differences("swiglu", "softmax_topk", 0.6, True)
    P.test_backward_matches_finite_differences("gelu", "sigmoid_topk", 0.6, False)
    P.test_backward_matches_finite_differences("relu", "softmax_full", 0.0, True)
    P.test_score_gradient_sums_to_zero_for_softmax_gatings()
    P.test_top1_gate_of_one_has_no_score_gradient("softmax_topk")
    P.test_top1_gate_of_one_has_no_score_gradient("sigmoid_topk")
    P.test_fully_dropped_token_gets_no_gradient()
    P.test_identical_experts_leave_the_router_without_gradient()
    P.test_balance_loss_gradient_vanishes_at_uniform_load()
    P.test_gradients_are_linear_in_dy()
    P.test_two_expert_layer_worked_by_hand()


_orig = {n: getattr(BW, n) for n in (
    "silu_grad", "gelu_grad", "expert_backward", "combine_backward", "gate_jacobian",
    "gate_backward", "balance_loss_backward", "router_backward")}


def m_silu_grad_sigmoid_only(z):
    return O.sigmoid(z)


def m_gelu_grad_cdf_only(z):
    return _orig["gelu_grad"](z) - np.asarray(z) * np.exp(-0.5 * np.asarray(z) ** 2) / np.sqrt(2 * np.pi)


def m_expert_w1_w3_swapped(xr, w1, w2, w3, act, dout):
    dx, a1, a2, a3 = _orig["expert_backward"](xr, w1, w2, w3, act, dout)
    return (dx, a3, a2, a1) if a3 is not None else (dx, a1, a2, a3)


def m_expert_no_up_path_in_dx(xr, w1, w2, w3, act, dout):
    dx, a1, a2, a3 = _orig["expert_backward"](xr, w1, w2, w3, act, dout)
    if act != "swiglu":
        return dx, a1, a2, a3
    z = np.asarray(xr) @ np.asarray(w1).T
    dh = np.asarray(dout) @ np.asarray(w2)
    du = dh * O.silu(z)
    return dx - du @ np.asarray(w3), a1, a2, a3


def m_expert_dw2_transposed_operands(xr, w1, w2, w3, act, dout):
    dx, a1, a2, a3 = _orig["expert_backward"](xr, w1, w2, w3, act, dout)
    # dW2 from the wrong row of each operand pair: rows reversed
    _, _, b2, _ = _orig["expert_backward"](xr[::-1], w1, w2, w3, act, dout)
    return dx, a1, b2, a3


def m_combine_no_gate_scale(x, topk_idx, gates, kept_mask, w1, w2, w3, act, dy, shared=None):
    ones = np.ones_like(np.asarray(gates, dtype=np.float64))
    r = _orig["combine_backward"](x, topk_idx, ones, kept_mask, w1, w2, w3, act, dy, shared)
    r["dgate"] = _orig["combine_backward"](x, topk_idx, gates, kept_mask, w1, w2, w3, act, dy,
                                           shared)["dgate"]
    return r


def m_combine_dgate_on_dropped(x, topk_idx, gates, kept_mask, w1, w2, w3, act, dy, shared=None):
    r = _orig["combine_backward"](x, topk_idx, gates, kept_mask, w1, w2, w3, act, dy, shared)
    allk = np.ones_like(np.asarray(kept_mask, dtype=bool))
    r["dgate"] = _orig["combine_backward"](x, topk_idx, gates, allk, w1, w2, w3, act, dy,
                                           shared)["dgate"]
    return r


def m_combine_no_shared(x, topk_idx, gates, kept_mask, w1, w2, w3, act, dy, shared=None):
    r = _orig["combine_backward"](x, topk_idx, gates, kept_mask, w1, w2, w3, act, dy, None)
    if shared is not None:
        r["dws1"] = np.zeros_like(np.asarray(shared[0]))
        r["dws3"] = np.zeros_like(np.asarray(shared[1]))
        r["dws2"] = np.zeros_like(np.asarray(shared[2]))
    return r


def m_jacobian_sign(s, topk_idx, gating):
    J = _orig["gate_jacobian"](s, topk_idx, gating)
    return -J if gating == "softmax_topk" else J


def m_jacobian_transposed_kk(s, topk_idx, gating):
    # d g_l / d s_j in place of d g_j / d s_l (differs for sigmoid gates)
    if gating != "sigmoid_topk":
        return _orig["gate_jacobian"](s, topk_idx, gating)
    J = _orig["gate_jacobian"](s, topk_idx, gating)
    idx = np.asarray(topk_idx)
    jkk = np.take_along_axis(J, idx[:, None, :], axis=2)          # [T, j, l]
    out = np.zeros_like(J)
    np.put_along_axis(out, idx[:, None, :].repeat(idx.shape[1], 1),
                      np.swapaxes(jkk, 1, 2), axis=2)
    return out


def m_sigmoid_jacobian_no_derivative(s, topk_idx, gating):
    if gating != "sigmoid_topk":
        return _orig["gate_jacobian"](s, topk_idx, gating)
    s = np.asarray(s, dtype=np.float64)
    idx = np.asarray(topk_idx)
    T, E = s.shape
    k = idx.shape[1]
    g = O.gate_values(s, idx, gating)
    sig = O.sigmoid(np.take_along_axis(s, idx, axis=-1))
    jkk = (np.eye(k)[None] - g[:, :, None]) / sig.sum(axis=-1)[:, None, None]
    onehot = np.zeros((T, k, E))
    np.put_along_axis(onehot, idx[:, :, None], 1.0, axis=2)
    return np.einsum("tjl,tle->tje", jkk, onehot)


def m_full_softmax_kept_only(s, topk_idx, gating):
    if gating != "softmax_full":
        return _orig["gate_jacobian"](s, topk_idx, gating)
    J = _orig["gate_jacobian"](s, topk_idx, gating)
    mask = np.zeros(J.shape[::2][:1] + (J.shape[2],), dtype=bool)
    np.put_along_axis(mask, np.asarray(topk_idx), True, axis=1)
    return J * mask[:, None, :]


def m_gate_backward_ignores_dgate_weights(s, topk_idx, dgate, gating):
    J = BW.gate_jacobian(s, topk_idx, gating)
    return np.einsum("tje,tj->te", J, np.ones_like(np.asarray(dgate)) * np.asarray(dgate).mean())


def m_balance_no_n(s, counts, alpha):
    return _orig["balance_loss_backward"](s, counts, alpha) / np.asarray(s).shape[1]


def m_balance_p_for_f(s, counts, alpha):
    T = np.asarray(s).shape[0]
    fake = O.softmax_probs(s).mean(axis=0) * T
    return _orig["balance_loss_backward"](s, fake, alpha)


def m_balance_sign(s, counts, alpha):
    return -_orig["balance_loss_backward"](s, counts, alpha)


def m_router_no_dx(x, w_router, ds):
    dw, dx = _orig["router_backward"](x, w_router, ds)
    return dw, 0.0 * dx


def m_router_dw_mean(x, w_router, ds):
    dw, dx = _orig["router_backward"](x, w_router, ds)
    return dw / np.asarray(x).shape[0], dx


MUTANTS = {
    "silu_grad_sigmoid_only": ("silu_grad", m_silu_grad_sigmoid_only),
    "gelu_grad_cdf_only": ("gelu_grad", m_gelu_grad_cdf_only),
    "expert_w1_w3_swapped": ("expert_backward", m_expert_w1_w3_swapped),
    "expert_no_up_path_in_dx": ("expert_backward", m_expert_no_up_path_in_dx),
    "expert_dw2_wrong_rows": ("expert_backward", m_expert_dw2_transposed_operands),
    "combine_no_gate_scale": ("combine_backward", m_combine_no_gate_scale),
    "combine_dgate_on_dropped": ("combine_backward", m_combine_dgate_on_dropped),
    "combine_no_shared": ("combine_backward", m_combine_no_shared),
    "jacobian_sign": ("gate_jacobian", m_jacobian_sign),
    "jacobian_transposed": ("gate_jacobian", m_jacobian_transposed_kk),
    "sigmoid_jacobian_no_derivative": ("gate_jacobian", m_sigmoid_jacobian_no_derivative),
    "full_softmax_kept_only": ("gate_jacobian", m_full_softmax_kept_only),
    "gate_backward_flat_dgate": ("gate_backward", m_gate_backward_ignores_dgate_weights),
    "balance_no_n": ("balance_loss_backward", m_balance_no_n),
    "balance_p_for_f": ("balance_loss_backward", m_balance_p_for_f),
    "balance_sign": ("balance_loss_backward", m_balance_sign),
    "router_no_dx": ("router_backward", m_router_no_dx),
    "router_dw_mean": ("router_backward", m_router_dw_mean),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    fn, impl = MUTANTS[name]
    monkeypatch.setattr(BW, fn, impl)
    with pytest.raises(AssertionError):
        _battery()


def test_battery_passes_unmutated():
    _battery()
