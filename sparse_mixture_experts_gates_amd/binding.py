"""ctypes binding of libmoe_mi355x.so (C ABI in include/moe.h).

Argument marshalling only: torch tensors (device memory) are checked and
turned into pointers, outputs are allocated with torch.empty, and each call
enqueues on torch's current HIP stream.  Every step of the layer runs in the
library's HIP kernels.  If the library has not been built, the first call
raises -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MOE_MI355X_LIB") or os.path.join(_HERE, "libmoe_mi355x.so")

MOE_F32, MOE_BF16 = 0, 1
ACTS = {"relu": 0, "gelu": 1, "swiglu": 2}
GATINGS = {"softmax_topk": 0, "sigmoid_topk": 1, "softmax_full": 2}
PRIORITIES = {"token": 0, "slot": 1}
DECODE_MAX_ROWS = 64
STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED",
          3: "MOE_ERR_WORKSPACE", 4: "MOE_ERR_HIP"}

EXPORTS = ("moe_status_str", "moe_check_config", "moe_workspace_size", "moe_capacity",
           "moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_forward",
           "moe_routing_stats", "moe_profile_enable", "moe_profile_read",
           "moe_train_workspace_size", "moe_forward_train", "moe_saved_routing",
           "moe_backward_workspace_size", "moe_backward", "moe_forward_noalloc")


class MoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class MoeConfig(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("act", ctypes.c_int32), ("gating", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("capacity_factor", ctypes.c_float),
                ("num_shared", ctypes.c_int32), ("d_ff_shared", ctypes.c_int32),
                ("capacity_priority", ctypes.c_int32)]


_lib_handle = None
_vp, _i64, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
_cfgp = ctypes.POINTER(MoeConfig)


def lib():
    """Load the library (once).  Raises if it is missing."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m sparse_mixture_experts_gates_amd.build` (there is no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_status_str.argtypes = [ctypes.c_int]
        L.moe_check_config.argtypes = [_cfgp, _i64]
        L.moe_workspace_size.argtypes = [_cfgp, _i64, ctypes.POINTER(_sz)]
        L.moe_capacity.argtypes = [_cfgp, _i64, ctypes.POINTER(_i64)]
        L.moe_route.argtypes = [_cfgp, _i64] + [_vp] * 8 + [_sz, _vp]
        L.moe_permute.argtypes = [_cfgp, _i64] + [_vp] * 9 + [_sz, _vp]
        L.moe_expert_ffn.argtypes = [_cfgp, _i64] + [_vp] * 12 + [_sz, _vp]
        L.moe_combine.argtypes = [_cfgp, _i64] + [_vp] * 5 + [_vp]
        L.moe_forward.argtypes = [_cfgp, _i64] + [_vp] * 16 + [_sz, _vp]
        L.moe_forward_noalloc.argtypes = [_cfgp, _i64] + [_vp] * 15 + [_vp]
        L.moe_routing_stats.argtypes = ([_cfgp, _i64] + [_vp] * 4 + [ctypes.c_float] * 2
                                        + [_vp] * 6 + [_sz, _vp])
        L.moe_train_workspace_size.argtypes = [_cfgp, _i64, ctypes.POINTER(_sz)]
        L.moe_forward_train.argtypes = [_cfgp, _i64] + [_vp] * 12 + [_sz, _vp]
        L.moe_saved_routing.argtypes = [_cfgp, _i64, _vp] + [ctypes.POINTER(_vp)] * 7
        L.moe_backward_workspace_size.argtypes = [_cfgp, _i64, ctypes.POINTER(_sz)]
        L.moe_backward.argtypes = ([_cfgp, _i64] + [_vp] * 9 + [_sz, _vp, ctypes.c_float]
                                   + [_vp] * 11 + [_sz, _vp])
        L.moe_profile_enable.argtypes = [ctypes.c_int32]
        L.moe_profile_read.restype = ctypes.c_int32
        L.moe_profile_read.argtypes = [ctypes.POINTER(ctypes.c_char_p),
                                       ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_int32), ctypes.c_int32]
        for fn in ("moe_check_config", "moe_workspace_size", "moe_capacity", "moe_route",
                   "moe_permute", "moe_expert_ffn", "moe_combine", "moe_forward",
                   "moe_forward_noalloc",
                   "moe_routing_stats", "moe_profile_enable", "moe_train_workspace_size",
                   "moe_forward_train", "moe_saved_routing", "moe_backward_workspace_size",
                   "moe_backward"):
            getattr(L, fn).restype = ctypes.c_int
        _lib_handle = L
    return _lib_handle


def config(d, num_experts, top_k, d_ff, act="swiglu", gating="softmax_topk",
           dtype="bf16", capacity_factor=0.0, num_shared=0, d_ff_shared=0,
           capacity_priority="token"):
    return MoeConfig(d, num_experts, top_k, d_ff, ACTS[act], GATINGS[gating],
                     MOE_BF16 if dtype == "bf16" else MOE_F32, float(capacity_factor),
                     num_shared, d_ff_shared, PRIORITIES[capacity_priority])


def config_for(w, T=None):
    """MoeConfig of a workloads.Workload."""
    return config(w.d, w.E, w.k, w.d_ff, w.act, w.gating, w.dtype, w.capacity_factor,
                  w.num_shared, w.d_ff_shared, w.capacity_priority)


def _check(st, where):
    if st != 0:
        raise MoeError(st, where)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be in device memory")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"tensor on {t.device}, but the current device is "
                         f"cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _arg(t: Optional[torch.Tensor], name, numel, dtype):
    """Device pointer of ``t`` once it holds exactly the ``numel`` elements of
    ``dtype`` that the library reads or writes through it (None passes)."""
    if t is None:
        return None
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    return _ptr(t)


def _weights(cfg, w1, w3, w2, ws1, ws3, ws2):
    """Checked pointers of the expert and shared-expert weights, in the
    library's argument order (w1, w3, w2, ws1, ws3, ws2)."""
    dt, E, d, f = _dt(cfg), cfg.num_experts, cfg.d, cfg.d_ff
    S, fs = cfg.num_shared, cfg.d_ff_shared
    return (_arg(w1, "w1", E * f * d, dt), _arg(w3, "w3", E * f * d, dt),
            _arg(w2, "w2", E * d * f, dt), _arg(ws1, "ws1", S * fs * d, dt),
            _arg(ws3, "ws3", S * fs * d, dt), _arg(ws2, "ws2", S * d * fs, dt))


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt(cfg):
    return torch.bfloat16 if cfg.dtype == MOE_BF16 else torch.float32


def check_config(cfg, T):
    return lib().moe_check_config(ctypes.byref(cfg), T)


def workspace_size(cfg, T):
    n = _sz(0)
    _check(lib().moe_workspace_size(ctypes.byref(cfg), T, ctypes.byref(n)), "moe_workspace_size")
    return n.value


def capacity(cfg, T):
    c = _i64(0)
    _check(lib().moe_capacity(ctypes.byref(cfg), T, ctypes.byref(c)), "moe_capacity")
    return c.value


def workspace(cfg, T, device="cuda"):
    return torch.empty(max(workspace_size(cfg, T), 256), dtype=torch.uint8, device=device)


def route(cfg, x, w_router, logit_offset=None, select_bias=None, want_logits=False, ws=None):
    T = x.shape[0]
    k, E = cfg.top_k, cfg.num_experts
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    gate = torch.empty((T, k), dtype=torch.float32, device=x.device)
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device) if want_logits else None
    dt, d = _dt(cfg), cfg.d
    _check(lib().moe_route(ctypes.byref(cfg), T, _arg(x, "x", T * d, dt),
                           _arg(w_router, "w_router", E * d, dt),
                           _arg(logit_offset, "logit_offset", E, torch.float32),
                           _arg(select_bias, "select_bias", E, torch.float32),
                           _ptr(logits), _ptr(idx), _ptr(gate), _ptr(ws),
                           0 if ws is None else ws.numel(), _stream()), "moe_route")
    return idx, gate, logits


def permute(cfg, topk_idx, x=None, gather=True, ws=None):
    T = topk_idx.shape[0]
    k, E, dev = cfg.top_k, cfg.num_experts, topk_idx.device
    out = dict(
        expert_counts=torch.empty(E, dtype=torch.int32, device=dev),
        expert_offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
        perm_src=torch.empty(T * k, dtype=torch.int32, device=dev),
        slot_pos=torch.empty(T * k, dtype=torch.int32, device=dev),
        num_dropped=torch.empty(1, dtype=torch.int32, device=dev),
        x_perm=(torch.empty((T * k, cfg.d), dtype=_dt(cfg), device=dev) if gather else None))
    if ws is None:
        ws = workspace(cfg, T, dev)
    _check(lib().moe_permute(ctypes.byref(cfg), T, _arg(topk_idx, "topk_idx", T * k, torch.int32),
                             _arg(x, "x", T * cfg.d, _dt(cfg)),
                             _ptr(out["expert_counts"]), _ptr(out["expert_offsets"]),
                             _ptr(out["perm_src"]), _ptr(out["slot_pos"]),
                             _ptr(out["num_dropped"]), _ptr(out["x_perm"]), _ptr(ws),
                             ws.numel(), _stream()), "moe_permute")
    return out


def expert_ffn(cfg, T, x_perm, expert_offsets, w1, w2, w3=None, x=None, ws1=None, ws3=None,
               ws2=None, ws=None):
    dev = x_perm.device
    eout = torch.empty((T * cfg.top_k, cfg.d), dtype=_dt(cfg), device=dev)
    sout = (torch.empty((cfg.num_shared, T, cfg.d), dtype=_dt(cfg), device=dev)
            if cfg.num_shared > 0 else None)
    if ws is None:
        ws = workspace(cfg, T, dev)
    dt, d = _dt(cfg), cfg.d
    _check(lib().moe_expert_ffn(ctypes.byref(cfg), T, _arg(x, "x", T * d, dt),
                                _arg(x_perm, "x_perm", T * cfg.top_k * d, dt),
                                _arg(expert_offsets, "expert_offsets", cfg.num_experts + 1,
                                     torch.int32),
                                *_weights(cfg, w1, w3, w2, ws1, ws3, ws2),
                                _ptr(eout), _ptr(sout), _ptr(ws), ws.numel(), _stream()),
           "moe_expert_ffn")
    return eout, sout


def combine(cfg, T, expert_out, slot_pos, topk_gate, shared_out=None):
    y = torch.empty((T, cfg.d), dtype=_dt(cfg), device=expert_out.device)
    dt, d, k = _dt(cfg), cfg.d, cfg.top_k
    _check(lib().moe_combine(ctypes.byref(cfg), T, _arg(expert_out, "expert_out", T * k * d, dt),
                             _arg(slot_pos, "slot_pos", T * k, torch.int32),
                             _arg(topk_gate, "topk_gate", T * k, torch.float32),
                             _arg(shared_out, "shared_out", cfg.num_shared * T * d, dt),
                             _ptr(y), _stream()),
           "moe_combine")
    return y


def forward(cfg, x, w_router, w1, w2, w3=None, *, logit_offset=None, select_bias=None,
            ws1=None, ws3=None, ws2=None, ws=None, y=None, outputs=True):
    """The whole layer.  Returns (y, topk_idx, topk_gate, expert_counts,
    num_dropped); the last four are None when outputs=False."""
    T = x.shape[0]
    dev = x.device
    if y is None:
        y = torch.empty((T, cfg.d), dtype=_dt(cfg), device=dev)
    idx = gate = counts = dropped = None
    if outputs:
        idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=dev)
        gate = torch.empty((T, cfg.top_k), dtype=torch.float32, device=dev)
        counts = torch.empty(cfg.num_experts, dtype=torch.int32, device=dev)
        dropped = torch.empty(1, dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(cfg, T, dev)
    dt, d, E = _dt(cfg), cfg.d, cfg.num_experts
    _check(lib().moe_forward(ctypes.byref(cfg), T, _arg(x, "x", T * d, dt),
                             _arg(w_router, "w_router", E * d, dt),
                             _arg(logit_offset, "logit_offset", E, torch.float32),
                             _arg(select_bias, "select_bias", E, torch.float32),
                             *_weights(cfg, w1, w3, w2, ws1, ws3, ws2),
                             _arg(y, "y", T * d, dt), _ptr(idx), _ptr(gate),
                             _ptr(counts), _ptr(dropped), _ptr(ws), ws.numel(), _stream()),
           "moe_forward")
    return y, idx, gate, counts, dropped


NOALLOC_SCRATCH_BYTES = 256 << 20   # MOE_NOALLOC_SCRATCH_BYTES


def forward_noalloc(cfg, x, w_router, w1, w2, w3=None, *, logit_offset=None, select_bias=None,
                    ws1=None, ws3=None, ws2=None, y=None, outputs=None):
    """moe_forward_noalloc: the whole layer with the library's own scratch
    array as its workspace.  ``outputs`` may be a (y, topk_idx, topk_gate,
    expert_counts, num_dropped) tuple of preallocated tensors; otherwise they
    are allocated here (in torch, before the call).  Returns that tuple."""
    T = x.shape[0]
    dev = x.device
    dt, d, E = _dt(cfg), cfg.d, cfg.num_experts
    if outputs is None:
        outputs = (torch.empty((T, d), dtype=dt, device=dev) if y is None else y,
                   torch.empty((T, cfg.top_k), dtype=torch.int32, device=dev),
                   torch.empty((T, cfg.top_k), dtype=torch.float32, device=dev),
                   torch.empty(E, dtype=torch.int32, device=dev),
                   torch.empty(1, dtype=torch.int32, device=dev))
    y, idx, gate, counts, dropped = outputs
    _check(lib().moe_forward_noalloc(ctypes.byref(cfg), T, _arg(x, "x", T * d, dt),
                                     _arg(w_router, "w_router", E * d, dt),
                                     _arg(logit_offset, "logit_offset", E, torch.float32),
                                     _arg(select_bias, "select_bias", E, torch.float32),
                                     *_weights(cfg, w1, w3, w2, ws1, ws3, ws2),
                                     _arg(y, "y", T * d, dt),
                                     _arg(idx, "topk_idx", T * cfg.top_k, torch.int32),
                                     _arg(gate, "topk_gate", T * cfg.top_k, torch.float32),
                                     _arg(counts, "expert_counts", E, torch.int32),
                                     _arg(dropped, "num_dropped", 1, torch.int32), _stream()),
           "moe_forward_noalloc")
    return outputs


def forward_inputs(cfg, inp, **kw):
    """forward() on a dict from workloads.make_inputs."""
    return forward(cfg, inp["x"], inp["w_router"], inp["w1"], inp["w2"], inp.get("w3"),
                   logit_offset=inp.get("logit_offset"), select_bias=inp.get("select_bias"),
                   ws1=inp.get("ws1"), ws3=inp.get("ws3"), ws2=inp.get("ws2"), **kw)


def routing_stats(cfg, logits, expert_counts, num_dropped=None, select_bias=None, gamma=0.0,
                  alpha=0.01, bias_out=None, ws=None, out=None):
    """Balance signals of one batch.  Returns dict(f, P, loss, drop_rate,
    bias); drop_rate needs num_dropped, bias needs select_bias (bias_out may
    be select_bias itself for an in-place update).  ``out`` may be an earlier
    result dict whose tensors are then reused."""
    T = logits.shape[0]
    dev = logits.device
    E = cfg.num_experts
    if out is not None:
        f, P, loss, rate = out["f"], out["P"], out["loss"], out["drop_rate"]
    else:
        f = torch.empty(E, dtype=torch.float32, device=dev)
        P = torch.empty(E, dtype=torch.float32, device=dev)
        loss = torch.empty(1, dtype=torch.float32, device=dev)
        rate = torch.empty(1, dtype=torch.float32, device=dev) if num_dropped is not None else None
    if select_bias is not None and bias_out is None:
        bias_out = torch.empty(E, dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(cfg, T, dev)
    f32, i32 = torch.float32, torch.int32
    _check(lib().moe_routing_stats(ctypes.byref(cfg), T, _arg(logits, "logits", T * E, f32),
                                   _arg(expert_counts, "expert_counts", E, i32),
                                   _arg(num_dropped, "num_dropped", 1, i32),
                                   _arg(select_bias, "select_bias", E, f32), float(gamma),
                                   float(alpha), _arg(f, "f", E, f32), _arg(P, "P", E, f32),
                                   _arg(loss, "loss", 1, f32), _arg(rate, "drop_rate", 1, f32),
                                   _arg(bias_out, "bias_out", E, f32), _ptr(ws), ws.numel(),
                                   _stream()),
           "moe_routing_stats")
    return dict(f=f, P=P, loss=loss, drop_rate=rate, bias=bias_out)


# ------------------------------------------------------------------ training
def train_workspace_size(cfg, T):
    n = _sz(0)
    _check(lib().moe_train_workspace_size(ctypes.byref(cfg), T, ctypes.byref(n)),
           "moe_train_workspace_size")
    return n.value


def backward_workspace_size(cfg, T):
    n = _sz(0)
    _check(lib().moe_backward_workspace_size(ctypes.byref(cfg), T, ctypes.byref(n)),
           "moe_backward_workspace_size")
    return n.value


def forward_train(cfg, x, w_router, w1, w2, w3=None, *, logit_offset=None, select_bias=None,
                  ws1=None, ws3=None, ws2=None, saved=None, y=None):
    """Training forward.  Returns (y, saved): ``saved`` is the uint8 buffer
    that moe_backward reads (keep it unchanged until then)."""
    T = x.shape[0]
    dev = x.device
    if y is None:
        y = torch.empty((T, cfg.d), dtype=_dt(cfg), device=dev)
    if saved is None:
        saved = torch.empty(max(train_workspace_size(cfg, T), 1), dtype=torch.uint8, device=dev)
    dt, d, E = _dt(cfg), cfg.d, cfg.num_experts
    if saved.dtype != torch.uint8:
        raise ValueError(f"saved: dtype {saved.dtype}, expected torch.uint8")
    _check(lib().moe_forward_train(ctypes.byref(cfg), T, _arg(x, "x", T * d, dt),
                                   _arg(w_router, "w_router", E * d, dt),
                                   _arg(logit_offset, "logit_offset", E, torch.float32),
                                   _arg(select_bias, "select_bias", E, torch.float32),
                                   *_weights(cfg, w1, w3, w2, ws1, ws3, ws2),
                                   _arg(y, "y", T * d, dt), _ptr(saved), saved.numel(),
                                   _stream()),
           "moe_forward_train")
    return y, saved


def forward_train_inputs(cfg, inp, **kw):
    """forward_train() on a dict from workloads.make_inputs."""
    return forward_train(cfg, inp["x"], inp["w_router"], inp["w1"], inp["w2"], inp.get("w3"),
                         logit_offset=inp.get("logit_offset"),
                         select_bias=inp.get("select_bias"), ws1=inp.get("ws1"),
                         ws3=inp.get("ws3"), ws2=inp.get("ws2"), **kw)


def saved_routing(cfg, T, saved):
    """Views (torch tensors) of the routing a training forward kept in saved:
    logits, topk_idx, topk_gate, expert_counts, num_dropped, expert_offsets,
    slot_pos."""
    ptrs = [_vp() for _ in range(7)]
    _check(lib().moe_saved_routing(ctypes.byref(cfg), T, _ptr(saved),
                                   *[ctypes.byref(p) for p in ptrs]), "moe_saved_routing")
    base = saved.data_ptr()
    k, E = cfg.top_k, cfg.num_experts
    spec = [("logits", (T, E), torch.float32), ("topk_idx", (T, k), torch.int32),
            ("topk_gate", (T, k), torch.float32), ("expert_counts", (E,), torch.int32),
            ("num_dropped", (1,), torch.int32), ("expert_offsets", (E + 1,), torch.int32),
            ("slot_pos", (T * k,), torch.int32)]
    out = {}
    for p, (name, shape, dt) in zip(ptrs, spec):
        off = p.value - base
        n = 1
        for v in shape:
            n *= v
        out[name] = saved[off:off + n * 4].view(dt).view(shape)
    return out


def backward(cfg, x, w_router, w1, w2, w3, saved, dy, *, ws1=None, ws3=None, ws2=None,
             aux_alpha=0.0, ws=None, grads=None, want_gate_grads=False):
    """Gradients of one layer from a training forward's ``saved`` buffer.
    Returns dict(dx, dw_router, dw1, dw3, dw2, dws1, dws3, dws2, d_gate,
    d_logits); ``grads`` may be an earlier result dict whose tensors are
    reused."""
    T = x.shape[0]
    dev = x.device
    glu = cfg.act == ACTS["swiglu"]
    S = cfg.num_shared
    if grads is None:
        grads = dict(
            dx=torch.empty_like(x), dw_router=torch.empty(w_router.shape, dtype=torch.float32,
                                                          device=dev),
            dw1=torch.empty_like(w1), dw3=torch.empty_like(w3) if glu else None,
            dw2=torch.empty_like(w2),
            dws1=torch.empty_like(ws1) if S else None, dws3=torch.empty_like(ws3) if S else None,
            dws2=torch.empty_like(ws2) if S else None,
            d_gate=torch.empty((T, cfg.top_k), dtype=torch.float32, device=dev)
            if want_gate_grads else None,
            d_logits=torch.empty((T, cfg.num_experts), dtype=torch.float32, device=dev)
            if want_gate_grads else None)
    if ws is None:
        ws = torch.empty(max(backward_workspace_size(cfg, T), 1), dtype=torch.uint8, device=dev)
    g = grads
    dt, d, E, k = _dt(cfg), cfg.d, cfg.num_experts, cfg.top_k
    f32 = torch.float32
    if saved.dtype != torch.uint8:
        raise ValueError(f"saved: dtype {saved.dtype}, expected torch.uint8")
    weights = _weights(cfg, w1, w3, w2, ws1, ws3, ws2)
    dweights = _weights(cfg, g["dw1"], g["dw3"], g["dw2"], g["dws1"], g["dws3"], g["dws2"])
    _check(lib().moe_backward(ctypes.byref(cfg), T, _arg(x, "x", T * d, dt),
                              _arg(w_router, "w_router", E * d, dt), *weights, _ptr(saved),
                              saved.numel(), _arg(dy, "dy", T * d, dt), float(aux_alpha),
                              _arg(g["dx"], "dx", T * d, dt),
                              _arg(g["dw_router"], "dw_router", E * d, f32),
                              dweights[0], dweights[1], dweights[2], dweights[3], dweights[4],
                              dweights[5], _arg(g["d_gate"], "d_gate", T * k, f32),
                              _arg(g["d_logits"], "d_logits", T * E, f32), _ptr(ws), ws.numel(),
                              _stream()), "moe_backward")
    return g


def profile_enable(on=True):
    _check(lib().moe_profile_enable(1 if on else 0), "moe_profile_enable")


def profile_read(max_names=64):
    names = (ctypes.c_char_p * max_names)()
    ms = (ctypes.c_double * max_names)()
    cnt = (ctypes.c_int32 * max_names)()
    n = lib().moe_profile_read(names, ms, cnt, max_names)
    if n < 0:
        raise MoeError(4, "moe_profile_read")
    return {names[i].decode(): (ms[i], cnt[i]) for i in range(n)}
