"""Seeded synthetic workloads for the sparse MoE layer.

This module only draws inputs: it holds none of the layer's arithmetic, and
both the HIP path and the CPU oracle consume what it produces.  Every tensor
has its own generator, seeded from (seed, tensor tag), so a workload is
reproducible on one device type.  (torch's CPU and GPU generators produce
different streams; a test always feeds the same drawn tensors to both sides.)

Recipe (one line per tensor; "N(0, v)" names the variance v):

* x ~ N(0, 1); router W_r [E, d] ~ N(0, 1/d); W1, W3 [E, d_ff, d] ~ N(0, 1/d);
  W2 [E, d, d_ff] ~ N(0, 1/d_ff); shared Ws1, Ws3 [S, d_ff_s, d] ~ N(0, 1/d),
  Ws2 [S, d, d_ff_s] ~ N(0, 1/d_ff_s).
* values are float32 standard normals times sqrt(v), rounded once to the
  layer dtype (round-to-nearest-even for bf16).
* skewed routers: ``offset_normal`` adds o ~ N(0, v) to every token's score
  for expert e; ``offset_zipf`` ranks expert e at e+1 and adds
  o_e = -s ln(e+1) (a Zipf(s) prior on the scores; the normaliser is a uniform
  shift and is left out).
* ``bias_normal`` draws the selection-only balancing bias b ~ N(0, v).
* backward pass: the output gradient dy [T, d] ~ N(0, 1) in the layer dtype
  (``make_output_grad``), standing in for the gradient a loss would send back.

Named workloads follow the layer shapes used for measurement: a toy fp32
layer, a Switch-style top-1 layer with capacity, a Mixtral-shape layer, a
DeepSeek-V3-shape layer with a shared expert and sigmoid gates, and a
gpt-oss-120b-shape layer run as a skewed prefill and as an 8-token decode.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional, Tuple

import torch

TAG_X, TAG_WR, TAG_W1, TAG_W3, TAG_W2 = 1, 2, 3, 4, 5
TAG_OFFSET, TAG_BIAS, TAG_WS1, TAG_WS3, TAG_WS2, TAG_X_DECODE = 6, 7, 8, 9, 10, 11
TAG_DY = 12


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    k: int
    d_ff: int
    act: str                      # "relu" | "gelu" | "swiglu"
    gating: str = "softmax_topk"  # | "sigmoid_topk" | "softmax_full"
    dtype: str = "bf16"           # "bf16" | "f32"
    capacity_factor: float = 0.0  # <= 0: no capacity limit
    offset: Optional[Tuple[str, float]] = None   # ("normal", var) | ("zipf", s)
    bias: Optional[Tuple[str, float]] = None     # ("normal", var)
    num_shared: int = 0
    d_ff_shared: int = 0
    capacity_priority: str = "token"   # "token" or "slot": which slots claim capacity first
    x_tag: int = TAG_X
    seed: int = 0

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def scaled(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    "toy_fp32": Workload("toy_fp32", T=512, d=64, E=8, k=2, d_ff=256,
                         act="gelu", dtype="f32"),
    "switch_bf16": Workload("switch_bf16", T=8192, d=768, E=8, k=1, d_ff=3072,
                            act="relu", capacity_factor=1.25,
                            offset=("normal", 0.5)),
    # the Switch layer with the variant gate p_i (the selected expert's
    # probability under a softmax over all E scores) instead of 1.0
    "switch_softmax_full_bf16": Workload("switch_softmax_full_bf16", T=8192, d=768, E=8, k=1,
                                         d_ff=3072, act="relu", gating="softmax_full",
                                         capacity_factor=1.25, offset=("normal", 0.5)),
    "mixtral_bf16": Workload("mixtral_bf16", T=4096, d=4096, E=8, k=2,
                             d_ff=14336, act="swiglu"),
    "deepseek_v3_bf16": Workload("deepseek_v3_bf16", T=8192, d=7168, E=256,
                                 k=8, d_ff=2048, act="swiglu",
                                 gating="sigmoid_topk", bias=("normal", 0.1),
                                 num_shared=1, d_ff_shared=2048),
    "gptoss_prefill_bf16": Workload("gptoss_prefill_bf16", T=16384, d=2880,
                                    E=128, k=4, d_ff=2880, act="swiglu",
                                    offset=("zipf", 1.1)),
    "gptoss_decode_bf16": Workload("gptoss_decode_bf16", T=8, d=2880, E=128,
                                   k=4, d_ff=2880, act="swiglu",
                                   x_tag=TAG_X_DECODE),
}


def _gen(device, seed, tag):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + int(tag))
    return g


def _normal(shape, var, tag, w: Workload, device, dtype):
    """float32 N(0,1) * sqrt(var), rounded once to ``dtype``; 3-D tensors are
    drawn one leading slice at a time from the same generator."""
    g = _gen(device, w.seed, tag)
    std = math.sqrt(var)
    out = torch.empty(shape, dtype=dtype, device=device)
    if len(shape) == 3:
        for e in range(shape[0]):
            z = torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32)
            out[e].copy_((z * std).to(dtype))
            del z
    else:
        z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        out.copy_((z * std).to(dtype))
    return out


def make_inputs(w: Workload, device="cpu", with_weights=True):
    """Draw every input of workload ``w`` on ``device``; returns a dict of
    tensors (missing optional inputs are None)."""
    dt = w.torch_dtype
    inp = {}
    inp["x"] = _normal((w.T, w.d), 1.0, w.x_tag, w, device, dt)
    inp["w_router"] = _normal((w.E, w.d), 1.0 / w.d, TAG_WR, w, device, dt)
    if with_weights:
        inp["w1"] = _normal((w.E, w.d_ff, w.d), 1.0 / w.d, TAG_W1, w, device, dt)
        inp["w3"] = (_normal((w.E, w.d_ff, w.d), 1.0 / w.d, TAG_W3, w, device, dt)
                     if w.act == "swiglu" else None)
        inp["w2"] = _normal((w.E, w.d, w.d_ff), 1.0 / w.d_ff, TAG_W2, w, device, dt)
        if w.num_shared > 0:
            S, f = w.num_shared, w.d_ff_shared
            inp["ws1"] = _normal((S, f, w.d), 1.0 / w.d, TAG_WS1, w, device, dt)
            inp["ws3"] = _normal((S, f, w.d), 1.0 / w.d, TAG_WS3, w, device, dt)
            inp["ws2"] = _normal((S, w.d, f), 1.0 / f, TAG_WS2, w, device, dt)
        else:
            inp["ws1"] = inp["ws3"] = inp["ws2"] = None
    off = None
    if w.offset is not None:
        kind, p = w.offset
        if kind == "normal":
            off = _normal((w.E,), p, TAG_OFFSET, w, device, torch.float32)
        elif kind == "zipf":
            off = torch.tensor([-p * math.log(e + 1.0) for e in range(w.E)],
                               dtype=torch.float32, device=device)
        else:
            raise ValueError(kind)
    inp["logit_offset"] = off
    b = None
    if w.bias is not None:
        kind, p = w.bias
        assert kind == "normal"
        b = _normal((w.E,), p, TAG_BIAS, w, device, torch.float32)
    inp["select_bias"] = b
    return inp


def make_output_grad(w: Workload, device="cpu"):
    """The output gradient dy [T, d] of workload ``w`` (N(0, 1), layer dtype)."""
    return _normal((w.T, w.d), 1.0, TAG_DY, w, device, w.torch_dtype)
