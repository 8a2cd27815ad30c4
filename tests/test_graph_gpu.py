"""moe_forward inside a captured HIP graph (torch.cuda.CUDAGraph): every
replay must give the eager result bit for bit, with eager work and
synchronisations between the replays, also after the inputs are overwritten
in place.  The library records no memset or allocation, so its launches are
all it puts into the graph."""

import pytest
import torch

from sparse_mixture_experts_gates_amd import binding as B
from sparse_mixture_experts_gates_amd.workloads import WORKLOADS, make_inputs

from tests.moe_check import bits

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


@pytest.mark.parametrize("name,kw", [
    ("mixtral_small", dict(T=300, d=256, d_ff=320)),
    ("decode_small", dict(T=8, d=192, E=32, d_ff=192)),
    ("deepseek_small", dict(T=200, d=192, E=64, d_ff=128, d_ff_shared=192)),
    ("persistent", dict(T=500, d=256, E=64, k=2, d_ff=512)),   # work-queue GEMM
])
def test_forward_replays_match_eager(name, kw):
    base = {"mixtral_small": "mixtral_bf16", "decode_small": "gptoss_decode_bf16",
            "deepseek_small": "deepseek_v3_bf16", "persistent": "mixtral_bf16"}[name]
    w = WORKLOADS[base].scaled(**kw)
    print(f"[graph] {name}", flush=True)
    inp = make_inputs(w, "cuda")
    cfg = B.config_for(w)
    ws = B.workspace(cfg, w.T)
    y = torch.empty((w.T, w.d), dtype=w.torch_dtype, device="cuda")

    def step():
        B.forward_inputs(cfg, inp, ws=ws, y=y, outputs=False)

    step()
    torch.cuda.synchronize()
    y_eager = y.clone()

    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cs):
            step()
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()

    other = B.forward_inputs(cfg, inp)[0]          # eager work with its own buffers
    for i in range(4):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(y), bits(y_eager)), f"replay {i} differs from eager"
        other = B.forward_inputs(cfg, inp)[0]
        torch.cuda.synchronize()
        assert torch.equal(bits(other), bits(y_eager))

    # new inputs written in place: replay == eager on the new inputs
    inp["x"].copy_(torch.flip(inp["x"], dims=[0]))
    g.replay()
    torch.cuda.synchronize()
    ref = B.forward_inputs(cfg, inp)[0]
    torch.cuda.synchronize()
    assert torch.equal(bits(y), bits(ref))
    print(f"[graph] {name} ok", flush=True)


@pytest.mark.parametrize("name,kw", [
    ("mixtral_small", dict(T=300, d=256, d_ff=320)),
    ("deepseek_small", dict(T=200, d=192, E=64, d_ff=128, d_ff_shared=192)),
    ("split_dx", dict(T=300, d=256, d_ff=2048)),                  # dX in K parts
])
def test_training_step_replays_match_eager(name, kw):
    """moe_forward_train + moe_backward captured together: every replay gives
    the eager y and gradients bit for bit (the backward's fills are kernels,
    its tile counters are reset by kernels, nothing is allocated)."""
    from sparse_mixture_experts_gates_amd.workloads import make_output_grad
    base = {"mixtral_small": "mixtral_bf16", "deepseek_small": "deepseek_v3_bf16",
            "split_dx": "mixtral_bf16"}[name]
    w = WORKLOADS[base].scaled(**kw)
    print(f"[graph-train] {name}", flush=True)
    inp = make_inputs(w, "cuda")
    dy = make_output_grad(w, "cuda")
    cfg = B.config_for(w)
    y, saved = B.forward_train_inputs(cfg, inp)
    bws = torch.empty(B.backward_workspace_size(cfg, w.T), dtype=torch.uint8, device="cuda")
    g = B.backward(cfg, inp["x"], inp["w_router"], inp["w1"], inp["w2"], inp["w3"], saved, dy,
                   ws1=inp["ws1"], ws3=inp["ws3"], ws2=inp["ws2"], ws=bws, want_gate_grads=True)

    def step():
        B.forward_train_inputs(cfg, inp, saved=saved, y=y)
        B.backward(cfg, inp["x"], inp["w_router"], inp["w1"], inp["w2"], inp["w3"], saved, dy,
                   ws1=inp["ws1"], ws3=inp["ws3"], ws2=inp["ws2"], ws=bws, grads=g,
                   aux_alpha=0.01)

    step()
    torch.cuda.synchronize()
    eager = {"y": y.clone(), **{k: v.clone() for k, v in g.items() if v is not None}}

    graph = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cs):
            step()
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()

    for i in range(4):
        # eager work with its own buffers between replays
        B.forward_inputs(cfg, inp)
        y.zero_()
        for v in g.values():
            if v is not None:
                v.zero_()
        graph.replay()
        torch.cuda.synchronize()
        got = {"y": y, **{k: v for k, v in g.items() if v is not None}}
        for k, v in eager.items():
            assert torch.equal(bits(got[k]), bits(v)), f"replay {i}: {k} differs from eager"
