"""moe_forward_noalloc through the C ABI against moe_forward.

The allocation-free entry point uses the library's per-GPU scratch array as
its workspace and shares every kernel with moe_forward, so on the same
inputs all five outputs (y, indices, gates, counts, drops) must agree bit for
bit.  Several calls run in a row on the one array, each smaller than the one
before, so a later call finds the earlier call's contents in it: a
Mixtral-shape prefill on the persistent (work-queue) GEMMs, a
DeepSeek-V3-style layer with sigmoid gates and a shared expert, then a decode
batch.  A batch whose workspace exceeds the array is refused before any GPU
work (tests/test_abi.py checks that on the host)."""

import pytest
import torch

from sparse_mixture_experts_gates_amd import binding as B
from sparse_mixture_experts_gates_amd.workloads import WORKLOADS

from tests.moe_check import bits

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

W = WORKLOADS
CALLS = [
    ("mixtral_1536", W["mixtral_bf16"].scaled(T=1536)),
    ("deepseek_small", W["deepseek_v3_bf16"].scaled(T=600, d=192, E=64, d_ff=128,
                                                    d_ff_shared=192)),
    ("decode", W["gptoss_decode_bf16"]),
]


def test_noalloc_matches_forward_on_successive_smaller_calls():
    from sparse_mixture_experts_gates_amd.workloads import make_inputs
    for name, w in CALLS:
        print(f"[noalloc] {name} T={w.T} d={w.d} E={w.E} k={w.k} d_ff={w.d_ff}", flush=True)
        inp = make_inputs(w, "cuda")
        cfg = B.config_for(w)
        assert B.workspace_size(cfg, w.T) <= B.NOALLOC_SCRATCH_BYTES
        ref = B.forward_inputs(cfg, inp)
        out = B.forward_noalloc(cfg, inp["x"], inp["w_router"], inp["w1"], inp["w2"],
                                inp["w3"], logit_offset=inp["logit_offset"],
                                select_bias=inp["select_bias"], ws1=inp["ws1"],
                                ws3=inp["ws3"], ws2=inp["ws2"])
        torch.cuda.synchronize()
        for what, a, b in zip(("y", "topk_idx", "topk_gate", "expert_counts", "num_dropped"),
                              ref, out):
            assert torch.equal(bits(a), bits(b)), f"{name}: {what} differs from moe_forward"
        del inp, ref, out
        torch.cuda.empty_cache()
