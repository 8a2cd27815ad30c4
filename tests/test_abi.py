"""The C-ABI library: it loads, exports every symbol include/moe.h declares,
and rejects bad arguments on the host before touching the GPU (no compute
call is made here)."""

import ctypes
import os
import re

import pytest

from sparse_mixture_experts_gates_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH),
                                reason="libmoe_mi355x.so not built (run __graft_entry__.build())")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_forward",
              "moe_routing_stats", "moe_workspace_size", "moe_capacity", "moe_status_str"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(B.LIB_PATH)
    for n in declared_functions():
        assert hasattr(L, n), n
    assert set(declared_functions()) == set(B.EXPORTS)


def test_config_struct_layout():
    assert ctypes.sizeof(B.MoeConfig) == 44


def test_status_strings():
    for s in range(5):
        assert B.lib().moe_status_str(s).decode().startswith(B.STATUS[s])


def cfg(**kw):
    base = dict(d=256, num_experts=8, top_k=2, d_ff=512, act="swiglu",
                gating="softmax_topk", dtype="bf16")
    base.update(kw)
    return B.config(**base)


def test_config_validation():
    ok = cfg()
    assert B.check_config(ok, 100) == 0
    assert B.check_config(ok, 0) == 0
    assert B.check_config(ok, -1) == 1
    assert B.check_config(cfg(top_k=9), 10) == 1           # k > E
    assert B.check_config(cfg(top_k=0), 10) == 1
    assert B.check_config(cfg(d=0), 10) == 1
    c = cfg(); c.act = 7
    assert B.check_config(c, 10) == 1
    c = cfg(); c.gating = -1
    assert B.check_config(c, 10) == 1
    c = cfg(); c.dtype = 5
    assert B.check_config(c, 10) == 1
    c = cfg(); c.capacity_factor = float("nan")
    assert B.check_config(c, 10) == 1
    c = cfg(); c.capacity_priority = 2
    assert B.check_config(c, 10) == 1
    assert B.check_config(cfg(capacity_priority="slot"), 10) == 0
    assert B.check_config(cfg(d=100), 10) == 2              # bf16 needs multiples of 64
    assert B.check_config(cfg(d=102, dtype="f32"), 10) == 2
    assert B.check_config(cfg(d=100, dtype="f32"), 10) == 0
    assert B.check_config(cfg(d=64, d_ff=36, dtype="f32"), 10) == 0
    assert B.check_config(cfg(num_experts=300, top_k=2), 10) == 2
    assert B.check_config(cfg(num_experts=64, top_k=17), 10) == 2
    assert B.check_config(cfg(num_shared=1, d_ff_shared=0), 10) == 1
    assert B.check_config(cfg(num_shared=1, d_ff_shared=128), 10) == 0


def test_capacity_and_workspace_on_host():
    c = cfg(d=768, d_ff=3072, top_k=1, act="relu", capacity_factor=1.25)
    assert B.capacity(c, 8192) == 1280
    assert B.capacity(cfg(), 8192) == -1
    assert B.capacity(cfg(capacity_factor=1.0, top_k=2), 10) == 2   # floor(1*2*10/8)
    w = B.workspace_size(cfg(), 1000)
    assert w > 2000 * 256 * 2
    assert B.workspace_size(cfg(), 0) >= 0
    with pytest.raises(B.MoeError):
        B.workspace_size(cfg(top_k=9), 10)


def test_entry_points_reject_bad_arguments_before_any_gpu_work():
    L = B.lib()
    c = cfg()
    p = ctypes.c_void_p(4096)          # aligned, never dereferenced
    mis = ctypes.c_void_p(4096 + 2)    # misaligned
    n = None
    # null required pointers
    assert L.moe_route(ctypes.byref(c), 10, n, p, n, n, n, p, p, n, 0, n) == 1
    assert L.moe_route(ctypes.byref(c), 10, mis, p, n, n, n, p, p, n, 0, n) == 1
    bad = cfg(top_k=9)
    assert L.moe_route(ctypes.byref(bad), 10, p, p, n, n, n, p, p, n, 0, n) == 1
    assert L.moe_permute(ctypes.byref(c), 10, n, n, n, p, p, p, n, n, p, 1 << 30, n) == 1
    # workspace too small
    assert L.moe_permute(ctypes.byref(c), 10, p, n, n, p, p, p, n, n, p, 16, n) == 3
    assert L.moe_expert_ffn(ctypes.byref(c), 10, n, p, p, p, n, p, n, n, n, p, n, p, 1 << 30, n) == 1  # swiglu needs w3
    assert L.moe_combine(ctypes.byref(c), 10, p, p, p, n, n, n) == 1
    assert L.moe_forward(ctypes.byref(c), 10, p, p, n, n, p, p, p, n, n, n, p, n, n, n, n, p, 16, n) == 3
    assert L.moe_forward(ctypes.byref(c), 10, p, p, n, n, p, n, p, n, n, n, p, n, n, n, n, p, 1 << 40, n) == 1
    sh = cfg(num_shared=1, d_ff_shared=128)
    assert L.moe_forward(ctypes.byref(sh), 10, p, p, n, n, p, p, p, n, n, n, p, n, n, n, n, p, 1 << 40, n) == 1
    # routing statistics: required pointers, optional pairs, scalars, workspace
    f32 = ctypes.c_float
    st = L.moe_routing_stats
    assert st(ctypes.byref(c), 10, n, p, n, n, f32(0), f32(0.01), p, p, p, n, n, p, 1 << 30, n) == 1
    assert st(ctypes.byref(c), 10, p, p, n, n, f32(0), f32(0.01), p, p, p, p, n, p, 1 << 30, n) == 1  # rate needs dropped
    assert st(ctypes.byref(c), 10, p, p, p, n, f32(0), f32(0.01), p, p, p, p, p, p, 1 << 30, n) == 1  # bias needs bias in
    assert st(ctypes.byref(c), 10, p, p, n, p, f32(-1), f32(0.01), p, p, p, n, p, p, 1 << 30, n) == 1
    assert st(ctypes.byref(c), 10, p, p, n, n, f32(0), f32(float("nan")), p, p, p, n, n, p, 1 << 30, n) == 1
    assert st(ctypes.byref(c), 10, mis, p, n, n, f32(0), f32(0.01), p, p, p, n, n, p, 1 << 30, n) == 1
    assert st(ctypes.byref(c), 10, p, p, n, n, f32(0), f32(0.01), p, p, p, n, n, p, 16, n) == 3
    assert st(ctypes.byref(c), 0, n, n, n, n, f32(0), f32(0.01), n, n, n, n, n, n, 0, n) == 0
    # T = 0 is a valid no-op for every entry point
    assert L.moe_route(ctypes.byref(c), 0, p, p, n, n, n, p, p, n, 0, n) == 0
    assert L.moe_permute(ctypes.byref(c), 0, p, n, n, p, p, p, n, n, n, 0, n) == 0
    assert L.moe_expert_ffn(ctypes.byref(c), 0, n, p, p, p, p, p, n, n, n, p, n, n, 0, n) == 0
    assert L.moe_combine(ctypes.byref(c), 0, p, p, p, n, p, n) == 0
    assert L.moe_forward(ctypes.byref(c), 0, p, p, n, n, p, p, p, n, n, n, p, n, n, n, n, n, 0, n) == 0
    assert L.moe_forward(ctypes.byref(c), 0, n, n, n, n, n, n, n, n, n, n, n, n, n, n, n, n, 0, n) == 0
    assert L.moe_forward(ctypes.byref(bad), 0, n, n, n, n, n, n, n, n, n, n, n, n, n, n, n, n, 0, n) == 1


def test_binding_refuses_host_tensors():
    import torch
    c = cfg()
    with pytest.raises(ValueError):
        B.route(c, torch.zeros((4, 256), dtype=torch.bfloat16),
                torch.zeros((8, 256), dtype=torch.bfloat16))


def test_binding_checks_dtype_and_size_of_each_argument():
    """The binding compares every tensor with what the library will read or
    write through its pointer (dtype, then element count, then device memory
    and layout), before the call."""
    import torch
    c = cfg()
    w2 = torch.zeros((c.num_experts, c.d, c.d_ff), dtype=torch.bfloat16)
    n = c.num_experts * c.d * c.d_ff
    with pytest.raises(ValueError, match="w2: dtype"):
        B._arg(w2.float(), "w2", n, torch.bfloat16)
    with pytest.raises(ValueError, match="w2: .* elements"):
        B._arg(w2[:, :-1], "w2", n, torch.bfloat16)
    with pytest.raises(ValueError, match="device memory"):
        B._arg(w2, "w2", n, torch.bfloat16)
    assert B._arg(None, "w2", n, torch.bfloat16) is None
    x = torch.zeros((4, c.d), dtype=torch.bfloat16)
    wr = torch.zeros((c.num_experts, c.d), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="x: dtype"):
        B.route(c, x.float(), wr)
    with pytest.raises(ValueError, match="x: .* elements"):
        B.forward(c, x[:, :-16], wr, w2, w2, w2, ws=torch.zeros(1, dtype=torch.uint8))


def test_training_entry_points_reject_bad_arguments_before_any_gpu_work():
    L = B.lib()
    c = cfg()
    by = ctypes.byref
    p = ctypes.c_void_p(1 << 20)      # 256-byte aligned, never dereferenced
    n = None
    f32 = ctypes.c_float
    big = 1 << 40
    c32 = cfg(dtype="f32")
    ft = L.moe_forward_train
    assert ft(by(c32), 10, p, p, n, n, p, p, p, n, n, n, p, p, big, n) == 2   # bf16 only
    assert ft(by(c), 10, p, p, n, n, p, n, p, n, n, n, p, p, big, n) == 1     # SwiGLU needs w3
    assert ft(by(c), 10, p, p, n, n, p, p, p, n, n, n, p, n, big, n) == 1     # saved buffer
    assert ft(by(c), 10, p, p, n, n, p, p, p, n, n, n, p, p, 16, n) == 3      # saved too small
    assert ft(by(c), 0, n, n, n, n, n, n, n, n, n, n, n, n, 0, n) == 0

    def bw(T=10, saved_bytes=big, aux=0.0, dw3=p, ws_bytes=big, cfg_=c):
        # x, w_router, w1, w3, w2, ws1, ws3, ws2, saved, saved_bytes, dy, aux,
        # dx, dw_router, dw1, dw3, dw2, dws1, dws3, dws2, d_gate, d_logits,
        # workspace, ws_bytes, stream
        return L.moe_backward(by(cfg_), T, p, p, p, p, p, n, n, n, p, saved_bytes, p, f32(aux),
                              p, p, p, dw3, p, n, n, n, n, n, p, ws_bytes, n)
    assert bw(cfg_=c32) == 2
    assert bw(aux=-1.0) == 1
    assert bw(aux=float("nan")) == 1
    assert bw(aux=float("inf")) == 1
    assert bw(dw3=None) == 1
    assert bw(saved_bytes=16) == 3
    assert bw(ws_bytes=16) == 3
    assert L.moe_backward(by(c), 0, *([n] * 9), 0, n, f32(0), *([n] * 10), n, 0, n) == 0
    sh = cfg(num_shared=1, d_ff_shared=128)
    assert bw(cfg_=sh) == 1                     # shared experts need their weights and grads


def test_training_sizes_and_saved_views_on_host():
    c = cfg()
    T = 1000
    tr = B.train_workspace_size(c, T)
    assert tr > B.workspace_size(c, T)
    assert B.backward_workspace_size(c, T) > 0
    with pytest.raises(B.MoeError):
        B.train_workspace_size(cfg(dtype="f32"), T)
    L = B.lib()
    base = 1 << 30
    ptrs = [ctypes.c_void_p() for _ in range(7)]
    assert L.moe_saved_routing(ctypes.byref(c), T, ctypes.c_void_p(base),
                               *[ctypes.byref(q) for q in ptrs]) == 0
    offs = [q.value - base for q in ptrs]
    sizes = [T * 8 * 4, T * 2 * 4, T * 2 * 4, 8 * 4, 4, 9 * 4, T * 2 * 4]
    spans = sorted(zip(offs, sizes))
    for (o, s_), (o2, _) in zip(spans, spans[1:]):
        assert 0 <= o and o + s_ <= o2          # disjoint, inside the buffer
    assert spans[-1][0] + spans[-1][1] <= tr


def test_noalloc_refuses_a_batch_beyond_its_scratch_before_touching_the_gpu():
    """moe_forward_noalloc sizes the batch's workspace on the host first: a
    Mixtral-shape batch of 4096 tokens needs more than the 256 MiB scratch
    array and is refused with MOE_ERR_WORKSPACE (no pointer is dereferenced
    and no HIP call is made, so this runs without a GPU)."""
    c = B.config(4096, 8, 2, 14336, "swiglu")
    assert B.workspace_size(c, 4096) > B.NOALLOC_SCRATCH_BYTES
    assert B.workspace_size(c, 3638) <= B.NOALLOC_SCRATCH_BYTES
    p = ctypes.c_void_p(1 << 20)          # aligned stand-ins, never read
    st = B.lib().moe_forward_noalloc(ctypes.byref(c), 4096, p, p, None, None, p, p, p,
                                     None, None, None, p, None, None, None, None, None)
    assert st == 3
