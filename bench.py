"""Throughput of the MoE layer forward pass on one MI355X.

One step = one moe_forward over one batch of seeded synthetic input already
resident in HBM: router GEMM + top-k + gates, histogram/scan/permutation and
row gather, the two grouped expert GEMMs (and shared expert), and the
gate-weighted combine.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--graph] [--cold-runs N] [--copy-calib MiB]
                    [--no-backward] [--no-per-config]

Prints one JSON line.  `value` is tokens/s of the headline workload (the
Mixtral-shape prefill) over K back-to-back steps; `roofline` reports its
dominant kernel (the first grouped GEMM) against the bf16 MFMA peak, timed
with HIP events recorded by the library around each of its launches inside a
second timed region; `subsystems` gives every kernel's time and its rate
against its own bound (router, permutation, gather, combine in GB/s of
algorithmic bytes; expert GEMMs in TFLOP/s, or GB/s for a decode batch);
`cold` times N single steps each after a 1 GiB write that evicts L2 and the
Infinity Cache; `next_rows` times the routing statistics call and the
training step (moe_forward_train + moe_backward, per kernel);
`per_config` repeats the step measurement for every other workload (the toy
fp32 layer, the Switch layer with both gatings, DeepSeek-V3, gpt-oss prefill
and decode; the small ones also as a replayed HIP graph); `cpu_baseline` times
the CPU oracle on a bounded token sample of the headline workload.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec + active TFLOP/s (prefill), GB/s (decode) at 1 GPU"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def algorithmic_work(w, counts):
    """Algorithmic FLOPs and bytes of one forward, and of the first expert GEMM.

    FLOPs: router 2 T d E; per kept routed row n_mat * 2 d d_ff (n_mat = 3 for
    SwiGLU, 2 otherwise), of which the first GEMM is (n_mat - 1) * 2 d d_ff;
    shared experts 3 * 2 T d d_ff_s each.  Bytes: x in + y out, the router
    weights, the weights of every expert that receives a row, shared weights,
    and 8 bytes of routing output per slot.  Padding rows and the round trips
    of intermediates are not counted."""
    b = 2 if w.dtype == "bf16" else 4
    n_mat = 3 if w.act == "swiglu" else 2
    kept = int(sum(counts))
    active = sum(1 for c in counts if c > 0)
    f_router = 2 * w.T * w.d * w.E
    f_ffn1 = kept * (n_mat - 1) * 2 * w.d * w.d_ff
    f_ffn2 = kept * 2 * w.d * w.d_ff
    f_shared = w.num_shared * 3 * 2 * w.T * w.d * w.d_ff_shared
    flops = f_router + f_ffn1 + f_ffn2 + f_shared
    byt = (2 * w.T * w.d * b + w.E * w.d * b + active * n_mat * w.d * w.d_ff * b
           + w.num_shared * 3 * w.d * w.d_ff_shared * b + 8 * w.T * w.k)
    ffn1_bytes = active * (n_mat - 1) * w.d * w.d_ff * b + kept * (w.d + w.d_ff) * b
    return dict(flops=flops, bytes=byt, ffn1_flops=f_ffn1, ffn1_bytes=ffn1_bytes,
                kept=kept, active=active)


KERNEL_SOURCES = ("ffn.hip", "common.h", "plan.h", "launch.h")


def kernel_source_digest():
    """sha256 of the sources the expert GEMM kernels and their plans are built
    from."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "sparse_mixture_experts_gates_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (profiles/<kernel>_<workload>_traffic.json: FETCH_SIZE and WRITE_SIZE in
    KiB per dispatch, each scaled by the factor a plain copy of known size
    gives), or None when there is none or the kernel source changed since."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        d = json.load(fh)
    if d.get("source_sha256") != kernel_source_digest():
        return None
    return d["traffic_bytes"]


def cpu_baseline(w, inp, flops_per_token, budget_s=15.0):
    """Time the CPU oracle (as it stands) on a bounded sample of tokens."""
    import numpy as np
    from oracle import moe_oracle as O
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in info
                                 if i.get("user_api") == "blas"})) or blas
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))

    def host(t):
        return None if t is None else t.float().cpu().numpy()

    x = host(inp["x"])
    wr = host(inp["w_router"])
    w1, w2, w3 = host(inp["w1"]), host(inp["w2"]), host(inp["w3"])
    sh = None
    if w.num_shared:
        sh = (host(inp["ws1"]), host(inp["ws3"]), host(inp["ws2"]))
    off = host(inp["logit_offset"])
    bias = host(inp["select_bias"])

    def run(n):
        t0 = time.perf_counter()
        O.forward(x[:n], wr, w1, w2, w3, k=w.k, act=w.act, gating=w.gating,
                  capacity_factor=float(np.float32(w.capacity_factor)), logit_offset=off,
                  select_bias=bias, shared=sh, capacity_priority=w.capacity_priority)
        return time.perf_counter() - t0

    n = min(w.T, 64)
    dt = run(n)
    while dt < budget_s * 0.66 and n < w.T:
        n = min(w.T, max(2 * n, int(n * budget_s / max(dt, 1e-3))))
        dt = run(n)
    reps = 1
    while dt < budget_s * 0.66:   # the whole batch is quick: repeat it
        dt += run(n)
        reps += 1
    what = f"first {n} of the {w.T} tokens" if n < w.T else f"all {w.T} tokens"
    return {"value": reps * n / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "blas": blas, "gflops": reps * n * flops_per_token / dt / 1e9,
            "sample": f"{what} of {w.name}, {reps} pass(es) of the numpy float64 oracle "
                      f"forward (all routed experts touched by them), {dt:.1f} s"}


def backward_work(w, counts):
    """Algorithmic FLOPs of one backward pass: per kept routed row, each
    expert matrix is used twice more (input gradient and weight gradient),
    2 * n_mat * 2 d d_ff; the shared experts likewise over all tokens; the
    router 2 * 2 T d E (dW_r and its dx term).  The dominant GEMMs: dX and the
    dW of W1 (and W3)."""
    n_mat = 3 if w.act == "swiglu" else 2
    kept = int(sum(counts))
    per = 2 * w.d * w.d_ff
    f = {"bwd_dh": kept * per, "bwd_dw2": kept * per, "bwd_dx": kept * (n_mat - 1) * per,
         "bwd_dw1": kept * per}
    if n_mat == 3:
        f["bwd_dw3"] = kept * per
    shared = w.num_shared * 2 * 3 * 2 * w.T * w.d * w.d_ff_shared
    total = sum(f.values()) + shared + 4 * w.T * w.d * w.E
    return total, f


def measure_backward(B, w, inp, cfg, counts, steps, warmup):
    """Training step of the layer: moe_forward_train, then moe_backward on a
    seeded output gradient; both timed over `steps` back-to-back calls, then
    per kernel with the library's HIP events."""
    import torch
    from sparse_mixture_experts_gates_amd.workloads import make_output_grad
    dy = make_output_grad(w, "cuda:0")
    y, saved = B.forward_train_inputs(cfg, inp)
    g = B.backward(cfg, inp["x"], inp["w_router"], inp["w1"], inp["w2"], inp["w3"], saved, dy,
                   ws1=inp["ws1"], ws3=inp["ws3"], ws2=inp["ws2"])
    bws = torch.empty(B.backward_workspace_size(cfg, w.T), dtype=torch.uint8, device="cuda:0")

    def fwd():
        B.forward_train_inputs(cfg, inp, saved=saved, y=y)

    def bwd():
        B.backward(cfg, inp["x"], inp["w_router"], inp["w1"], inp["w2"], inp["w3"], saved, dy,
                   ws1=inp["ws1"], ws3=inp["ws3"], ws2=inp["ws2"], ws=bws, grads=g)

    for _ in range(warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    out = {}
    for name, fn in (("forward_train", fwd), ("backward", bwd)):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name + "_ms"] = e0.elapsed_time(e1) / steps
    B.profile_enable(True)
    for _ in range(steps):
        bwd()
    torch.cuda.synchronize()
    prof = B.profile_read()
    B.profile_enable(False)
    kern = {k: v[0] / max(v[1], 1) for k, v in prof.items()}
    total, per = backward_work(w, counts)
    out["tflops"] = total / (out["backward_ms"] * 1e-3) / 1e12
    out["frac_of_bf16_peak"] = out["tflops"] / PEAK_BF16_TFLOPS
    out["step_tokens_per_s"] = w.T / ((out["forward_train_ms"] + out["backward_ms"]) * 1e-3)
    out["kernels_ms"] = {k: round(v, 5) for k, v in sorted(kern.items())}
    gemms = {}
    for k, fl in per.items():
        if k in kern and kern[k] > 0:
            tf = fl / (kern[k] * 1e-3) / 1e12
            gemms[k] = {"ms": kern[k], "tflops": tf, "frac": tf / PEAK_BF16_TFLOPS}
    out["gemms"] = gemms
    return out


def subsystem_work(w, kept_counts, active):
    """Algorithmic work of each kernel of one step, by the profiler's kernel
    name: (bound, amount, unit) with bytes for the HBM-bound kernels and
    FLOPs for the expert GEMMs (bytes when the batch is a decode batch).

    route: x and W_r read, the k indices and gates written; permute: the k
    indices read, perm_src / slot_pos written; gather (stepwise path only):
    each kept row read and written; combine: each kept expert-output row and
    the shared outputs read, the gates and slot positions read, y written."""
    b = 2 if w.dtype == "bf16" else 4
    n_mat = 3 if w.act == "swiglu" else 2
    kept = int(sum(kept_counts))
    R = w.T * w.k
    decode = R <= 64
    out = {
        "route": ("hbm", w.T * w.d * b + w.E * w.d * b + 8 * R, "B"),
        "permute": ("hbm", 4 * R + 8 * R, "B"),
        # small batches: router and permutation in one launch pair
        "route_permute": ("hbm", w.T * w.d * b + w.E * w.d * b + 8 * R + 12 * R, "B"),
        "gather": ("hbm", 2 * kept * w.d * b, "B"),
        "combine": ("hbm", kept * w.d * b + w.num_shared * w.T * w.d * b + 8 * R
                    + w.T * w.d * b, "B"),
    }
    if decode:
        out["ffn1"] = ("hbm", active * (n_mat - 1) * w.d * w.d_ff * b + kept * (w.d + w.d_ff) * b, "B")
        out["ffn2"] = ("hbm", active * w.d * w.d_ff * b + kept * (w.d + w.d_ff) * b, "B")
    else:
        out["ffn1"] = ("mfma", kept * (n_mat - 1) * 2 * w.d * w.d_ff, "FLOP")
        out["ffn2"] = ("mfma", kept * 2 * w.d * w.d_ff, "FLOP")
    if w.num_shared:
        out["ffn1_shared"] = ("mfma", w.num_shared * 2 * 2 * w.T * w.d * w.d_ff_shared, "FLOP")
        out["ffn2_shared"] = ("mfma", w.num_shared * 2 * w.T * w.d * w.d_ff_shared, "FLOP")
    return out


def rate_of(kind, amount, ms, peak_flops):
    if ms is None or not ms > 0:
        return None
    if kind == "hbm":
        gbs = amount / (ms * 1e-3) / 1e9
        return {"ms": ms, "bound": "hbm", "GB_s": gbs, "frac": gbs / PEAK_HBM_GBS}
    tf = amount / (ms * 1e-3) / 1e12
    return {"ms": ms, "bound": "mfma", "TFLOP_s": tf, "frac": tf / peak_flops}


def measure_workload(B, w, steps, warmup, graph=False, gather=True, dev="cuda:0"):
    """Inputs, warm-up, K timed back-to-back steps (and, with graph=True, K
    replays of one captured step), per-kernel times from the library's HIP
    events, and the batch's routing.  Returns (result dict, inputs, cfg)."""
    import torch
    from sparse_mixture_experts_gates_amd.workloads import make_inputs
    inp = make_inputs(w, dev)
    cfg = B.config_for(w)
    ws = B.workspace(cfg, w.T, dev)
    y = torch.empty((w.T, w.d), dtype=w.torch_dtype, device=dev)

    def step():
        B.forward(cfg, inp["x"], inp["w_router"], inp["w1"], inp["w2"], inp["w3"],
                  logit_offset=inp["logit_offset"], select_bias=inp["select_bias"],
                  ws1=inp["ws1"], ws3=inp["ws3"], ws2=inp["ws2"], ws=ws, y=y, outputs=False)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    _, _, _, cnt_dev, drp_dev = B.forward_inputs(cfg, inp, ws=ws)
    torch.cuda.synchronize()
    cnt = cnt_dev.cpu().tolist()
    dropped = int(drp_dev.item())
    kept_counts = [min(c, B.capacity(cfg, w.T)) for c in cnt] if w.capacity_factor > 0 else cnt
    work = algorithmic_work(w, kept_counts)

    def timed(fn):
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    ms = timed(step)
    ms_graph = None
    if graph:
        # the library launches on torch's current stream, so a capture on a
        # side stream records every kernel of the step
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
        for _ in range(warmup):
            g.replay()
        ms_graph = timed(g.replay)

    # per-kernel times: the same steps with the library's per-launch events
    B.profile_enable(True)
    torch.cuda.synchronize()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    prof = B.profile_read()
    B.profile_enable(False)
    kern = {k: v[0] / max(v[1], 1) for k, v in prof.items()}
    # the row gather as a pass of its own (the stepwise moe_permute with
    # x_perm; moe_forward folds it into the first GEMM's loads)
    if gather and w.T * w.k > 0:
        idx, _, _ = B.route(cfg, inp["x"], inp["w_router"], inp["logit_offset"],
                            inp["select_bias"], ws=ws)
        B.permute(cfg, idx, inp["x"], gather=True, ws=ws)
        torch.cuda.synchronize()
        B.profile_enable(True)
        for _ in range(steps):
            B.permute(cfg, idx, inp["x"], gather=True, ws=ws)
        torch.cuda.synchronize()
        gp = B.profile_read()
        B.profile_enable(False)
        if "gather" in gp:
            kern["gather"] = gp["gather"][0] / max(gp["gather"][1], 1)

    active = work["active"]
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    decode = w.T * w.k <= B.DECODE_MAX_ROWS
    subs = {}
    if "permute" not in kern and "permute_scatter" in kern:   # chunked permutation
        kern["permute"] = sum(kern.pop(n) for n in ("permute_count", "permute_scan",
                                                     "permute_scatter") if n in kern)
    for name, (kind, amount, unit) in subsystem_work(w, kept_counts, active).items():
        r = rate_of(kind, amount, kern.get(name), peak)
        if r is not None:
            r["algorithmic_" + ("bytes" if unit == "B" else "flops")] = amount
            subs[name] = r
    for name, v in kern.items():          # plans, split reduce, chunked permutation
        if name not in subs:
            subs[name] = {"ms": v}
    tflops = work["flops"] / (ms * 1e-3) / 1e12
    gbs = work["bytes"] / (ms * 1e-3) / 1e9
    res = {
        "workload": w.name,
        "config": {"T": w.T, "d": w.d, "E": w.E, "k": w.k, "d_ff": w.d_ff, "act": w.act,
                   "gating": w.gating, "dtype": w.dtype, "capacity_factor": w.capacity_factor,
                   "num_shared": w.num_shared, "d_ff_shared": w.d_ff_shared},
        "bound": "hbm" if decode else ("mfma" if w.T * w.k >= 4096 else "latency"),
        "ms_per_step": ms,
        "tokens_per_s": w.T / (ms * 1e-3),
        "active_tflops": tflops,
        "frac_of_peak": tflops / peak,
        "peak_tflops": peak,
        "algorithmic_gbs": gbs,
        "frac_of_hbm": gbs / PEAK_HBM_GBS,
        "routing": {"kept_rows": work["kept"], "active_experts": active, "dropped": dropped},
        "subsystems": subs,
    }
    if ms_graph is not None:
        res["hip_graph"] = {"ms_per_step": ms_graph, "tokens_per_s": w.T / (ms_graph * 1e-3),
                            "algorithmic_gbs": work["bytes"] / (ms_graph * 1e-3) / 1e9,
                            "frac_of_hbm": work["bytes"] / (ms_graph * 1e-3) / 1e9 / PEAK_HBM_GBS,
                            "active_tflops": work["flops"] / (ms_graph * 1e-3) / 1e12}
    ctx = dict(inp=inp, cfg=cfg, ws=ws, y=y, step=step, work=work, kern=kern,
               kept_counts=kept_counts, cnt_dev=cnt_dev, drp_dev=drp_dev)
    return res, ctx


PER_CONFIG = ("toy_fp32", "switch_bf16", "switch_softmax_full_bf16", "deepseek_v3_bf16",
              "gptoss_prefill_bf16", "gptoss_decode_bf16")
GRAPHED = ("toy_fp32", "switch_bf16", "switch_softmax_full_bf16", "gptoss_decode_bf16")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time replays of one step captured in a HIP graph")
    ap.add_argument("--cold-runs", type=int, default=20,
                    help="extra single-step runs, each after writing 1 GiB to flush L2 and "
                         "the Infinity Cache (median / min / p90 reported; 0 = skip)")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the training-step measurement (forward_train + backward)")
    ap.add_argument("--no-per-config", action="store_true",
                    help="measure the headline workload only")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the layer is "
              "built and measured on a single MI355X; multi-GPU sharding is not part of "
              "this build.", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_mixture_experts_gates_amd import binding as B
    from sparse_mixture_experts_gates_amd.workloads import WORKLOADS

    w = WORKLOADS[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    head, ctx = measure_workload(B, w, args.steps, args.warmup, graph=args.graph)
    inp, cfg, ws, step = ctx["inp"], ctx["cfg"], ctx["ws"], ctx["step"]
    work, kern = ctx["work"], ctx["kern"]
    ms = head["ms_per_step"]

    if args.copy_calib:
        n = args.copy_calib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # cold runs: each step after a 1 GiB write that evicts L2 and the 256 MB
    # Infinity Cache (the flush is not timed)
    cold = None
    if args.cold_runs > 0:
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        times = []
        for i in range(args.cold_runs):
            flush.fill_(float(i))
            c0.record()
            step()
            c1.record()
            torch.cuda.synchronize()
            times.append(c0.elapsed_time(c1))
        del flush
        times.sort()
        cold = {"runs": len(times), "median_ms": times[len(times) // 2], "min_ms": times[0],
                "p90_ms": times[min(len(times) - 1, int(0.9 * len(times)))],
                "tokens_per_s_median": w.T / (times[len(times) // 2] * 1e-3)}

    # routing statistics of the batch (balance signals; not part of the
    # forward step): they read the scores, which the forward keeps internal
    _, _, logits = B.route(cfg, inp["x"], inp["w_router"], inp["logit_offset"],
                           inp["select_bias"], want_logits=True, ws=ws)
    bias_in = (inp["select_bias"] if inp["select_bias"] is not None
               else torch.zeros(w.E, dtype=torch.float32, device=dev))
    stats_out = torch.empty(w.E, dtype=torch.float32, device=dev)
    cnt_dev, drp_dev = ctx["cnt_dev"], ctx["drp_dev"]
    st_res = B.routing_stats(cfg, logits, cnt_dev, drp_dev, bias_in, gamma=1e-3, alpha=0.01,
                             bias_out=stats_out, ws=ws)
    torch.cuda.synchronize()
    B.profile_enable(True)
    for _ in range(args.steps):
        B.routing_stats(cfg, logits, cnt_dev, drp_dev, bias_in, gamma=1e-3, alpha=0.01,
                        bias_out=stats_out, ws=ws, out=st_res)
    torch.cuda.synchronize()
    sp = B.profile_read()
    B.profile_enable(False)
    st_ms = sp["routing_stats"][0] / max(sp["routing_stats"][1], 1) if "routing_stats" in sp \
        else float("nan")
    # bytes: the scores once, counts, bias in and out, f, P
    st_bytes = w.T * w.E * 4 + 5 * w.E * 4
    next_rows = {"routing_stats": {
        "ms": st_ms, "bound": "hbm", "algorithmic_bytes": st_bytes,
        "achieved_gbs": st_bytes / (st_ms * 1e-3) / 1e9,
        "frac": st_bytes / (st_ms * 1e-3) / 1e9 / PEAK_HBM_GBS}}

    dom = "ffn1"
    dom_ms = kern.get(dom, float("nan"))
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    decode = w.T * w.k <= B.DECODE_MAX_ROWS
    if decode:   # small batch: the expert GEMMs stream the active experts' weights
        roof = {"kernel": dom, "bound": "hbm",
                "achieved": work["ffn1_bytes"] / (dom_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "algorithmic_bytes_per_launch": work["ffn1_bytes"]}
    else:
        roof = {"kernel": dom, "bound": "mfma",
                "achieved": work["ffn1_flops"] / (dom_ms * 1e-3) / 1e12, "peak": peak,
                "unit": "TFLOP/s", "algorithmic_flops_per_launch": work["ffn1_flops"]}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(dom, w.name)
    roof["avg_ms"] = dom_ms
    res = {
        "metric": METRIC,
        "value": w.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "hip_graph": False,
        "config": {"workload": w.name, "T": w.T, "d": w.d, "E": w.E, "k": w.k,
                   "d_ff": w.d_ff, "act": w.act, "gating": w.gating,
                   "capacity_factor": w.capacity_factor, "num_shared": w.num_shared,
                   "d_ff_shared": w.d_ff_shared, "parallelism": "none (1 GPU)"},
        "active_tflops": head["active_tflops"],
        "active_tflops_frac_of_peak": head["frac_of_peak"],
        "algorithmic_gbs": head["algorithmic_gbs"],
        "algorithmic_gbs_frac_of_hbm": head["frac_of_hbm"],
        "routing": head["routing"],
        "kernels_ms": {k: round(v, 5) for k, v in sorted(kern.items())},
        "subsystems": head["subsystems"],
        "roofline": roof,
        "next_rows": next_rows,
        "cold": cold,
    }
    if "hip_graph" in head:
        res["graph_replay"] = head["hip_graph"]
    if w.dtype == "bf16" and not args.no_backward:
        next_rows["backward"] = measure_backward(B, w, inp, cfg, ctx["kept_counts"], args.steps,
                                                 args.warmup)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, inp, work["flops"] / w.T)
    del inp, ctx, ws, step, logits
    torch.cuda.empty_cache()
    if not args.no_per_config:
        per = {}
        for name in PER_CONFIG:
            if name == w.name:
                continue
            r, c = measure_workload(B, WORKLOADS[name], args.steps, args.warmup,
                                    graph=name in GRAPHED)
            del c
            torch.cuda.empty_cache()
            per[name] = r
        res["per_config"] = per
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
