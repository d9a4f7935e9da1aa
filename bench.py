"""Benchmark: MoE layer forward on one MI355X.

A step is one moe_layer_forward call (router -> permutation -> grouped
gate_up + SwiGLU -> grouped down -> combine) over one batch of seeded
synthetic input already resident in HBM, on torch's current stream.  The
library records caller-supplied HIP events between its stages, so each
stage's average duration is measured live over the timed steps.

Prints one JSON line.  Headline workload: the Qwen3-30B-A3B-shaped prefill
layer, T = 4096 tokens, H = 2048, I = 768, E = 128, top_k = 8, bf16.  With
no --workload the same line also carries, under "workloads", the decode
layer (T = 64; its layer_hbm_frac is the decode HBM figure), the skewed
batch (T = 16384, Zipf(1.2) popularity), the tiny float32 layer and one
expert-parallel rank's share, each timed the same way.

Byte counts: a kernel's algorithmic bytes are what the method must move
(hit experts' weights once, the hidden states it reads, the router's and
the layer's outputs); this implementation's intermediates (h, the per-slot
expert outputs, index maps) are reported separately as bytes moved.

Other modes:
  --workload NAME        one named workload alone (prefill, decode, skewed,
                         tiny_fp32, ep_rank_235b)
  --no-extra             the prefill headline alone
  --copy-calibration     only run a plain 1 GiB device copy (for scaling the
                         rocprofv3 FETCH_SIZE / WRITE_SIZE counters)
  --router sigmoid-groups  a sigmoid, node-limited, biased router variant
  --shared-I IS          add a shared expert (FeedForward) of intermediate
                         size IS
  --backward             time the layer backward instead (one training
                         forward first, then moe_layer_backward per step)
  --workload ep_rank_235b  one expert-parallel rank: rank-major reshuffle,
                         grouped SwiGLU, reverse reshuffle

The headline ms_per_step (and value) is the mean over K replays of the layer
call captured once in a HIP graph, as a serving loop runs it: the same
kernels on the same inputs with bit-identical outputs, without the host's
launch gaps.  The eager stream's mean over K steps is eager_ms_per_step; the
per-stage durations and the roofline come from those eager steps' events.
The backward and the EP-rank modes time the eager stream.

Besides the mean over the timed steps, each line reports per-step median and
minimum, warm and cold (a 512 MB scratch write before each step evicts L2
and the MALL), and, as context only, torch's batched bf16 GEMM at the
average expert's shape.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed tokens/s per MoE layer fwd (bf16); % MFMA peak; decode HBM GB/s"
PEAK_BF16_FLOPS = 2.5e15      # MI355X dense bf16 MFMA (published)
PEAK_F32_FLOPS = 157.3e12     # MI355X fp32 (published)
PEAK_HBM = 8.0e12             # MI355X HBM3E bytes/s (published)
KERNELS = ("route", "permute", "gate_up_swiglu", "down", "combine")  # stage order


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="time one named workload alone (default: the prefill headline, "
                         "with the decode, skewed, tiny and EP-rank workloads beside it)")
    ap.add_argument("--no-extra", action="store_true",
                    help="time the prefill headline alone")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--router", default="softmax", choices=["softmax", "sigmoid-groups"],
                    help="softmax: the default router; sigmoid-groups: sigmoid scores, route "
                         "scale 2.5, 8 expert groups of which 4 are kept, a selection-only "
                         "expert bias")
    ap.add_argument("--shared-I", type=int, default=0,
                    help="intermediate size of a shared expert (0: none)")
    ap.add_argument("--backward", action="store_true",
                    help="time moe_layer_backward (after one moe_layer_forward_train)")
    return ap.parse_args()


BWD_STAGES = ("permute", "dgrad_down_swiglu_dw", "dgrad_gate_up_dx", "wgrad_down",
              "wgrad_gate_up", "router_wgrad")


def algorithmic_backward(wl, counts, Is=0):
    """Per-stage algorithmic FLOPs and HBM bytes of one layer backward.
    Weights and weight gradients count once per expert (every expert's
    gradient is written); rows count once per read or write."""
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.top_k
    es = 2
    N = T * k
    hit = int((counts > 0).sum())
    f = {
        "permute": 0.0,
        # dout . down^T, then <., h> for the routing weights' gradient
        "dgrad_down_swiglu_dw": 2.0 * N * H * I + 2.0 * N * I,
        "dgrad_gate_up_dx": 2.0 * N * 2 * I * H,
        "wgrad_down": 2.0 * N * I * H,
        "wgrad_gate_up": 2.0 * N * H * 2 * I,
        "router_wgrad": 2.0 * N * H if wl.norm_topk_prob else 2.0 * T * E * H,
    }
    b = {
        # ids in; counts, offsets and the three index maps out
        "permute": N * 4 + 3 * N * 4,
        # down, dout and G in; dG and hw out; logits in, dL out
        "dgrad_down_swiglu_dw": hit * I * H * es + T * H * es + 2 * N * 2 * I * es + N * I * es
        + 2 * T * E * 4,
        "dgrad_gate_up_dx": hit * H * 2 * I * es + N * 2 * I * es + 2 * N * H * es + T * H * es,
        "wgrad_down": N * I * es + T * H * es + E * I * H * es,
        "wgrad_gate_up": N * 2 * I * es + T * H * es + E * H * 2 * I * es,
        "router_wgrad": T * H * es + T * E * 4 + E * H * 4,
    }
    if Is:
        # the shared expert: its dgrads run in the third stage, its wgrads
        # after the router's weight gradient
        f["dgrad_gate_up_dx"] += 6.0 * T * H * Is
        b["dgrad_gate_up_dx"] += 3 * H * Is * es + 3 * T * 2 * Is * es + 2 * T * H * es
        f["router_wgrad"] += 6.0 * T * H * Is
        b["router_wgrad"] += 3 * H * Is * es + 3 * T * Is * es + 2 * T * H * es
    return f, b


def dense_gemm_context(wl):
    """Context only (never on the path): torch's batched bf16 GEMM over the
    experts at the average expert's gate_up shape, as a ceiling check."""
    import torch
    E, H, I = wl.E, wl.H, wl.I
    m = max(16, wl.T * wl.top_k // E)
    g = torch.Generator(device="cuda").manual_seed(7)
    a = torch.randn(E, m, H, device="cuda", generator=g).to(torch.bfloat16)
    b = torch.randn(E, H, 2 * I, device="cuda", generator=g).to(torch.bfloat16).contiguous()
    for _ in range(3):
        torch.bmm(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        torch.bmm(a, b)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    return {"torch_bmm_bf16": f"{E} x [{m},{H}] x [{H},{2 * I}]",
            "ms": round(ms, 4), "tflops": round(2.0 * E * m * H * 2 * I / (ms * 1e-3) / 1e12, 1)}


def cpu_baseline_backward(wl, dout, budget_s=12.0):
    import numpy as np
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    args = [t.float().numpy() for t in (wl.hidden_states, wl.router_weight, wl.gate_up, wl.down)]
    bias = wl.router_bias.numpy() if wl.router_bias is not None else None
    d = dout.float().numpy()
    runs, t0 = 0, time.perf_counter()
    while True:
        O.moe_layer_backward(args[0], args[1], bias, args[2], args[3], wl.top_k,
                             wl.norm_topk_prob, d)
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s or runs >= 3:
            break
    return {"value": wl.T * wl.top_k * runs / el, "unit": "routed tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"whole {wl.name} workload ({wl.T} tokens), forward recomputed inside, "
                      f"{runs} run(s), {el:.1f} s, float64 NumPy"}


def bench_ep_rank(args, wl, cpu=True):
    """One expert-parallel rank: rows received rank-major from R source
    ranks (built untimed with the library's router and torch indexing), then
    the timed span moe_permute (rank-major reshuffle) -> moe_grouped_swiglu
    (rows gathered in the loads, outputs scattered back to rank-major)."""
    import numpy as np
    import torch

    import mixture_experts_layer_17_amd as moe
    from mixture_experts_layer_17_amd import _lib
    dev = torch.device("cuda:0")
    R, H, I, El, k = wl.R, wl.H, wl.I, wl.E_local, wl.top_k
    wr = wl.router_weight.to(dev)
    rows, C = [], torch.zeros(R, El, dtype=torch.int32)
    for r in range(R):
        xr = wl.source_hidden[r].to(dev)
        _, ids, _, _ = moe.route(xr, wr, k, wl.norm_topk_prob)
        loc = ids.long() - wl.local_lo
        t_idx = torch.arange(xr.shape[0], device=dev).unsqueeze(1).expand_as(loc)
        sel = (loc >= 0) & (loc < El)
        e_sel, t_sel = loc[sel], t_idx[sel]
        order = torch.sort(e_sel * xr.shape[0] + t_sel, stable=True).indices
        rows.append(xr[t_sel[order]])
        C[r] = torch.bincount(e_sel, minlength=El).to(torch.int32).cpu()
    x_rm = torch.cat(rows).contiguous()
    N = x_rm.shape[0]
    C_d = C.to(dev)
    gu, dn = wl.gate_up.to(dev), wl.down.to(dev)
    perm = {n: torch.empty(sz, dtype=torch.int32, device=dev)
            for n, sz in (("counts", El), ("offsets", El + 1), ("sorted_token", N),
                          ("sorted_slot", N), ("slot_pos", N))}
    y = torch.empty(N, H, dtype=wl.dtype, device=dev)
    L = moe.lib
    nb_p = L.moe_workspace_size(_lib.MOE_OP_PERMUTE, 0, 0, 0, El, 1, R, N, _lib.MOE_BF16)
    nb_g = L.moe_workspace_size(_lib.MOE_OP_GROUPED_SWIGLU, 0, H, I, El, 1, 0, N, _lib.MOE_BF16)
    ws_p = torch.empty(max(nb_p, 1), dtype=torch.uint8, device=dev)
    ws_g = torch.empty(max(nb_g, 1), dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream(dev)
    P = lambda t: t.data_ptr()  # noqa: E731

    def step(evs=None):
        if evs:
            evs[0].record(s)
        st = L.moe_permute(None, 0, 1, P(C_d), R, N, El, P(perm["counts"]), P(perm["offsets"]),
                           P(perm["sorted_token"]), P(perm["sorted_slot"]), P(perm["slot_pos"]),
                           P(ws_p), nb_p, s.cuda_stream)
        if evs:
            evs[1].record(s)
        st = st or L.moe_grouped_swiglu(P(x_rm), N, P(perm["sorted_token"]),
                                        P(perm["sorted_token"]), P(perm["offsets"]), N, H, I, El,
                                        P(gu), P(dn), _lib.MOE_BF16, P(y), P(ws_g), nb_g,
                                        s.cuda_stream)
        if evs:
            evs[2].record(s)
        if st != 0:
            raise RuntimeError(f"EP rank step failed with status {st}")

    for _ in range(args.warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(s)
    for i in range(args.steps):
        step(evs[i])
    end.record(s)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_per_step = start.elapsed_time(end) / args.steps
    perm_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    gemm_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    steps = [e[0].elapsed_time(e[2]) for e in evs]
    counts = C.sum(0).numpy()
    hit = int((counts > 0).sum())
    flops = 6.0 * N * H * I
    bytes_ = hit * 3 * H * I * 2 + 2 * N * H * 2
    roof = {"bound": "mfma", "achieved": round(flops / (gemm_ms * 1e-3) / 1e12, 2),
            "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof.update(traffic=None, kernel="grouped_swiglu (both GEMMs)", algorithmic_flops=int(flops),
                algorithmic_bytes=int(bytes_))
    result = {
        "metric": "routed rows/s per EP-rank expert pass (rank-major reshuffle + grouped SwiGLU "
                  "+ reverse), bf16",
        "value": round(N / (ms_per_step * 1e-3), 1), "unit": "routed rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded Gaussian source tokens routed by the library's router",
        "config": {"workload": wl.name, "R": R, "T_per_rank": wl.T_per_rank, "H": H, "I": I,
                   "E": wl.E, "E_local": El, "top_k": k, "routed_rows": N, "experts_hit": hit},
        "layer_tflops": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "layer_mfma_frac": round(flops / (ms_per_step * 1e-3) / PEAK_BF16_FLOPS, 4),
        "roofline": roof,
        "kernels": {"permute_rank_major": {"avg_us": round(perm_ms * 1e3, 2)},
                    "grouped_swiglu": {"avg_us": round(gemm_ms * 1e3, 2),
                                       "tflops": roof["achieved"]}},
        "step_ms": {"warm_median": round(float(np.median(steps)), 4),
                    "warm_min": round(float(np.min(steps)), 4)},
        "wall_s_timed": round(t_wall, 3),
    }
    if cpu and not args.no_cpu_baseline:
        from oracle import moe_oracle as O
        n0 = int(C[0].sum())
        xs = x_rm[:n0].float().cpu().numpy()
        gu_c, dn_c = wl.gate_up.float().numpy(), wl.down.float().numpy()
        t0 = time.perf_counter()
        O.ep_rank_forward(xs, C[:1].numpy(), gu_c, dn_c)
        el = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": n0 / el, "unit": "routed rows/s", "cores":
                                  os.cpu_count(), "kind": "oracle",
                                  "sample": f"source rank 0's {n0} received rows, one run, "
                                            f"{el:.1f} s, float64 NumPy"}
    return result


def bench_backward(args, wl):
    import numpy as np
    import torch

    import workloads
    import mixture_experts_layer_17_amd as moe
    from mixture_experts_layer_17_amd import _lib
    dev = torch.device("cuda:0")
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.top_k
    N = T * k
    norm = wl.norm_topk_prob
    x, wr, gu, dn = (t.to(dev).contiguous() for t in (wl.hidden_states, wl.router_weight,
                                                       wl.gate_up, wl.down))
    bias = wl.router_bias.to(dev) if wl.router_bias is not None else None
    dout_cpu = torch.randn(T, H, generator=torch.Generator().manual_seed(100)).to(wl.dtype)
    dout = dout_cpu.to(dev)
    Is = args.shared_I
    sh = sh_t = None
    if Is:
        w1, w2, w3 = workloads.shared_expert_weights(H, Is, wl.dtype)
        sh_t = (torch.cat([w1.t(), w3.t()], dim=1).contiguous().to(dev),
                w2.t().contiguous().to(dev))
        sh = moe.shared_expert(*sh_t)
    _, saved = moe.layer_forward_train(x, wr, gu, dn, k, norm, router_bias=bias, shared=sh_t)
    g = dict(dx=torch.empty(T, H, dtype=wl.dtype, device=dev),
             dwr=torch.empty(E, H, dtype=torch.float32, device=dev),
             db=torch.empty(E, dtype=torch.float32, device=dev),
             dgu=torch.empty(E, H, 2 * I, dtype=wl.dtype, device=dev),
             ddn=torch.empty(E, I, H, dtype=wl.dtype, device=dev),
             dw=torch.empty(T, k, dtype=torch.float32, device=dev),
             dsgu=torch.empty(H, 2 * Is, dtype=wl.dtype, device=dev) if Is else None,
             dsdn=torch.empty(Is, H, dtype=wl.dtype, device=dev) if Is else None)
    L = moe.lib
    nws = L.moe_workspace_size(_lib.MOE_OP_LAYER_BACKWARD, T, H, I, E, k, Is, N, _lib.MOE_BF16)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream(dev)
    P = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    nst = len(BWD_STAGES) + 1

    def new_event():
        ev = ctypes.c_void_p()
        if hip.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev

    sv = _lib.TrainSaved(P(saved["gate_up_out"]), P(saved["expert_out"]),
                         P(saved["shared_gate_up_out"]))
    gr = _lib.LayerGrads(P(g["dx"]), P(g["dwr"]), P(g["db"]), P(g["dgu"]), P(g["ddn"]),
                         P(g["dw"]), P(g["dsgu"]), P(g["dsdn"]))
    sh_p = ctypes.addressof(sh) if sh is not None else None

    def step(evs=None):
        st = L.moe_layer_backward(P(x), P(wr), P(gu), P(dn), T, H, I, E, k, int(norm),
                                  _lib.MOE_BF16, None, sh_p, P(saved["router_logits"]),
                                  P(saved["topk_ids"]), P(saved["topk_weights"]),
                                  ctypes.addressof(sv), P(dout), ctypes.addressof(gr), P(ws), nws,
                                  evs, s.cuda_stream)
        if st != 0:
            raise RuntimeError(f"moe_layer_backward failed with status {st}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev_arrays = [(ctypes.c_void_p * nst)(*[new_event() for _ in range(nst)])
                 for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(s)
    for i in range(args.steps):
        step(ev_arrays[i])
    end.record(s)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_per_step = start.elapsed_time(end) / args.steps
    f = ctypes.c_float()
    per = {}
    for j, name in enumerate(BWD_STAGES):
        acc = []
        for arr in ev_arrays:
            if hip.hipEventElapsedTime(ctypes.byref(f), arr[j], arr[j + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            acc.append(f.value)
        per[name] = float(np.mean(acc))
    for arr in ev_arrays:
        for j in range(nst):
            hip.hipEventDestroy(arr[j])
    flops, bytes_ = algorithmic_backward(wl, saved["num_tokens_per_expert"].cpu().numpy(), Is)
    kern = {}
    for name in BWD_STAGES:
        t_s = per[name] * 1e-3
        kern[name] = {"avg_us": round(per[name] * 1e3, 2),
                      "tflops": round(flops[name] / t_s / 1e12, 2),
                      "gbps": round(bytes_[name] / t_s / 1e9, 1),
                      "mfma_frac": round(flops[name] / t_s / PEAK_BF16_FLOPS, 4),
                      "hbm_frac": round(bytes_[name] / t_s / PEAK_HBM, 4)}
    dom = max(BWD_STAGES, key=lambda n_: per[n_])
    t_dom = per[dom] * 1e-3
    if bytes_[dom] / PEAK_HBM >= flops[dom] / PEAK_BF16_FLOPS:
        roof = {"bound": "hbm", "achieved": round(bytes_[dom] / t_dom / 1e9, 1),
                "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(flops[dom] / t_dom / 1e12, 2),
                "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    # the counters were taken for the layer without a shared expert
    roof["traffic"] = load_traffic(dom, wl.name) if Is == 0 else None
    roof["kernel"] = dom
    roof["algorithmic_bytes"] = int(bytes_[dom])
    roof["algorithmic_flops"] = int(flops[dom])
    total_f = sum(flops.values())
    result = {
        "metric": "routed tokens/s per MoE layer backward (bf16)",
        "value": round(N / (ms_per_step * 1e-3), 1),
        "unit": "routed tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded Gaussian inputs, output gradient and random-init weights",
        "config": {"workload": wl.name, "T": T, "H": H, "I": I, "E": E, "top_k": k,
                   "norm_topk_prob": norm, "routed_rows": N, "pass": "backward",
                   "shared_I": Is},
        "layer_tflops": round(total_f / (ms_per_step * 1e-3) / 1e12, 2),
        "layer_mfma_frac": round(total_f / (ms_per_step * 1e-3) / PEAK_BF16_FLOPS, 4),
        "roofline": roof,
        "kernels": kern,
        "wall_s_timed": round(t_wall, 3),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_backward(wl, dout_cpu)
    print(json.dumps(result), flush=True)


def algorithmic(wl, counts, Is=0, fused=False):
    """Per-kernel algorithmic FLOPs and HBM bytes for one layer pass.

    Bytes count what the method itself must move: each hit expert's weights
    once, the router weight, the hidden states each kernel has to read, the
    router's outputs and the layer output.  The intermediates of this
    implementation (h between the GEMMs, the per-slot expert outputs Y
    between the second GEMM and the combine, the index maps) are not
    algorithmic; they are returned separately as ``moved`` (bytes each
    kernel actually reads and writes, intermediates included).  The layer's
    algorithmic bytes count the hidden states once."""
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.top_k
    es = 2 if wl.dtype.itemsize == 2 else 4
    N = T * k
    hit = int((counts > 0).sum())
    f = {
        "route": 2.0 * T * H * E,
        "permute": 0.0,
        "gate_up_swiglu": 2.0 * N * H * 2 * I,
        "down": 2.0 * N * I * H,
        "combine": 2.0 * N * H,
    }
    b = {
        "route": T * H * es + E * H * es + T * E * 4 + T * k * 8,
        "permute": 0,
        "gate_up_swiglu": hit * H * 2 * I * es + T * H * es,
        "down": hit * I * H * es,
        "combine": T * H * es,
    }
    moved = {
        "route": b["route"],
        "permute": N * 4 * 5,
        "gate_up_swiglu": b["gate_up_swiglu"] + N * I * es,
        "down": b["down"] + N * I * es + N * H * es,
        "combine": b["combine"] + N * H * es + N * 4,
    }
    layer_b = hit * 3 * H * I * es + E * H * es + 2 * T * H * es + T * E * 4 + T * k * 8
    if Is and fused:
        # the shared expert inside the grouped launches: its weights once; x
        # is read once more, its h and output are intermediates
        f["gate_up_swiglu"] += 2.0 * T * H * 2 * Is
        b["gate_up_swiglu"] += H * 2 * Is * es
        moved["gate_up_swiglu"] += H * 2 * Is * es + T * H * es + T * Is * es
        f["down"] += 2.0 * T * Is * H
        b["down"] += Is * H * es
        moved["down"] += Is * H * es + T * Is * es + T * H * es
        moved["combine"] += T * H * es
    elif Is:
        # on its own, in the last stage with the combine
        f["combine"] += 2.0 * T * H * 2 * Is + 2.0 * T * Is * H
        b["combine"] += 3 * H * Is * es
        moved["combine"] += 3 * H * Is * es + T * H * es + 2 * T * Is * es + 2 * T * H * es
    if Is:
        layer_b += 3 * H * Is * es
    return f, b, moved, layer_b, hit


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))


def cpu_baseline(wl, budget_s=12.0, shared=None):
    """The CPU oracle, as it stands, on this host: the whole workload, run
    until about budget_s seconds of work are done (at least once)."""
    import numpy as np
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    x = wl.hidden_states.float().numpy()
    wr = wl.router_weight.float().numpy()
    gu = wl.gate_up.float().numpy()
    dn = wl.down.float().numpy()
    bias = wl.router_bias.numpy() if wl.router_bias is not None else None
    runs, t0 = 0, time.perf_counter()
    while True:
        O.moe_layer_forward(x, wr, bias, gu, dn, wl.top_k, wl.norm_topk_prob, shared=shared)
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s or runs >= 5:
            break
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": wl.T * wl.top_k * runs / el, "unit": "routed tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"whole {wl.name} workload ({wl.T} tokens, all experts), {runs} run(s), "
                      f"{el:.1f} s, float64 NumPy per-expert loop on {cpu}, "
                      f"affinity {len(os.sched_getaffinity(0))} cpus"}


def source_sha(path):
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def load_traffic(kernel: str, workload: str):
    """HBM traffic of a kernel from committed rocprofv3 counter summaries,
    only while the kernel source still matches the one measured."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        t = json.load(fh)
    # every source the measured kernels are built from must be unchanged
    shas = t.get("sources") or {t["source"]: t.get("source_sha256")}
    for rel, sha in shas.items():
        src = os.path.join(ROOT, rel)
        if not os.path.exists(src) or source_sha(src) != sha:
            return None
    return t.get("traffic_bytes")


def graph_replay(torch, step, s, steps, warmup):
    """The same layer call captured once in a HIP graph (as a serving loop
    would run it), replayed `warmup` times untimed, then `steps` times: the
    per-step time without the host's launch gaps."""
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(stream=torch.cuda.current_stream().cuda_stream)
        for _ in range(max(warmup, 1)):
            g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        for _ in range(steps):
            g.replay()
        b.record(s)
        torch.cuda.synchronize()
        return {"ms_per_step": round(a.elapsed_time(b) / steps, 4), "steps": steps}
    except RuntimeError as err:   # reported, never fatal to the bench line
        return {"error": str(err)[:200]}


def run_forward(args, wl, router="softmax", Is=0, context=True):
    """Times moe_layer_forward_ex on one workload; returns the measured
    fields of the JSON line (no CPU baseline)."""
    import numpy as np
    import torch

    import mixture_experts_layer_17_amd as moe
    import workloads
    from mixture_experts_layer_17_amd import _lib

    dev = torch.device("cuda:0")
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.top_k
    N = T * k
    bf16 = wl.dtype == torch.bfloat16
    dt = _lib.MOE_BF16 if bf16 else _lib.MOE_F32
    x, wr, gu, dn = (t.to(dev).contiguous() for t in (wl.hidden_states, wl.router_weight,
                                                       wl.gate_up, wl.down))
    bias = wl.router_bias.to(dev) if wl.router_bias is not None else None
    f32, i32 = torch.float32, torch.int32
    logits = torch.empty(T, E, dtype=f32, device=dev)
    ids = torch.empty(T, k, dtype=i32, device=dev)
    w = torch.empty(T, k, dtype=f32, device=dev)
    counts = torch.empty(E, dtype=i32, device=dev)
    out = torch.empty(T, H, dtype=wl.dtype, device=dev)
    L = moe.lib

    cfg = None
    if router == "sigmoid-groups":
        g = torch.Generator().manual_seed(1)
        ebias = (torch.randn(E, generator=g) * 0.05).to(dev)
        cfg = moe.router_config("sigmoid", 2.5, ebias, 8, 4)
    cfg_p = ctypes.addressof(cfg) if cfg is not None else None
    sh_p = None
    fused = False
    kernels = KERNELS
    if Is:
        w1, w2, w3 = workloads.shared_expert_weights(H, Is, wl.dtype)
        sgu = torch.cat([w1.t(), w3.t()], dim=1).contiguous().to(dev)
        sdn = w2.t().contiguous().to(dev)
        sh = moe.shared_expert(sgu, sdn)
        sh_p = ctypes.addressof(sh)
        # bf16 with Is a multiple of 128: the library runs the shared expert
        # inside the two grouped GEMM launches, else in the last stage
        fused = bf16 and Is % 128 == 0
        if not fused:
            kernels = KERNELS[:-1] + ("shared_ffn_combine",)
    nws = L.moe_workspace_size(_lib.MOE_OP_LAYER, T, H, I, E, k, Is, N, dt)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream(dev)
    sp = s.cuda_stream
    P = lambda t: t.data_ptr() if t is not None else None  # noqa: E731

    # HIP events for the per-stage split, recorded by the library between its
    # kernels on the same stream (the layer is launched exactly as users do)
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    nst = len(KERNELS) + 1

    def new_event():
        ev = ctypes.c_void_p()
        if hip.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev

    def step(evs=None, stream=None):
        st = L.moe_layer_forward_ex(P(x), P(wr), P(bias), P(gu), P(dn), T, H, I, E, k,
                                    int(wl.norm_topk_prob), dt, cfg_p, sh_p, P(out), P(logits),
                                    P(ids), P(w), P(counts), P(ws), nws, evs,
                                    sp if stream is None else stream)
        if st != 0:
            raise RuntimeError(f"moe_layer_forward failed with status {st}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev_arrays = []
    for _ in range(args.steps):
        arr = (ctypes.c_void_p * nst)(*[new_event() for _ in range(nst)])
        ev_arrays.append(arr)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(s)
    for i in range(args.steps):
        step(ev_arrays[i])
    end.record(s)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    per_kernel_ms = {}
    f = ctypes.c_float()
    for j, kname in enumerate(kernels):
        acc = []
        for arr in ev_arrays:
            if hip.hipEventElapsedTime(ctypes.byref(f), arr[j], arr[j + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            acc.append(f.value)
        per_kernel_ms[kname] = float(np.mean(acc))

    def step_times(arrs):
        out_ = []
        for arr in arrs:
            if hip.hipEventElapsedTime(ctypes.byref(f), arr[0], arr[nst - 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out_.append(f.value)
        return out_

    warm = step_times(ev_arrays)
    # cold: a 512 MB scratch write before each step evicts L2 and the MALL;
    # each step is timed on its own by its first and last stage events
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for i in range(args.steps):
        scratch.fill_(i & 255)
        step(ev_arrays[i])
    torch.cuda.synchronize()
    cold = step_times(ev_arrays)
    del scratch
    for arr in ev_arrays:
        for j in range(nst):
            hip.hipEventDestroy(arr[j])
    graph = graph_replay(torch, step, s, args.steps, args.warmup)
    ctx = dense_gemm_context(wl) if (context and bf16) else None

    c_np = counts.cpu().numpy()
    flops, bytes_, moved, layer_bytes, hit = algorithmic(wl, c_np, Is, fused)
    flops = dict(zip(kernels, flops.values()))
    bytes_ = dict(zip(kernels, bytes_.values()))
    moved = dict(zip(kernels, moved.values()))
    peak_f = PEAK_BF16_FLOPS if bf16 else PEAK_F32_FLOPS
    kern = {}
    for kname in kernels:
        t_s = per_kernel_ms[kname] * 1e-3
        kern[kname] = {
            "avg_us": round(per_kernel_ms[kname] * 1e3, 2),
            "tflops": round(flops[kname] / t_s / 1e12, 2),
            "gbps": round(bytes_[kname] / t_s / 1e9, 1),
            "gbps_moved": round(moved[kname] / t_s / 1e9, 1),
            "mfma_frac": round(flops[kname] / t_s / peak_f, 4),
            "hbm_frac": round(bytes_[kname] / t_s / PEAK_HBM, 4),
        }
    dom = max(kernels, key=lambda n: per_kernel_ms[n])
    t_dom = per_kernel_ms[dom] * 1e-3
    hbm_floor = bytes_[dom] / PEAK_HBM
    mfma_floor = flops[dom] / peak_f
    if hbm_floor >= mfma_floor:
        roof = {"bound": "hbm", "achieved": round(bytes_[dom] / t_dom / 1e9, 1),
                "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(flops[dom] / t_dom / 1e12, 2),
                "peak": peak_f / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    # the counters were taken for the softmax router without a shared expert
    plain = Is == 0 and router == "softmax"
    roof["traffic"] = load_traffic(dom, wl.name) if plain else None
    roof["kernel"] = dom
    roof["algorithmic_bytes"] = int(bytes_[dom])
    roof["algorithmic_flops"] = int(flops[dom])
    roof["bytes_moved"] = int(moved[dom])

    layer_flops = sum(flops.values())
    # the headline step time is the graph replay's (the same kernels on the
    # same inputs, bit-identical outputs, without the host's launch gaps);
    # the eager stream's time stays next to it
    eager_ms = ms_per_step
    if "ms_per_step" in graph:
        ms_per_step = graph["ms_per_step"]
    t_layer = ms_per_step * 1e-3
    return {
        "value": round(N / t_layer, 1),
        "ms_per_step": round(ms_per_step, 4),
        "dtype": "bf16" if bf16 else "f32",
        "config": {"workload": wl.name, "T": T, "H": H, "I": I, "E": E, "top_k": k,
                   "norm_topk_prob": wl.norm_topk_prob, "routed_rows": N,
                   "experts_hit": hit, "router": router, "shared_I": Is},
        "layer_tflops": round(layer_flops / t_layer / 1e12, 2),
        "layer_mfma_frac": round(layer_flops / t_layer / peak_f, 4),
        "layer_algorithmic_bytes": int(layer_bytes),
        "layer_hbm_gbps": round(layer_bytes / t_layer / 1e9, 1),
        "layer_hbm_frac": round(layer_bytes / t_layer / PEAK_HBM, 4),
        "roofline": roof,
        "kernels": kern,
        "step_ms": {"warm_median": round(float(np.median(warm)), 4),
                    "warm_min": round(float(np.min(warm)), 4),
                    "cold_median": round(float(np.median(cold)), 4),
                    "cold_min": round(float(np.min(cold)), 4)},
        "timing": "hip_graph_replay" if "ms_per_step" in graph else "eager_stream",
        "eager_ms_per_step": round(eager_ms, 4),
        "graph": graph,
        "context": ctx,
        "wall_s_timed": round(t_wall, 3),
    }


def compact(r: dict) -> dict:
    """The fields of a secondary workload kept in the headline line."""
    keep = ("value", "unit", "ms_per_step", "eager_ms_per_step", "dtype", "layer_tflops",
            "layer_mfma_frac", "layer_hbm_gbps", "layer_hbm_frac", "roofline", "step_ms")
    c = {k_: r[k_] for k_ in keep if k_ in r}
    c["config"] = r["config"]
    c["kernels_us"] = {n: v["avg_us"] for n, v in r["kernels"].items()}
    return c


# Secondary workloads timed next to the headline when bench.py runs with no
# --workload: the decode layer (graded on its HBM fraction), the skewed
# batch, the tiny float32 layer and one expert-parallel rank's share.
EXTRA_WORKLOADS = ("qwen3_30b_a3b_decode", "qwen3_30b_a3b_skewed", "tiny_fp32", "ep_rank_235b")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", args.gpus))
    if args.gpus > 1 or world > 1:
        print("bench.py measures one GPU only: the MoE layer forward here has no multi-GPU "
              "path (no collectives); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch

    import mixture_experts_layer_17_amd  # noqa: F401  (fails loudly without libmoe.so)
    import workloads

    name = args.workload or "qwen3_30b_a3b_prefill"
    wl = workloads.make(name)
    if not hasattr(wl, "T"):
        print(json.dumps(bench_ep_rank(args, wl)), flush=True)
        return
    if args.backward:
        bench_backward(args, wl)
        return
    r = run_forward(args, wl, args.router, args.shared_I)
    result = {"metric": METRIC, "value": r["value"], "unit": "routed tokens/s", "n_gpus": 1,
              "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["ms_per_step"],
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": r["dtype"],
              "data": "synthetic: seeded Gaussian inputs and random-init weights of the named "
                      "layer shape"}
    result.update({k_: v for k_, v in r.items() if k_ not in result})
    result["host"] = platform.node()
    del wl
    if args.workload is None and not args.no_extra:
        extra = {}
        for xname in EXTRA_WORKLOADS:
            xw = workloads.make(xname)
            if hasattr(xw, "T"):
                xr = run_forward(args, xw, context=False)
                xr["unit"] = "routed tokens/s"
            else:
                xr = bench_ep_rank(args, xw, cpu=False)
            extra[xname] = compact(xr)
            del xw
            torch.cuda.empty_cache()
        result["workloads"] = extra
    if not args.no_cpu_baseline:
        sh_w = (tuple(t.float().numpy() for t in workloads.shared_expert_weights(
            r["config"]["H"], args.shared_I, workloads.make(name).dtype))
            if args.shared_I else None)
        result["cpu_baseline"] = cpu_baseline(workloads.make(name), shared=sh_w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
