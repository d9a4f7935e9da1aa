"""moe_layer_forward_noalloc -- the layer forward whose workspace is the
library's static device scratch array -- against moe_layer_forward_ex with a
caller workspace, through the C ABI (MI355X only).

Two calls in a row on the same GPU, the second with fewer tokens (so the
array still holds the first call's contents), each bit-identical to the
workspace entry point on the same inputs: the two run the same kernels in
the same order, so every output matches exactly.  Every case prints its
name (flushed) before touching the GPU."""
from __future__ import annotations

import ctypes

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mixture_experts_layer_17_amd as m
    return m


def _noalloc(moe, x, wr, gu, dn, k, norm, shared=None):
    T, H = x.shape
    E = wr.shape[0]
    I = gu.shape[2] // 2
    dev = x.device
    out = torch.empty(T, H, dtype=x.dtype, device=dev)
    logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    w = torch.empty(T, k, dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    sh = moe.shared_expert(*shared) if shared is not None else None
    dt = moe._lib.MOE_BF16 if x.dtype == torch.bfloat16 else moe._lib.MOE_F32
    st = moe.lib.moe_layer_forward_noalloc(
        x.data_ptr(), wr.data_ptr(), None, gu.data_ptr(), dn.data_ptr(), T, H, I, E, k,
        int(norm), dt, None, ctypes.addressof(sh) if sh is not None else None, out.data_ptr(),
        logits.data_ptr(), ids.data_ptr(), w.data_ptr(), counts.data_ptr(), None,
        torch.cuda.current_stream(dev).cuda_stream)
    assert st == 0, f"moe_layer_forward_noalloc: {moe._lib.STATUS.get(st, st)}"
    return out, logits, ids, w, counts


# (workload, token counts of the two calls): decode-sized calls take the
# small-batch router; 1024 and 600 tokens the split-K router with the
# permutation's first pass folded into it, near the array's limit
@pytest.mark.parametrize("shared_I", [0, 768])
@pytest.mark.parametrize("name,Ts", [("qwen3_30b_a3b_decode", (64, 16)),
                                     ("qwen3_30b_a3b_prefill", (1024, 600))])
def test_noalloc_matches_workspace_entry_point(moe, name, Ts, shared_I):
    wl = workloads.make(name)
    x_all, wr, gu, dn = (t.to(DEV) for t in (wl.hidden_states, wl.router_weight, wl.gate_up,
                                             wl.down))
    shared = None
    if shared_I:
        w1, w2, w3 = workloads.shared_expert_weights(wl.H, shared_I, wl.dtype)
        shared = (torch.cat([w1.t(), w3.t()], dim=1).contiguous().to(DEV),
                  w2.t().contiguous().to(DEV))
    for T in Ts:   # the second call is smaller
        say(f"noalloc layer T={T} H={wl.H} I={wl.I} E={wl.E} k={wl.top_k} shared_I={shared_I}")
        x = x_all[:T].contiguous()
        got = _noalloc(moe, x, wr, gu, dn, wl.top_k, wl.norm_topk_prob, shared)
        ref = moe.layer_forward(x, wr, gu, dn, wl.top_k, wl.norm_topk_prob, shared=shared)
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "logits", "ids", "weights", "counts"), got, ref):
            assert torch.equal(a, b), f"T={T}: {name} differs from moe_layer_forward_ex"
        assert int(got[4].sum()) == T * wl.top_k
