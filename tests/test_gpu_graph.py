"""The layer forward captured once in a HIP graph and replayed (MI355X only).

A serving loop that cannot afford host launch gaps captures the layer call
once and replays it.  The forward enqueues kernels only (no memset, copy,
allocation or host synchronisation inside the call), so every replay must
give the eager call's outputs bit for bit.  Each replay is preceded by
eager work of the program's own (another layer call on other tokens and a
fill of the captured outputs) and a synchronisation, and every replay is
checked, not only the first.
"""
from __future__ import annotations

import pytest
import torch

import workloads

pytestmark = [pytest.mark.gpu]

DEV = "cuda"


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mixture_experts_layer_17_amd as m
    return m


def _shared(H, Is, dtype):
    w1, w2, w3 = workloads.shared_expert_weights(H, Is, dtype)
    return (torch.cat([w1.t(), w3.t()], dim=1).contiguous().to(DEV),
            w2.t().contiguous().to(DEV))


@pytest.mark.parametrize("name,T,Is", [("qwen3_30b_a3b_decode", None, 0),
                                       ("graph_small", 300, 256)])
def test_layer_forward_graph_replays_match_eager(moe, name, T, Is):
    print(f"\n[case] graph replay {name} T={T} shared_I={Is}", flush=True)
    if T is None:
        wl = workloads.make(name)
    else:
        wl = workloads.make_layer(name, T=T, H=512, I=256, E=16, top_k=4, seed=21)
    x, wr, gu, dn = (t.to(DEV) for t in (wl.hidden_states, wl.router_weight, wl.gate_up,
                                          wl.down))
    k, norm = wl.top_k, wl.norm_topk_prob
    sh = _shared(wl.H, Is, wl.dtype) if Is else None
    buf = moe.LayerBuffers(wl.T, wl.H, wl.I, wl.E, k, wl.dtype, DEV, Is)
    ref = [t.clone() for t in moe.layer_forward(x, wr, gu, dn, k, norm, buffers=buf, shared=sh)]
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.layer_forward(x, wr, gu, dn, k, norm, buffers=buf, shared=sh)
    torch.cuda.synchronize()

    x2 = torch.flip(x, dims=[0]).contiguous()
    for r in range(4):
        # eager work between replays: clear what the replay must rewrite, run
        # the layer on other tokens with its own buffers
        for t in (buf.out, buf.logits, buf.weights):
            t.fill_(float("nan"))
        buf.ids.fill_(-1)
        buf.counts.fill_(-1)
        moe.layer_forward(x2, wr, gu, dn, k, norm, shared=sh)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (buf.out, buf.logits, buf.ids, buf.weights, buf.counts)
        for what, a, b in zip(("out", "logits", "ids", "weights", "counts"), got, ref):
            assert torch.equal(a, b), f"replay {r}: {what} differs from the eager call"
    print("  4 replays bit-identical to the eager call", flush=True)
