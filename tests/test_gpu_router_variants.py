"""Router variants and the expert-bias update on the GPU against the oracle
(MI355X only): sigmoid / softmax scores, route scale, selection-only expert
bias, node-limited groups, the selection accumulator, and the layer forward
with a variant router.

Selection is decided in float32 on both sides but through different exp
implementations, so the oracle's selection runs on the GPU's own float32
logits and a token whose selection (or group) boundary is closer than a few
float32 ulps of the keys may still differ; such tokens are checked for
validity, every other token bit for bit, and the layer is compared on every
token against the oracle run on the GPU's routing.  Every case prints its
name (flushed) before touching the GPU.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from oracle import moe_oracle as O
from tests import parity_util as U

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

DEV = "cuda"


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mixture_experts_layer_17_amd as m
    return m


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def _variant_ref(logits, k, norm, v):
    return O.route_variant(logits, k, norm, v["score_func"], v["route_scale"], v.get("bias"),
                           v.get("groups", 0), v.get("limited", 0))


def check_route(moe, wl, v, norm, T=None):
    x = wl.hidden_states[:T] if T else wl.hidden_states
    say(f"route variant {wl.name} T={x.shape[0]} E={wl.E} k={wl.top_k} norm={norm} {v}")
    E, k = wl.E, wl.top_k
    bias = v.get("bias")
    tpe = torch.zeros(E, dtype=torch.float32, device=DEV)
    cfg = moe.router_config(v["score_func"], v["route_scale"],
                            torch.as_tensor(bias, dtype=torch.float32, device=DEV)
                            if bias is not None else None,
                            v.get("groups", 0), v.get("limited", 0), tpe)
    xg, wrg = x.to(DEV), wl.router_weight.to(DEV)
    logits, ids, w, counts = moe.route(xg, wrg, k, norm, config=cfg)
    torch.cuda.synchronize()
    logits, ids, w, counts = (t.cpu().numpy() for t in (logits, ids, w, counts))
    ref_logits = O.router_logits(x.float().numpy(), wl.router_weight.float().numpy())
    U.assert_close(torch.as_tensor(logits), ref_logits, wl.dtype, "router logits")
    # the oracle's selection from the GPU's own float32 logits
    rid, rw, rs, rkey = _variant_ref(logits, k, norm, v)
    dec, same = U.variant_routing_check(ids, rkey, rs, k, v.get("groups", 0),
                                        v.get("limited", 0), ref_ids=rid)
    # weights: the oracle's scores at the GPU's ids (from the same logits)
    ref_w = np.take_along_axis(rs, ids.astype(np.int64), axis=1)
    if norm:
        ref_w = ref_w / ref_w.sum(axis=1, keepdims=True)
    assert np.allclose(w, ref_w, rtol=1e-5, atol=1e-7), "routing weights"
    # counts and the accumulator agree with the ids
    hist = O.expert_counts(ids, E)
    assert np.array_equal(counts, hist), "counts"
    assert np.array_equal(tpe.cpu().numpy(), hist.astype(np.float32)), "tokens_per_expert"
    print(f"  decided {dec.sum()}/{len(dec)}, matching {same.sum()}", flush=True)
    return dict(logits=logits, ids=ids, w=w, same=same, decided=dec)


DEEPSEEK_LIKE = dict(score_func="sigmoid", route_scale=2.5, groups=8, limited=4)


def _bias(E, seed=0, scale=0.05):
    return (np.random.default_rng(seed).standard_normal(E) * scale).astype(np.float32)


@pytest.mark.parametrize("name,T", [("qwen3_30b_a3b_decode", None),
                                    ("qwen3_30b_a3b_prefill", None)])
def test_sigmoid_groups_bias(moe, name, T):
    wl = workloads.make(name)
    check_route(moe, wl, dict(DEEPSEEK_LIKE, bias=_bias(wl.E)), norm=True, T=T)


def test_softmax_bias_scale(moe):
    wl = workloads.make("qwen3_30b_a3b_decode")
    check_route(moe, wl, dict(score_func="softmax", route_scale=1.5, bias=_bias(wl.E, 1)),
                norm=False)


def test_sigmoid_plain_prefill_slice(moe):
    # no bias, no groups: the sigmoid order is the logit order
    wl = workloads.make("qwen3_30b_a3b_prefill")
    check_route(moe, wl, dict(score_func="sigmoid", route_scale=1.0), norm=False, T=1024)


def test_tiny_fp32_one_group(moe):
    wl = workloads.make("tiny_fp32")
    check_route(moe, wl, dict(score_func="sigmoid", route_scale=1.0, groups=4, limited=1,
                              bias=_bias(wl.E, 2, 0.5)), norm=True)


def test_256_experts(moe):
    g = torch.Generator().manual_seed(3)
    T, H, E, k = 64, 256, 256, 8
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    wr = (torch.randn(E, H, generator=g) * 0.02).to(torch.bfloat16)

    class WL:
        name, dtype, top_k = "synthetic E=256", torch.bfloat16, k
    wl = WL()
    wl.E, wl.hidden_states, wl.router_weight = E, x, wr
    check_route(moe, wl, dict(score_func="sigmoid", route_scale=1.0, groups=16, limited=3,
                              bias=_bias(E, 4)), norm=True)


def test_layer_forward_variant(moe):
    wl = workloads.make("qwen3_30b_a3b_decode")
    v = dict(DEEPSEEK_LIKE, bias=_bias(wl.E, 5))
    say(f"layer forward with variant router {wl.name}")
    dev = torch.device(DEV)
    cfg = moe.router_config(v["score_func"], v["route_scale"],
                            torch.as_tensor(v["bias"], device=dev), v["groups"], v["limited"])
    x, wr, gu, dn = (t.to(dev) for t in (wl.hidden_states, wl.router_weight, wl.gate_up, wl.down))
    buf = moe.LayerBuffers(wl.T, wl.H, wl.I, wl.E, wl.top_k, wl.dtype, dev)
    out, logits, ids, w, counts = moe.layer_forward(x, wr, gu, dn, wl.top_k, True, config=cfg,
                                                    buffers=buf)
    torch.cuda.synchronize()
    internals = {n: t.cpu().numpy() for n, t in buf.internals().items() if n != "expert_out"}
    out, logits, ids, w, counts = (t.cpu().numpy() for t in (out.float(), logits, ids, w, counts))
    rid, rw, rs, rkey = _variant_ref(logits, wl.top_k, True, v)
    U.variant_routing_check(ids, rkey, rs, wl.top_k, v["groups"], v["limited"], ref_ids=rid)
    U.permutation_check(counts, internals, ids, wl.E)
    # the oracle's layer with the variant router, on the GPU's routing
    router = dict(score_func=v["score_func"], route_scale=v["route_scale"],
                  expert_bias=v["bias"], n_groups=v["groups"], n_limited=v["limited"])
    ref = O.moe_layer_forward(wl.hidden_states.float().numpy(), wl.router_weight.float().numpy(),
                              None, wl.gate_up.float().numpy(), wl.down.float().numpy(),
                              wl.top_k, True, ids=ids, router=router)
    assert np.allclose(w, ref["weights"], rtol=1e-4, atol=1e-7), "routing weights"
    U.assert_close(torch.as_tensor(out), ref["out"], wl.dtype, "layer output")


def test_update_expert_bias(moe):
    say("update_expert_bias E=128")
    r = np.random.default_rng(9)
    for E, nrec in ((128, 1), (128, 2), (7, 1), (256, 3)):
        bias = r.standard_normal(E).astype(np.float32) * 0.1
        tpe = r.integers(0, 3000, E).astype(np.float32)
        ref_b, ref_t = O.update_expert_bias(bias, tpe, 1e-3, nrec)
        bg = torch.as_tensor(bias, device=DEV).clone()
        tg = torch.as_tensor(tpe, device=DEV).clone()
        moe.update_expert_bias(bg, tg, 1e-3, nrec)
        torch.cuda.synchronize()
        assert np.allclose(bg.cpu().numpy(), ref_b, rtol=0, atol=2e-7), (E, nrec)
        assert not tg.cpu().numpy().any()
