"""Layer backward on the GPU against the oracle's gradients, through the C
ABI (MI355X only).

The training forward runs first; its routing is checked with the forward's
protocol (decided tokens bit-exact, the rest a valid top-k of the device's
own float32 logits), and the oracle's backward then takes the device's
routing decision, so every gradient is compared element by element.

Gradient tolerance: max|gpu - ref| <= 1e-2 * max|ref| per tensor.  The
device keeps the pre-activations, dG, w*h and dX in bf16 (relative rounding
2^-9 each) and sums in float32; the oracle is float64 throughout.  The
router's weight and bias gradients are sums over tokens of dL (times x),
and with renormalised weights each token's dL row sums to zero, so those
sums cancel by construction (badly with few experts: at E = 4, top-2 the
largest bias gradient is 1/13 of its sum of absolute terms).  A sum's
rounding error scales with the sum of the absolute values of its terms
(the standard forward error bound of summation), so for these two the
scale is max of sum_t |dL[t, e]| (times |x|) instead of max|ref|.

Every case prints its name (flushed) before touching the GPU.
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
GRAD_REL = 1e-2


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mixture_experts_layer_17_amd as m
    return m


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def _np32(t):
    return t.float().cpu().numpy()


def grad_close(gpu, ref, what, scale=None):
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    if scale is None:
        scale = np.abs(r).max() if r.size else 0.0
    err = np.abs(g - r).max() if r.size else 0.0
    assert err <= GRAD_REL * scale, f"{what}: max|gpu-ref| = {err:.3e} > {GRAD_REL * scale:.3e}"
    return err / scale if scale else 0.0


def _shared_layout(w1, w2, w3):
    return torch.cat([w1.t(), w3.t()], dim=1).contiguous(), w2.t().contiguous()


def run_backward(moe, wl, seed=0, router=None, shared=None):
    """``router``: a router variant as the oracle's keyword dict (score_func,
    route_scale, expert_bias, n_groups, n_limited), or None.  ``shared``:
    FeedForward weights (w1, w2, w3) in nn.Linear layout, or None."""
    say(f"backward {wl.name} T={wl.T} H={wl.H} I={wl.I} E={wl.E} k={wl.top_k} "
        f"norm={wl.norm_topk_prob} router={router}")
    k, norm = wl.top_k, wl.norm_topk_prob
    x, wr, gu, dn = (t.to(DEV) for t in (wl.hidden_states, wl.router_weight, wl.gate_up, wl.down))
    b = wl.router_bias.to(DEV) if wl.router_bias is not None else None
    cfg = None
    if router is not None:
        eb = router.get("expert_bias")
        cfg = moe.router_config(router["score_func"], router.get("route_scale", 1.0),
                                torch.as_tensor(eb, dtype=torch.float32, device=DEV)
                                if eb is not None else None,
                                router.get("n_groups", 0), router.get("n_limited", 0))
    g = torch.Generator().manual_seed(100 + seed)
    dout = torch.randn(wl.T, wl.H, generator=g).to(wl.dtype)
    sh = tuple(t.to(DEV) for t in _shared_layout(*shared)) if shared is not None else None
    out, saved = moe.layer_forward_train(x, wr, gu, dn, k, norm, router_bias=b, config=cfg,
                                         shared=sh)
    grads = moe.layer_backward(x, wr, gu, dn, k, norm, saved, dout.to(DEV), config=cfg, shared=sh)
    torch.cuda.synchronize()
    logits = saved["router_logits"].cpu().numpy()
    ids = saved["topk_ids"].cpu().numpy()
    xs, wrs, gus, dns = (_np32(t) for t in (wl.hidden_states, wl.router_weight, wl.gate_up,
                                            wl.down))
    bias = wl.router_bias.numpy() if wl.router_bias is not None else None
    sh_np = tuple(_np32(t) for t in shared) if shared is not None else None
    ref_L = O.router_logits(xs, wrs, bias)
    U.assert_close(torch.as_tensor(logits), ref_L, wl.dtype, "router logits")
    if router is None:
        decided, same = U.routing_check(logits, ids, ref_L, O.select_topk(ref_L, k), k)
    else:
        # the variant's selection from the device's own logits, by the
        # decided-token protocol
        rid, _, rs, rkey = O.route_variant(logits, k, norm, **router)
        decided, same = U.variant_routing_check(ids, rkey, rs, k, router.get("n_groups", 0),
                                                router.get("n_limited", 0), ref_ids=rid)
    ref = O.moe_layer_backward(xs, wrs, bias, gus, dns, k, norm, _np32(dout), ids=ids,
                               router=router, shared=sh_np)
    f = ref["forward"]
    # what the training forward kept
    U.assert_close(out.cpu(), f["out"], wl.dtype, "layer output")
    U.assert_close(saved["expert_out"].cpu(), O.unpermute(f["y"], f["slot_pos"]), wl.dtype,
                   "saved expert outputs")
    G = np.concatenate([xs[f["sorted_token"][f["offsets"][e]:f["offsets"][e + 1]]] @ gus[e]
                        for e in range(wl.E)], axis=0) if wl.T else np.zeros((0, 2 * wl.I))
    U.assert_close(saved["gate_up_out"].cpu(), G, wl.dtype, "saved pre-activations")
    rel = {}
    # sums over tokens of the routing Jacobian's output: scale by the sum of
    # the absolute terms
    adl = np.abs(ref["d_logits"])
    sum_scale = {"d_router_bias": adl.sum(axis=0).max() if adl.size else 0.0,
                 "d_router_weight": (adl.T @ np.abs(xs.astype(np.float64))).max()
                 if adl.size else 0.0}
    for name in ("d_topk_weights", "dx", "d_router_weight", "d_router_bias", "d_down",
                 "d_gate_up"):
        refn = ref["d_weights"] if name == "d_topk_weights" else ref[name]
        rel[name] = grad_close(_np32(grads[name]), refn, name, sum_scale.get(name))
        if name in sum_scale:
            # the same error against max|ref| (reported; the bar above is the
            # sum's error bound)
            mr = np.abs(refn).max() if np.size(refn) else 0.0
            err = np.abs(_np32(grads[name]).astype(np.float64) - refn).max() if mr else 0.0
            rel[name + " vs max|ref|"] = err / mr if mr else 0.0
    if shared is not None:
        w1, w2, w3 = sh_np
        U.assert_close(saved["shared_gate_up_out"].cpu(),
                       np.concatenate([xs @ w1.T, xs @ w3.T], axis=1), wl.dtype,
                       "saved shared pre-activations")
        d1, d2, d3 = ref["d_shared"]
        rel["d_shared_gate_up"] = grad_close(_np32(grads["d_shared_gate_up"]),
                                             np.concatenate([d1.T, d3.T], axis=1),
                                             "d_shared_gate_up")
        rel["d_shared_down"] = grad_close(_np32(grads["d_shared_down"]), d2.T, "d_shared_down")
    print("  routed as the oracle: %d/%d; relative errors %s" % (
        same.sum(), wl.T, {k_: f"{v:.1e}" for k_, v in rel.items()}), flush=True)
    return grads, ref


@pytest.mark.parametrize("shape", [
    dict(T=37, H=256, I=128, E=8, top_k=2),      # ragged tiles, a few rows per expert
    dict(T=300, H=512, I=256, E=16, top_k=4),    # several K-blocks per expert in wgrad
    dict(T=1, H=256, I=128, E=8, top_k=8),       # one token, k = E
    dict(T=500, H=384, I=128, E=1, top_k=1),     # one expert, H not a multiple of 256
    dict(T=200, H=256, I=128, E=64, top_k=2),    # empty experts get zero gradients
])
def test_backward_small(moe, shape):
    wl = workloads.make_layer(f"bwd_{shape['T']}_{shape['E']}", norm_topk_prob=True, seed=11,
                              **shape)
    grads, ref = run_backward(moe, wl)
    empty = np.flatnonzero(ref["forward"]["counts"] == 0)
    assert not grads["d_gate_up"].cpu()[empty].any() and not grads["d_down"].cpu()[empty].any()


def test_backward_no_renorm_with_bias(moe):
    wl = workloads.make_layer("bwd_plain", T=160, H=256, I=128, E=16, top_k=4,
                              norm_topk_prob=False, seed=12,
                              router_bias=workloads.zipf_router_bias(16))
    run_backward(moe, wl)


@pytest.mark.parametrize("norm,router", [
    (True, dict(score_func="sigmoid", route_scale=2.5)),
    (False, dict(score_func="sigmoid", route_scale=2.5, n_groups=8, n_limited=4)),
    (False, dict(score_func="softmax", route_scale=1.5)),
])
def test_backward_router_variant_small(moe, norm, router):
    wl = workloads.make_layer("bwd_variant", T=200, H=256, I=128, E=64, top_k=4,
                              norm_topk_prob=norm, seed=14)
    r = dict(router)
    r["expert_bias"] = (np.random.default_rng(3).standard_normal(64) * 0.05).astype(np.float32)
    run_backward(moe, wl, router=r)


def test_backward_router_variant_decode(moe):
    wl = workloads.make("qwen3_30b_a3b_decode")
    r = dict(score_func="sigmoid", route_scale=2.5, n_groups=8, n_limited=4,
             expert_bias=(np.random.default_rng(1).standard_normal(128) * 0.05).astype(np.float32))
    run_backward(moe, wl, router=r)


@pytest.mark.parametrize("name,T,I,Is", [
    ("bwd_shared_small", 150, 128, 256),       # shared wgrads inside the routed launches
    ("bwd_shared_apart", 150, 256, 128),       # Is does not fit the tile: on their own
    ("qwen3_30b_a3b_decode", None, None, 768),
    ("qwen3_30b_a3b_prefill", None, None, 768)])
def test_backward_shared_expert(moe, name, T, I, Is):
    if T is None:
        wl = workloads.make(name)
    else:
        wl = workloads.make_layer(name, T=T, H=256, I=I, E=16, top_k=4, seed=15)
    run_backward(moe, wl, shared=workloads.shared_expert_weights(wl.H, Is, wl.dtype, seed=2))


def test_backward_decode(moe):
    run_backward(moe, workloads.make("qwen3_30b_a3b_decode"))


def test_backward_prefill(moe):
    run_backward(moe, workloads.make("qwen3_30b_a3b_prefill"))


def test_backward_deterministic(moe):
    wl = workloads.make_layer("bwd_det", T=256, H=256, I=128, E=16, top_k=4, seed=13)
    say("backward determinism")
    x, wr, gu, dn = (t.to(DEV) for t in (wl.hidden_states, wl.router_weight, wl.gate_up, wl.down))
    dout = torch.randn(wl.T, wl.H, generator=torch.Generator().manual_seed(5)).to(wl.dtype).to(DEV)
    _, saved = moe.layer_forward_train(x, wr, gu, dn, 4, True)
    a = moe.layer_backward(x, wr, gu, dn, 4, True, saved, dout)
    b = moe.layer_backward(x, wr, gu, dn, 4, True, saved, dout)
    torch.cuda.synchronize()
    for name in a:
        if a[name] is not None:
            assert torch.equal(a[name], b[name]), name


def test_backward_unsupported_is_reported(moe):
    say("backward: float32 and I % 128 != 0 are refused before any launch")
    wl = workloads.make("tiny_fp32")
    x, wr, gu, dn = (t.to(DEV) for t in (wl.hidden_states, wl.router_weight, wl.gate_up, wl.down))
    with pytest.raises(moe.MoEError):
        moe.layer_forward_train(x, wr, gu, dn, wl.top_k, True)
    wl = workloads.make_layer("bwd_i64", T=16, H=256, I=64, E=4, top_k=2)
    x, wr, gu, dn = (t.to(DEV) for t in (wl.hidden_states, wl.router_weight, wl.gate_up, wl.down))
    with pytest.raises(moe.MoEError):
        moe.layer_forward_train(x, wr, gu, dn, 2, True)


def test_backward_zero_tokens(moe):
    say("backward: T = 0 gives exact zero weight gradients")
    wl = workloads.make_layer("bwd_empty", T=8, H=256, I=128, E=8, top_k=2, seed=16)
    x, wr, gu, dn = (t.to(DEV) for t in (wl.hidden_states, wl.router_weight, wl.gate_up, wl.down))
    x0 = x[:0].contiguous()
    sh = _shared_layout(*workloads.shared_expert_weights(256, 128, wl.dtype))
    sh = tuple(t.to(DEV) for t in sh)
    _, saved = moe.layer_forward_train(x0, wr, gu, dn, 2, True, shared=sh)
    dout = torch.empty(0, wl.H, dtype=wl.dtype, device=DEV)
    g = moe.layer_backward(x0, wr, gu, dn, 2, True, saved, dout, shared=sh)
    torch.cuda.synchronize()
    assert g["dx"].shape == (0, wl.H)
    for name in ("d_router_weight", "d_router_bias", "d_gate_up", "d_down", "d_shared_gate_up",
                 "d_shared_down"):
        assert not g[name].cpu().any(), name
