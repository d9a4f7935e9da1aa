"""HIP path against the CPU oracle, through the C ABI (MI355X only).

Every case prints its name (flushed) before touching the GPU.
"""
from __future__ import annotations

import ctypes

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


def _np32(t):
    return t.float().numpy()


def shared_layout(w1, w2, w3):
    """FeedForward's nn.Linear weights in the library's layout: gate_up
    [H, 2 Is] = (w1^T | w3^T), down [Is, H] = w2^T."""
    return torch.cat([w1.t(), w3.t()], dim=1).contiguous(), w2.t().contiguous()


def run_layer(moe, wl, shared=None):
    """Full layer on the GPU vs the oracle's per-expert loop, by the routing
    protocol: logits within tolerance; the GPU's ids equal the oracle's
    selection on the GPU's float32 logits on every token (and the oracle's
    own ids on every decided token); the layer's counts, offsets and
    permutation bit for bit against the oracle's of the GPU's ids; expert
    outputs, routing weights and the layer output against the oracle's layer
    run on the GPU's ids, on every token.  ``shared`` = (w1, w2, w3): a
    shared expert in nn.Linear layout."""
    say(f"layer {wl.name} T={wl.T} H={wl.H} I={wl.I} E={wl.E} k={wl.top_k} {wl.dtype}"
        + (f" shared Is={shared[0].shape[0]}" if shared is not None else ""))
    x = wl.hidden_states.to(DEV)
    wr = wl.router_weight.to(DEV)
    gu = wl.gate_up.to(DEV)
    dn = wl.down.to(DEV)
    b = wl.router_bias.to(DEV) if wl.router_bias is not None else None
    sh = tuple(t.to(DEV) for t in shared_layout(*shared)) if shared is not None else None
    Is = shared[0].shape[0] if shared is not None else 0
    buf = moe.LayerBuffers(wl.T, wl.H, wl.I, wl.E, wl.top_k, wl.dtype, x.device, Is)
    out, logits, ids, w, counts = moe.layer_forward(x, wr, gu, dn, wl.top_k, wl.norm_topk_prob,
                                                    router_bias=b, shared=sh, buffers=buf)
    torch.cuda.synchronize()
    internals = {n: t.cpu() for n, t in buf.internals().items()}
    out, logits, ids, w, counts = (t.cpu() for t in (out, logits, ids, w, counts))
    xs, wrs = _np32(wl.hidden_states), _np32(wl.router_weight)
    bias_np = wl.router_bias.numpy() if wl.router_bias is not None else None
    # the oracle's own routing, then its whole layer on the GPU's routing
    ref_L, own_ids, _ = O.route(xs, wrs, bias_np, wl.top_k, wl.norm_topk_prob)
    U.assert_close(logits, ref_L, wl.dtype, "router logits")
    decided, same = U.routing_check(logits.numpy(), ids.numpy(), ref_L, own_ids, wl.top_k)
    ref = O.moe_layer_forward(xs, wrs, bias_np, _np32(wl.gate_up), _np32(wl.down), wl.top_k,
                              wl.norm_topk_prob, ids=ids.numpy(),
                              shared=tuple(_np32(t) for t in shared) if shared is not None
                              else None)
    every = np.ones(wl.T, dtype=bool)
    U.weights_check(w, ref["weights"], logits, ref_L, every)
    U.permutation_check(counts.numpy(), {n: t.numpy() for n, t in internals.items()
                                         if n != "expert_out"}, ids.numpy(), wl.E)
    U.assert_close(internals["expert_out"], O.unpermute(ref["y"], ref["slot_pos"]), wl.dtype,
                   "expert outputs (flat slot order)")
    U.assert_close(out, ref["out"], wl.dtype, "layer output")
    print(f"  tokens the oracle routes the same from its own logits: {same.sum()}/{wl.T}, "
          f"undecided {(~decided).sum()}", flush=True)
    return dict(out=out, logits=logits, ids=ids, w=w, counts=counts, ref=ref, same=same,
                own_ids=own_ids, ref_logits=ref_L)


# ----------------------------------------------------------------- layers

def test_layer_tiny_fp32(moe):
    run_layer(moe, workloads.make("tiny_fp32"))


@pytest.mark.parametrize("shape", [
    dict(T=1000, H=256, I=128, E=8, top_k=2),     # wide tiles, ~250 rows per expert
    dict(T=300, H=256, I=128, E=16, top_k=4),     # 64-row tiles
    dict(T=37, H=256, I=128, E=32, top_k=4),      # 16-row tiles, ragged
    dict(T=200, H=384, I=192, E=8, top_k=2),      # narrow-tile fallback
    dict(T=129, H=512, I=64, E=6, top_k=6),       # k = E
    dict(T=70, H=256, I=128, E=1, top_k=1),       # one expert
    dict(T=200, H=256, I=128, E=32, top_k=8),     # ~50 rows per expert
    dict(T=150, H=512, I=192, E=8, top_k=2),      # K-blocks not a multiple of the stages
    dict(T=800, H=256, I=128, E=4, top_k=2),      # ~400 rows per expert: 320-row tiles, plain weight copies
    dict(T=300, H=256, I=128, E=4, top_k=2),      # ~150 rows per expert: 128-row tiles, plain weight copies
])
def test_layer_small_bf16(moe, shape):
    wl = workloads.make_layer(f"small_{shape['T']}", norm_topk_prob=True, seed=1, **shape)
    run_layer(moe, wl)


# Batches on the split-K router path (T > 512), where top_k of 8, 16 or 32
# folds the permutation's first pass into the selection kernel: a ragged last
# block of 16 tokens, 256- and 512-slot blocks, and float32.
@pytest.mark.parametrize("shape", [
    dict(T=777, H=256, I=128, E=32, top_k=8, dtype=torch.bfloat16),
    dict(T=700, H=256, I=128, E=64, top_k=16, dtype=torch.bfloat16),
    dict(T=600, H=128, I=64, E=40, top_k=32, dtype=torch.bfloat16),
    dict(T=900, H=256, I=64, E=16, top_k=8, dtype=torch.float32),
])
def test_layer_router_folded_permutation(moe, shape):
    wl = workloads.make_layer(f"fold_{shape['T']}_{shape['top_k']}", norm_topk_prob=True, seed=3,
                              **shape)
    run_layer(moe, wl)


def test_layer_no_renorm(moe):
    wl = workloads.make_layer("no_renorm", T=96, H=256, I=128, E=16, top_k=4,
                              norm_topk_prob=False, seed=2)
    run_layer(moe, wl)


def test_layer_prefill_4096(moe):
    run_layer(moe, workloads.make("qwen3_30b_a3b_prefill"))


def test_layer_decode_64(moe):
    run_layer(moe, workloads.make("qwen3_30b_a3b_decode"))


def test_layer_skewed_16384(moe):
    r = run_layer(moe, workloads.make("qwen3_30b_a3b_skewed"))
    c = r["counts"].numpy()
    assert (c == 0).any() and c.max() > 10 * c.mean()


def test_integer_logits_route_bit_exact(moe):
    """Exact-integer router inputs: GPU and oracle logits are identical, ties
    are frequent, and routing must match bit for bit on every token."""
    wl = workloads.integer_grid_layer(T=4096, H=2048, I=128, E=128, top_k=8)
    r = run_layer(moe, wl)
    assert np.array_equal(r["logits"].numpy(), r["ref_logits"])
    assert r["same"].all()
    assert np.array_equal(r["ids"].numpy(), r["own_ids"])


def test_all_ties_zero_router(moe):
    """Zero router weight: all logits equal, every token picks experts
    0..k-1, the other experts are empty, weights are exactly 1/k."""
    wl = workloads.make_layer("ties", T=50, H=256, I=64, E=16, top_k=4, seed=3)
    wl.router_weight.zero_()
    r = run_layer(moe, wl)
    assert np.array_equal(r["ids"].numpy(), np.tile(np.arange(4), (50, 1)))
    assert np.all(r["w"].numpy() == 0.25)
    assert r["counts"].numpy().tolist() == [50] * 4 + [0] * 12


def test_layer_deterministic(moe):
    wl = workloads.make_layer("det", T=512, H=512, I=256, E=32, top_k=4, seed=4)
    x, wr, gu, dn = (t.to(DEV) for t in (wl.hidden_states, wl.router_weight, wl.gate_up, wl.down))
    say("determinism")
    a = moe.layer_forward(x, wr, gu, dn, 4)[0].clone()
    b = moe.layer_forward(x, wr, gu, dn, 4)[0].clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ------------------------------------------------------------ shared expert

@pytest.mark.parametrize("T,H,Is,dtype", [
    (4096, 2048, 768, torch.bfloat16),    # prefill tokens, Qwen3-30B-A3B width
    (64, 2048, 768, torch.bfloat16),      # decode tokens
    (300, 256, 256, torch.bfloat16),      # several row tiles, ragged tail
    (1, 256, 128, torch.bfloat16),        # one token
    (200, 384, 192, torch.bfloat16),      # Is not a multiple of 128: narrow-tile fallback
    (37, 128, 64, torch.float32),
    (513, 256, 128, torch.float32),
])
def test_shared_expert_alone(moe, T, H, Is, dtype):
    say(f"shared expert T={T} H={H} Is={Is} {dtype}")
    g = torch.Generator().manual_seed(T + Is)
    x = torch.randn(T, H, generator=g).to(dtype)
    w1, w2, w3 = workloads.shared_expert_weights(H, Is, dtype, seed=T)
    gu, dn = shared_layout(w1, w2, w3)
    out = moe.shared_expert_forward(x.to(DEV), gu.to(DEV), dn.to(DEV))
    torch.cuda.synchronize()
    ref = O.feed_forward(_np32(x), _np32(w1), _np32(w2), _np32(w3))
    U.assert_close(out.cpu(), ref, dtype, "shared expert")


@pytest.mark.parametrize("name,Is", [("qwen3_30b_a3b_decode", 768),
                                     ("qwen3_30b_a3b_prefill", 768),
                                     ("tiny_fp32", 128)])
def test_layer_with_shared_expert(moe, name, Is):
    wl = workloads.make(name)
    run_layer(moe, wl, shared=workloads.shared_expert_weights(wl.H, Is, wl.dtype))


@pytest.mark.parametrize("T,H,I,E,k,Is", [
    (37, 256, 128, 32, 4, 192),     # Is not a multiple of 128: shared GEMMs on their own
    (37, 256, 128, 32, 4, 256),     # inside the grouped launches, ragged tail
    (1000, 256, 128, 8, 2, 384),    # inside, many dense row tiles next to wide expert tiles
    (1, 512, 64, 6, 6, 128),        # one token, k = E
])
def test_layer_shared_small(moe, T, H, I, E, k, Is):
    wl = workloads.make_layer(f"shared_{T}_{Is}", T=T, H=H, I=I, E=E, top_k=k, seed=7,
                              norm_topk_prob=False)
    run_layer(moe, wl, shared=workloads.shared_expert_weights(H, Is, wl.dtype, seed=7))


def test_layer_shared_zero_tokens(moe):
    say("layer with shared expert, T = 0")
    H, I, E, Is = 256, 128, 8, 128
    x = torch.empty(0, H, dtype=torch.bfloat16, device=DEV)
    wr = torch.zeros(E, H, dtype=torch.bfloat16, device=DEV)
    gu = torch.zeros(E, H, 2 * I, dtype=torch.bfloat16, device=DEV)
    dn = torch.zeros(E, I, H, dtype=torch.bfloat16, device=DEV)
    sh = (torch.zeros(H, 2 * Is, dtype=torch.bfloat16, device=DEV),
          torch.zeros(Is, H, dtype=torch.bfloat16, device=DEV))
    out, _, _, _, counts = moe.layer_forward(x, wr, gu, dn, 2, True, shared=sh)
    torch.cuda.synchronize()
    assert out.shape == (0, H) and not counts.cpu().any()


# ------------------------------------------------------------ sub-steps

@pytest.mark.parametrize("T,E,k", [(4096, 128, 8), (16384, 128, 8), (1, 8, 8), (777, 256, 3),
                                   (5000, 4, 1)])
def test_permute_bit_exact(moe, T, E, k):
    say(f"permute T={T} E={E} k={k}")
    pop = torch.tensor([1.0 / (1 + e) ** 1.2 for e in range(E)])
    ids = workloads.random_topk_ids(T, E, k, seed=T + E, popularity=pop)
    r = moe.permute(ids.to(DEV), E)
    torch.cuda.synchronize()
    ss, st, sp = O.permutation(ids.numpy(), E)
    c = O.expert_counts(ids.numpy(), E)
    assert np.array_equal(r["counts"].cpu().numpy(), c)
    assert np.array_equal(r["offsets"].cpu().numpy(), O.expert_offsets(c))
    assert np.array_equal(r["sorted_slot"].cpu().numpy(), ss)
    assert np.array_equal(r["sorted_token"].cpu().numpy(), st)
    assert np.array_equal(r["slot_pos"].cpu().numpy(), sp)


def test_gather_and_combine(moe):
    say("gather + combine")
    T, E, k, H = 333, 16, 4, 256
    ids = workloads.random_topk_ids(T, E, k, seed=5)
    g = torch.Generator().manual_seed(6)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    w = torch.rand(T, k, generator=g)
    perm = moe.permute(ids.to(DEV), E)
    xp = moe.gather_rows(x.to(DEV), perm["sorted_token"])
    # expert-major rows through slot_pos, weighted
    out1 = moe.combine(xp, T, k, topk_weights=w.to(DEV), slot_pos=perm["slot_pos"])
    # unweighted: each token's k copies of itself
    out2 = moe.combine(xp, T, k, slot_pos=perm["slot_pos"])
    torch.cuda.synchronize()
    _, st, sp = O.permutation(ids.numpy(), E)
    xg = O.gather_rows(_np32(x), st)
    assert np.array_equal(xp.cpu().float().numpy(), xg)
    ref1 = O.combine(O.unpermute(xg, sp), w.numpy())
    U.assert_close(out1.cpu(), ref1, torch.bfloat16, "weighted combine")
    U.assert_close(out2.cpu(), k * _np32(x), torch.bfloat16, "plain un-permute")


def test_route_c_abi_direct(moe):
    """moe_route called through ctypes with raw device pointers."""
    say("route via C ABI")
    wl = workloads.make("tiny_fp32")
    x, wr = wl.hidden_states.to(DEV), wl.router_weight.to(DEV)
    T, E, k = wl.T, wl.E, wl.top_k
    logits = torch.empty(T, E, device=DEV)
    ids = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, k, device=DEV)
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    st = moe.lib.moe_route(x.data_ptr(), wr.data_ptr(), None, T, wl.H, E, k, 1, 0,
                           logits.data_ptr(), ids.data_ptr(), w.data_ptr(), counts.data_ptr(),
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    L, rid, rw = O.route(_np32(wl.hidden_states), _np32(wl.router_weight), None, k, True)
    U.assert_close(logits.cpu(), L, torch.float32, "logits")
    U.routing_check(logits.cpu().numpy(), ids.cpu().numpy(), L, rid, k)
    assert np.array_equal(counts.cpu().numpy(), np.bincount(ids.cpu().numpy().ravel(), minlength=E))


def test_grouped_swiglu_expert_major(moe):
    """Grouped experts on seeded expert-major rows (no router), y expert-major."""
    say("grouped swiglu expert-major")
    E, H, I = 8, 256, 128
    counts = np.array([0, 300, 1, 0, 129, 64, 17, 0], np.int32)
    N = int(counts.sum())
    g = torch.Generator().manual_seed(7)
    x = torch.randn(N, H, generator=g).to(torch.bfloat16)
    gu = (0.05 * torch.randn(E, H, 2 * I, generator=g)).to(torch.bfloat16)
    dn = (0.05 * torch.randn(E, I, H, generator=g)).to(torch.bfloat16)
    offs = torch.tensor(O.expert_offsets(counts), dtype=torch.int32)
    y = moe.grouped_swiglu(x.to(DEV), offs.to(DEV), gu.to(DEV), dn.to(DEV), N)
    h = moe.grouped_gate_up_swiglu(x.to(DEV), offs.to(DEV), gu.to(DEV), N)
    torch.cuda.synchronize()
    ref = O.grouped_swiglu(_np32(x), counts, _np32(gu), _np32(dn))
    U.assert_close(y.cpu(), ref, torch.bfloat16, "grouped swiglu")
    # h alone: per-expert gate/up SwiGLU
    hr = np.zeros((N, I))
    o = O.expert_offsets(counts)
    for e in range(E):
        if counts[e]:
            G = _np32(x)[o[e]:o[e + 1]].astype(np.float64) @ _np32(gu)[e].astype(np.float64)
            hr[o[e]:o[e + 1]] = O.silu(G[:, :I]) * G[:, I:]
    U.assert_close(h.cpu(), hr, torch.bfloat16, "gate_up swiglu")


# ---------------------------------------------------------------- EP rank

def test_ep_rank_reshuffle_and_experts(moe):
    """One EP rank of the 235B-A22B-shaped layer: rank-major received rows ->
    expert-major -> grouped SwiGLU -> back to rank-major, vs the oracle."""
    wl = workloads.make("ep_rank_235b")
    say(f"ep rank R={wl.R} T/rank={wl.T_per_rank} H={wl.H} I={wl.I} E_loc={wl.E_local}")
    xs = [_np32(t) for t in wl.source_hidden]
    rows, C, _ = O.dispatch_rank_major(xs, _np32(wl.router_weight), wl.top_k,
                                       wl.norm_topk_prob, wl.local_lo, wl.E_local)
    N = rows.shape[0]
    ref = O.ep_rank_forward(rows, C, _np32(wl.gate_up), _np32(wl.down))
    rows_d = torch.from_numpy(rows).to(torch.bfloat16).to(DEV)
    C_d = torch.from_numpy(C).to(DEV)
    perm = moe.permute_rank_major(C_d, N)
    y = moe.grouped_swiglu(rows_d, perm["offsets"], wl.gate_up.to(DEV), wl.down.to(DEV), N,
                           row_index=perm["sorted_token"], out_index=perm["sorted_token"])
    torch.cuda.synchronize()
    src = O.reshuffle_rank_to_expert(C)
    assert np.array_equal(perm["sorted_token"].cpu().numpy(), src)
    assert np.array_equal(perm["counts"].cpu().numpy(), C.sum(axis=0))
    inv = np.empty(N, np.int64)
    inv[src] = np.arange(N)
    assert np.array_equal(perm["slot_pos"].cpu().numpy(), inv)
    U.assert_close(y.cpu(), ref["y_rm"], torch.bfloat16, "ep rank output (rank-major)")


def test_rank_major_small_with_empty_blocks(moe):
    say("rank-major small")
    C = np.array([[3, 0, 2], [0, 0, 5], [1, 4, 0], [0, 0, 0]], np.int32)
    N = int(C.sum())
    perm = moe.permute_rank_major(torch.from_numpy(C).to(DEV), N)
    torch.cuda.synchronize()
    assert np.array_equal(perm["sorted_token"].cpu().numpy(), O.reshuffle_rank_to_expert(C))
    assert np.array_equal(perm["offsets"].cpu().numpy(), O.expert_offsets(C.sum(axis=0)))


# ---------------------------------------------------------- edge / errors

def test_empty_inputs(moe):
    say("T = 0")
    H, I, E, k = 256, 128, 8, 2
    x = torch.empty(0, H, dtype=torch.bfloat16, device=DEV)
    wr = torch.randn(E, H, device=DEV).to(torch.bfloat16)
    gu = torch.zeros(E, H, 2 * I, dtype=torch.bfloat16, device=DEV)
    dn = torch.zeros(E, I, H, dtype=torch.bfloat16, device=DEV)
    out, logits, ids, w, counts = moe.layer_forward(x, wr, gu, dn, k)
    torch.cuda.synchronize()
    assert out.shape == (0, H) and counts.cpu().tolist() == [0] * E


def test_invalid_arguments_rejected(moe):
    say("argument validation")
    s = torch.cuda.current_stream().cuda_stream
    buf = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    p = buf.data_ptr()
    L = moe.lib
    assert L.moe_route(p, p, None, 4, 128, 0, 1, 1, 1, None, p, p, None, s) == -2   # E = 0
    assert L.moe_route(p, p, None, 4, 128, 8, 9, 1, 1, None, p, p, None, s) == -2   # k > E
    assert L.moe_route(p, p, None, 4, 128, 8, 2, 1, 7, None, p, p, None, s) == -3   # dtype
    assert L.moe_route(p + 2, p, None, 4, 128, 8, 2, 1, 1, None, p, p, None, s) == -7
    assert L.moe_route(None, p, None, 4, 128, 8, 2, 1, 1, None, p, p, None, s) == -1
    assert L.moe_layer_forward(p, p, None, p, p, 4, 100, 64, 8, 2, 1, 1, p, None, None, None,
                               None, p, 1 << 20, None, s) == -2                         # H % 128
    assert L.moe_layer_forward(p, p, None, p, p, 4, 128, 64, 8, 2, 1, 1, p, None, None, None,
                               None, p, 16, None, s) == -4                              # workspace
    assert L.moe_permute(None, 4, 2, None, 0, 8, 8, p, p, p, p, p, p, 1 << 20, s) == -1
    assert L.moe_permute(None, 0, 1, p, 1000, 8, 8, p, p, p, p, p, p, 1 << 20, s) == -2  # R*E
    torch.cuda.synchronize()
