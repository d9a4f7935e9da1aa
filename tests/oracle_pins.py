"""Pins for the CPU oracle: checks against facts fixed by the pages and by
mathematics, not against the oracle's own formulas.

Each ``pin_*`` function raises ``AssertionError`` when the oracle is wrong.
They are plain functions so that a test can also plant a mistake in the
oracle and confirm that some pin catches it.

What pins what:

* router logits: one-hot tokens (closed form), zero weights (logit = bias),
  small-integer inputs (exact integer dot products by brute force);
* top-k: all-equal logits (closed form of the lower-id tie rule), large bias
  on a chosen set, -0.0 vs +0.0, brute force over all k-subsets;
* routing weights: renormalised weights sum to one, k = 1 gives 1, uniform
  logits give 1/k and 1/E exactly, the two-expert sigmoid closed form, the
  full softmax against scipy's;
* counts / permutation: sum invariant, numpy's bincount and stable argsort,
  bijection, gather-then-inverse identity;
* expert FFN / combine: the all-expert masked path of the Qwen3-Omni issue
  (brute force), identical experts (dense SwiGLU via torch), E = 1, k = E soft
  mixture, zero token, the scalar closed form at H = I = 1, permute + combine
  with an identity expert;
* expert-parallel rank: a hand-worked reshuffle, and equality with the
  token-choice layer when one rank owns every expert;
* router variants (sigmoid / softmax scores, route scale, selection-only
  expert bias, node-limited groups): equal scores make the bias order the
  selection (closed form), sigmoid weights against scipy's expit, the
  softmax variant against the default router, a hand-worked group example,
  and the group invariant on random inputs;
* expert-bias update: hand-worked steps, zero-mean steps, recomputation;
* shared expert: the FeedForward formula by scalar loops on tiny inputs
  (nn.Linear convention, gate w1 and up w3 kept apart), the closed form at
  H = Is = 1, routed experts that are copies of the shared one (the output is
  (1 + sum of the routing weights) times the FFN), zero routed outputs, and
  the all-expert brute-force path;
* layer backward: central finite differences of the (pinned) forward on every
  input and weight entry of small layers, with and without renormalisation
  and with a router bias; the closed form of the scalar layer; the softmax
  gradient summing to zero per token; zero gradients for experts without
  rows.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import scipy.special
import torch

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


def _layer(T, H, I, E, seed=0, std=0.3):
    r = _rng(seed)
    x = r.standard_normal((T, H)).astype(np.float32)
    wr = (r.standard_normal((E, H)) * std).astype(np.float32)
    gu = (r.standard_normal((E, H, 2 * I)) * std).astype(np.float32)
    dn = (r.standard_normal((E, I, H)) * std).astype(np.float32)
    return x, wr, gu, dn


def _torch_swiglu(x, gu, dn):
    """Dense SwiGLU with torch's own SiLU (an independent implementation)."""
    xt = torch.as_tensor(np.asarray(x, np.float64))
    gut = torch.as_tensor(np.asarray(gu, np.float64))
    dnt = torch.as_tensor(np.asarray(dn, np.float64))
    I = gut.shape[1] // 2
    G = xt @ gut
    h = torch.nn.functional.silu(G[:, :I]) * G[:, I:]
    return (h @ dnt).numpy()


# --------------------------------------------------------------------- logits

def pin_logits_onehot():
    """A one-hot token selects one column of the router weight:
    ``L[t, e] = Wr[e, h_t] + b[e]`` with a single product, so exact."""
    r = _rng(1)
    T, H, E = 12, 16, 8
    hs = r.integers(0, H, T)
    x = np.zeros((T, H), np.float32)
    x[np.arange(T), hs] = 1.0
    wr = r.standard_normal((E, H)).astype(np.float32)
    b = r.standard_normal(E).astype(np.float32)
    L = O.router_logits(x, wr, b)
    expect = (wr[:, hs].T.astype(np.float64) + b.astype(np.float64)).astype(np.float32)
    assert L.dtype == np.float32
    assert np.array_equal(L, expect), "one-hot logits"


def pin_logits_zero_weight():
    b = np.array([0.5, -1.25, 3.0, 0.0], np.float32)
    L = O.router_logits(np.ones((3, 8), np.float32), np.zeros((4, 8), np.float32), b)
    assert np.array_equal(L, np.tile(b, (3, 1))), "zero router weight gives the bias"


def pin_logits_integer_exact():
    """Small integers: the exact dot product by brute force in Python ints."""
    r = _rng(2)
    T, H, E = 5, 7, 4
    x = r.integers(-3, 4, (T, H))
    wr = r.integers(-3, 4, (E, H))
    L = O.router_logits(x.astype(np.float32), wr.astype(np.float32))
    for t in range(T):
        for e in range(E):
            s = 0
            for h in range(H):
                s += int(x[t, h]) * int(wr[e, h])
            assert L[t, e] == s, "integer logits"


# --------------------------------------------------------------------- top-k

def pin_topk_all_ties():
    """All logits equal: the lower-id rule gives experts 0..k-1 for every
    token, and counts ``[T]*k + [0]*(E-k)``."""
    T, E, k = 6, 8, 3
    L = np.zeros((T, E), np.float32)
    ids = O.select_topk(L, k)
    assert np.array_equal(ids, np.tile(np.arange(k), (T, 1))), "tie rule"
    c = O.expert_counts(ids, E)
    assert np.array_equal(c, np.array([T] * k + [0] * (E - k))), "tie counts"


def pin_topk_bias_set():
    """A +100 bias on a chosen set S routes every token to S, in order of
    decreasing bias (ties to the lower id)."""
    r = _rng(3)
    T, H, E, k = 10, 8, 8, 3
    x = r.standard_normal((T, H)).astype(np.float32)
    wr = (0.01 * r.standard_normal((E, H))).astype(np.float32)
    b = np.zeros(E, np.float32)
    b[6], b[1], b[4] = 100.0, 100.0, 101.0
    L = O.router_logits(x, wr, b)
    ids = O.select_topk(L, k)
    assert set(map(tuple, np.sort(ids, axis=1))) == {(1, 4, 6)}, "bias set"
    assert np.all(ids[:, 0] == 4), "largest bias first"


def pin_topk_negzero():
    """-0.0 and +0.0 are equal logits: the lower id wins either way."""
    L = np.array([[-1.0, 0.0, -0.0, -2.0], [-1.0, -0.0, 0.0, -2.0]], np.float32)
    ids = O.select_topk(L, 2)
    assert np.array_equal(ids, [[1, 2], [1, 2]]), "signed zero tie"


def pin_topk_bruteforce():
    """Distinct logits: the top-k set maximises the sum over all k-subsets;
    order is decreasing logit."""
    r = _rng(4)
    T, E, k = 20, 6, 3
    L = r.standard_normal((T, E)).astype(np.float32)
    ids = O.select_topk(L, k)
    for t in range(T):
        best = max(itertools.combinations(range(E), k),
                   key=lambda s: sum(float(L[t, e]) for e in s))
        assert set(ids[t].tolist()) == set(best), "top-k set"
        vals = [float(L[t, e]) for e in ids[t]]
        assert all(vals[i] > vals[i + 1] for i in range(k - 1)), "top-k order"


# ------------------------------------------------------------------- weights

def pin_weights_sum_to_one():
    x, wr, _, _ = _layer(32, 16, 4, 8, seed=5)
    L, ids, w = O.route(x, wr, None, 3, True)
    assert np.all(np.abs(w.sum(axis=1) - 1.0) < 1e-12), "renormalised sum"
    assert np.all((w > 0) & (w <= 1)), "weights in (0, 1]"


def pin_weights_k1_norm():
    x, wr, _, _ = _layer(16, 8, 4, 4, seed=6)
    _, _, w = O.route(x, wr, None, 1, True)
    assert np.all(w == 1.0), "k=1 renormalised weight is exactly 1"


def pin_weights_uniform():
    """Equal logits: softmax is 1/E; renormalised top-k is 1/k (powers of 2,
    so exact)."""
    L = np.zeros((4, 8), np.float32)
    ids = O.select_topk(L, 2)
    assert np.all(O.routing_weights(L, ids, True) == 0.5)
    assert np.all(O.routing_weights(L, ids, False) == 0.125)


def pin_weights_two_expert_closed_form():
    """E = 2, k = 1, no renormalisation: the selected weight is
    ``1 / (1 + exp(-(L_max - L_min)))``."""
    L = np.array([[0.3, -1.2], [2.0, 2.5], [-0.7, -0.7]], np.float32)
    ids = O.select_topk(L, 1)
    w = O.routing_weights(L, ids, False)
    for t in range(3):
        a, b = float(L[t].max()), float(L[t].min())
        assert abs(w[t, 0] - 1.0 / (1.0 + math.exp(-(a - b)))) < 1e-15


def pin_weights_full_softmax():
    r = _rng(7)
    L = r.standard_normal((9, 5)).astype(np.float32) * 4
    ids = O.select_topk(L, 5)
    w = O.routing_weights(L, ids, False)
    sm = scipy.special.softmax(L.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(sm, ids.astype(np.int64), 1), rtol=1e-13, atol=0)


# ----------------------------------------------------- counts / permutation

def pin_counts_and_permutation():
    r = _rng(8)
    T, E, k = 50, 7, 3
    ids = np.stack([r.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    c = O.expert_counts(ids, E)
    assert c.sum() == T * k and np.all(c <= T)
    assert np.array_equal(c, np.bincount(ids.ravel(), minlength=E))
    o = O.expert_offsets(c)
    assert o[0] == 0 and o[-1] == T * k and np.array_equal(np.diff(o), c)
    ss, st, sp = O.permutation(ids, E)
    ref = np.argsort(ids.ravel(), kind="stable")
    assert np.array_equal(ss, ref), "stable expert-major order"
    assert np.array_equal(st, ref // k)
    assert np.array_equal(np.sort(sp), np.arange(T * k)), "bijection"
    flat_t = np.repeat(np.arange(T), k)
    assert np.array_equal(st[sp], flat_t), "sorted_token[slot_pos[t*k+j]] == t"
    x = r.standard_normal((T, 4))
    back = O.unpermute(O.gather_rows(x, st), sp).reshape(T, k, 4)
    for j in range(k):
        assert np.array_equal(back[:, j], x), "gather then inverse is identity"


# ------------------------------------------------------------ experts/layer

def pin_brute_vs_loop():
    """Per-expert loop with index-add equals the all-expert masked path
    (the two forward paths of ``SpeedupMoeExperts``)."""
    x, wr, gu, dn = _layer(24, 16, 8, 6, seed=9)
    for k, norm in ((2, True), (3, False), (6, True)):
        a = O.moe_layer_forward(x, wr, None, gu, dn, k, norm)["out"]
        b = O.moe_layer_forward_brute(x, wr, None, gu, dn, k, norm)
        assert np.allclose(a, b, rtol=1e-12, atol=1e-12), "loop vs brute"


def pin_identical_experts():
    """Identical experts with renormalised weights: the output is the dense
    SwiGLU of the token whatever the routing."""
    x, wr, gu, dn = _layer(16, 12, 6, 5, seed=10)
    gu[:] = gu[0]
    dn[:] = dn[0]
    out = O.moe_layer_forward(x, wr, None, gu, dn, 2, True)["out"]
    assert np.allclose(out, _torch_swiglu(x, gu[0], dn[0]), rtol=1e-11, atol=1e-12)


def pin_single_expert_dense():
    x, wr, gu, dn = _layer(8, 10, 4, 1, seed=11)
    out = O.moe_layer_forward(x, wr, None, gu, dn, 1, False)["out"]
    assert np.allclose(out, _torch_swiglu(x, gu[0], dn[0]), rtol=1e-11, atol=1e-12)


def pin_soft_mixture():
    """k = E with renormalisation is the softmax-weighted sum of all experts."""
    x, wr, gu, dn = _layer(8, 8, 4, 4, seed=12)
    out = O.moe_layer_forward(x, wr, None, gu, dn, 4, True)["out"]
    L = (x.astype(np.float64) @ wr.astype(np.float64).T).astype(np.float32)
    p = scipy.special.softmax(L.astype(np.float64), axis=1)
    ref = sum(p[:, e:e + 1] * _torch_swiglu(x, gu[e], dn[e]) for e in range(4))
    assert np.allclose(out, ref, rtol=1e-11, atol=1e-12)


def pin_zero_token():
    x, wr, gu, dn = _layer(6, 8, 4, 4, seed=13)
    x[2] = 0.0
    out = O.moe_layer_forward(x, wr, None, gu, dn, 2, True)["out"]
    assert np.all(out[2] == 0.0), "silu(0) * 0 = 0"


def pin_scalar_closed_form():
    """H = I = 1, E = 2, k = 1: ``out = w * silu(x g) * (x u) * d`` with the
    gate in column 0 of ``gate_up`` and the up projection in column 1."""
    with open(os.path.join(GOLDEN, "scalar_layer.json")) as f:
        case = json.load(f)
    x = np.array(case["x"], np.float32).reshape(-1, 1)
    wr = np.array(case["router_weight"], np.float32).reshape(2, 1)
    gu = np.array(case["gate_up"], np.float32).reshape(2, 1, 2)
    dn = np.array(case["down"], np.float32).reshape(2, 1, 1)
    res = O.moe_layer_forward(x, wr, None, gu, dn, 1, case["norm_topk_prob"])
    for t, xv in enumerate(x[:, 0].tolist()):
        e = 0 if xv * float(wr[0, 0]) >= xv * float(wr[1, 0]) else 1
        if xv * float(wr[0, 0]) == xv * float(wr[1, 0]):
            e = 0
        g, u, d = float(gu[e, 0, 0]), float(gu[e, 0, 1]), float(dn[e, 0, 0])
        z = xv * g
        ref = (z / (1.0 + math.exp(-z))) * (xv * u) * d
        assert res["ids"][t, 0] == e
        assert abs(res["out"][t, 0] - ref) <= 1e-15 * max(1.0, abs(ref)), "scalar closed form"
    assert np.allclose(res["out"][:, 0], case["expected_out"], rtol=1e-12, atol=1e-15)


def pin_identity_expert_roundtrip():
    """Permute, apply an identity 'expert', combine with renormalised weights:
    the tokens come back."""
    r = _rng(14)
    T, E, k, H = 30, 6, 3, 5
    x = r.standard_normal((T, H))
    L = r.standard_normal((T, E)).astype(np.float32)
    ids = O.select_topk(L, k)
    w = O.routing_weights(L, ids, True)
    _, st, sp = O.permutation(ids, E)
    y = O.gather_rows(x, st)
    out = O.combine(O.unpermute(y, sp), w)
    assert np.allclose(out, x, rtol=1e-13, atol=1e-13)


def pin_token_subset():
    x, wr, gu, dn = _layer(20, 8, 4, 5, seed=15)
    full = O.moe_layer_forward(x, wr, None, gu, dn, 2, True)["out"]
    toks = [0, 7, 19, 3]
    sub = O.moe_layer_forward_tokens(x, wr, None, gu, dn, 2, True, toks)["out"]
    assert np.allclose(sub, full[toks], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------ EP rank

def pin_reshuffle_worked_example():
    """Hand-worked reshuffle: rank-major blocks (r0,e0)=[0], (r0,e1)=[1,2],
    (r1,e0)=[3,4,5], (r1,e1)=[] become expert-major e0: 0,3,4,5; e1: 1,2."""
    with open(os.path.join(GOLDEN, "reshuffle_example.json")) as f:
        case = json.load(f)
    src = O.reshuffle_rank_to_expert(np.array(case["counts_rank_major"]))
    assert src.tolist() == case["expert_major_source_rows"]


def pin_reshuffle_properties():
    r = _rng(16)
    C = r.integers(0, 5, (4, 3))
    C[1, 2] = 0
    src = O.reshuffle_rank_to_expert(C)
    N = int(C.sum())
    assert np.array_equal(np.sort(src), np.arange(N)), "bijection"
    x = r.standard_normal((N, 2))
    back = np.empty_like(x)
    back[src] = x[src]
    assert np.array_equal(back, x)


def pin_ep_equals_token_choice():
    """One rank owning every expert: the rank-major path, combined on the
    source side with the routing weights, equals the token-choice layer."""
    r = _rng(17)
    R, T, H, I, E, k = 3, 10, 8, 4, 4, 2
    xs = [r.standard_normal((T, H)).astype(np.float32) for _ in range(R)]
    wr = (0.5 * r.standard_normal((E, H))).astype(np.float32)
    gu = (0.3 * r.standard_normal((E, H, 2 * I))).astype(np.float32)
    dn = (0.3 * r.standard_normal((E, I, H))).astype(np.float32)
    rows, C, meta = O.dispatch_rank_major(xs, wr, k, True, 0, E)
    res = O.ep_rank_forward(rows, C, gu, dn)
    assert np.array_equal(res["counts"], C.sum(axis=0))
    for rr in range(R):
        ref = O.moe_layer_forward(xs[rr], wr, None, gu, dn, k, True)
        out = np.zeros((T, H))
        for i, (src_r, t, j) in enumerate(meta):
            if src_r == rr:
                out[t] += ref["weights"][t, j] * res["y_rm"][i]
        assert np.allclose(out, ref["out"], rtol=1e-12, atol=1e-13)



def pin_page_shape_examples():
    """The shapes the moe.py page's docstring examples print."""
    with open(os.path.join(GOLDEN, "page_shape_examples.json")) as f:
        case = json.load(f)
    g = case["grouped_experts"]
    r = _rng(18)
    x = r.standard_normal((g["tokens"], g["dim"]))
    gu = r.standard_normal((g["num_experts"], g["dim"], 2 * g["hidden_dim"]))
    dn = r.standard_normal((g["num_experts"], g["hidden_dim"], g["dim"]))
    assert list(O.grouped_swiglu(x, g["counts"], gu, dn).shape) == g["out_shape"]
    c = case["router"]
    x = r.standard_normal((c["tokens"], c["dim"])).astype(np.float32)
    wr = r.standard_normal((c["num_experts"], c["dim"])).astype(np.float32)
    L, ids, w = O.route(x, wr, None, c["top_k"], False)
    assert list(w.shape) == c["scores_shape"] and list(ids.shape) == c["indices_shape"]
    assert list(O.expert_counts(ids, c["num_experts"]).shape) == c["counts_shape"]
    m = case["moe"]
    b, s, d = m["input_shape"]
    x = r.standard_normal((b * s, d)).astype(np.float32)
    wr = r.standard_normal((m["num_experts"], d)).astype(np.float32)
    gu = r.standard_normal((m["num_experts"], d, 2 * m["hidden_dim"]))
    dn = r.standard_normal((m["num_experts"], m["hidden_dim"], d))
    out = O.moe_layer_forward(x, wr, None, gu, dn, m["top_k"], True)["out"]
    assert list(out.reshape(b, s, d).shape) == m["out_shape"]


# ---- router variants -------------------------------------------------------

def pin_variant_bias_steers_selection():
    # zero logits: every sigmoid score is 0.5 * scale, so the selection
    # follows the bias alone and the weights do not see it
    T, E, k, scale = 5, 8, 3, 2.5
    L = np.zeros((T, E), np.float32)
    bias = np.array([0.3, -0.2, 0.9, 0.1, 0.5, -0.7, 0.0, 0.2])
    ids, w, s, _ = O.route_variant(L, k, False, "sigmoid", scale, bias)
    assert (ids == np.array([2, 4, 0])[None, :]).all()
    assert np.array_equal(w, np.full((T, k), 0.5 * scale))
    ids, w, _, _ = O.route_variant(L, k, True, "sigmoid", scale, bias)
    assert np.allclose(w, 1.0 / k, rtol=0, atol=1e-15)
    # softmax of equal logits is 1/E
    ids, w, _, _ = O.route_variant(L, k, False, "softmax", 1.0, bias)
    assert (ids == np.array([2, 4, 0])[None, :]).all() and np.allclose(w, 1.0 / E, atol=1e-15)


def pin_variant_sigmoid_matches_expit():
    r = _rng(7)
    L = r.standard_normal((40, 16)).astype(np.float32) * 3
    k, scale = 4, 1.7
    ids, w, s, _ = O.route_variant(L, k, False, "sigmoid", scale)
    # sigmoid is monotone: without bias or groups the logit order decides
    assert np.array_equal(ids, O.select_topk(L, k))
    ref = scipy.special.expit(L.astype(np.float64)) * scale
    assert np.allclose(w, np.take_along_axis(ref, ids.astype(np.int64), 1), rtol=1e-14, atol=0)
    assert np.allclose(s, ref, rtol=1e-14, atol=0)


def pin_variant_softmax_equals_default_router():
    x, wr, _, _ = _layer(24, 32, 8, 16, seed=3)
    L, ids, w = O.route(x, wr, None, 4, True)
    ids2, w2, _, _ = O.route_variant(L, 4, True, "softmax", 1.0)
    assert np.array_equal(ids, ids2) and np.allclose(w, w2, rtol=1e-12, atol=0)


def pin_variant_groups_worked_example():
    # E = 8 in 4 groups of 2; group maxima 5, 4.5, 4, 3 (sigmoid keeps the
    # order).  Two groups kept: experts 0-3 only.
    L = np.array([[0, 5, 4.5, 1, 4, 0, 3, 2]], np.float32)
    ids, _, _, _ = O.route_variant(L, 3, False, "sigmoid", 1.0, None, 4, 2)
    assert ids.tolist() == [[1, 2, 3]]
    ids, _, _, _ = O.route_variant(L, 3, False, "sigmoid")
    assert ids.tolist() == [[1, 2, 4]]          # unrestricted: expert 4 wins
    ids, _, _, _ = O.route_variant(L, 2, False, "sigmoid", 1.0, None, 4, 1)
    assert ids.tolist() == [[1, 0]]             # only group 0
    # the bias moves selection inside the kept groups but not the groups
    ids, w, s, _ = O.route_variant(L, 2, False, "sigmoid", 1.0, np.array([0, 0, 0, 0, 9, 9, 0, 0.]),
                                   4, 2)
    assert ids.tolist() == [[1, 2]]
    assert np.allclose(w, scipy.special.expit(np.array([[5.0, 4.5]])), rtol=1e-14)


def pin_variant_groups_invariant():
    r = _rng(11)
    T, E, G, lim, k = 60, 32, 8, 3, 6
    L = r.standard_normal((T, E)).astype(np.float32)
    bias = r.standard_normal(E) * 0.3
    ids, w, s, key = O.route_variant(L, k, False, "sigmoid", 1.0, bias, G, lim)
    epg = E // G
    gmax = s.reshape(T, G, epg).max(axis=2)
    for t in range(T):
        groups = set(int(e) // epg for e in ids[t])
        assert len(groups) <= lim
        # the kept groups are the lim largest group maxima
        kept = sorted(range(G), key=lambda g: (-np.float32(gmax[t, g]), g))[:lim]
        allowed = [e for e in range(E) if e // epg in kept]
        assert set(int(e) // epg for e in ids[t]) <= set(kept)
        # and the selection is the k largest keys among them
        best = sorted(allowed, key=lambda e: (-np.float32(s[t, e] + bias[e]), e))[:k]
        assert ids[t].tolist() == best
        assert np.allclose(w[t], s[t, ids[t]], rtol=0, atol=0)


def pin_update_expert_bias_worked():
    b, z = O.update_expert_bias(np.zeros(4), np.array([3, 1, 2, 2.0]), lr=0.1)
    assert np.allclose(b, [-0.1, 0.1, 0.0, 0.0], atol=1e-15) and not z.any()
    # the step is centred: mean load 2, signs (+, +, +, -), mean step 0.05
    b, _ = O.update_expert_bias(np.array([1.0, 2, 3, 4]), np.array([1, 1, 1, 5.0]), lr=0.1)
    assert np.allclose(b, [1.05, 2.05, 3.05, 3.85], atol=1e-15)
    # counts accumulated over two forward passes are halved first
    b2, _ = O.update_expert_bias(np.array([1.0, 2, 3, 4]), np.array([2, 2, 2, 10.0]), lr=0.1,
                                 num_recomputations=2)
    assert np.allclose(b2, b, atol=1e-15)
    r = _rng(5)
    d, _ = O.update_expert_bias(np.zeros(64), r.integers(0, 100, 64).astype(float), lr=0.01)
    assert abs(d.sum()) < 1e-12


# ---- shared expert ----------------------------------------------------------

def _ffn_loops(x, w1, w2, w3):
    """FeedForward row by row with scalar loops: a linear layer with weight
    W [out, in] maps x to y[o] = sum_i W[o][i] x[i]."""
    out = []
    for row in np.asarray(x, np.float64).tolist():
        h = []
        for i in range(len(w1)):
            g = sum(a * b for a, b in zip(np.asarray(w1[i], np.float64).tolist(), row))
            u = sum(a * b for a, b in zip(np.asarray(w3[i], np.float64).tolist(), row))
            h.append(g / (1.0 + math.exp(-g)) * u)
        out.append([sum(a * b for a, b in zip(np.asarray(w2[o], np.float64).tolist(), h))
                    for o in range(len(w2))])
    return np.array(out)


def _ffn_weights(r, H, Is, scale=0.5):
    return (r.standard_normal((Is, H)) * scale, r.standard_normal((H, Is)) * scale,
            r.standard_normal((Is, H)) * scale)


def pin_feed_forward_loops():
    r = _rng(21)
    x = r.standard_normal((3, 4))
    w1, w2, w3 = _ffn_weights(r, 4, 5)
    assert np.allclose(O.feed_forward(x, w1, w2, w3), _ffn_loops(x, w1, w2, w3),
                       rtol=1e-13, atol=1e-15)


def pin_feed_forward_scalar():
    # H = Is = 1: out = c * silu(a x) * (b x), gate a = w1, up b = w3, down c = w2
    for x, a, b, c in ((1.5, 2.0, -0.5, 3.0), (-2.0, 0.25, 4.0, -1.0), (0.0, 1.0, 1.0, 1.0),
                       (3.0, 0.0, 2.0, 5.0)):
        z = a * x
        ref = c * (z / (1.0 + math.exp(-z))) * (b * x)
        got = O.feed_forward([[x]], [[a]], [[c]], [[b]])
        assert got.shape == (1, 1) and abs(got[0, 0] - ref) <= 1e-15 * max(1.0, abs(ref))
    # silu(0) = 0 kills the row whatever the up projection is
    assert O.feed_forward([[1.0]], [[0.0]], [[7.0]], [[9.0]])[0, 0] == 0.0


def _routed_copies(w1, w2, w3, E):
    """Routed experts in the concatenated layout that equal FeedForward(w1, w2,
    w3): gate columns x w1^T first, then up x w3^T; down is w2^T."""
    gu = np.concatenate([np.asarray(w1).T, np.asarray(w3).T], axis=1)
    return np.repeat(gu[None], E, 0), np.repeat(np.asarray(w2).T[None], E, 0)


def pin_shared_equals_routed_copies():
    r = _rng(22)
    T, H, Is, E, k = 12, 6, 4, 5, 2
    x = r.standard_normal((T, H))
    wr = r.standard_normal((E, H)).astype(np.float32)
    w1, w2, w3 = _ffn_weights(r, H, Is)
    gu, dn = _routed_copies(w1, w2, w3, E)
    ffn = _ffn_loops(x, w1, w2, w3)
    for norm in (True, False):
        res = O.moe_layer_forward(x, wr, None, gu, dn, k, norm, shared=(w1, w2, w3))
        wsum = res["weights"].sum(axis=1, keepdims=True)
        if norm:
            assert np.allclose(wsum, 1.0, atol=1e-15)
        else:
            assert np.all(wsum < 1.0)
        # the routed part is the FFN times the weight sum; the shared part is
        # added once, unweighted
        assert np.allclose(res["out"], (1.0 + wsum) * ffn, rtol=1e-12, atol=1e-13)
        assert np.allclose(res["shared_out"], ffn, rtol=1e-12, atol=1e-13)


def pin_shared_zero_routed():
    r = _rng(23)
    T, H, I, Is, E, k = 9, 8, 6, 10, 4, 3
    x = r.standard_normal((T, H))
    wr = r.standard_normal((E, H)).astype(np.float32)
    gu = r.standard_normal((E, H, 2 * I))
    w1, w2, w3 = _ffn_weights(r, H, Is)
    res = O.moe_layer_forward(x, wr, None, gu, np.zeros((E, I, H)), k, True, shared=(w1, w2, w3))
    assert np.allclose(res["out"], _ffn_loops(x, w1, w2, w3), rtol=1e-12, atol=1e-13)
    # a shared expert with zero down projection adds nothing
    dn = r.standard_normal((E, I, H))
    a = O.moe_layer_forward(x, wr, None, gu, dn, k, True, shared=(w1, np.zeros((H, Is)), w3))
    b = O.moe_layer_forward(x, wr, None, gu, dn, k, True)
    assert np.array_equal(a["out"], b["out"]) and b["shared_out"] is None


def pin_shared_brute_and_tokens():
    r = _rng(24)
    T, H, I, Is, E, k = 16, 8, 4, 12, 6, 2
    x = r.standard_normal((T, H)).astype(np.float32)
    wr = r.standard_normal((E, H)).astype(np.float32)
    gu = r.standard_normal((E, H, 2 * I)) * 0.5
    dn = r.standard_normal((E, I, H)) * 0.5
    sh = _ffn_weights(r, H, Is)
    full = O.moe_layer_forward(x, wr, None, gu, dn, k, False, shared=sh)["out"]
    brute = O.moe_layer_forward_brute(x, wr, None, gu, dn, k, False, shared=sh)
    assert np.allclose(full, brute, rtol=1e-12, atol=1e-12)
    toks = [3, 0, 15, 7]
    sub = O.moe_layer_forward_tokens(x, wr, None, gu, dn, k, False, toks, shared=sh)["out"]
    assert np.allclose(sub, full[toks], rtol=1e-12, atol=1e-12)


# ---- layer backward -----------------------------------------------------------

def _fd_layer(seed, norm, with_bias, T=4, H=6, I=3, E=5, k=2, eps=1e-3, router=None):
    r = _rng(seed)
    x = r.standard_normal((T, H))
    wr = r.standard_normal((E, H)) * 0.7
    b = r.standard_normal(E) * 0.3 if with_bias else None
    gu = r.standard_normal((E, H, 2 * I)) * 0.5
    dn = r.standard_normal((E, I, H)) * 0.5
    dout = r.standard_normal((T, H))
    g = O.moe_layer_backward(x, wr, b, gu, dn, k, norm, dout, router=router)
    ids0 = g["forward"]["ids"]

    def loss(x_, wr_, b_, gu_, dn_):
        f = O.moe_layer_forward(x_, wr_, b_, gu_, dn_, k, norm, router=router)
        assert np.array_equal(f["ids"], ids0), "perturbation changed the routing"
        return float((f["out"] * dout).sum())

    args = [x, wr, b, gu, dn]
    names = ["dx", "d_router_weight", "d_router_bias", "d_gate_up", "d_down"]
    for a, name in enumerate(names):
        if args[a] is None:
            continue
        fd = np.zeros_like(args[a])
        for idx in np.ndindex(args[a].shape):
            plus = [t.copy() if t is not None else None for t in args]
            minus = [t.copy() if t is not None else None for t in args]
            plus[a][idx] += eps
            minus[a][idx] -= eps
            fd[idx] = (loss(*plus) - loss(*minus)) / (2 * eps)
        an = g[name]
        err = np.abs(fd - an).max()
        # float32 logits add ~1e-7 / eps of noise to the differences
        assert err <= 2e-4 * max(1.0, np.abs(an).max()), f"{name}: finite differences off by {err}"
    return g


def pin_backward_finite_differences_renorm():
    g = _fd_layer(31, True, True)
    # renormalised: only the selected logits get a gradient
    mask = np.zeros_like(g["d_logits"], dtype=bool)
    np.put_along_axis(mask, g["forward"]["ids"].astype(np.int64), True, axis=1)
    assert np.all(g["d_logits"][~mask] == 0.0)


def pin_backward_finite_differences_plain():
    _fd_layer(32, False, False)


def pin_backward_finite_differences_k1_bias():
    _fd_layer(33, False, True, T=3, H=4, I=2, E=3, k=1)


def pin_backward_variant_sigmoid_renorm():
    _fd_layer(41, True, True, router=dict(score_func="sigmoid", route_scale=2.5))


def pin_backward_variant_sigmoid_groups_bias():
    # bias and groups steer the selection only; the gradient flows through
    # the unbiased sigmoid scores
    _fd_layer(42, False, False, T=5, E=6, k=2,
              router=dict(score_func="sigmoid", route_scale=1.5,
                          expert_bias=np.array([0.3, -0.2, 0.1, 0.0, 0.4, -0.1]),
                          n_groups=3, n_limited=2))


def pin_backward_variant_softmax_scaled():
    _fd_layer(43, False, True, router=dict(score_func="softmax", route_scale=1.7))


def pin_backward_variant_jacobian_matches_default():
    # the softmax variant with scale 1 is the default router: the Jacobian
    # path and the closed forms agree
    r = _rng(44)
    T, H, I, E, k = 12, 8, 4, 7, 3
    x = r.standard_normal((T, H))
    wr = r.standard_normal((E, H))
    gu = r.standard_normal((E, H, 2 * I)) * 0.4
    dn = r.standard_normal((E, I, H)) * 0.4
    dout = r.standard_normal((T, H))
    for norm in (True, False):
        a = O.moe_layer_backward(x, wr, None, gu, dn, k, norm, dout)
        b = O.moe_layer_backward(x, wr, None, gu, dn, k, norm, dout,
                                 router=dict(score_func="softmax", route_scale=1.0))
        assert np.array_equal(a["forward"]["ids"], b["forward"]["ids"])
        assert np.allclose(a["d_logits"], b["d_logits"], rtol=1e-12, atol=1e-14)
        assert np.allclose(a["dx"], b["dx"], rtol=1e-12, atol=1e-13)


def pin_backward_shared_expert_finite_differences():
    r = _rng(45)
    T, H, I, Is, E, k, eps = 4, 5, 3, 4, 4, 2, 1e-3
    x = r.standard_normal((T, H))
    wr = r.standard_normal((E, H))
    gu = r.standard_normal((E, H, 2 * I)) * 0.5
    dn = r.standard_normal((E, I, H)) * 0.5
    sh = [t * 1.0 for t in _ffn_weights(r, H, Is)]
    dout = r.standard_normal((T, H))
    g = O.moe_layer_backward(x, wr, None, gu, dn, k, True, dout, shared=tuple(sh))
    ids0 = g["forward"]["ids"]

    def loss(x_, sh_):
        f = O.moe_layer_forward(x_, wr, None, gu, dn, k, True, shared=tuple(sh_))
        assert np.array_equal(f["ids"], ids0)
        return float((f["out"] * dout).sum())

    for w_i in range(3):
        fd = np.zeros_like(sh[w_i])
        for idx in np.ndindex(sh[w_i].shape):
            p_, m_ = [t.copy() for t in sh], [t.copy() for t in sh]
            p_[w_i][idx] += eps
            m_[w_i][idx] -= eps
            fd[idx] = (loss(x, p_) - loss(x, m_)) / (2 * eps)
        assert np.abs(fd - g["d_shared"][w_i]).max() <= 2e-4 * max(1.0, np.abs(fd).max())
    fd = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += eps
        xm[idx] -= eps
        fd[idx] = (loss(xp, sh) - loss(xm, sh)) / (2 * eps)
    assert np.abs(fd - g["dx"]).max() <= 2e-4 * max(1.0, np.abs(fd).max())
    # the shared expert's gradients alone, against scalar loops at H = Is = 1
    a_, b_, c_, xv, dv = 0.7, -1.2, 0.9, 1.3, -0.4
    sgm = lambda z: 1.0 / (1.0 + math.exp(-z))  # noqa: E731
    z = a_ * xv
    ffb = O.feed_forward_backward([[xv]], [[a_]], [[c_]], [[b_]], [[dv]])
    dsilu = sgm(z) * (1 + z * (1 - sgm(z)))
    assert abs(ffb["d_w2"][0, 0] - dv * z * sgm(z) * b_ * xv) < 1e-12
    assert abs(ffb["d_w1"][0, 0] - dv * c_ * b_ * xv * dsilu * xv) < 1e-12
    assert abs(ffb["d_w3"][0, 0] - dv * c_ * z * sgm(z) * xv) < 1e-12


def pin_backward_scalar_closed_form():
    # H = I = 1, E = 2, k = 1, renormalised: w = 1, so the router gets no
    # gradient, and out = silu(x g) (x u) d
    x = np.array([[0.7], [-1.3], [2.0]])
    wr = np.array([[1.0], [-0.5]])
    gu = np.array([[[0.8, -1.1]], [[0.4, 0.9]]])
    dn = np.array([[[1.5]], [[-0.6]]])
    dout = np.array([[0.3], [-2.0], [1.1]])
    g = O.moe_layer_backward(x, wr, None, gu, dn, 1, True, dout)
    assert np.all(g["d_router_weight"] == 0) and np.all(g["d_router_bias"] == 0)
    sg = lambda z: 1.0 / (1.0 + math.exp(-z))  # noqa: E731
    dgu = np.zeros_like(gu)
    ddn = np.zeros_like(dn)
    for t in range(3):
        xv, dv = float(x[t, 0]), float(dout[t, 0])
        e = int(g["forward"]["ids"][t, 0])
        a, b, c = float(gu[e, 0, 0]), float(gu[e, 0, 1]), float(dn[e, 0, 0])
        z = a * xv
        s = sg(z)
        silu_z, dsilu = z * s, s * (1 + z * (1 - s))
        # out = silu(a x) (b x) c
        assert abs(g["dx"][t, 0] - dv * c * (dsilu * a * b * xv + silu_z * b)) < 1e-12
        dgu[e, 0, 0] += dv * c * dsilu * xv * b * xv
        dgu[e, 0, 1] += dv * c * silu_z * xv
        ddn[e, 0, 0] += dv * silu_z * b * xv
        assert abs(g["d_weights"][t, 0] - dv * silu_z * b * xv * c) < 1e-12
    assert np.allclose(g["d_gate_up"], dgu, rtol=0, atol=1e-12)
    assert np.allclose(g["d_down"], ddn, rtol=0, atol=1e-12)


def pin_backward_softmax_gradient_sums_to_zero():
    r = _rng(34)
    T, H, I, E, k = 20, 8, 4, 12, 3
    x = r.standard_normal((T, H))
    wr = r.standard_normal((E, H))
    gu = r.standard_normal((E, H, 2 * I)) * 0.3
    dn = r.standard_normal((E, I, H)) * 0.3
    dout = r.standard_normal((T, H))
    for norm in (True, False):
        g = O.moe_layer_backward(x, wr, None, gu, dn, k, norm, dout)
        assert np.allclose(g["d_logits"].sum(axis=1), 0.0, atol=1e-13)
        assert np.allclose(g["d_router_bias"], g["d_logits"].sum(axis=0), atol=1e-13)


def pin_backward_idle_experts_get_zero():
    r = _rng(35)
    T, H, I, E, k = 10, 8, 4, 6, 2
    x = r.standard_normal((T, H))
    wr = np.zeros((E, H))
    b = np.array([5.0, 4.0, 0.0, 0.0, 0.0, 0.0])    # every token picks experts 0 and 1
    gu = r.standard_normal((E, H, 2 * I))
    dn = r.standard_normal((E, I, H))
    g = O.moe_layer_backward(x, wr, b, gu, dn, k, False, r.standard_normal((T, H)))
    assert np.all(g["d_gate_up"][2:] == 0) and np.all(g["d_down"][2:] == 0)
    assert np.abs(g["d_gate_up"][:2]).max() > 0 and np.abs(g["d_down"][:2]).max() > 0


def pin_routing_decision_from_outside():
    # the oracle's own ids reproduce the default path bit for bit
    x, wr, gu, dn = _layer(16, 12, 6, 5, seed=36)
    a = O.moe_layer_forward(x, wr, None, gu, dn, 2, True)
    b = O.moe_layer_forward(x, wr, None, gu, dn, 2, True, ids=a["ids"])
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["weights"], b["weights"])
    # a forced choice with k = 1 renormalised: weight 1, the chosen expert's FFN
    forced = (np.arange(16) % 5).astype(np.int32)[:, None]
    c = O.moe_layer_forward(x, wr, None, gu, dn, 1, True, ids=forced)
    assert np.all(c["weights"] == 1.0)
    for t in range(16):
        e = int(forced[t, 0])
        ref = O.swiglu_expert(np.asarray(x)[t:t + 1], gu[e], dn[e])
        assert np.allclose(c["out"][t:t + 1], ref, rtol=1e-13, atol=1e-15)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
