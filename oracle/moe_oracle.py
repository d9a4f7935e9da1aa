"""CPU oracle for the Mixture-of-Experts layer: the forward, its router
variants and shared expert, and the layer backward.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, obviously correct
statement of what the layer computes.  Only the test suite, the package's
smoke check and the benchmark's CPU-baseline leg may import it; the library
and its binding never do, and this module never imports them.

Precision.  Every floating-point step runs in float64 (NumPy).  The one place
the pages fix a precision that decides an integer is the router: the gate
output is taken in float32 before the softmax and the top-k (MindSpore
hyper-parallel ``moe.py``, ``TokenChoiceTopKRouter.forward`` runs the gate
on float32 inputs so that the scores are stable; Qwen3-Omni issue #115,
``SpeedupMoeSparseMoeBlock.forward``: ``softmax(..., dtype=float)``).  So the
router logits are rounded once to float32 and the top-k decision is taken on
those float32 values; everything after that is float64 again.

Pages and sections cited below:

* [QO] Qwen3-Omni issue #115, "Training: Extremely Slow Deepspeed Engine
  initialization ...": ``SpeedupMoeExperts`` (concatenated experts
  ``gate_up_proj [E, H, 2I]``, ``down_proj [E, I, H]``; per-expert training
  loop and all-expert ``bmm`` eval path) and ``SpeedupMoeSparseMoeBlock.forward``
  (gate -> fp32 softmax -> top-k -> optional renormalisation).
* [HP] MindSpore hyper-parallel coverage page for ``moe.py``:
  ``TokenChoiceTopKRouter.forward``, ``_run_experts_for_loop``,
  ``MoE.permutation``, ``MoE.unpermutation``, ``MoE.forward``, and
  ``FeedForward`` (the always-active shared expert).
* [TP] transformers PR "Qwen3 moe": ``Ep2DpParallel._token_dispatch`` (layout of
  the rows one expert-parallel rank receives) and ``_token_combine``.
* [ED] transformers "Expert parallelism" docs, section "Token dispatch"
  (contiguous expert blocks per rank; combine with routing weights on the
  source rank).

Readings where the pages leave a step open (each also listed in the design
notes): logits stay float32 (not bf16) before the softmax; the top-k ranks the
float32 logits (softmax is monotone, so the selected set is the same) with
ties going to the lower expert id and ``-0.0 == +0.0``; slots of one token are
ordered by that key; the routing weight multiplies the expert output in the
combine (as [QO] does), not the expert input; no epsilon in the
renormalisation.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "router_logits", "select_topk", "routing_weights", "route",
    "router_scores", "limited_group_mask", "route_variant", "update_expert_bias",
    "expert_counts", "expert_offsets", "permutation", "gather_rows",
    "silu", "swiglu_expert", "grouped_swiglu", "combine", "unpermute", "feed_forward",
    "moe_layer_forward", "moe_layer_forward_brute", "moe_layer_forward_tokens",
    "silu_grad", "moe_layer_backward", "routing_weight_jacobian", "feed_forward_backward",
    "dispatch_rank_major", "reshuffle_rank_to_expert", "ep_rank_forward",
]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Router  ([QO] SpeedupMoeSparseMoeBlock.forward; [HP] TokenChoiceTopKRouter.forward)
# ---------------------------------------------------------------------------

def router_logits(x, w_router, bias=None) -> np.ndarray:
    """Router logits ``L[t, e] = sum_h x[t, h] * Wr[e, h] (+ b[e])``.

    ``Wr`` has the ``nn.Linear(H, E)`` layout ``[E, H]`` ([QO] ``self.gate``;
    [HP] ``self.gate = nn.Linear(dim, num_experts)``).  The optional per-expert
    bias is added to the logit (it is the skewed workload's popularity knob).
    Computed in float64, rounded once to float32 (the gate is taken in float32
    on both pages)."""
    L = _f64(x) @ _f64(w_router).T
    if bias is not None:
        L = L + _f64(bias)[None, :]
    L32 = L.astype(np.float32)
    if not np.all(np.isfinite(L32)):
        raise ValueError("router logits must be finite")
    return L32


def select_topk(logits32: np.ndarray, k: int) -> np.ndarray:
    """Top-k experts per token ([QO] ``torch.topk(routing_weights, top_k)``;
    [HP] ``scores_with_bias.topk``).

    Experts are ranked by the key (-logit, expert id): larger float32 logit
    first, equal logits (float equality, so -0.0 equals +0.0) go to the lower
    id.  Returns ``ids[T, k]`` int32 in that order."""
    L = np.asarray(logits32, dtype=np.float32)
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("top_k must be in [1, E]")
    eid = np.broadcast_to(np.arange(E, dtype=np.int64), L.shape)
    # np.lexsort sorts by the last key first; -L compares -0.0 == +0.0.
    order = np.lexsort((eid, -L.astype(np.float64)), axis=-1)
    return order[:, :k].astype(np.int32)


def routing_weights(logits32: np.ndarray, ids: np.ndarray, norm_topk_prob: bool) -> np.ndarray:
    """Routing weights of the selected experts ([QO] forward: fp32 softmax
    over all experts, keep the top-k probabilities, divide by their sum when
    ``norm_topk_prob``).  Softmax uses the max-subtracted form; float64."""
    L = _f64(logits32)
    m = L.max(axis=1, keepdims=True)
    p = np.exp(L - m)
    p = p / p.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if norm_topk_prob:
        w = w / w.sum(axis=1, keepdims=True)
    return w


def route(x, w_router, bias, top_k: int, norm_topk_prob: bool):
    """Router logits, top-k ids and routing weights for every token."""
    L = router_logits(x, w_router, bias)
    ids = select_topk(L, top_k)
    w = routing_weights(L, ids, norm_topk_prob)
    return L, ids, w


# ---------------------------------------------------------------------------
# Router variants  ([HP] TokenChoiceTopKRouter.forward and
# _get_node_limited_routing_scores; MoE.update_expert_bias)
# ---------------------------------------------------------------------------

def router_scores(logits32, score_func: str = "sigmoid", route_scale: float = 1.0) -> np.ndarray:
    """Routing scores ([HP] ``TokenChoiceTopKRouter.forward``): the float32
    gate output through a sigmoid (the page's default) or a softmax over the
    experts, then multiplied by ``route_scale``.  Float64."""
    L = _f64(logits32)
    if score_func == "sigmoid":
        s = 1.0 / (1.0 + np.exp(-L))
    elif score_func == "softmax":
        p = np.exp(L - L.max(axis=1, keepdims=True))
        s = p / p.sum(axis=1, keepdims=True)
    else:
        raise ValueError(f"unknown score function {score_func!r}: use sigmoid or softmax")
    return s * float(route_scale)


def limited_group_mask(scores, n_groups: int, n_limited: int) -> np.ndarray:
    """Node-limited routing ([HP] ``_get_node_limited_routing_scores``):
    experts are cut into ``n_groups`` contiguous groups, a group's score is the
    largest score among its experts, and each token keeps the ``n_limited``
    groups with the largest group scores.  Returns the boolean ``[T, E]`` mask
    of experts that stay selectable.  The group ranking is decided on float32
    group scores (the page works in float32), ties going to the lower group
    id."""
    S = _f64(scores)
    T, E = S.shape
    if n_groups < 1 or E % n_groups or not 1 <= n_limited <= n_groups:
        raise ValueError("need E % n_groups == 0 and 1 <= n_limited <= n_groups")
    epg = E // n_groups
    gs = S.reshape(T, n_groups, epg).max(axis=2).astype(np.float32)
    gid = np.broadcast_to(np.arange(n_groups), gs.shape)
    keep = np.lexsort((gid, -gs.astype(np.float64)), axis=-1)[:, :n_limited]
    mask = np.zeros((T, n_groups), dtype=bool)
    np.put_along_axis(mask, keep, True, axis=1)
    return np.repeat(mask, epg, axis=1)


def route_variant(logits32, top_k: int, norm_topk_prob: bool = False, score_func: str = "sigmoid",
                  route_scale: float = 1.0, expert_bias=None, n_groups: int = 0,
                  n_limited: int = 0):
    """Generalised token-choice router ([HP] ``TokenChoiceTopKRouter.forward``).

    1. scores = score_func(float32 logits) * route_scale;
    2. with node-limited routing, experts outside the token's best groups are
       not selectable;
    3. the selection key is score + expert_bias (the bias steers selection
       only), decided in float32; the top-k keys are taken in descending
       order, equal keys going to the lower expert id;
    4. the routing weights are the unbiased scores of the selected experts,
       divided by their sum when ``norm_topk_prob``.

    Returns ``(ids[T, k] int32, weights[T, k] float64, scores[T, E] float64,
    keys[T, E] float32)`` where non-selectable experts have key -inf."""
    s = router_scores(logits32, score_func, route_scale)
    T, E = s.shape
    if not 1 <= top_k <= E:
        raise ValueError("top_k must be in [1, E]")
    key = s + (0.0 if expert_bias is None else _f64(expert_bias)[None, :])
    key32 = key.astype(np.float32)
    if n_groups:
        allowed = limited_group_mask(s, n_groups, n_limited)
        if top_k > allowed[0].sum():
            raise ValueError("top_k exceeds the experts of the kept groups")
        key32 = np.where(allowed, key32, np.float32(-np.inf))
    eid = np.broadcast_to(np.arange(E), s.shape)
    ids = np.lexsort((eid, -key32.astype(np.float64)), axis=-1)[:, :top_k].astype(np.int32)
    w = np.take_along_axis(s, ids.astype(np.int64), axis=1)
    if norm_topk_prob:
        w = w / w.sum(axis=1, keepdims=True)
    return ids, w, s, key32


def update_expert_bias(expert_bias, tokens_per_expert, lr: float = 1e-3,
                       num_recomputations: int = 1):
    """Auxiliary-loss-free bias step ([HP] ``MoE.update_expert_bias``): the
    accumulated token counts are divided by the number of forward passes per
    step, every expert's bias moves by ``lr`` toward the mean load
    (``lr * sign(mean - load)``), the step is centred to zero mean, and the
    accumulator is cleared.  Returns ``(new_bias, new_tokens_per_expert)``."""
    tpe = _f64(tokens_per_expert)
    if num_recomputations > 1:
        tpe = tpe / num_recomputations
    delta = float(lr) * np.sign(tpe.mean() - tpe)
    delta = delta - delta.mean()
    return _f64(expert_bias) + delta, np.zeros_like(tpe)


# ---------------------------------------------------------------------------
# Histogram and permutation  ([HP] MoE.permutation, TokenChoiceTopKRouter.forward)
# ---------------------------------------------------------------------------

def expert_counts(ids: np.ndarray, E: int) -> np.ndarray:
    """Tokens per expert ([HP] ``torch.bincount(selected_experts.flatten(),
    minlength=num_experts)``): count each (token, slot) pair once."""
    c = np.zeros(E, dtype=np.int64)
    for e in np.asarray(ids).reshape(-1):
        c[int(e)] += 1
    return c.astype(np.int32)


def expert_offsets(counts: np.ndarray) -> np.ndarray:
    """Start row of each expert's group in expert-major order, plus the end:
    ``o[0] = 0, o[e + 1] = o[e] + c[e]``."""
    o = np.zeros(len(counts) + 1, dtype=np.int64)
    for e, c in enumerate(counts):
        o[e + 1] = o[e] + int(c)
    return o.astype(np.int32)


def permutation(ids: np.ndarray, E: int):
    """Token-major -> expert-major order ([HP] ``MoE.permutation``: a stable
    argsort of the flattened expert ids; ``token_indices = flat // top_k``).

    Written out directly: for each expert in ascending id, the flat slots
    ``t * k + j`` that chose it, in ascending slot order (so ascending token,
    since a token never picks one expert twice).

    Returns ``(sorted_slot[N], sorted_token[N], slot_pos[N])``:
    ``sorted_slot[p]`` is the flat slot at expert-major position ``p``,
    ``sorted_token[p] = sorted_slot[p] // k`` its token, and ``slot_pos`` the
    inverse (``slot_pos[sorted_slot[p]] = p``)."""
    ids = np.asarray(ids)
    T, k = ids.shape
    flat = ids.reshape(-1)
    order: List[int] = []
    for e in range(E):
        order.extend(int(i) for i in np.flatnonzero(flat == e))
    sorted_slot = np.asarray(order, dtype=np.int64)
    slot_pos = np.empty(T * k, dtype=np.int64)
    slot_pos[sorted_slot] = np.arange(T * k)
    return (sorted_slot.astype(np.int32), (sorted_slot // k).astype(np.int32),
            slot_pos.astype(np.int32))


def gather_rows(x, index) -> np.ndarray:
    """``x[index]`` ([HP] ``routed_x = x_flat[token_indices]``)."""
    return np.asarray(x)[np.asarray(index, dtype=np.int64)]


# ---------------------------------------------------------------------------
# Experts  ([QO] SpeedupMoeExperts; [HP] _run_experts_for_loop)
# ---------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """SiLU, ``z * sigmoid(z) = z / (1 + exp(-z))``."""
    z = _f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_expert(x_rows, gate_up_e, down_e) -> np.ndarray:
    """One expert on its rows ([QO] training path: ``gate_up = state @
    gate_up_proj[e]``; ``gate, up = gate_up.chunk(2)``; ``up * act(gate)``;
    ``@ down_proj[e]``).  Gate is the first I columns of ``gate_up``."""
    gu = _f64(gate_up_e)
    I2 = gu.shape[1]
    I = I2 // 2
    G = _f64(x_rows) @ gu
    g, u = G[:, :I], G[:, I:]
    h = silu(g) * u
    return h @ _f64(down_e)


def grouped_swiglu(x_rows_expert_major, counts, gate_up, down) -> np.ndarray:
    """Per-expert SwiGLU over rows already in expert-major order, split by
    ``counts`` ([HP] ``_run_experts_for_loop``; empty experts are skipped)."""
    X = np.asarray(x_rows_expert_major)
    N = X.shape[0]
    H = np.asarray(down).shape[2]
    Y = np.zeros((N, H), dtype=np.float64)
    start = 0
    for e, n in enumerate(np.asarray(counts).tolist()):
        if n == 0:
            continue
        Y[start:start + n] = swiglu_expert(X[start:start + n], gate_up[e], down[e])
        start += n
    return Y


def combine(y_slot_major, weights) -> np.ndarray:
    """Weighted sum of each token's k expert outputs in slot order:
    ``out[t] = sum_j w[t, j] * y[t * k + j]`` ([QO] ``expert_out * routing_weights``
    then ``index_add_`` into the token rows; [HP] ``MoE.unpermutation``)."""
    w = _f64(weights)
    T, k = w.shape
    Y = _f64(y_slot_major).reshape(T, k, -1)
    out = np.zeros((T, Y.shape[2]), dtype=np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * Y[:, j, :]
    return out


def unpermute(y_expert_major, slot_pos) -> np.ndarray:
    """Expert-major rows back to flat-slot order: ``y_slot[i] = y[slot_pos[i]]``."""
    return _f64(y_expert_major)[np.asarray(slot_pos, dtype=np.int64)]


# ---------------------------------------------------------------------------
# Shared expert  ([HP] FeedForward; MoE.forward adds its output to the
# unpermuted routed output)
# ---------------------------------------------------------------------------

def feed_forward(x, w1, w2, w3) -> np.ndarray:
    """[HP] ``FeedForward.forward``: ``w2(silu(w1(x)) * w3(x))`` with the
    weights as ``nn.Linear`` stores them (``w1``, ``w3``: [Is, H]; ``w2``:
    [H, Is]; no bias), so a linear layer maps a row ``x`` to ``x W^T``."""
    x = _f64(x)
    return (silu(x @ _f64(w1).T) * (x @ _f64(w3).T)) @ _f64(w2).T


def _add_shared(out, x, shared):
    """[HP] ``MoE.forward``: the shared expert sees every token (``x_flat``)
    and its output is added, unweighted, after the unpermutation."""
    if shared is None:
        return out, None
    s = feed_forward(x, *shared)
    return out + s, s


# ---------------------------------------------------------------------------
# The layer  ([QO] SpeedupMoeSparseMoeBlock.forward + SpeedupMoeExperts training
# path; [HP] MoE.forward)
# ---------------------------------------------------------------------------

def moe_layer_forward(x, w_router, bias, gate_up, down, top_k: int,
                      norm_topk_prob: bool, shared=None, ids=None, router=None) -> dict:
    """Full layer: route, permute, per-expert SwiGLU loop, combine, and the
    optional shared expert ``shared = (w1, w2, w3)`` (``FeedForward`` weights).
    ``ids`` replaces the top-k decision with one taken elsewhere (a device's
    top-k of its own float32 logits, checked separately); the routing weights
    are then this module's at those ids.  ``router`` selects a router variant
    ([HP] ``TokenChoiceTopKRouter``): a dict of ``route_variant``'s keyword
    arguments ``score_func``, ``route_scale``, ``expert_bias``, ``n_groups``,
    ``n_limited``.

    Returns a dict with ``logits`` (float32 [T, E]), ``ids`` ([T, k]),
    ``weights`` ([T, k] float64), ``counts``, ``offsets``, ``sorted_slot``,
    ``sorted_token``, ``slot_pos``, ``y`` (expert-major expert outputs, float64
    [N, H]), ``shared_out`` (float64 [T, H] or None) and ``out`` (float64
    [T, H])."""
    x = np.asarray(x)
    E = np.asarray(w_router).shape[0]
    if router is not None:
        L = router_logits(x, w_router, bias)
        if ids is None:
            ids, w, _, _ = route_variant(L, top_k, norm_topk_prob, **router)
        else:
            ids = np.asarray(ids, dtype=np.int32)
            sc = router_scores(L, router.get("score_func", "sigmoid"), router.get("route_scale", 1.0))
            w = np.take_along_axis(sc, ids.astype(np.int64), axis=1)
            if norm_topk_prob:
                w = w / w.sum(axis=1, keepdims=True)
    elif ids is None:
        L, ids, w = route(x, w_router, bias, top_k, norm_topk_prob)
    else:
        L = router_logits(x, w_router, bias)
        ids = np.asarray(ids, dtype=np.int32)
        w = routing_weights(L, ids, norm_topk_prob)
    counts = expert_counts(ids, E)
    offsets = expert_offsets(counts)
    sorted_slot, sorted_token, slot_pos = permutation(ids, E)
    y = np.zeros((ids.size, np.asarray(down).shape[2]), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        y[lo:hi] = swiglu_expert(gather_rows(x, sorted_token[lo:hi]), gate_up[e], down[e])
    out, shared_out = _add_shared(combine(unpermute(y, slot_pos), w), x, shared)
    return dict(logits=L, ids=ids, weights=w, counts=counts, offsets=offsets,
                sorted_slot=sorted_slot, sorted_token=sorted_token,
                slot_pos=slot_pos, y=y, shared_out=shared_out, out=out)


def moe_layer_forward_brute(x, w_router, bias, gate_up, down, top_k: int,
                            norm_topk_prob: bool, shared=None) -> np.ndarray:
    """Every expert applied to every token, then masked by the selection and
    weighted ([QO] ``SpeedupMoeExperts`` eval path: ``bmm`` over all experts,
    one-hot mask times routing weights, sum over experts).  Small inputs only."""
    L, ids, w = route(x, w_router, bias, top_k, norm_topk_prob)
    E = np.asarray(w_router).shape[0]
    T = np.asarray(x).shape[0]
    out = np.zeros((T, np.asarray(down).shape[2]), dtype=np.float64)
    for e in range(E):
        y_all = swiglu_expert(x, gate_up[e], down[e])          # [T, H]
        mask_w = np.where(ids == e, w, 0.0).sum(axis=1)        # [T]
        out += mask_w[:, None] * y_all
    return _add_shared(out, x, shared)[0]


def moe_layer_forward_tokens(x, w_router, bias, gate_up, down, top_k: int,
                             norm_topk_prob: bool, tokens: Sequence[int],
                             shared=None) -> dict:
    """The layer output for a chosen subset of tokens only.  Each token is
    routed and combined on its own, so its row equals the full layer's row
    ([QO] per-token reading of the forward).  Used to spot-check large
    workloads."""
    xs = np.asarray(x)[np.asarray(tokens, dtype=np.int64)]
    L, ids, w = route(xs, w_router, bias, top_k, norm_topk_prob)
    out = np.zeros((xs.shape[0], np.asarray(down).shape[2]), dtype=np.float64)
    for j in range(top_k):
        for e in np.unique(ids[:, j]):
            rows = np.flatnonzero(ids[:, j] == e)
            out[rows] += w[rows, j:j + 1] * swiglu_expert(xs[rows], gate_up[int(e)], down[int(e)])
    out, _ = _add_shared(out, xs, shared)
    return dict(logits=L, ids=ids, weights=w, out=out)


# ---------------------------------------------------------------------------
# The layer backward: the gradient of moe_layer_forward (the pages train this
# layer with autograd: [QO] SpeedupMoeExperts' training path, [HP] MoE.forward)
# ---------------------------------------------------------------------------

def silu_grad(z: np.ndarray) -> np.ndarray:
    """d/dz silu(z) = s(z) (1 + z (1 - s(z))) with s the logistic sigmoid."""
    z = _f64(z)
    with np.errstate(over="ignore"):
        sg = 1.0 / (1.0 + np.exp(-z))
    return sg * (1.0 + z * (1.0 - sg))


def routing_weight_jacobian(logits32, ids, norm_topk_prob: bool, score_func: str = "softmax",
                            route_scale: float = 1.0) -> np.ndarray:
    """``J[t, j, e] = d w[t, j] / d L[t, e]`` for the routing weights of a
    router variant ([HP] ``TokenChoiceTopKRouter.forward``): scores
    ``s = score_func(L) * route_scale`` (softmax: ``ds_a/dL_e = scale
    p_a (delta_ae - p_e)``; sigmoid: ``scale sg_a (1 - sg_a) delta_ae``), the
    selected scores, and with renormalisation ``w_j = s_j / Z``,
    ``dw_j/dL_e = (ds_j/dL_e - w_j sum_i ds_i/dL_e) / Z`` over the selection.
    The selection itself (bias, groups) has no gradient.  Float64 [T, k, E]."""
    L = _f64(logits32)
    T, E = L.shape
    ii = np.asarray(ids, dtype=np.int64)
    eye = np.eye(E)
    if score_func == "softmax":
        p = np.exp(L - L.max(axis=1, keepdims=True))
        p = p / p.sum(axis=1, keepdims=True)
        s = route_scale * p
        ds = route_scale * p[:, :, None] * (eye[None] - p[:, None, :])      # [T, a, e]
    elif score_func == "sigmoid":
        sg = 1.0 / (1.0 + np.exp(-L))
        s = route_scale * sg
        ds = (route_scale * sg * (1.0 - sg))[:, :, None] * eye[None]
    else:
        raise ValueError(f"unknown score function {score_func!r}: use sigmoid or softmax")
    dsel = np.take_along_axis(ds, ii[:, :, None], axis=1)                  # [T, k, E]
    if not norm_topk_prob:
        return dsel
    ssel = np.take_along_axis(s, ii, axis=1)
    Z = ssel.sum(axis=1)
    w = ssel / Z[:, None]
    return (dsel - w[:, :, None] * dsel.sum(axis=1)[:, None, :]) / Z[:, None, None]


def feed_forward_backward(x, w1, w2, w3, dout) -> dict:
    """Gradients of ``sum(dout * feed_forward(x, w1, w2, w3))`` ([HP]
    ``FeedForward``): with ``a = x w1^T``, ``b = x w3^T``,
    ``h = silu(a) * b``: ``dh = dout w2``, ``d_w2 = dout^T h``,
    ``da = dh * b * silu'(a)``, ``db = dh * silu(a)``, ``d_w1 = da^T x``,
    ``d_w3 = db^T x``, ``dx = da w1 + db w3``.  Float64, nn.Linear layouts."""
    X, D = _f64(x), _f64(dout)
    w1, w2, w3 = _f64(w1), _f64(w2), _f64(w3)
    a, b = X @ w1.T, X @ w3.T
    h = silu(a) * b
    dh = D @ w2
    da = dh * b * silu_grad(a)
    db = dh * silu(a)
    return dict(dx=da @ w1 + db @ w3, d_w1=da.T @ X, d_w2=D.T @ h, d_w3=db.T @ X)


def moe_layer_backward(x, w_router, bias, gate_up, down, top_k: int, norm_topk_prob: bool,
                       dout, ids=None, router=None, shared=None) -> dict:
    """Gradients of ``sum(dout * out)`` for the layer of ``moe_layer_forward``.

    The routing decision (which experts) is piecewise constant, so gradients
    flow through the routing weights' values, the experts and the combine
    only.  Steps, from the output back:

    * combine: ``out[t] = sum_j w[t, j] y[t, j]`` gives
      ``d_weights[t, j] = <dout[t], y[t, j]>`` and ``dy[t, j] = w[t, j] dout[t]``;
    * expert e on its rows: ``y = h Wd``, ``h = silu(g) * u``, ``[g | u] = X Wgu``:
      ``dWd = h^T dy``, ``dh = dy Wd^T``, ``du = dh silu(g)``,
      ``dg = dh u silu'(g)``, ``dWgu = X^T [dg | du]``,
      ``dX = [dg | du] Wgu^T`` added into each row's token;
    * routing weights: ``w = softmax(L)[ids]`` gives
      ``dL = p (g - <g, p>)`` with ``g`` the scattered ``d_weights``; with
      renormalisation ``w`` is the softmax over the selected logits, so
      ``dL[ids] = w (d_weights - <d_weights, w>)`` and zero elsewhere;
    * router: ``dx += dL Wr``, ``dWr = dL^T x``, ``db = sum_t dL``.

    Returns float64 ``dx``, ``d_router_weight``, ``d_router_bias``,
    ``d_gate_up``, ``d_down``, ``d_weights`` [T, k] and ``d_logits`` [T, E],
    plus the forward's dict under ``forward``.  ``ids`` and ``router`` as in
    ``moe_layer_forward``; with a router variant the logits' gradient is
    ``sum_j d_weights[t, j] J[t, j, e]`` with ``routing_weight_jacobian``.
    With a shared expert ``shared = (w1, w2, w3)`` (added unweighted, [HP]
    ``MoE.forward``) its ``feed_forward_backward`` adds to ``dx`` and the
    result carries ``d_shared = (d_w1, d_w2, d_w3)``."""
    fwd = moe_layer_forward(x, w_router, bias, gate_up, down, top_k, norm_topk_prob, ids=ids,
                            router=router, shared=shared)
    X = _f64(x)
    D = _f64(dout)
    T, H = X.shape
    k = top_k
    gu, dn = _f64(gate_up), _f64(down)
    E, I = gu.shape[0], gu.shape[2] // 2
    ids, w = fwd["ids"], fwd["weights"]
    # combine
    y_slot = unpermute(fwd["y"], fwd["slot_pos"]).reshape(T, k, H)
    d_w = np.einsum("th,tjh->tj", D, y_slot)
    dy = (w[:, :, None] * D[:, None, :]).reshape(T * k, H)
    # experts
    dx = np.zeros((T, H))
    dgu = np.zeros_like(gu)
    ddn = np.zeros_like(dn)
    offsets, sorted_slot = fwd["offsets"], fwd["sorted_slot"]
    for e in range(E):
        slots = sorted_slot[offsets[e]:offsets[e + 1]].astype(np.int64)
        if slots.size == 0:
            continue
        tok = slots // k
        Xe = X[tok]
        G = Xe @ gu[e]
        g, u = G[:, :I], G[:, I:]
        h = silu(g) * u
        dY = dy[slots]
        ddn[e] = h.T @ dY
        dh = dY @ dn[e].T
        dG = np.concatenate([dh * u * silu_grad(g), dh * silu(g)], axis=1)
        dgu[e] = Xe.T @ dG
        np.add.at(dx, tok, dG @ gu[e].T)
    # routing weights -> logits
    L = _f64(fwd["logits"])
    ii = ids.astype(np.int64)
    dL = np.zeros((T, E))
    if router is not None:
        sf, sc = router.get("score_func", "sigmoid"), router.get("route_scale", 1.0)
        for t0 in range(0, T, 256):          # [T, k, E] Jacobians, 256 tokens at a time
            J = routing_weight_jacobian(L[t0:t0 + 256].astype(np.float32), ids[t0:t0 + 256],
                                        norm_topk_prob, sf, sc)
            dL[t0:t0 + 256] = np.einsum("tj,tje->te", d_w[t0:t0 + 256], J)
    elif norm_topk_prob:
        inner = (d_w * w).sum(axis=1, keepdims=True)
        np.put_along_axis(dL, ii, w * (d_w - inner), axis=1)
    else:
        p = np.exp(L - L.max(axis=1, keepdims=True))
        p = p / p.sum(axis=1, keepdims=True)
        gsc = np.zeros((T, E))
        np.put_along_axis(gsc, ii, d_w, axis=1)
        dL = p * (gsc - (gsc * p).sum(axis=1, keepdims=True))
    # router
    Wr = _f64(w_router)
    dx += dL @ Wr
    d_shared = None
    if shared is not None:
        sg = feed_forward_backward(X, *shared, D)
        dx += sg["dx"]
        d_shared = (sg["d_w1"], sg["d_w2"], sg["d_w3"])
    return dict(dx=dx, d_router_weight=dL.T @ X, d_router_bias=dL.sum(axis=0),
                d_gate_up=dgu, d_down=ddn, d_weights=d_w, d_logits=dL, d_shared=d_shared,
                forward=fwd)


# ---------------------------------------------------------------------------
# One expert-parallel rank  ([TP] Ep2DpParallel; [ED] "Token dispatch")
# ---------------------------------------------------------------------------

def dispatch_rank_major(source_hidden: Sequence, w_router, top_k: int,
                        norm_topk_prob: bool, local_lo: int, E_local: int):
    """Rows one EP rank receives, laid out rank-major.

    Each source rank routes its own tokens with the shared router, keeps the
    (token, expert) pairs whose expert lies in this rank's contiguous block
    ``[local_lo, local_lo + E_local)`` ([ED]: experts are cut into contiguous
    blocks), orders them by (local expert, token) and sends them; the receiver
    concatenates by source rank ([TP] ``_token_dispatch``: the all-to-all
    returns rows grouped by source rank, each block ordered by local expert).

    Returns ``(rows[N, H] float32, counts_rm[R, E_local] int32, meta)`` with
    ``meta[i] = (source rank, token, slot j)`` of received row ``i``."""
    rows, meta = [], []
    R = len(source_hidden)
    C = np.zeros((R, E_local), dtype=np.int64)
    for r, xr in enumerate(source_hidden):
        xr = np.asarray(xr)
        L, ids, _ = route(xr, w_router, None, top_k, norm_topk_prob)
        for el in range(E_local):
            e = local_lo + el
            tok, slot = np.nonzero(ids == e)       # row-major: ascending token
            C[r, el] = len(tok)
            rows.append(xr[tok])
            meta.extend((r, int(t), int(j)) for t, j in zip(tok, slot))
    H = np.asarray(source_hidden[0]).shape[1]
    R_rm = np.concatenate(rows, axis=0) if rows else np.zeros((0, H), np.float32)
    return R_rm, C.astype(np.int32), meta


def reshuffle_rank_to_expert(counts_rm: np.ndarray) -> np.ndarray:
    """Index map from expert-major position to rank-major row.

    Received rows are blocks ``(source rank r, local expert e)`` in rank-major
    order; the experts need blocks ``(e, r)``.  Block order within a block is
    kept.  Returns ``src[p]``: the rank-major row placed at expert-major
    position ``p`` ([TP] ``_reshuffle_indices`` / the comment that the
    received rows "need to be reshuffled")."""
    C = np.asarray(counts_rm, dtype=np.int64)
    R, El = C.shape
    start = np.zeros((R, El), dtype=np.int64)
    pos = 0
    for r in range(R):
        for e in range(El):
            start[r, e] = pos
            pos += C[r, e]
    src: List[int] = []
    for e in range(El):
        for r in range(R):
            src.extend(range(int(start[r, e]), int(start[r, e] + C[r, e])))
    return np.asarray(src, dtype=np.int32)


def ep_rank_forward(rows_rm, counts_rm, gate_up_local, down_local) -> dict:
    """Reshuffle received rows to expert-major, run the local experts, and put
    the outputs back in rank-major order.  No routing weight is applied here:
    the source rank combines ([ED] "Token dispatch"; [TP] ``_token_combine``
    returns the raw expert outputs)."""
    src = reshuffle_rank_to_expert(counts_rm)
    counts_em = np.asarray(counts_rm, dtype=np.int64).sum(axis=0)
    X = gather_rows(rows_rm, src)
    Y_em = grouped_swiglu(X, counts_em, gate_up_local, down_local)
    Y_rm = np.zeros_like(Y_em)
    Y_rm[src.astype(np.int64)] = Y_em
    return dict(src=src, counts=counts_em.astype(np.int32), y_em=Y_em, y_rm=Y_rm)
