"""Plant plausible mistakes in the oracle (on the CPU) and check that some
pin fails for each: the pins are sensitive enough to be trusted."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests import oracle_pins as P

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _some_pin_fails():
    for pin in P.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


def _swapped_gate_up(x_rows, gate_up_e, down_e):
    gu = np.asarray(gate_up_e, np.float64)
    I = gu.shape[1] // 2
    G = np.asarray(x_rows, np.float64) @ gu
    return (O.silu(G[:, I:]) * G[:, :I]) @ np.asarray(down_e, np.float64)


def _sigmoid_not_silu(z):
    return 1.0 / (1.0 + np.exp(-np.asarray(z, np.float64)))


def _higher_id_ties(logits32, k):
    L = np.asarray(logits32, np.float32)
    eid = np.broadcast_to(np.arange(L.shape[1]), L.shape)
    return np.lexsort((-eid, -L.astype(np.float64)), axis=-1)[:, :k].astype(np.int32)


def _no_renorm(logits32, ids, norm):
    return _orig["routing_weights"](logits32, ids, False)


def _weights_twice(y, w):
    return _orig["combine"](y, np.asarray(w) ** 2)


def _unstable_perm(ids, E):
    ss, st, sp = _orig["permutation"](ids, E)
    k = ids.shape[1]
    flat = np.asarray(ids).reshape(-1)
    ss = ss.copy()
    for e in range(E):
        sel = np.flatnonzero(flat[ss] == e)
        ss[sel] = ss[sel][::-1]
    sp = np.empty_like(ss)
    sp[ss] = np.arange(len(ss))
    return ss, ss // k, sp


def _bf16_logits(x, w_router, bias=None):
    L = _orig["router_logits"](x, w_router, bias)
    u = L.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


def _drop_bias(x, w_router, bias=None):
    return _orig["router_logits"](x, w_router, None)


def _off_by_one_offsets(counts):
    o = _orig["expert_offsets"](counts)
    o[1:] += 1
    return o


def _biased_weights(logits32, top_k, norm_topk_prob=False, score_func="sigmoid", route_scale=1.0,
                    expert_bias=None, n_groups=0, n_limited=0):
    ids, w, s, key = _orig["route_variant"](logits32, top_k, norm_topk_prob, score_func,
                                            route_scale, expert_bias, n_groups, n_limited)
    if expert_bias is not None:
        w = w + np.asarray(expert_bias, np.float64)[ids]
    return ids, w, s, key


def _group_sum_mask(scores, n_groups, n_limited):
    S = np.asarray(scores, np.float64)
    T, E = S.shape
    epg = E // n_groups
    gs = S.reshape(T, n_groups, epg).sum(axis=2)
    keep = np.argsort(-gs, axis=1, kind="stable")[:, :n_limited]
    mask = np.zeros((T, n_groups), dtype=bool)
    np.put_along_axis(mask, keep, True, axis=1)
    return np.repeat(mask, epg, axis=1)


def _uncentred_bias_update(expert_bias, tokens_per_expert, lr=1e-3, num_recomputations=1):
    tpe = np.asarray(tokens_per_expert, np.float64)
    if num_recomputations > 1:
        tpe = tpe / num_recomputations
    return np.asarray(expert_bias, np.float64) + lr * np.sign(tpe.mean() - tpe), np.zeros_like(tpe)


def _ffn_gate_up_swapped(x, w1, w2, w3):
    return _orig["feed_forward"](x, w3, w2, w1)


def _shared_weighted(out, x, shared):
    # the shared output scaled as if it carried a routing weight
    if shared is None:
        return out, None
    s = 0.5 * _orig["feed_forward"](x, *shared)
    return out + s, s


def _silu_grad_no_product_rule(z):
    return 1.0 / (1.0 + np.exp(-np.asarray(z, np.float64)))


def _backward_without_router_dx(x, w_router, bias, gate_up, down, top_k, norm, dout, **kw):
    g = _orig["moe_layer_backward"](x, w_router, bias, gate_up, down, top_k, norm, dout, **kw)
    g["dx"] = g["dx"] - g["d_logits"] @ np.asarray(w_router, np.float64)
    return g


def _jacobian_without_renorm_coupling(logits32, ids, norm, score_func="softmax", route_scale=1.0):
    # renormalisation treated as a constant divisor (the coupling term dropped)
    J = _orig["routing_weight_jacobian"](logits32, ids, False, score_func, route_scale)
    if not norm:
        return J
    L = np.asarray(logits32, np.float64)
    s = (1.0 / (1.0 + np.exp(-L))) if score_func == "sigmoid" else \
        np.exp(L - L.max(1, keepdims=True)) / np.exp(L - L.max(1, keepdims=True)).sum(1, keepdims=True)
    Z = np.take_along_axis(s * route_scale, np.asarray(ids, np.int64), 1).sum(1)
    return J / Z[:, None, None]


def _ffn_backward_swapped_up_gate(x, w1, w2, w3, dout):
    g = _orig["feed_forward_backward"](x, w1, w2, w3, dout)
    g["d_w1"], g["d_w3"] = g["d_w3"], g["d_w1"]
    return g


def _backward_unweighted_down_grad(x, w_router, bias, gate_up, down, top_k, norm, dout, **kw):
    # the down-projection gradient taken from dout without the routing weight
    g = _orig["moe_layer_backward"](x, w_router, bias, gate_up, down, top_k, norm, dout, **kw)
    f = g["forward"]
    k = top_k
    wsum = np.zeros(np.asarray(down).shape[0])
    for e in range(len(wsum)):
        sl = f["sorted_slot"][f["offsets"][e]:f["offsets"][e + 1]]
        wsum[e] = f["weights"].reshape(-1)[sl].mean() if len(sl) else 1.0
    g["d_down"] = g["d_down"] / wsum[:, None, None]
    return g


_orig = {n: getattr(O, n) for n in ("routing_weights", "combine", "permutation",
                                     "router_logits", "expert_offsets", "route_variant",
                                     "feed_forward", "moe_layer_backward",
                                     "routing_weight_jacobian", "feed_forward_backward")}

MUTATIONS = {
    "swiglu_expert": _swapped_gate_up,
    "silu": _sigmoid_not_silu,
    "select_topk": _higher_id_ties,
    "routing_weights": _no_renorm,
    "combine": _weights_twice,
    "permutation": _unstable_perm,
    "router_logits": _bf16_logits,
    "expert_offsets": _off_by_one_offsets,
    "route_variant": _biased_weights,
    "limited_group_mask": _group_sum_mask,
    "update_expert_bias": _uncentred_bias_update,
    "feed_forward": _ffn_gate_up_swapped,
    "_add_shared": _shared_weighted,
    "silu_grad": _silu_grad_no_product_rule,
    "moe_layer_backward": _backward_without_router_dx,
    "routing_weight_jacobian": _jacobian_without_renorm_coupling,
    "feed_forward_backward": _ffn_backward_swapped_up_gate,
}


def test_unweighted_down_grad_is_caught(monkeypatch):
    monkeypatch.setattr(O, "moe_layer_backward", _backward_unweighted_down_grad)
    assert _some_pin_fails()


def test_unmutated_oracle_passes_all_pins():
    assert not _some_pin_fails()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    monkeypatch.setattr(O, name, MUTATIONS[name])
    assert _some_pin_fails(), f"no pin catches a mistake in {name}"


def test_drop_bias_is_caught(monkeypatch):
    monkeypatch.setattr(O, "router_logits", _drop_bias)
    assert _some_pin_fails()
