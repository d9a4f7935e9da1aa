"""Comparison rules between the HIP path and the CPU oracle.

Tolerances (float): max|gpu - ref| <= rel * max|ref| + abs with
rel = 1e-2, abs = 1e-3 for bf16 workloads and rel = 1e-5, abs = 0 for the
float32 workload.

Routing: the top-k is a decision taken in float32 on float32 logits.  The
GPU and the oracle sum the router dot products in different orders, so their
logits differ by a few ulps (delta_t = max_e |gpu - ref| on token t).  The
protocol therefore runs the oracle's selection on the GPU's own float32
logits: the GPU's ids must equal it bit for bit on every token, the layer's
counts, offsets and permutation must equal the oracle's of those ids bit for
bit, and the oracle's layer run on those ids is compared with the GPU's
output on every token.  Against the oracle's own logits, a token is
*decided* when every gap between consecutive entries of the oracle's ordering
up to position k exceeds 2 * delta_t (or delta_t is 0): then no perturbation
of that size can change the selection or its order, and the GPU's ids must
equal the oracle's bit for bit; the remaining near-tie tokens must pick
experts within 2 * delta_t of the oracle's k-th logit.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import moe_oracle as O

BF16_REL, BF16_ABS = 1e-2, 1e-3
F32_REL, F32_ABS = 1e-5, 0.0


def tol(dtype):
    return (BF16_REL, BF16_ABS) if dtype == torch.bfloat16 else (F32_REL, F32_ABS)


def np64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def assert_close(gpu, ref, dtype, what: str, rows=None):
    g, r = np64(gpu), np64(ref)
    if rows is not None:
        scale = np.abs(r).max() if r.size else 0.0
        g, r = g[rows], r[rows]
    else:
        scale = np.abs(r).max() if r.size else 0.0
    rel, ab = tol(dtype)
    err = np.abs(g - r).max() if r.size else 0.0
    bound = rel * scale + ab
    assert err <= bound, f"{what}: max|gpu-ref| = {err:.3e} > {bound:.3e} (max|ref| = {scale:.3e})"
    return err, bound


def routing_check(gpu_logits, gpu_ids, ref_logits32, ref_ids, k: int):
    """The routing protocol for the default router.  Returns (decided mask,
    mask of tokens the oracle routes the same from its own logits).

    1. The GPU's ids must equal, bit for bit and on every token, the oracle's
       selection (``O.select_topk``) applied to the GPU's own float32 logits.
    2. Decided tokens (every gap at the oracle's selection boundary above
       2 * delta_t) must route as the oracle does from its own logits.
    3. The remaining near-tie tokens must pick experts whose oracle logits
       are within 2 * delta_t of the oracle's k-th logit."""
    gL = np.asarray(gpu_logits, dtype=np.float32)
    rL = np.asarray(ref_logits32, dtype=np.float32)
    gI = np.asarray(gpu_ids, dtype=np.int64)
    rI = np.asarray(ref_ids, dtype=np.int64)
    T, E = rL.shape
    own = O.select_topk(gL, k).astype(np.int64)
    badself = np.flatnonzero(np.any(own != gI, axis=1))
    assert badself.size == 0, (f"{badself.size} tokens: gpu ids are not the oracle's top-k of the "
                               f"gpu logits, e.g. token {badself[:5].tolist()}")
    delta = np.abs(gL.astype(np.float64) - rL.astype(np.float64)).max(axis=1)
    order = np.lexsort((np.broadcast_to(np.arange(E), rL.shape), -rL.astype(np.float64)), axis=-1)
    sorted_vals = np.take_along_axis(rL.astype(np.float64), order, axis=1)
    upto = min(k + 1, E)
    gaps = sorted_vals[:, :upto - 1] - sorted_vals[:, 1:upto]
    decided = (delta == 0) | np.all(gaps > 2 * delta[:, None], axis=1)
    same = np.all(gI == rI, axis=1)
    bad = np.flatnonzero(decided & ~same)
    assert bad.size == 0, (f"{bad.size} decided tokens route differently, e.g. token {bad[0]}: "
                           f"gpu {gI[bad[0]].tolist()} ref {rI[bad[0]].tolist()}")
    for t in np.flatnonzero(~same):
        kth = sorted_vals[t, k - 1]
        assert np.all(rL[t, gI[t]] >= kth - 2 * delta[t]), f"token {t}: invalid selection"
    return decided, same


def variant_key_tol(keys32):
    """Per-token bound on how far the device's float32 selection keys
    (float32 sigmoid / softmax times the scale, plus the bias) can sit from
    the oracle's (float64 scores rounded once): 1e-5 of the row's largest
    key plus 1e-6, i.e. tens of float32 ulps."""
    key = np.asarray(keys32, dtype=np.float64)
    return 1e-5 * np.nanmax(np.abs(np.where(np.isfinite(key), key, 0)), axis=1) + 1e-6


def variant_routing_check(gpu_ids, keys32, scores, k: int, n_groups: int = 0, n_limited: int = 0,
                          ref_ids=None):
    """The routing protocol for a router variant, with the oracle's keys and
    scores computed from the GPU's own float32 logits (``O.route_variant``).
    The device computes the scores with its own float32 exp, so keys agree
    to ``variant_key_tol`` only:

    * decided tokens -- the k-th / (k+1)-th key gap and, with groups, the
      gap between the last kept and the first dropped group score exceed
      2 * tol -- must select exactly the oracle's ids, in order;
    * every other token must select k distinct experts in at most
      ``n_limited`` groups, each from a group whose score is within 2 * tol
      of the last kept one, with keys within 2 * tol of the oracle's k-th
      key among the experts the device's groups allow.

    Returns (decided, same)."""
    gI = np.asarray(gpu_ids, dtype=np.int64)
    key = np.asarray(keys32, dtype=np.float64)
    sc = np.asarray(scores, dtype=np.float64)
    T, E = key.shape
    rI = np.asarray(ref_ids, dtype=np.int64)
    tol = variant_key_tol(keys32)
    # keys of experts outside the kept groups are -inf, so the gap is the
    # one among the selectable experts
    srt = -np.sort(-key, axis=1)
    nxt = srt[:, k] if k < E else np.full(T, -np.inf)
    decided = (srt[:, k - 1] - nxt) > 2 * tol
    if n_groups:
        gs = -np.sort(-sc.reshape(T, n_groups, E // n_groups).max(axis=2), axis=1)
        if n_limited < n_groups:
            decided &= (gs[:, n_limited - 1] - gs[:, n_limited]) > 2 * tol
    same = np.all(gI == rI, axis=1)
    bad = np.flatnonzero(decided & ~same)
    assert bad.size == 0, (f"{bad.size} decided tokens differ, e.g. token {bad[0]}: "
                           f"{gI[bad[0]].tolist()} vs {rI[bad[0]].tolist()}")
    assert ((gI >= 0) & (gI < E)).all(), "expert id out of range"
    assert all(len(set(r)) == k for r in gI.tolist()), "repeated expert in a token's selection"
    if n_groups:
        epg = E // n_groups
        gmax = sc.reshape(T, n_groups, epg).max(axis=2)
        last_kept = -np.sort(-gmax, axis=1)[:, n_limited - 1]
        for t in np.flatnonzero(~same):
            groups = np.unique(gI[t] // epg)
            assert groups.size <= n_limited, f"token {t}: more than {n_limited} groups"
            assert np.all(gmax[t, groups] >= last_kept[t] - 2 * tol[t]), f"token {t}: group"
    for t in np.flatnonzero(~same):
        fin = key[t][np.isfinite(key[t])]
        kth = np.sort(fin)[::-1][k - 1] if fin.size >= k else -np.inf
        # experts outside the oracle's kept groups (key -inf) passed the
        # group check above
        sel = key[t, gI[t]]
        ok = ~np.isfinite(sel) | (sel >= kth - 2 * tol[t])
        assert ok.all(), f"token {t}: invalid selection {gI[t].tolist()}"
    return decided, same


def permutation_check(counts, internals, gpu_ids, E: int):
    """The layer's own histogram, offsets and permutation, bit for bit
    against the oracle's (``O.expert_counts``, ``O.expert_offsets``,
    ``O.permutation``) of the GPU's ids."""
    ids = np.asarray(gpu_ids)
    c = O.expert_counts(ids, E)
    assert np.array_equal(np.asarray(counts), c), "counts"
    o = O.expert_offsets(c)
    assert np.array_equal(np.asarray(internals["offsets"]), o), "expert offsets"
    ss, st, sp = O.permutation(ids, E)
    assert np.array_equal(np.asarray(internals["sorted_slot"]), ss), "sorted_slot"
    assert np.array_equal(np.asarray(internals["sorted_token"]), st), "sorted_token"
    assert np.array_equal(np.asarray(internals["slot_pos"]), sp), "slot_pos"


def weights_check(gpu_w, ref_w, gpu_logits, ref_logits32, rows):
    """|gpu_w - ref_w| <= (3 delta_t + 2e-5) * ref_w on the given tokens: a
    logit error delta moves exp(L_j - max) / sum by at most a factor
    exp(3 delta); float32 exp, sum and division add ~1e-5 relative."""
    gw, rw = np64(gpu_w)[rows], np64(ref_w)[rows]
    delta = np.abs(np64(gpu_logits) - np64(ref_logits32)).max(axis=1)[rows]
    bound = (3 * delta[:, None] + 2e-5) * rw + 1e-12
    assert np.all(np.abs(gw - rw) <= bound), \
        f"routing weights: worst excess {np.max(np.abs(gw - rw) - bound):.3e}"
