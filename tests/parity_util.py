"""Comparison rules between the HIP path and the CPU oracle.

Tolerances (float): max|gpu - ref| <= rel * max|ref| + abs with
rel = 1e-2, abs = 1e-3 for bf16 workloads and rel = 1e-5, abs = 0 for the
float32 workload.

Routing: the top-k is a decision taken in float32 on float32 logits.  The
GPU and the oracle sum the router dot products in different orders, so their
logits differ by a few ulps (delta_t = max_e |gpu - ref| on token t).  A
token is *decided* when every gap between consecutive entries of the
oracle's ordering up to position k exceeds 2 * delta_t (or delta_t is 0):
then no perturbation of that size can change the selection or its order,
and the GPU's ids must equal the oracle's bit for bit.  For the remaining
(near-tie) tokens the GPU's ids must still be the exact top-k of its own
logits under the lower-id tie rule, and its selected experts must be within
2 * delta_t of the oracle's k-th logit.
"""
from __future__ import annotations

import numpy as np
import torch

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


def topk_by_rule(L: np.ndarray, k: int) -> np.ndarray:
    """Top-k ids of float32 rows under (-logit, id) ordering (numpy's lexsort)."""
    L = np.asarray(L, dtype=np.float32)
    eid = np.broadcast_to(np.arange(L.shape[1]), L.shape)
    return np.lexsort((eid, -L.astype(np.float64)), axis=-1)[:, :k]


def routing_check(gpu_logits, gpu_ids, ref_logits32, ref_ids, k: int):
    """Returns (decided mask, ids_equal mask).  Asserts the rules above."""
    gL = np.asarray(gpu_logits, dtype=np.float32)
    rL = np.asarray(ref_logits32, dtype=np.float32)
    gI = np.asarray(gpu_ids, dtype=np.int64)
    rI = np.asarray(ref_ids, dtype=np.int64)
    T, E = rL.shape
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
    # GPU ids are the exact top-k of the GPU's own logits (tie rule included)
    selfk = topk_by_rule(gL, k)
    badself = np.flatnonzero(np.any(selfk != gI, axis=1))
    assert badself.size == 0, f"gpu ids are not the top-k of gpu logits at token {badself[:5]}"
    # near-tie tokens: the GPU's choice is valid under the oracle's logits
    for t in np.flatnonzero(~same):
        kth = sorted_vals[t, k - 1]
        assert np.all(rL[t, gI[t]] >= kth - 2 * delta[t]), f"token {t}: invalid selection"
    return decided, same


def weights_check(gpu_w, ref_w, gpu_logits, ref_logits32, rows):
    """|gpu_w - ref_w| <= (3 delta_t + 2e-5) * ref_w on the given tokens: a
    logit error delta moves exp(L_j - max) / sum by at most a factor
    exp(3 delta); float32 exp, sum and division add ~1e-5 relative."""
    gw, rw = np64(gpu_w)[rows], np64(ref_w)[rows]
    delta = np.abs(np64(gpu_logits) - np64(ref_logits32)).max(axis=1)[rows]
    bound = (3 * delta[:, None] + 2e-5) * rw + 1e-12
    assert np.all(np.abs(gw - rw) <= bound), \
        f"routing weights: worst excess {np.max(np.abs(gw - rw) - bound):.3e}"
