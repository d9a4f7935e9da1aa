"""libmoe: MI355X-native MoE layer forward (router -> permutation -> grouped
SwiGLU experts -> combine) as hand-written HIP kernels behind a C ABI.

This module is the thin Python binding: it checks tensors, allocates outputs
and workspace with torch, and passes device pointers and torch's current
stream to libmoe.so.  Every step of the computation runs in the library's
kernels; importing fails if the library is missing.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib

lib = _lib.load()

__all__ = ["lib", "route", "permute", "permute_rank_major", "gather_rows",
           "grouped_gate_up_swiglu", "grouped_down", "grouped_swiglu", "combine",
           "layer_forward", "workspace_size", "router_config", "update_expert_bias",
           "shared_expert", "shared_expert_forward", "layer_forward_train", "layer_backward",
           "LayerBuffers", "MoEError"]

MoEError = _lib.MoEError


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.MOE_BF16
    if t.dtype == torch.float32:
        return _lib.MOE_F32
    raise TypeError(f"unsupported dtype {t.dtype}; bf16 or float32")


def _chk(t: Optional[torch.Tensor], name: str, dtype=None, shape=None):
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _call(name: str, *args):
    st = getattr(lib, name)(*args)
    if st != 0:
        raise MoEError(name, st)


def workspace_size(op: int, T=0, H=0, I=0, E=0, top_k=0, R=0, N=0, dtype=torch.bfloat16) -> int:
    dt = _lib.MOE_BF16 if dtype == torch.bfloat16 else _lib.MOE_F32
    n = lib.moe_workspace_size(op, T, H, I, E, top_k, R, N, dt)
    if n == ctypes_size_max():
        raise ValueError("invalid sizes for workspace query")
    return n


def ctypes_size_max() -> int:
    import ctypes
    return ctypes.c_size_t(-1).value


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> Tuple[int, int, torch.Tensor]:
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError("workspace too small")
        return ws.data_ptr(), ws.numel() * ws.element_size(), ws
    t = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    return t.data_ptr(), nbytes, t


def router_config(score_func: str = "sigmoid", route_scale: float = 1.0,
                  expert_bias: Optional[torch.Tensor] = None, num_expert_groups: int = 0,
                  num_limited_groups: int = 0,
                  tokens_per_expert: Optional[torch.Tensor] = None) -> "_lib.RouterConfig":
    """A router variant (struct moe_router_config): score function, route
    scale, selection-only expert bias [E] float32, node-limited groups and an
    optional float32 [E] accumulator of selections."""
    funcs = {"softmax": _lib.MOE_SCORE_SOFTMAX, "sigmoid": _lib.MOE_SCORE_SIGMOID}
    if score_func not in funcs:
        raise ValueError(f"unknown score function {score_func!r}: use sigmoid or softmax")
    _chk(expert_bias, "expert_bias", torch.float32)
    _chk(tokens_per_expert, "tokens_per_expert", torch.float32)
    cfg = _lib.RouterConfig(funcs[score_func], float(route_scale),
                            expert_bias.data_ptr() if expert_bias is not None else None,
                            int(num_expert_groups), int(num_limited_groups),
                            tokens_per_expert.data_ptr() if tokens_per_expert is not None else None)
    cfg._keep = (expert_bias, tokens_per_expert)   # the tensors outlive the struct's use
    return cfg


def _cfg_ptr(cfg):
    import ctypes
    return ctypes.addressof(cfg) if cfg is not None else None


def update_expert_bias(expert_bias: torch.Tensor, tokens_per_expert: torch.Tensor,
                       lr: float = 1e-3, num_recomputations: int = 1) -> None:
    """In place: one auxiliary-loss-free bias step; clears the accumulator."""
    E = expert_bias.shape[0]
    _chk(expert_bias, "expert_bias", torch.float32, (E,))
    _chk(tokens_per_expert, "tokens_per_expert", torch.float32, (E,))
    _call("moe_update_expert_bias", expert_bias.data_ptr(), tokens_per_expert.data_ptr(), E,
          float(lr), int(num_recomputations), _stream(expert_bias.device))


def route(x: torch.Tensor, router_weight: torch.Tensor, top_k: int,
          norm_topk_prob: bool = True, router_bias: Optional[torch.Tensor] = None,
          with_logits: bool = True, with_counts: bool = True, config=None):
    """Router logits, top-k ids and routing weights (and tokens per expert).
    ``config`` (from ``router_config``) selects a router variant."""
    T, H = x.shape
    E = router_weight.shape[0]
    dev = x.device
    _chk(x, "x")
    _chk(router_weight, "router_weight", x.dtype, (E, H))
    _chk(router_bias, "router_bias", torch.float32, (E,))
    logits = torch.empty(T, E, dtype=torch.float32, device=dev) if with_logits else None
    ids = torch.empty(T, top_k, dtype=torch.int32, device=dev)
    w = torch.empty(T, top_k, dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev) if with_counts else None
    _call("moe_route_cfg", x.data_ptr(), router_weight.data_ptr(),
          _chk(router_bias, "router_bias"), T, H, E, top_k, int(norm_topk_prob), _dt(x),
          _cfg_ptr(config), _chk(logits, "logits"), ids.data_ptr(), w.data_ptr(),
          _chk(counts, "counts"), _stream(dev))
    return logits, ids, w, counts


def permute(topk_ids: torch.Tensor, num_experts: int, workspace=None) -> dict:
    """Histogram, offsets and the stable expert-major permutation of the
    (token, slot) pairs."""
    T, k = topk_ids.shape
    _chk(topk_ids, "topk_ids", torch.int32)
    dev = topk_ids.device
    N = T * k
    E = num_experts
    out = dict(counts=torch.empty(E, dtype=torch.int32, device=dev),
               offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
               sorted_token=torch.empty(N, dtype=torch.int32, device=dev),
               sorted_slot=torch.empty(N, dtype=torch.int32, device=dev),
               slot_pos=torch.empty(N, dtype=torch.int32, device=dev))
    nb = lib.moe_workspace_size(_lib.MOE_OP_PERMUTE, T, 0, 0, E, k, 0, N, _lib.MOE_BF16)
    wp, wb, _keep = _workspace(nb, dev, workspace)
    _call("moe_permute", topk_ids.data_ptr(), T, k, None, 0, N, E, out["counts"].data_ptr(),
          out["offsets"].data_ptr(), out["sorted_token"].data_ptr(),
          out["sorted_slot"].data_ptr(), out["slot_pos"].data_ptr(), wp, wb, _stream(dev))
    return out


def permute_rank_major(counts_rank_major: torch.Tensor, N: int, workspace=None) -> dict:
    """Expert-major order of rows received rank-major (blocks (rank, expert))."""
    R, E = counts_rank_major.shape
    _chk(counts_rank_major, "counts_rank_major", torch.int32)
    dev = counts_rank_major.device
    out = dict(counts=torch.empty(E, dtype=torch.int32, device=dev),
               offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
               sorted_token=torch.empty(N, dtype=torch.int32, device=dev),
               sorted_slot=torch.empty(N, dtype=torch.int32, device=dev),
               slot_pos=torch.empty(N, dtype=torch.int32, device=dev))
    nb = lib.moe_workspace_size(_lib.MOE_OP_PERMUTE, 0, 0, 0, E, 1, R, N, _lib.MOE_BF16)
    wp, wb, _keep = _workspace(nb, dev, workspace)
    _call("moe_permute", None, 0, 1, counts_rank_major.data_ptr(), R, N, E,
          out["counts"].data_ptr(), out["offsets"].data_ptr(), out["sorted_token"].data_ptr(),
          out["sorted_slot"].data_ptr(), out["slot_pos"].data_ptr(), wp, wb, _stream(dev))
    return out


def gather_rows(x: torch.Tensor, row_index: torch.Tensor) -> torch.Tensor:
    N = row_index.shape[0]
    _chk(x, "x")
    _chk(row_index, "row_index", torch.int32)
    out = torch.empty(N, x.shape[1], dtype=x.dtype, device=x.device)
    _call("moe_gather_rows", x.data_ptr(), x.shape[0], row_index.data_ptr(), N, x.shape[1],
          _dt(x), out.data_ptr(), _stream(x.device))
    return out


def grouped_gate_up_swiglu(x: torch.Tensor, offsets: torch.Tensor, gate_up: torch.Tensor,
                           N: int, row_index: Optional[torch.Tensor] = None,
                           out: Optional[torch.Tensor] = None, workspace=None) -> torch.Tensor:
    """h[p] = SwiGLU gate/up of x[row_index[p]] for expert-major rows p."""
    E, H, I2 = gate_up.shape
    I = I2 // 2
    _chk(x, "x")
    _chk(gate_up, "gate_up", x.dtype)
    _chk(offsets, "offsets", torch.int32, (E + 1,))
    _chk(row_index, "row_index", torch.int32)
    dev = x.device
    h = out if out is not None else torch.empty(N, I, dtype=x.dtype, device=dev)
    _chk(h, "h", x.dtype, (N, I))
    nb = lib.moe_workspace_size(_lib.MOE_OP_GATE_UP, 0, H, I, E, 1, 0, N, _dt(x))
    wp, wb, _keep = _workspace(nb, dev, workspace)
    _call("moe_grouped_gate_up_swiglu", x.data_ptr(), x.shape[0], _chk(row_index, "row_index"),
          offsets.data_ptr(), N, H, I, E, gate_up.data_ptr(), _dt(x), h.data_ptr(), wp, wb,
          _stream(dev))
    return h


def grouped_down(h: torch.Tensor, offsets: torch.Tensor, down: torch.Tensor,
                 out_index: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 workspace=None) -> torch.Tensor:
    """y[out_index[p]] = h[p] @ down[expert of p]."""
    E, I, H = down.shape
    N = h.shape[0]
    _chk(h, "h")
    _chk(down, "down", h.dtype)
    _chk(offsets, "offsets", torch.int32, (E + 1,))
    _chk(out_index, "out_index", torch.int32)
    dev = h.device
    y = out if out is not None else torch.empty(N, H, dtype=h.dtype, device=dev)
    _chk(y, "y", h.dtype, (N, H))
    nb = lib.moe_workspace_size(_lib.MOE_OP_DOWN, 0, H, I, E, 1, 0, N, _dt(h))
    wp, wb, _keep = _workspace(nb, dev, workspace)
    _call("moe_grouped_down", h.data_ptr(), offsets.data_ptr(), _chk(out_index, "out_index"), N,
          H, I, E, down.data_ptr(), _dt(h), y.data_ptr(), wp, wb, _stream(dev))
    return y


def grouped_swiglu(x: torch.Tensor, offsets: torch.Tensor, gate_up: torch.Tensor,
                   down: torch.Tensor, N: int, row_index: Optional[torch.Tensor] = None,
                   out_index: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                   workspace=None) -> torch.Tensor:
    """Both grouped GEMMs: y[out_index[p]] = SwiGLU_e(x[row_index[p]])."""
    E, H, I2 = gate_up.shape
    I = I2 // 2
    _chk(x, "x")
    _chk(gate_up, "gate_up", x.dtype)
    _chk(down, "down", x.dtype, (E, I, H))
    _chk(offsets, "offsets", torch.int32, (E + 1,))
    dev = x.device
    y = out if out is not None else torch.empty(N, H, dtype=x.dtype, device=dev)
    _chk(y, "y", x.dtype, (N, H))
    nb = lib.moe_workspace_size(_lib.MOE_OP_GROUPED_SWIGLU, 0, H, I, E, 1, 0, N, _dt(x))
    wp, wb, _keep = _workspace(nb, dev, workspace)
    _call("moe_grouped_swiglu", x.data_ptr(), x.shape[0], _chk(row_index, "row_index"),
          _chk(out_index, "out_index"), offsets.data_ptr(), N, H, I, E, gate_up.data_ptr(),
          down.data_ptr(), _dt(x), y.data_ptr(), wp, wb, _stream(dev))
    return y


def combine(y: torch.Tensor, T: int, top_k: int, topk_weights: Optional[torch.Tensor] = None,
            slot_pos: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[t] = sum_j w[t, j] * y[src(t, j)] in float32, j ascending."""
    H = y.shape[1]
    _chk(y, "y")
    _chk(topk_weights, "topk_weights", torch.float32, (T, top_k))
    _chk(slot_pos, "slot_pos", torch.int32)
    o = out if out is not None else torch.empty(T, H, dtype=y.dtype, device=y.device)
    _chk(o, "out", y.dtype, (T, H))
    _call("moe_combine", y.data_ptr(), _chk(slot_pos, "slot_pos"),
          _chk(topk_weights, "topk_weights"), T, top_k, H, _dt(y), o.data_ptr(),
          _stream(y.device))
    return o


class LayerBuffers:
    """Preallocated outputs and workspace for repeated layer_forward calls
    (``shared_I``: the shared expert's intermediate size, 0 for none)."""

    def __init__(self, T, H, I, E, top_k, dtype, device, shared_I=0):
        self.out = torch.empty(T, H, dtype=dtype, device=device)
        self.logits = torch.empty(T, E, dtype=torch.float32, device=device)
        self.ids = torch.empty(T, top_k, dtype=torch.int32, device=device)
        self.weights = torch.empty(T, top_k, dtype=torch.float32, device=device)
        self.counts = torch.empty(E, dtype=torch.int32, device=device)
        dt = _lib.MOE_BF16 if dtype == torch.bfloat16 else _lib.MOE_F32
        nb = lib.moe_workspace_size(_lib.MOE_OP_LAYER, T, H, I, E, top_k, shared_I, T * top_k,
                                    dt)
        self.workspace = torch.empty(max(nb, 1), dtype=torch.uint8, device=device)
        self.ws_bytes = nb
        self._dims = (T, H, I, E, top_k, shared_I, dt, dtype)

    def internals(self) -> dict:
        """Views of what the last layer_forward on these buffers left in the
        workspace (moe_layer_workspace_offset): expert offsets, the
        permutation and the expert outputs in flat slot order."""
        T, H, I, E, k, Is, dt, dtype = self._dims
        N = T * k

        def view(piece, n, elt):
            off = lib.moe_layer_workspace_offset(piece, T, H, I, E, k, Is, dt)
            if off == ctypes_size_max():
                raise ValueError("invalid sizes for workspace views")
            nbytes = n * torch.empty(0, dtype=elt).element_size()
            return self.workspace[off:off + nbytes].view(elt)

        return dict(offsets=view(_lib.MOE_LAYER_WS_OFFSETS, E + 1, torch.int32),
                    sorted_token=view(_lib.MOE_LAYER_WS_SORTED_TOKEN, N, torch.int32),
                    sorted_slot=view(_lib.MOE_LAYER_WS_SORTED_SLOT, N, torch.int32),
                    slot_pos=view(_lib.MOE_LAYER_WS_SLOT_POS, N, torch.int32),
                    expert_out=view(_lib.MOE_LAYER_WS_EXPERT_OUT, N * H, dtype).view(N, H))


def shared_expert(gate_up: torch.Tensor, down: torch.Tensor) -> "_lib.SharedExpert":
    """struct moe_shared_expert for FeedForward weights in the library's layout:
    ``gate_up`` [H, 2 Is] (w1^T | w3^T) and ``down`` [Is, H] (w2^T)."""
    H, Is2 = gate_up.shape
    _chk(gate_up, "shared gate_up", gate_up.dtype, (H, Is2))
    _chk(down, "shared down", gate_up.dtype, (Is2 // 2, H))
    sh = _lib.SharedExpert(gate_up.data_ptr(), down.data_ptr(), Is2 // 2)
    sh._keep = (gate_up, down)
    return sh


def shared_expert_forward(x: torch.Tensor, gate_up: torch.Tensor,
                          down: torch.Tensor) -> torch.Tensor:
    """The shared expert (FeedForward) on every row of ``x`` [T, H]."""
    T, H = x.shape
    Is = gate_up.shape[1] // 2
    _chk(x, "x")
    _chk(gate_up, "gate_up", x.dtype, (H, 2 * Is))
    _chk(down, "down", x.dtype, (Is, H))
    out = torch.empty(T, H, dtype=x.dtype, device=x.device)
    nb = lib.moe_workspace_size(_lib.MOE_OP_SHARED, T, H, Is, 1, 1, 0, T, _dt(x))
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=x.device)
    _call("moe_shared_expert_forward", x.data_ptr(), gate_up.data_ptr(), down.data_ptr(), T, H,
          Is, _dt(x), out.data_ptr(), ws.data_ptr(), nb, _stream(x.device))
    return out


def layer_forward(x: torch.Tensor, router_weight: torch.Tensor, gate_up: torch.Tensor,
                  down: torch.Tensor, top_k: int, norm_topk_prob: bool = True,
                  router_bias: Optional[torch.Tensor] = None,
                  buffers: Optional[LayerBuffers] = None, config=None, shared=None):
    """The whole MoE layer forward; returns (out, router_logits, topk_ids,
    topk_weights, num_tokens_per_expert).  ``config`` (from
    ``router_config``) selects a router variant; ``shared`` = (gate_up [H,
    2 Is], down [Is, H]) adds a shared expert."""
    T, H = x.shape
    E = router_weight.shape[0]
    I = gate_up.shape[2] // 2
    _chk(x, "x")
    _chk(router_weight, "router_weight", x.dtype, (E, H))
    _chk(gate_up, "gate_up", x.dtype, (E, H, 2 * I))
    _chk(down, "down", x.dtype, (E, I, H))
    _chk(router_bias, "router_bias", torch.float32, (E,))
    sh = None
    if shared is not None:
        _chk(shared[0], "shared gate_up", x.dtype)
        sh = shared_expert(*shared)
    Is = sh.intermediate_size if sh is not None else 0
    b = buffers if buffers is not None else LayerBuffers(T, H, I, E, top_k, x.dtype, x.device,
                                                         Is)
    _call("moe_layer_forward_ex", x.data_ptr(), router_weight.data_ptr(),
          _chk(router_bias, "router_bias"), gate_up.data_ptr(), down.data_ptr(), T, H, I, E,
          top_k, int(norm_topk_prob), _dt(x), _cfg_ptr(config), _cfg_ptr(sh), b.out.data_ptr(),
          b.logits.data_ptr(), b.ids.data_ptr(), b.weights.data_ptr(), b.counts.data_ptr(),
          b.workspace.data_ptr(), b.ws_bytes, None, _stream(x.device))
    return b.out, b.logits, b.ids, b.weights, b.counts


def layer_forward_train(x: torch.Tensor, router_weight: torch.Tensor, gate_up: torch.Tensor,
                        down: torch.Tensor, top_k: int, norm_topk_prob: bool = True,
                        router_bias: Optional[torch.Tensor] = None, config=None, shared=None):
    """The layer forward that also keeps what the backward needs.  Returns
    (out, saved) where ``saved`` holds router_logits, topk_ids, topk_weights,
    num_tokens_per_expert, gate_up_out [T*k, 2I] (expert-major
    pre-activations), expert_out [T*k, H] (flat slot order) and, with a
    shared expert ``shared = (gate_up [H, 2Is], down [Is, H])``,
    shared_gate_up_out [T, 2Is]."""
    T, H = x.shape
    E = router_weight.shape[0]
    I = gate_up.shape[2] // 2
    _chk(x, "x")
    _chk(router_weight, "router_weight", x.dtype, (E, H))
    _chk(gate_up, "gate_up", x.dtype, (E, H, 2 * I))
    _chk(down, "down", x.dtype, (E, I, H))
    _chk(router_bias, "router_bias", torch.float32, (E,))
    sh = shared_expert(*shared) if shared is not None else None
    Is = sh.intermediate_size if sh is not None else 0
    b = LayerBuffers(T, H, I, E, top_k, x.dtype, x.device, Is)
    N = T * top_k
    g = torch.empty(N, 2 * I, dtype=x.dtype, device=x.device)
    y = torch.empty(N, H, dtype=x.dtype, device=x.device)
    gs = torch.empty(T, 2 * Is, dtype=x.dtype, device=x.device) if Is else None
    sv = _lib.TrainSaved(g.data_ptr(), y.data_ptr(), gs.data_ptr() if gs is not None else None)
    _call("moe_layer_forward_train", x.data_ptr(), router_weight.data_ptr(),
          _chk(router_bias, "router_bias"), gate_up.data_ptr(), down.data_ptr(), T, H, I, E,
          top_k, int(norm_topk_prob), _dt(x), _cfg_ptr(config), _cfg_ptr(sh), b.out.data_ptr(),
          b.logits.data_ptr(), b.ids.data_ptr(), b.weights.data_ptr(), b.counts.data_ptr(),
          _cfg_ptr(sv), b.workspace.data_ptr(), b.ws_bytes, None, _stream(x.device))
    saved = dict(router_logits=b.logits, topk_ids=b.ids, topk_weights=b.weights,
                 num_tokens_per_expert=b.counts, gate_up_out=g, expert_out=y,
                 shared_gate_up_out=gs)
    return b.out, saved


def layer_backward(x: torch.Tensor, router_weight: torch.Tensor, gate_up: torch.Tensor,
                   down: torch.Tensor, top_k: int, norm_topk_prob: bool, saved: dict,
                   dout: torch.Tensor, with_bias_grad: bool = True, config=None,
                   shared=None) -> dict:
    """Gradients of sum(dout * out) given ``saved`` from layer_forward_train
    (same config and shared expert): dx, d_router_weight (float32),
    d_router_bias (float32), d_gate_up, d_down, d_topk_weights (float32) and,
    with a shared expert, d_shared_gate_up [H, 2Is] and d_shared_down
    [Is, H]."""
    T, H = x.shape
    E = router_weight.shape[0]
    I = gate_up.shape[2] // 2
    dev = x.device
    _chk(dout, "dout", x.dtype, (T, H))
    sh = shared_expert(*shared) if shared is not None else None
    Is = sh.intermediate_size if sh is not None else 0
    N = T * top_k
    g = dict(dx=torch.empty(T, H, dtype=x.dtype, device=dev),
             d_router_weight=torch.empty(E, H, dtype=torch.float32, device=dev),
             d_router_bias=torch.empty(E, dtype=torch.float32, device=dev) if with_bias_grad
             else None,
             d_gate_up=torch.empty(E, H, 2 * I, dtype=x.dtype, device=dev),
             d_down=torch.empty(E, I, H, dtype=x.dtype, device=dev),
             d_topk_weights=torch.empty(T, top_k, dtype=torch.float32, device=dev),
             d_shared_gate_up=torch.empty(H, 2 * Is, dtype=x.dtype, device=dev) if Is else None,
             d_shared_down=torch.empty(Is, H, dtype=x.dtype, device=dev) if Is else None)
    P = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
    gr = _lib.LayerGrads(P(g["dx"]), P(g["d_router_weight"]), P(g["d_router_bias"]),
                         P(g["d_gate_up"]), P(g["d_down"]), P(g["d_topk_weights"]),
                         P(g["d_shared_gate_up"]), P(g["d_shared_down"]))
    sv = _lib.TrainSaved(P(saved["gate_up_out"]), P(saved["expert_out"]),
                         P(saved.get("shared_gate_up_out")))
    nb = lib.moe_workspace_size(_lib.MOE_OP_LAYER_BACKWARD, T, H, I, E, top_k, Is, N, _dt(x))
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    _call("moe_layer_backward", x.data_ptr(), router_weight.data_ptr(), gate_up.data_ptr(),
          down.data_ptr(), T, H, I, E, top_k, int(norm_topk_prob), _dt(x), _cfg_ptr(config),
          _cfg_ptr(sh), saved["router_logits"].data_ptr(), saved["topk_ids"].data_ptr(),
          saved["topk_weights"].data_ptr(), _cfg_ptr(sv), dout.data_ptr(), _cfg_ptr(gr),
          ws.data_ptr(), nb, None, _stream(dev))
    return g
