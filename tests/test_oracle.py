"""The CPU oracle against its pins (no GPU)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import moe_oracle as O
from tests import oracle_pins as P

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_skewed_workload_shape_of_load():
    """The Zipf(1.2) logit bias leaves some experts empty and makes the
    largest group more than 10x the mean (skewed 30B-A3B layer)."""
    wl = workloads.make("qwen3_30b_a3b_skewed")
    x = wl.hidden_states.float().numpy()
    wr = wl.router_weight.float().numpy()
    L = O.router_logits(x, wr, wl.router_bias.numpy())
    ids = O.select_topk(L, wl.top_k)
    c = O.expert_counts(ids, wl.E)
    assert c.sum() == wl.T * wl.top_k
    assert (c == 0).sum() >= 1
    assert c.max() > 10 * c.mean()


def test_workloads_are_deterministic():
    a = workloads.make("tiny_fp32")
    b = workloads.make("tiny_fp32")
    for f in ("hidden_states", "router_weight", "gate_up", "down"):
        assert torch.equal(getattr(a, f), getattr(b, f))
    assert a.hidden_states.dtype == torch.float32
    c = workloads.make("qwen3_30b_a3b_decode")
    assert c.gate_up.shape == (128, 2048, 1536) and c.gate_up.dtype == torch.bfloat16
    assert c.down.shape == (128, 768, 2048)


def test_integer_grid_logits_are_exact():
    wl = workloads.integer_grid_layer(T=32, H=2048, I=64, E=128, top_k=8)
    x = wl.hidden_states.double().numpy()
    wr = wl.router_weight.double().numpy()
    L64 = x @ wr.T
    assert np.array_equal(L64.astype(np.float32).astype(np.float64), L64)
    # frequent exact ties exercise the lower-id rule
    L32 = O.router_logits(x, wr)
    assert any(len(set(row.tolist())) < len(row) for row in L32)
