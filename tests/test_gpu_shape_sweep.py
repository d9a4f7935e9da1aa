"""Seeded sweep of layer shapes against the oracle (MI355X only).

The shapes are drawn once, from a fixed seed, over the ranges the library
accepts: T from 1 to 700 tokens, H any multiple of 128 up to 1024, I any
multiple of 64 (forward) or 128 (backward) up to 512, E from 1 to 64 experts,
top_k up to min(E, 8), renormalised or not, with and without a router bias,
bf16 and (forward) fp32.  They reach tile configurations, ragged tails and
empty experts that the named cases do not; the bars are the same as theirs.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from tests.test_gpu_backward import run_backward
from tests.test_gpu_parity import run_layer

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mixture_experts_layer_17_amd as m
    return m


def _draw(n, seed, i_step, fp32_every):
    rs = np.random.RandomState(seed)
    shapes = []
    for j in range(n):
        E = int(rs.randint(1, 65))
        shapes.append(dict(
            T=int(rs.choice([1, 2, 5, 17, 64, 100, 255, 301, 512, 700])),
            H=128 * int(rs.randint(1, 9)),
            I=i_step * int(rs.randint(1, 512 // i_step + 1)),
            E=E,
            top_k=int(rs.randint(1, min(E, 8) + 1)),
            norm=bool(rs.randint(0, 2)),
            bias=bool(rs.randint(0, 2)),
            fp32=fp32_every > 0 and j % fp32_every == fp32_every - 1,
            seed=100 + j))
    return shapes


FORWARD = _draw(16, 7, 64, 4)
BACKWARD = _draw(8, 8, 128, 0)


def _workload(s, tag):
    dtype = torch.float32 if s["fp32"] else torch.bfloat16
    bias = None
    if s["bias"]:
        g = torch.Generator().manual_seed(s["seed"] + 7)
        bias = torch.randn(s["E"], generator=g) * 0.05
    return workloads.make_layer(f"{tag}_{s['seed']}", T=s["T"], H=s["H"], I=s["I"], E=s["E"],
                                top_k=s["top_k"], norm_topk_prob=s["norm"], dtype=dtype,
                                seed=s["seed"], router_bias=bias)


@pytest.mark.parametrize("s", FORWARD, ids=lambda s: "T{T}_H{H}_I{I}_E{E}_k{top_k}".format(**s))
def test_layer_forward_shape_sweep(moe, s):
    run_layer(moe, _workload(s, "sweep"))


@pytest.mark.parametrize("s", BACKWARD, ids=lambda s: "T{T}_H{H}_I{I}_E{E}_k{top_k}".format(**s))
def test_layer_backward_shape_sweep(moe, s):
    run_backward(moe, _workload(s, "sweep_bwd"), seed=s["seed"])
