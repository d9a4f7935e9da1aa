"""The library's size limits against the oracle (MI355X only): the most
experts a router supports (E = 256, including top_k = E), long and short
contractions (H = 8192, I = 4096), on both router paths (T <= 512 and
T > 512), forward and backward.  Same bars as the named cases."""
from __future__ import annotations

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


@pytest.mark.parametrize("shape", [
    dict(T=300, H=256, I=128, E=256, top_k=8),      # most experts, small-batch router
    dict(T=1100, H=256, I=128, E=256, top_k=8),     # most experts, large-batch router
    dict(T=6, H=256, I=64, E=256, top_k=256),       # every expert chosen by every token
    dict(T=64, H=8192, I=128, E=8, top_k=2),        # long router and gate_up contraction
    dict(T=600, H=256, I=4096, E=4, top_k=2),       # long down contraction
    dict(T=48, H=128, I=64, E=256, top_k=3, dtype=torch.float32),
], ids=lambda s: "T{T}_H{H}_I{I}_E{E}_k{top_k}".format(**s))
def test_layer_forward_limits(moe, shape):
    wl = workloads.make_layer("limits", seed=31, **shape)
    run_layer(moe, wl)


@pytest.mark.parametrize("shape", [
    dict(T=300, H=256, I=128, E=256, top_k=8),
    dict(T=64, H=4096, I=128, E=8, top_k=2),
    dict(T=200, H=256, I=2048, E=4, top_k=2),
], ids=lambda s: "T{T}_H{H}_I{I}_E{E}_k{top_k}".format(**s))
def test_layer_backward_limits(moe, shape):
    wl = workloads.make_layer("limits_bwd", seed=32, **shape)
    run_backward(moe, wl, seed=32)
