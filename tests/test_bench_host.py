"""Host logic of bench.py (CPU only): the one-GPU guard, the algorithmic
FLOP and byte counts the roofline is computed from, and the rule that a
committed traffic record is used only while its kernel sources are
unchanged."""
from __future__ import annotations

import json
import os
import shutil
import subprocess
import sys
import types

import numpy as np
import torch

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _wl(T, H, I, E, k, dtype=torch.bfloat16):
    return types.SimpleNamespace(T=T, H=H, I=I, E=E, top_k=k, dtype=dtype)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_prefill_counts():
    # T 4096, H 2048, I 768, E 128, top-8, bf16, every expert hit
    wl = _wl(4096, 2048, 768, 128, 8)
    f, b, moved, layer_b, hit = bench.algorithmic(wl, np.ones(128, dtype=np.int64))
    N, es = 4096 * 8, 2
    assert hit == 128
    # gate_up: the hit experts' [H, 2I] weights once and the hidden states once
    assert b["gate_up_swiglu"] == 128 * 2048 * 1536 * es + 4096 * 2048 * es == 822083584
    # down: the hit experts' [I, H] weights once; the combine writes the output
    assert b["down"] == 128 * 768 * 2048 * es
    assert b["combine"] == 4096 * 2048 * es
    # intermediates are counted only as bytes moved: h written by gate_up,
    # read by down together with the per-slot outputs it writes
    assert moved["gate_up_swiglu"] - b["gate_up_swiglu"] == N * 768 * es
    assert moved["down"] - b["down"] == N * 768 * es + N * 2048 * es
    assert f["gate_up_swiglu"] == 4.0 * N * 2048 * 768
    assert f["down"] == 2.0 * N * 768 * 2048
    assert f["route"] == 2.0 * 4096 * 2048 * 128
    # the layer: all weights once, router weight, x in and out once, logits
    # and the routing outputs
    assert layer_b == 1244397568
    assert abs(sum(f.values()) - 3.115e11) < 1e9


def test_decode_counts_follow_the_hit_experts():
    wl = _wl(64, 2048, 768, 128, 8)
    counts = np.zeros(128, dtype=np.int64)
    counts[:100] = 5
    _, b, _, layer_b, hit = bench.algorithmic(wl, counts)
    assert hit == 100
    assert b["gate_up_swiglu"] == 100 * 2048 * 1536 * 2 + 64 * 2048 * 2
    assert layer_b == 100 * 3 * 2048 * 768 * 2 + 128 * 2048 * 2 + 2 * 64 * 2048 * 2 \
        + 64 * 128 * 4 + 64 * 8 * 8


def test_float32_counts_use_four_byte_elements():
    wl = _wl(64, 128, 64, 8, 2, dtype=torch.float32)
    _, b, _, _, _ = bench.algorithmic(wl, np.ones(8, dtype=np.int64))
    assert b["down"] == 8 * 64 * 128 * 4


def test_traffic_record_needs_unchanged_sources(tmp_path, monkeypatch):
    rec = json.load(open(os.path.join(
        ROOT, "profiles", "traffic_gate_up_swiglu_qwen3_30b_a3b_prefill.json")))
    # a copy of the tree's profiles and sources under a temporary root
    (tmp_path / "profiles").mkdir()
    shutil.copy(os.path.join(ROOT, "profiles",
                             "traffic_gate_up_swiglu_qwen3_30b_a3b_prefill.json"),
                tmp_path / "profiles")
    for rel in rec["sources"]:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_traffic("gate_up_swiglu", "qwen3_30b_a3b_prefill") == rec["traffic_bytes"]
    # one changed byte in any of the measured kernel's sources voids it
    first = tmp_path / next(iter(rec["sources"]))
    first.write_bytes(first.read_bytes() + b"\n")
    assert bench.load_traffic("gate_up_swiglu", "qwen3_30b_a3b_prefill") is None
    assert bench.load_traffic("gate_up_swiglu", "no_such_workload") is None


def test_compact_keeps_the_headline_fields():
    r = {"value": 1.0, "unit": "u", "ms_per_step": 2.0, "eager_ms_per_step": 3.0, "dtype": "bf16",
         "layer_tflops": 4.0, "layer_mfma_frac": 0.1, "layer_hbm_gbps": 5.0,
         "layer_hbm_frac": 0.2, "roofline": {"frac": 0.3}, "step_ms": {},
         "config": {"workload": "w"}, "kernels": {"gate_up_swiglu": {"avg_us": 7.0, "gbps": 1.0}},
         "context": {}, "cpu_baseline": {}}
    c = bench.compact(r)
    assert c["roofline"] == {"frac": 0.3} and c["layer_hbm_frac"] == 0.2
    assert c["config"] == {"workload": "w"} and c["kernels_us"] == {"gate_up_swiglu": 7.0}
    assert "cpu_baseline" not in c and "context" not in c
