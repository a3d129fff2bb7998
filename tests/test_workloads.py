"""Workload recipe and the sizing arithmetic the pages print (CPU only)."""
import json
import os

import torch

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def test_score_matrix_size_matches_page_example():
    """32 MB per head at N = 4096 in 2-byte elements; 32 heads x 40 layers
    is about 41 GB (the page mixes MiB and decimal GB)."""
    g = json.load(open(GOLDEN))["score_matrix_example"]
    per_head = workloads.score_matrix_bytes(g["N"], 1, g["elem_bytes"])
    assert per_head == g["bytes_per_head_MiB"] * 2**20
    total = workloads.score_matrix_bytes(g["N"], g["heads"] * g["layers"], g["elem_bytes"])
    assert abs(total / 2**20 / 1000 - g["total_GB_approx"]) / g["total_GB_approx"] < 0.01


def test_sram_figure_matches_page():
    g = json.load(open(GOLDEN))["a100_sram_example"]
    assert abs(g["sms"] * g["kb_per_sm"] / 1000 - g["total_MB_approx"]) < 1.0


def test_long_context_footprint_is_linear():
    """At N = 65536 the fused forward writes O + LSE = 520 MiB, while one bf16
    score matrix per head would take 256 GiB."""
    w = workloads.WORKLOADS["long_causal_64k"]
    assert workloads.fwd_output_bytes(w) == 545_259_520
    assert workloads.score_matrix_bytes(w.N, w.H) == 256 * 2**30


def test_draw_is_seeded_and_ordered():
    w = workloads.WORKLOADS["single_head_f32"]
    q, k, v, do = workloads.draw(w)
    q2, k2, v2, do2 = workloads.draw(w)
    for a, b in ((q, q2), (k, k2), (v, v2), (do, do2)):
        assert torch.equal(a, b)
    g = torch.Generator().manual_seed(w.seed)
    assert torch.equal(q, torch.randn(q.shape, generator=g))
    w2 = workloads.WORKLOADS["small_fwd_bf16"]
    q, k, v, do = workloads.draw(w2)
    assert do is None and q.dtype == torch.bfloat16


def test_flop_convention():
    w = workloads.WORKLOADS["train_dropout"]
    assert w.flops_fwd() == 549_755_813_888
    assert w.flops_bwd() == 1_374_389_534_720
