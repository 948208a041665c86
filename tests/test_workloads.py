"""Seeded inputs and the work/byte model (no GPU)."""
import json
import os

import numpy as np
import pytest
import torch

from io_aware_tiled_08_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _model_fn(name):
    return {
        "naive_score_bytes": W.naive_score_bytes,
        "naive_score_round_trip_bytes": W.naive_score_round_trip_bytes,
        "score_count": lambda N: W.naive_score_bytes(N, 1),
        "half_metric_flops": lambda N, d: W.metric_flops(1, 1, N, d, False) / 2,
        "roofline_ridge": W.roofline_ridge,
    }[name]


def test_model_against_page_arithmetic():
    with open(os.path.join(GOLDEN, "page_arithmetic.json")) as f:
        entries = json.load(f)["entries"]
    for e in entries:
        got = _model_fn(e["function"])(**e["args"])
        tol = e["tolerance_rel"] * e["expected"]
        assert abs(got - e["expected"]) <= tol, (e["source"], got)


def test_metric_flops_and_bytes():
    w = W.WORKLOADS[W.HEADLINE]
    assert w.flops() == 4 * 2 * 16 * 4096 * 4096 * 128
    assert abs(w.flops() - 2.749e11) / 2.749e11 < 1e-3
    c = W.WORKLOADS["batch_f16_d64_causal"]
    assert c.flops() == W.WORKLOADS["batch_f16_d64"].flops() / 2
    assert w.compulsory_bytes() == 4 * 2 * 16 * 4096 * 128 * 2 + 4 * 2 * 16 * 4096


def test_workload_table_matches_configs():
    t = W.WORKLOADS
    assert (t["single_head_f32"].B, t["single_head_f32"].N, t["single_head_f32"].d,
            t["single_head_f32"].dtype) == (1, 512, 64, "f32")
    assert (t["headline_f16_d128"].B, t["headline_f16_d128"].H,
            t["headline_f16_d128"].N, t["headline_f16_d128"].d) == (2, 16, 4096, 128)
    assert t["rescale_stress_bf16"].causal and t["long_context_bf16"].causal
    assert t["long_context_bf16"].sampled_rows == 256
    assert t["batch_f16_d64"].seed == t["batch_f16_d64_causal"].seed


def test_generation_is_deterministic_and_rounded():
    a = W.random_qkv(2, 3, 17, 8, "f16", seed=9)
    b = W.random_qkv(2, 3, 17, 8, "f16", seed=9)
    for x, y in zip(a, b):
        assert x.dtype == torch.float16 and torch.equal(x, y)
    c = W.random_qkv(2, 3, 17, 8, "f16", seed=10)
    assert not torch.equal(a[0], c[0])
    q32, _, _ = W.random_qkv(2, 3, 17, 8, "f32", seed=9)
    assert torch.equal(q32.to(torch.float16), a[0])  # RNE rounding of the draws
    qb, _, _ = W.random_qkv(2, 3, 17, 8, "bf16", seed=9)
    assert torch.equal(q32.to(torch.bfloat16), qb)


def test_rescale_stress_recipe():
    q, k, v = W.random_qkv(1, 2, 4096, 64, "f32", seed=4, kind="rescale_stress")
    norms = k[0, 0].double().norm(dim=-1).numpy()
    assert 2.9 < norms[-512:].mean() / norms[:512].mean() < 3.5
    assert float(v.abs().max()) <= 1.0 and float(v.min()) < -0.9
    assert abs(float(q.double().std()) - 1.0) < 0.05


def test_sample_rows():
    r = W.sample_rows(5, 1, 3, 1000, 256)
    assert r.shape == (1, 3, 256)
    for h in range(3):
        assert len(np.unique(r[0, h])) == 256 and np.all(np.diff(r[0, h]) > 0)
    assert np.array_equal(r, W.sample_rows(5, 1, 3, 1000, 256))
    assert W.sample_rows(5, 1, 1, 10, 256).shape == (1, 1, 10)


def test_default_scale_is_float32():
    s = W.default_scale(128)
    assert s == float(np.float32(s))
    assert abs(s - 128 ** -0.5) < 1e-8
