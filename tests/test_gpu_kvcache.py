"""Key/value-cache path (flash_attn_fwd_kvcache) vs the fp64 oracle on
identical seeded inputs (needs a gfx950 GPU).

Same tolerances as the square path: max-abs error against fp64 of 2e-3 for
fp16 and 1e-2 for bf16 inputs, on O and on LSE.  Outputs are pre-filled with
NaN so that an element the kernels fail to write shows up.
"""
import numpy as np
import pytest
import torch

import oracle
from io_aware_tiled_08_amd import (FlashAttnError, flash_attn_fwd_kvcache, kvcache_splits,
                                   kvcache_workspace_size)
from io_aware_tiled_08_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f16": 2e-3, "bf16": 1e-2}
DEV = "cuda:0"


def run_cache(q, k, v, scale, causal, num_splits=0, workspace=None, stream=None):
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full(tuple(q.shape[:3]), float("nan"), dtype=torch.float32, device=DEV)
    flash_attn_fwd_kvcache(qd, kd, vd, o, lse, scale=scale, causal=causal,
                           num_splits=num_splits, workspace=workspace, stream=stream)
    torch.cuda.synchronize()
    return o, lse


def check(o, lse, q, k, v, scale, causal, dtype, label, tol=None):
    tol = TOL[dtype] if tol is None else tol
    O_ref, L_ref = oracle.attention_forward(q, k, v, scale, causal)
    O = o.double().cpu().numpy()
    L = lse.double().cpu().numpy()
    assert np.isfinite(O).all() and np.isfinite(L).all(), f"{label}: non-finite output"
    err_o = float(np.max(np.abs(O - O_ref))) if O.size else 0.0
    err_l = float(np.max(np.abs(L - L_ref))) if L.size else 0.0
    print(f"{label}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
    assert err_o <= tol, f"{label}: O error {err_o:.3e} > {tol}"
    assert err_l <= tol, f"{label}: LSE error {err_l:.3e} > {tol}"


# (Nq, Nk): single tokens against short and ragged caches, multi-token steps,
# the square case, several query blocks, a cache of 4097 keys.
SHAPES = [(1, 1), (1, 31), (1, 33), (1, 1000), (3, 100), (16, 16), (32, 32), (33, 257),
          (70, 500), (5, 4097)]


@pytest.mark.parametrize("splits", [0, 1, 7])
@pytest.mark.parametrize("nq,nk", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_cache_sweep(dtype, d, causal, nq, nk, splits):
    q, k, v = W.random_cache_inputs(1, 2, nq, nk, d, dtype, seed=3000 + nq * 7 + nk)
    scale = W.default_scale(d)
    o, lse = run_cache(q, k, v, scale, causal, num_splits=splits)
    check(o, lse, q, k, v, scale, causal, dtype,
          f"{dtype} d={d} causal={causal} Nq={nq} Nk={nk} splits={splits}")


def test_more_queries_than_keys_without_mask():
    q, k, v = W.random_cache_inputs(2, 3, 40, 10, 64, "f16", seed=3100)
    o, lse = run_cache(q, k, v, 0.125, False, num_splits=2)
    check(o, lse, q, k, v, 0.125, False, "f16", "Nq=40 Nk=10")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_batch_head_indexing_and_negative_scale(dtype):
    q, k, v = W.random_cache_inputs(3, 5, 7, 333, 128, dtype, seed=3200)
    for scale in (-0.2, 0.0, 0.3):
        o, lse = run_cache(q, k, v, scale, True, num_splits=3)
        check(o, lse, q, k, v, scale, True, dtype, f"{dtype} B=3 H=5 scale={scale}",
              tol=TOL[dtype] * max(1.0, abs(scale) * 128 ** 0.5))


def test_splits_agree_with_one_split():
    """Every split count reaches the same answer within the tolerance."""
    q, k, v = W.random_cache_inputs(1, 4, 4, 3000, 128, "f16", seed=3300)
    ref = run_cache(q, k, v, 0.09, True, num_splits=1)
    for s in (2, 5, 16, 94, 256):
        o, lse = run_cache(q, k, v, 0.09, True, num_splits=s)
        assert float((o.float() - ref[0].float()).abs().max()) <= 2e-3, s
        assert float((lse - ref[1]).abs().max()) <= 2e-3, s


def test_deterministic():
    q, k, v = W.random_cache_inputs(2, 2, 3, 2000, 64, "bf16", seed=3400)
    a = run_cache(q, k, v, 0.125, True, num_splits=4)
    b = run_cache(q, k, v, 0.125, True, num_splits=4)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_shared_workspace_two_calls_second_smaller():
    """One caller-owned workspace reused by two calls on one stream, the
    second on a smaller problem: both results are right."""
    need = kvcache_workspace_size(2, 4, 8, 5000, 128, 6)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    q1, k1, v1 = W.random_cache_inputs(2, 4, 8, 5000, 128, "f16", seed=3500)
    q2, k2, v2 = W.random_cache_inputs(1, 2, 3, 900, 128, "f16", seed=3501)
    o1, l1 = run_cache(q1, k1, v1, 0.088, True, num_splits=6, workspace=ws)
    o2, l2 = run_cache(q2, k2, v2, 0.088, True, num_splits=6, workspace=ws)
    check(o1, l1, q1, k1, v1, 0.088, True, "f16", "first call")
    check(o2, l2, q2, k2, v2, 0.088, True, "f16", "second call")


def test_small_workspace_is_rejected():
    q, k, v = (x.to(DEV) for x in W.random_cache_inputs(1, 1, 1, 4096, 64, "f16", seed=3600))
    need = kvcache_workspace_size(1, 1, 1, 4096, 64, 8)
    assert need > 0 and kvcache_splits(1, 1, 1, 4096, 64, 8) == 8
    ws = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(FlashAttnError, match="FA_ERR_WORKSPACE"):
        flash_attn_fwd_kvcache(q, k, v, num_splits=8, workspace=ws)


def test_fp32_is_rejected():
    x = torch.zeros(1, 1, 4, 64, dtype=torch.float32, device=DEV)
    with pytest.raises(FlashAttnError, match="FA_ERR_DTYPE"):
        flash_attn_fwd_kvcache(x, x, x)


def test_side_stream():
    q, k, v = W.random_cache_inputs(1, 2, 2, 700, 64, "f16", seed=3700)
    s = torch.cuda.Stream()
    o, lse = run_cache(q, k, v, 0.125, True, num_splits=3, stream=s)
    check(o, lse, q, k, v, 0.125, True, "f16", "side stream")


def test_square_case_matches_square_kernel():
    """With Nq = Nk the cache path computes flash_attn_fwd's result."""
    from io_aware_tiled_08_amd import flash_attn_fwd
    q, k, v = (x.to(DEV) for x in W.random_qkv(1, 2, 300, 128, "f16", seed=3800))
    o1, l1 = flash_attn_fwd(q, k, v, causal=True)
    o2, l2 = flash_attn_fwd_kvcache(q, k, v, causal=True, num_splits=3)
    torch.cuda.synchronize()
    assert float((o1.float() - o2.float()).abs().max()) <= 2e-3
    assert float((l1 - l2).abs().max()) <= 2e-3


@pytest.mark.parametrize("name", sorted(W.CACHE_WORKLOADS))
def test_cache_workload_full(name):
    w = W.CACHE_WORKLOADS[name]
    q, k, v = W.cache_workload_inputs(w)
    o, lse = run_cache(q, k, v, w.scale, w.causal)
    check(o, lse, q, k, v, w.scale, w.causal, w.dtype, name)


@pytest.mark.parametrize("causal", [False, True])
def test_cache_graph_capture_replays(causal):
    """With a caller workspace the cache path enqueues the split and merge
    kernels, allocates nothing and clears no memory, so it can be captured in
    a HIP graph: three replays, with eager cache calls on other tensors
    between them, each bitwise equal to the eager call."""
    B, H, Nq, Nk, d = 2, 4, 3, 5000, 128
    q, k, v = W.random_cache_inputs(B, H, Nq, Nk, d, "bf16", seed=8800)
    scale = W.default_scale(d)
    assert kvcache_splits(B, H, Nq, Nk, d, 0) > 1
    ws = torch.empty(kvcache_workspace_size(B, H, Nq, Nk, d, 0), dtype=torch.uint8, device=DEV)
    o_ref, lse_ref = run_cache(q, k, v, scale, causal)
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty(B, H, Nq, dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up call on the capture stream
        flash_attn_fwd_kvcache(qd, kd, vd, o, lse, scale=scale, causal=causal, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        flash_attn_fwd_kvcache(qd, kd, vd, o, lse, scale=scale, causal=causal, workspace=ws)
    for rep in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), f"replay {rep}"
        # unrelated eager work between replays (other queries, its own workspace)
        o2, _ = run_cache(q.flip(2), k, v, scale, causal)
        assert torch.isfinite(o2).all()
