"""Backward pass (flash_attn_bwd) vs the fp64 oracle (needs a gfx950 GPU).

The kernel receives the forward output O rounded to the input type and the
exact LSE in float32, as flash_attn_fwd would hand them over.  Accuracy
contract (oracle.backward_error_bound): the bound per element that follows
from rounding P, dS and O to the input type (unit u = 2^-11 for fp16, 2^-8
for bf16), dS being formed from the rounded P, plus the rounding of dq, dk,
dv themselves (u |ref|) and fp32 accumulation (1e-5 max|ref| + 1e-6).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from io_aware_tiled_08_amd import FlashAttnError, flash_attn_bwd, lib
from io_aware_tiled_08_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
UNIT = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def run_bwd(q, k, v, do, scale, causal, dtype, stream=None):
    O, L = oracle.attention_forward(q, k, v, scale, causal)
    tdt = W.DTYPES[dtype]
    o = torch.from_numpy(O).to(tdt).to(DEV)
    lse = torch.from_numpy(L).to(torch.float32).to(DEV)
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    dq, dk, dv = (torch.full_like(qd, float("nan")) for _ in range(3))
    flash_attn_bwd(qd, kd, vd, o, lse, dod, dq, dk, dv, scale=scale, causal=causal, stream=stream)
    torch.cuda.synchronize()
    return dq, dk, dv


def check(got, q, k, v, do, scale, causal, dtype, label):
    u = UNIT[dtype]
    refs = oracle.attention_backward(q, k, v, do, scale, causal)[:3]
    bounds = oracle.backward_error_bound(q, k, v, do, scale, causal, u=u)
    for name, g, ref, b in zip(("dQ", "dK", "dV"), got, refs, bounds):
        G = g.double().cpu().numpy()
        assert np.isfinite(G).all(), f"{label} {name}: non-finite"
        tol = 1.2 * b + u * np.abs(ref) + 1e-5 * max(1.0, float(np.abs(ref).max())) + 1e-6
        err = np.abs(G - ref)
        print(f"{label} {name}: max|d|={err.max():.3e} max|ref|={np.abs(ref).max():.3e} "
              f"max err/tol={float((err / tol).max()):.3f}", flush=True)
        assert np.all(err <= tol), f"{label} {name}: outside the 16-bit backward bound"


@pytest.mark.parametrize("N", [1, 17, 64, 65, 127, 128, 129, 200, 256, 300])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_backward_sweep(dtype, d, causal, N):
    q, k, v = W.random_qkv(1, 2, N, d, dtype, seed=7000 + N)
    do = W.random_dout(1, 2, N, d, dtype, seed=7000 + N)
    scale = W.default_scale(d)
    got = run_bwd(q, k, v, do, scale, causal, dtype)
    check(got, q, k, v, do, scale, causal, dtype, f"{dtype} d={d} causal={causal} N={N}")


@pytest.mark.parametrize("scale", [-0.3, 0.0, 0.5])
def test_backward_batch_heads_and_scales(scale):
    q, k, v = W.random_qkv(2, 3, 150, 64, "f16", seed=7100)
    do = W.random_dout(2, 3, 150, 64, "f16", seed=7100)
    for causal in (False, True):
        got = run_bwd(q, k, v, do, scale, causal, "f16")
        check(got, q, k, v, do, scale, causal, "f16", f"B=2 H=3 scale={scale} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_backward_many_tiles(causal):
    q, k, v = W.random_qkv(1, 4, 1000, 128, "bf16", seed=7200)
    do = W.random_dout(1, 4, 1000, 128, "bf16", seed=7200)
    got = run_bwd(q, k, v, do, W.default_scale(128), causal, "bf16")
    check(got, q, k, v, do, W.default_scale(128), causal, "bf16", f"N=1000 causal={causal}")


@pytest.mark.parametrize("N", [600, 700])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_backward_causal_block_pairs(dtype, d, N):
    """Causal: a workgroup takes blocks i and n - 1 - i.  N = 600 gives 5 key
    blocks and 3 query blocks (an odd middle block runs alone), N = 700 gives
    6 and 3, both with a ragged last block; B*H = 15, so the grid is not a
    multiple of the eight XCDs either.  Every gradient against the oracle."""
    q, k, v = W.random_qkv(3, 5, N, d, dtype, seed=7300 + N + d)
    do = W.random_dout(3, 5, N, d, dtype, seed=7300 + N + d)
    got = run_bwd(q, k, v, do, W.default_scale(d), True, dtype)
    check(got, q, k, v, do, W.default_scale(d), True, dtype, f"pairs {dtype} d={d} N={N}")


def test_backward_deterministic_and_side_stream():
    q, k, v = W.random_qkv(1, 2, 333, 128, "f16", seed=7300)
    do = W.random_dout(1, 2, 333, 128, "f16", seed=7300)
    a = run_bwd(q, k, v, do, 0.088, True, "f16")
    b = run_bwd(q, k, v, do, 0.088, True, "f16", stream=torch.cuda.Stream())
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_graph_capture_replays(causal):
    """flash_attn_bwd with a caller workspace enqueues three kernels, allocates
    nothing and clears no memory, so it can be captured in a HIP graph: three
    replays, with eager backward calls on other tensors between them, each
    bitwise equal to the eager call."""
    B, H, N, d = 1, 3, 700, 128
    q, k, v = W.random_qkv(B, H, N, d, "f16", seed=7400)
    do = W.random_dout(B, H, N, d, "f16", seed=7400)
    scale = W.default_scale(d)
    O, L = oracle.attention_forward(q, k, v, scale, causal)
    o = torch.from_numpy(O).to(torch.float16).to(DEV)
    lse = torch.from_numpy(L).to(torch.float32).to(DEV)
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    ws = torch.empty(lib().flash_attn_bwd_workspace_size(B, H, N), dtype=torch.uint8, device=DEV)
    ref = run_bwd(q, k, v, do, scale, causal, "f16")
    grads = [torch.empty_like(qd) for _ in range(3)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up call on the capture stream
        flash_attn_bwd(qd, kd, vd, o, lse, dod, *grads, scale=scale, causal=causal, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        flash_attn_bwd(qd, kd, vd, o, lse, dod, *grads, scale=scale, causal=causal, workspace=ws)
    for rep in range(3):
        for g in grads:
            g.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, g, r in zip(("dQ", "dK", "dV"), grads, ref):
            assert torch.equal(g, r), f"replay {rep} {name}"
        # unrelated eager work between replays (one head, its own workspace)
        other = run_bwd(q[:, :1], k[:, :1], v[:, :1], do[:, :1], scale, causal, "f16")
        for g, r in zip(other, ref):
            assert torch.equal(g, r[:, :1])


def test_backward_workspace_and_dtype_errors():
    x = torch.zeros(1, 1, 8, 64, dtype=torch.float16, device=DEV)
    lse = torch.zeros(1, 1, 8, dtype=torch.float32, device=DEV)
    with pytest.raises(FlashAttnError, match="FA_ERR_WORKSPACE"):
        flash_attn_bwd(x, x, x, x, lse, x, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    # 8 bytes per row (D and LSE * log2(e)); one byte short, or the size of D
    # alone, is rejected before any kernel runs.
    for nbytes in (8 * 8 - 1, 4 * 8):
        with pytest.raises(FlashAttnError, match="FA_ERR_WORKSPACE"):
            flash_attn_bwd(x, x, x, x, lse, x,
                           workspace=torch.empty(nbytes, dtype=torch.uint8, device=DEV))
    ws = torch.empty(8 * 8, dtype=torch.uint8, device=DEV)
    dq, dk, dv = flash_attn_bwd(x, x, x, x, lse, x, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
    y = x.float()
    with pytest.raises(FlashAttnError, match="FA_ERR_DTYPE"):
        flash_attn_bwd(y, y, y, y, lse, y)


@pytest.mark.parametrize("name", sorted(W.BWD_WORKLOADS))
def test_backward_workload_sampled(name):
    """The benchmark's launches at full size (B=2 H=16 N=4096 d=128 fp16
    non-causal; B=1 H=16 N=8192 d=128 bf16 causal), O and LSE from the fp64
    forward: every output finite; four heads checked at 48 sampled query rows
    and 48 sampled key rows (plus the first and last) against the sampled
    oracle and its bound."""
    w = W.BWD_WORKLOADS[name]
    q, k, v = W.random_qkv(w.B, w.H, w.N, w.d, w.dtype, w.seed)
    do = W.random_dout(w.B, w.H, w.N, w.d, w.dtype, w.seed)
    print(f"backward at B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} causal={w.causal}", flush=True)
    got = run_bwd(q, k, v, do, w.scale, w.causal, w.dtype)
    for g in got:
        assert torch.isfinite(g).all()
    rng = np.random.default_rng([w.seed, 77])
    rows = np.unique(np.concatenate([[0, w.N - 1], rng.choice(w.N, 48, replace=False)]))
    cols = np.unique(np.concatenate([[0, w.N - 1], rng.choice(w.N, 48, replace=False)]))
    heads = [(b, h) for b in range(w.B) for h in (0, w.H - 1)] + [(w.B - 1, w.H // 2)]
    u = UNIT[w.dtype]
    ref = oracle.attention_backward_sampled(q, k, v, do, w.scale, w.causal, heads, rows, cols, u=u)
    for (b, h), (rq, rk, rv, bq, bk, bv) in ref.items():
        for name, g, r, bound in (("dQ", got[0][b, h][rows], rq, bq), ("dK", got[1][b, h][cols], rk, bk),
                                  ("dV", got[2][b, h][cols], rv, bv)):
            G = g.double().cpu().numpy()
            tol = 1.2 * bound + u * np.abs(r) + 1e-5 * max(1.0, float(np.abs(r).max())) + 1e-6
            err = np.abs(G - r)
            print(f"head ({b},{h}) {name}: max|d|={err.max():.3e} max err/tol={float((err / tol).max()):.3f}",
                  flush=True)
            assert np.all(err <= tol), f"head ({b},{h}) {name}: outside the 16-bit backward bound"
