"""HIP path vs the fp64 oracle on identical seeded inputs (needs a gfx950 GPU).

Tolerances: max-abs error against fp64 of 2e-3 for fp16, 1e-2 for bf16 and
1e-5 for fp32 inputs, applied to O and to LSE alike.  Only the unusual-scale
test departs from them, with the bound derived for its inputs (see there).
"""
import time

import numpy as np
import pytest
import torch

import oracle
from oracle_pool import forward_by_heads, host_cores
from io_aware_tiled_08_amd import FlashAttnError, flash_attn_fwd
from io_aware_tiled_08_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}
DEV = "cuda:0"


def gpu_forward(q, k, v, scale, causal, stream=None):
    """Runs the kernel with O and LSE pre-filled with NaN, so any element the
    kernel fails to write shows up."""
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full(tuple(q.shape[:3]), float("nan"), dtype=torch.float32, device=DEV)
    flash_attn_fwd(qd, kd, vd, o, lse, scale=scale, causal=causal, stream=stream)
    torch.cuda.synchronize()
    return o, lse


def check(o, lse, q, k, v, scale, causal, dtype, rows=None, label="", tol=None, ref=None):
    """Max-abs error of O and LSE against the oracle.  ``tol`` is a number or,
    for O, an array of per-element bounds (LSE then takes the fixed one);
    ``ref`` a precomputed oracle result for these inputs and rows."""
    tol = TOL[dtype] if tol is None else tol
    tol_l = tol if np.isscalar(tol) else TOL[dtype]
    O_ref, L_ref = oracle.attention_forward(q, k, v, scale, causal, rows=rows) if ref is None else ref
    O = o.double().cpu().numpy()
    L = lse.double().cpu().numpy()
    if rows is not None:
        idx = np.broadcast_to(rows, L.shape[:2] + rows.shape[-1:])
        O = np.take_along_axis(O, idx[..., None], axis=2)
        L = np.take_along_axis(L, idx, axis=2)
    assert np.isfinite(O).all() and np.isfinite(L).all(), f"{label}: non-finite output"
    d_o = np.abs(O - O_ref)
    err_o = float(np.max(d_o)) if O.size else 0.0
    err_l = float(np.max(np.abs(L - L_ref))) if L.size else 0.0
    ratio = float(np.max(d_o / tol)) if O.size else 0.0
    print(f"{label}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e} max|dO|/tol={ratio:.3f}", flush=True)
    assert ratio <= 1.0, f"{label}: O error {err_o:.3e}, {ratio:.3f} of its bound"
    assert err_l <= tol_l, f"{label}: LSE error {err_l:.3e} > {tol_l}"
    return err_o, err_l


SWEEP_N = [1, 2, 17, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300, 1000]


@pytest.mark.parametrize("N", SWEEP_N)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_sweep(dtype, d, causal, N):
    q, k, v = W.random_qkv(1, 2, N, d, dtype, seed=1000 + N)
    scale = W.default_scale(d)
    o, lse = gpu_forward(q, k, v, scale, causal)
    check(o, lse, q, k, v, scale, causal, dtype, label=f"{dtype} d={d} causal={causal} N={N}")


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_batch_and_head_indexing(dtype):
    q, k, v = W.random_qkv(3, 5, 100, 64, dtype, seed=77)
    for causal in (False, True):
        o, lse = gpu_forward(q, k, v, 0.125, causal)
        check(o, lse, q, k, v, 0.125, causal, dtype, label=f"B3H5 {dtype} causal={causal}")


@pytest.mark.parametrize("scale", [-0.2, 0.0, 1.5])
@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_unusual_scales(dtype, scale):
    """Scores here reach |scale| * sqrt(d) standard deviations (17 for 1.5 at
    d=128), far from the workloads' statistics.
    fp32: the products and sums of an fp32 dot product round relative to the
    score's size, and that error moves O and LSE by the same amount, so the
    bound grows with max(1, |scale| * sqrt(d)).
    fp16/bf16: the products are exact and the rounding of the scores is
    negligible; the errors are the rounding of each weight and of O to the
    input type, both relative.  With nearly one-hot rows O approaches single
    rows of V and the output rounding alone nears the fixed fp16 tolerance, so
    each element may use the derived bound of those two roundings
    (oracle.forward_error_bound_16) where it exceeds the fixed tolerance; LSE
    keeps the fixed tolerance."""
    q, k, v = W.random_qkv(1, 2, 200, 128, dtype, seed=5)
    for causal in (False, True):
        if dtype == "f32":
            tol = TOL[dtype] * max(1.0, abs(scale) * 128 ** 0.5)
        else:
            tol = np.maximum(TOL[dtype], oracle.forward_error_bound_16(q, k, v, scale, causal, dtype))
        o, lse = gpu_forward(q, k, v, scale, causal)
        check(o, lse, q, k, v, scale, causal, dtype, tol=tol,
              label=f"{dtype} scale={scale} causal={causal}")


def test_rescale_stress_small():
    """Growing score maxima along the sequence (the rescale-stress recipe at a
    size the oracle handles whole)."""
    q, k, v = W.random_qkv(1, 4, 3000, 128, "bf16", seed=44, kind="rescale_stress")
    o, lse = gpu_forward(q, k, v, W.default_scale(128), True)
    check(o, lse, q, k, v, W.default_scale(128), True, "bf16", label="stress bf16 N=3000")
    q, k, v = W.random_qkv(1, 4, 3000, 64, "f16", seed=45, kind="rescale_stress")
    o, lse = gpu_forward(q, k, v, W.default_scale(64), True)
    check(o, lse, q, k, v, W.default_scale(64), True, "f16", label="stress f16 N=3000")


def test_constant_v_and_dominant_key():
    N, d = 333, 64
    q, k, _ = W.random_qkv(1, 1, N, d, "f16", seed=9)
    v = torch.full((1, 1, N, d), 0.75, dtype=torch.float16)
    o, _ = gpu_forward(q, k, v, 0.125, False)
    assert torch.all(o.float().cpu() == 0.75)
    # One key aligned with every query by a wide margin: O is that key's V row.
    q = torch.zeros(1, 1, N, d, dtype=torch.float16)
    q[..., 0] = 1.0
    k = torch.zeros(1, 1, N, d, dtype=torch.float16)
    k[0, 0, 200, 0] = 60.0
    v = torch.randn(1, 1, N, d).to(torch.float16)
    o, lse = gpu_forward(q, k, v, 1.0, False)
    assert torch.allclose(o[0, 0].float().cpu(), v[0, 0, 200].float().expand(N, d), atol=1e-3)
    assert torch.allclose(lse.cpu(), torch.full((1, 1, N), 60.0), atol=1e-3)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("jump", [5.0, 12.0, 15.5, 17.0, 40.0, 118.0, 124.0, 180.0])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_score_jump_in_later_tile(dtype, jump, causal):
    """One key (in the third 128-key tile) whose score exceeds every earlier
    score of its row by `jump` log2 units, so the running maximum rises by
    that much in one tile and what was accumulated is rescaled by 2^-jump.
    The sizes straddle the lazy-rescale slack (2^8, below which the reference
    stays put and weights up to 2^jump enter P), the top of fp16 (2^16), and
    factors that underflow fp32 (2^-124 is subnormal, 2^-180 is zero)."""
    N, d, p = 700, 64, 300
    g = torch.Generator().manual_seed(int(jump * 10) + causal)
    q = 0.1 * torch.randn(1, 2, N, d, generator=g)
    k = 0.1 * torch.randn(1, 2, N, d, generator=g)
    q[..., 0] = 1.0
    k[:, :, p, 0] = jump / np.log2(np.e)  # scale 1: natural-log score of about jump * ln 2
    dt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    q, k = q.to(dt), k.to(dt)
    v = torch.randn(1, 2, N, d, generator=g).to(dt)
    o, lse = gpu_forward(q, k, v, 1.0, causal)
    check(o, lse, q, k, v, 1.0, causal, dtype, label=f"{dtype} jump={jump} causal={causal}")


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_deterministic(dtype):
    q, k, v = W.random_qkv(2, 2, 777, 128, dtype, seed=3)
    o1, l1 = gpu_forward(q, k, v, 0.09, True)
    o2, l2 = gpu_forward(q, k, v, 0.09, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_side_stream():
    q, k, v = W.random_qkv(1, 2, 500, 64, "f16", seed=8)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = gpu_forward(q, k, v, 0.125, True, stream=s)
    check(o, lse, q, k, v, 0.125, True, "f16", label="side stream")


def test_misaligned_pointer_is_rejected():
    x = torch.zeros(4 * 64 + 1, dtype=torch.float16, device=DEV)
    q = x[1:].view(1, 1, 4, 64)
    with pytest.raises(FlashAttnError, match="FA_ERR_ALIGN"):
        flash_attn_fwd(q, q, q)


def test_bad_head_dim_is_rejected():
    x = torch.zeros(1, 1, 4, 96, dtype=torch.float16, device=DEV)
    with pytest.raises(FlashAttnError, match="FA_ERR_HEAD_DIM"):
        flash_attn_fwd(x, x, x)


def test_empty_sequence():
    x = torch.zeros(1, 2, 0, 64, dtype=torch.float16, device=DEV)
    o, lse = flash_attn_fwd(x, x, x)
    assert o.shape == x.shape and lse.shape == (1, 2, 0)


# --- the named workloads, in the launch configuration the benchmark times ---

def _run_workload(name, rows=None):
    w = W.WORKLOADS[name]
    q, k, v = W.workload_inputs(w)
    print(f"workload {name}: B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} causal={w.causal}",
          flush=True)
    o, lse = gpu_forward(q, k, v, w.scale, w.causal)
    return w, q, k, v, o, lse


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["single_head_f32", "batch_f16_d64", "batch_f16_d64_causal",
                                  "headline_f16_d128", "rescale_stress_bf16"])
def test_workload_full(name):
    """Every row of every head against the oracle, at the fixed tolerances.
    The oracle runs head by head on the host's cores (tests/oracle_pool.py)."""
    w, q, k, v, o, lse = _run_workload(name)
    t0 = time.time()

    def progress(done, total):
        if done == total or done % max(1, total // 4) == 0:
            print(f"  oracle: {done}/{total} heads, {time.time() - t0:.1f} s", flush=True)

    ref = forward_by_heads(q, k, v, w.scale, w.causal, progress=progress)
    print(f"  oracle on {host_cores()} cores: {time.time() - t0:.1f} s", flush=True)
    check(o, lse, q, k, v, w.scale, w.causal, w.dtype, label=name, ref=ref)


def test_workload_long_context():
    name = "long_context_bf16"
    w, q, k, v, o, lse = _run_workload(name)
    rows = W.sample_rows(w.seed, w.B, w.H, w.N, w.sampled_rows)
    check(o, lse, q, k, v, w.scale, w.causal, w.dtype, rows=rows, label=name)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("N", [600, 700])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_causal_d64_block_pairs(dtype, N):
    """The small causal d=64 schedule runs 128-row blocks in pairs (block
    n-1-i, then block i, in one workgroup): an odd block count (600: five
    blocks, the middle one alone), a ragged last block (700: six blocks, 60
    rows in the last), and a grid of 45 workgroups (not a multiple of the
    eight XCDs), every row against the oracle."""
    q, k, v = W.random_qkv(3, 5, N, 64, dtype, seed=2200 + N)
    scale = W.default_scale(64)
    o, lse = gpu_forward(q, k, v, scale, True)
    check(o, lse, q, k, v, scale, True, dtype, label=f"{dtype} causal d=64 N={N} block pairs")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_causal_d64_many_blocks(dtype):
    """Causal d=64 with more than 512 blocks of 256 rows (here 640): the
    256-row schedule; the small causal d=64 cases above take the 128-row
    key-split schedule."""
    B, H, N, d = 8, 16, 1100, 64
    q, k, v = W.random_qkv(B, H, N, d, dtype, seed=2100)
    scale = W.default_scale(d)
    o, lse = gpu_forward(q, k, v, scale, True)
    rows = np.sort(np.concatenate([W.sample_rows(2100, B, H, N, 40),
                                   np.broadcast_to(np.array([0, 255, 256, 1099]), (B, H, 4))], axis=2), axis=2)
    check(o, lse, q, k, v, scale, True, dtype, rows=rows, label=f"{dtype} causal d=64 640 blocks")


@pytest.mark.parametrize("dtype,d,N,heads,scale", [
    ("f16", 128, 1000, 128, None),   # 512 blocks of 256 rows: two per CU, ragged last block
    ("bf16", 64, 1300, 128, None),   # 768 blocks: three per CU
    ("f16", 64, 700, 256, -0.11),    # negative scale: Q's sign flip on every next-block load
])
def test_many_unmasked_blocks(dtype, d, N, heads, scale):
    """Unmasked problems with at least two 256-row blocks per CU, where
    flash_attn_fwd runs each workgroup's blocks as one tile stream: sampled
    rows (plus every block's first and last rows) against the oracle."""
    B, H = 2, heads // 2
    q, k, v = W.random_qkv(B, H, N, d, dtype, seed=7000 + N)
    scale = W.default_scale(d) if scale is None else scale
    o, lse = gpu_forward(q, k, v, scale, False)
    base = {0, N - 1} | {x for b in range(0, N, 256) for x in (b, b + 255) if x < N}
    rng = np.random.default_rng([N, 17])
    extra = rng.choice(N, size=min(N, 24), replace=False)
    rows = np.array(sorted(base | {int(x) for x in extra}), dtype=np.int64)
    rows = np.broadcast_to(rows, (B, H, rows.size))
    check(o, lse, q, k, v, scale, False, dtype, rows=rows,
          label=f"{dtype} d={d} N={N} B*H={heads} scale={scale:.3f}")


@pytest.mark.parametrize("B,H,N,causal", [
    (1, 3, 700, True),      # one workgroup per block (the grid)
    (2, 16, 4096, False),   # two blocks per CU: the persistent tile stream
])
def test_graph_capture_replays(B, H, N, causal):
    """flash_attn_fwd enqueues one kernel, allocates nothing and clears no
    memory, so it can be captured in a HIP graph: three replays, with eager
    work on other tensors between them, each bitwise equal to the eager call."""
    q, k, v = (x.to(DEV) for x in W.random_qkv(B, H, N, 128, "f16", seed=9100 + N))
    scale = W.default_scale(128)
    o_ref, lse_ref = gpu_forward(q, k, v, scale, causal)
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up call on the capture stream
        flash_attn_fwd(q, k, v, o, lse, scale=scale, causal=causal)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        flash_attn_fwd(q, k, v, o, lse, scale=scale, causal=causal)
    for rep in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), f"replay {rep}"
        # unrelated eager work between replays
        o2, _ = gpu_forward(q[:, :1].contiguous(), k[:, :1].contiguous(), v[:, :1].contiguous(),
                            scale, causal)
        assert torch.equal(o2, o_ref[:, :1])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N", [
    (1, 1, 2100),  # B*H*N^2 over 2^20: the 32-row kernel
    (2, 8, 300),   # B*H*N^2 = 1.44e7: the 32-row kernel
    (4, 1, 512),   # B*H*N^2 = 2^20 (the limit): the 4-row kernel
    (1, 3, 37),    # ragged 4-row blocks
])
def test_f32_both_schedules(B, H, N, causal):
    """fp32 at d=64 runs on 4-row workgroups when B*H*N^2 <= 2^20, else on
    32-row workgroups; both against the oracle at 1e-5."""
    q, k, v = W.random_qkv(B, H, N, 64, "f32", seed=3300 + N)
    o, lse = gpu_forward(q, k, v, 0.125, causal)
    check(o, lse, q, k, v, 0.125, causal, "f32", label=f"f32 B={B} H={H} N={N} causal={causal}")
