"""8-bit forward pass (flash_attn_fwd_fp8) vs the fp64 oracle on the exact
values of the same e4m3 inputs (needs a gfx950 GPU).

Accuracy contract (oracle.fp8_weight_error_bound): the pass rounds its
softmax weights to e4m3, so per output element
    |O - O_exact| <= sum_j max(w_j/16, 2^-10) |v_j - O_exact| / (W - E)
and per row |LSE - LSE_exact| <= -ln(1 - E/W), w_j = exp(s_j - s_max),
W = sum w_j, E = sum max(w_j/16, 2^-10).  On top of that: the bfloat16
rounding of O (2^-9 relative, taken as 2^-8) and fp32 accumulation (1e-4
absolute).
"""
import numpy as np
import pytest
import torch

import oracle
from io_aware_tiled_08_amd import FlashAttnError, flash_attn_fwd_fp8
from io_aware_tiled_08_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_fp8(q, k, v, qs, ks, vs, scale, causal, stream=None):
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o = torch.full(tuple(q.shape), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full(tuple(q.shape[:3]), float("nan"), dtype=torch.float32, device=DEV)
    flash_attn_fwd_fp8(qd, kd, vd, o, lse, q_descale=qs, k_descale=ks, v_descale=vs,
                       scale=scale, causal=causal, stream=stream)
    torch.cuda.synchronize()
    return o, lse


def check(o, lse, q, k, v, qs, ks, vs, scale, causal, label, rows=None):
    Q, K, V = (oracle.dequantize_fp8(x, s) for x, s in ((q, qs), (k, ks), (v, vs)))
    O_ref, L_ref = oracle.attention_forward(Q, K, V, scale, causal, rows=rows)
    bO, bL = oracle.fp8_weight_error_bound(Q, K, V, scale, causal, rows=rows)
    O = o.double().cpu().numpy()
    L = lse.double().cpu().numpy()
    if rows is not None:
        idx = np.broadcast_to(rows, L.shape[:2] + rows.shape[-1:])
        O = np.take_along_axis(O, idx[..., None], axis=2)
        L = np.take_along_axis(L, idx, axis=2)
    assert np.isfinite(O).all() and np.isfinite(L).all(), f"{label}: non-finite output"
    tol_o = bO + 2.0 ** -8 * np.abs(O_ref) + 1e-4
    tol_l = bL + 1e-4
    err_o = np.abs(O - O_ref)
    err_l = np.abs(L - L_ref)
    frac = float(np.max(err_o / tol_o))
    print(f"{label}: max|dO|={err_o.max():.3e} (max err/bound {frac:.3f}) "
          f"max|dLSE|={err_l.max():.3e} (bound {bL.max():.2e})", flush=True)
    assert np.all(err_o <= tol_o), f"{label}: O outside the e4m3 weight-rounding bound"
    assert np.all(err_l <= tol_l), f"{label}: LSE outside the e4m3 weight-rounding bound"


@pytest.mark.parametrize("N", [1, 17, 64, 127, 128, 129, 255, 256, 257, 1000])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_fp8_sweep(d, causal, N):
    q, k, v, qs, ks, vs = W.random_qkv_fp8(1, 2, N, d, seed=5000 + N)
    scale = W.default_scale(d)
    o, lse = run_fp8(q, k, v, qs, ks, vs, scale, causal)
    check(o, lse, q, k, v, qs, ks, vs, scale, causal, f"fp8 d={d} causal={causal} N={N}")


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.4])
def test_fp8_batch_heads_and_scales(scale):
    q, k, v, qs, ks, vs = W.random_qkv_fp8(2, 3, 300, 128, seed=5100)
    for causal in (False, True):
        o, lse = run_fp8(q, k, v, qs, ks, vs, scale, causal)
        check(o, lse, q, k, v, qs, ks, vs, scale, causal, f"B=2 H=3 scale={scale} causal={causal}")


def test_fp8_descales_enter_scores_and_output():
    """Doubling k_descale doubles every score; doubling v_descale doubles O."""
    q, k, v, qs, ks, vs = W.random_qkv_fp8(1, 2, 200, 64, seed=5200)
    for f_k, f_v in ((1.0, 1.0), (2.0, 1.0), (1.0, 3.0), (0.25, 0.5)):
        o, lse = run_fp8(q, k, v, qs, ks * f_k, vs * f_v, 0.125, True)
        check(o, lse, q, k, v, qs, ks * f_k, vs * f_v, 0.125, True, f"k x{f_k} v x{f_v}")


def test_fp8_deterministic_and_side_stream():
    q, k, v, qs, ks, vs = W.random_qkv_fp8(1, 4, 700, 128, seed=5300)
    a = run_fp8(q, k, v, qs, ks, vs, 0.088, True)
    b = run_fp8(q, k, v, qs, ks, vs, 0.088, True, stream=torch.cuda.Stream())
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_fp8_rejects_bad_arguments():
    x = torch.zeros(1, 1, 8, 64).to(torch.float8_e4m3fn).to(DEV)
    with pytest.raises(FlashAttnError, match="FA_ERR_SCALE"):
        flash_attn_fwd_fp8(x, x, x, q_descale=1.0, k_descale=0.0, v_descale=1.0)
    with pytest.raises(FlashAttnError, match="FA_ERR_SCALE"):
        flash_attn_fwd_fp8(x, x, x, q_descale=1.0, k_descale=1.0, v_descale=float("nan"))
    with pytest.raises(TypeError):
        flash_attn_fwd_fp8(x.to(torch.float16), x, x, q_descale=1.0, k_descale=1.0, v_descale=1.0)


def test_fp8_headline_workload_sampled():
    """B=2 H=16 N=4096 d=128, the benchmark's launch, 64 sampled rows per head
    plus the rows around every 256-row block boundary."""
    B, H, N, d = 2, 16, 4096, 128
    q, k, v, qs, ks, vs = W.random_qkv_fp8(B, H, N, d, seed=8)
    o, lse = run_fp8(q, k, v, qs, ks, vs, W.default_scale(d), False)
    sampled = W.sample_rows(8, B, H, N, 64)
    edges = np.array(sorted({r for b0 in range(0, N, 256) for r in (b0 - 1, b0) if 0 <= r < N}))
    rows = np.concatenate([sampled, np.broadcast_to(edges, (B, H, len(edges)))], axis=2)
    rows = np.sort(rows, axis=2)
    check(o, lse, q, k, v, qs, ks, vs, W.default_scale(d), False, "headline fp8", rows=rows)
