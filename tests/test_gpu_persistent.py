"""Persistent schedule (flash_attn_fwd_persistent) vs the fp64 oracle, and
bitwise against flash_attn_fwd's 256-row kernel, which computes every query
block with the same code (needs a gfx950 GPU).

Tolerances as for flash_attn_fwd: max-abs error against fp64 of 2e-3 (fp16)
and 1e-2 (bf16) on O and LSE.
"""
import numpy as np
import pytest
import torch

import oracle
from io_aware_tiled_08_amd import FlashAttnError, flash_attn_fwd, flash_attn_fwd_persistent
from io_aware_tiled_08_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f16": 2e-3, "bf16": 1e-2}
DEV = "cuda:0"


def run(fn, q, k, v, scale, causal, **kw):
    """O and LSE pre-filled with NaN, so an element no block writes shows up."""
    o = torch.full_like(q, float("nan"))
    lse = torch.full(tuple(q.shape[:3]), float("nan"), dtype=torch.float32, device=DEV)
    fn(q, k, v, o, lse, scale=scale, causal=causal, **kw)
    torch.cuda.synchronize()
    return o, lse


def grid_is_256_rows(B, H, N, d, causal):
    """flash_attn_fwd takes the 128-row key-split schedule for causal d=64
    problems of at most 512 blocks of 256 rows; otherwise the 256-row kernel."""
    return not (d == 64 and causal and B * H * ((N + 255) // 256) <= 512)


def check_oracle(o, lse, q, k, v, scale, causal, dtype, label, rows=None):
    O_ref, L_ref = oracle.attention_forward(q, k, v, scale, causal, rows=rows)
    O = o.double().cpu().numpy()
    L = lse.double().cpu().numpy()
    if rows is not None:
        idx = np.broadcast_to(rows, L.shape[:2] + rows.shape[-1:])
        O = np.take_along_axis(O, idx[..., None], axis=2)
        L = np.take_along_axis(L, idx, axis=2)
    assert np.isfinite(O).all() and np.isfinite(L).all(), f"{label}: non-finite output"
    err_o = float(np.max(np.abs(O - O_ref)))
    err_l = float(np.max(np.abs(L - L_ref)))
    print(f"{label}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
    assert err_o <= TOL[dtype] and err_l <= TOL[dtype], label


@pytest.mark.parametrize("nwg", [0, 1, 5])
@pytest.mark.parametrize("N", [1, 255, 256, 257, 1000, 1300])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_persistent_sweep(d, causal, N, nwg):
    """B*H = 6 (not a multiple of 8), 1 to 36 blocks; one workgroup runs them
    all, five take several rounds each, 0 means one per CU (clamped to the
    block count)."""
    dtype = "f16" if (N + d) % 2 else "bf16"
    q, k, v = (x.to(DEV) for x in W.random_qkv(2, 3, N, d, dtype, seed=6000 + N))
    scale = W.default_scale(d)
    o, lse = run(flash_attn_fwd_persistent, q, k, v, scale, causal, num_workgroups=nwg)
    label = f"persistent {dtype} d={d} causal={causal} N={N} nwg={nwg}"
    check_oracle(o, lse, q.cpu(), k.cpu(), v.cpu(), scale, causal, dtype, label)
    if grid_is_256_rows(2, 3, N, d, causal):
        o2, lse2 = run(flash_attn_fwd, q, k, v, scale, causal)
        assert torch.equal(o, o2) and torch.equal(lse, lse2), f"{label}: differs from the grid kernel"


@pytest.mark.parametrize("nwg", [0, 8, 24, 40])
@pytest.mark.parametrize("causal", [False, True])
def test_persistent_xcd_orders(causal, nwg):
    """B*H = 16 and grids that are multiples of 8 take the XCD-aware item
    orders (the head-major remap when unmasked); 40 workgroups over 80 blocks
    leave a partial snake round when causal."""
    B, H, N, d = 2, 8, 1280, 128
    q, k, v = (x.to(DEV) for x in W.random_qkv(B, H, N, d, "f16", seed=6100))
    scale = W.default_scale(d)
    o, lse = run(flash_attn_fwd_persistent, q, k, v, scale, causal, num_workgroups=nwg)
    rows = np.array(sorted({0, 1, 255, 256, 511, 512, 767, 768, 1023, 1024, 1279} |
                           set(range(600, 640))), dtype=np.int64)
    check_oracle(o, lse, q.cpu(), k.cpu(), v.cpu(), scale, causal, "f16",
                 f"xcd causal={causal} nwg={nwg}", rows=rows)
    o2, lse2 = run(flash_attn_fwd, q, k, v, scale, causal)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("scale", [-0.2, 0.0])
def test_persistent_negative_and_zero_scale(scale):
    q, k, v = (x.to(DEV) for x in W.random_qkv(1, 2, 300, 128, "bf16", seed=6200))
    for causal in (False, True):
        o, lse = run(flash_attn_fwd_persistent, q, k, v, scale, causal, num_workgroups=3)
        check_oracle(o, lse, q.cpu(), k.cpu(), v.cpu(), scale, causal, "bf16",
                     f"scale={scale} causal={causal}")


@pytest.mark.parametrize("name", ["headline_f16_d128", "long_context_bf16"])
def test_persistent_workload_bitwise(name):
    """Full-size workloads: bitwise equal to the grid kernel, plus sampled
    rows against the oracle.  flash_attn_fwd itself runs unmasked problems of
    two or more blocks per CU on the persistent tile stream, so the grid
    kernel's reference comes from the first batch entry alone, few enough
    blocks for flash_attn_fwd to take the grid."""
    w = W.WORKLOADS[name]
    print(f"workload {name}: B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} causal={w.causal}",
          flush=True)
    q, k, v = (x.to(DEV) for x in W.workload_inputs(w))
    o, lse = run(flash_attn_fwd_persistent, q, k, v, w.scale, w.causal)
    if w.causal:
        o2, lse2 = run(flash_attn_fwd, q, k, v, w.scale, w.causal)
        assert torch.equal(o, o2) and torch.equal(lse, lse2), name
    else:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        assert w.H * ((w.N + 255) // 256) < 2 * cus, "first batch entry must take the grid"
        q1, k1, v1 = (x[:1].contiguous() for x in (q, k, v))
        o2, lse2 = run(flash_attn_fwd, q1, k1, v1, w.scale, w.causal)
        assert torch.equal(o[:1], o2) and torch.equal(lse[:1], lse2), name
    rows = W.sample_rows(w.seed, w.B, w.H, w.N, 64)
    check_oracle(o, lse, q.cpu(), k.cpu(), v.cpu(), w.scale, w.causal, w.dtype, name, rows=rows)


def test_persistent_rejects_fp32_and_negative_grid():
    x = torch.zeros(1, 1, 8, 64, device=DEV)
    with pytest.raises(FlashAttnError, match="FA_ERR_DTYPE"):
        flash_attn_fwd_persistent(x, x, x)
    y = x.half()
    with pytest.raises(FlashAttnError, match="FA_ERR_SHAPE"):
        flash_attn_fwd_persistent(y, y, y, num_workgroups=-2)


def test_persistent_side_stream_and_repeat():
    q, k, v = (x.to(DEV) for x in W.random_qkv(1, 4, 700, 64, "f16", seed=6300))
    a = run(flash_attn_fwd_persistent, q, k, v, 0.125, True, num_workgroups=7)
    b = run(flash_attn_fwd_persistent, q, k, v, 0.125, True, num_workgroups=7,
            stream=torch.cuda.Stream())
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
