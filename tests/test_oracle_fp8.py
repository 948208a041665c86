"""The 8-bit side of the oracle: e4m3 decoding and the accuracy contract of a
forward pass that rounds its softmax weights to e4m3, pinned against torch's
float8_e4m3fn conversion, values fixed by the format's definition, and a
simulation of that rounding on random inputs."""
import math

import numpy as np
import pytest
import torch

import oracle
from io_aware_tiled_08_amd import workloads as W


def test_decode_matches_torch_for_every_code():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    want = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode_e4m3(codes.numpy())
    nan = np.isnan(want)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(got[~nan], want[~nan])


def test_decode_fixed_values():
    # largest finite, smallest normal, smallest subnormal, one, NaN, -0
    table = {0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x38: 1.0, 0x39: 1.125,
             0xBE: -1.75, 0x00: 0.0, 0x80: -0.0}
    for c, v in table.items():
        assert oracle.decode_e4m3([c])[0] == v, hex(c)
    assert np.isnan(oracle.decode_e4m3([0x7F, 0xFF])).all()


def test_dequantize_applies_float32_descale():
    x = torch.tensor([1.0, -2.0, 448.0]).to(torch.float8_e4m3fn)
    got = oracle.dequantize_fp8(x, 0.1)
    assert np.array_equal(got, np.array([1.0, -2.0, 448.0]) * float(np.float32(0.1)))


def test_quantize_recipe_round_trip():
    x = np.random.default_rng(5).standard_normal((2, 3, 50, 16)).astype(np.float32)
    codes, s = W.quantize_e4m3(x)
    assert s == float(np.float32(np.abs(x).max() / 448.0))
    back = oracle.dequantize_fp8(codes, s)
    # |x| / s <= 448: every value rounds to a neighbour within half a unit
    rel = np.abs(back - x) / np.maximum(np.abs(x), 2.0 ** -6 * s)
    assert rel.max() <= 2.0 ** -4 + 1e-6
    assert np.abs(back).max() <= 448.0 * s * (1 + 1e-7)


def _round_e4m3(w):
    return torch.from_numpy(w).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def _simulated_fp8_pass(q, k, v, scale, causal, drop, rng, absolute_term=True):
    """The weight rounding of an 8-bit pass, simulated in float64: weights
    2^(c*s - m_ref) with m_ref = m_max - drop*U[0,1] (log2 units), rounded to
    e4m3, used in both sums.  Returns (O_hat, LSE_hat)."""
    Q, K, V = (oracle.as_f64(x) for x in (q, k, v))
    B, H, N, d = Q.shape
    c = float(np.float32(scale)) / math.log(2.0)
    O = np.zeros((B, H, N, d))
    L = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            S = Q[b, h] @ K[b, h].T * c  # log2 units
            if causal:
                S[np.triu(np.ones((N, N), bool), 1)] = -np.inf
            m_ref = S.max(axis=1, keepdims=True) - drop * rng.random((N, 1))
            w = np.exp2(S - m_ref)
            wh = _round_e4m3(w)
            O[b, h] = wh @ V[b, h] / wh.sum(axis=1, keepdims=True)
            L[b, h] = (m_ref[:, 0] + np.log2(wh.sum(axis=1))) * math.log(2.0)
    return O, L


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("temp", [0.3, 1.0, 3.0])
def test_bound_holds_for_simulated_rounding(causal, temp):
    """Random e4m3 inputs at three score temperatures: the simulated error of
    the weight rounding never exceeds the bound, and the bound is not vacuous
    (the largest error reaches a fair fraction of it)."""
    q, k, v, qs, ks, vs = W.random_qkv_fp8(1, 2, 200, 32, seed=41)
    Q, K, V = (oracle.dequantize_fp8(x, s) for x, s in ((q, qs), (k, ks), (v, vs)))
    scale = temp / math.sqrt(32)
    O, L = oracle.attention_forward(Q, K, V, scale, causal)
    bO, bL = oracle.fp8_weight_error_bound(Q, K, V, scale, causal)
    rng = np.random.default_rng(7)
    worst = 0.0
    for drop in (0.0, 4.0, 8.0):
        Oh, Lh = _simulated_fp8_pass(Q, K, V, scale, causal, drop, rng)
        assert np.all(np.abs(Oh - O) <= bO * (1 + 1e-9) + 1e-12)
        assert np.all(np.abs(Lh - L) <= bL * (1 + 1e-9) + 1e-12)
        worst = max(worst, float(np.max(np.abs(Oh - O) / (bO + 1e-300))))
    assert worst > 0.05


def test_weight_rounding_error_terms():
    """The per-weight ingredient of the bound: rounding a weight in (0, 1] to
    e4m3 moves it by at most max(2^-4 w, 2^-10), and both terms are needed
    (subnormal weights break the relative term alone; the absolute term alone
    fails near 1)."""
    w = np.exp2(-np.linspace(0.0, 12.0, 200_001))
    err = np.abs(_round_e4m3(w) - w)
    assert np.all(err <= np.maximum(2.0 ** -4 * w, 2.0 ** -10) * (1 + 1e-12))
    assert np.any(err > 2.0 ** -4 * w)
    assert np.any(err > 2.0 ** -10)
    # the bound is reached: a tie in the normal range, and half a subnormal step
    assert np.isclose(np.max(err / np.maximum(2.0 ** -4 * w, 2.0 ** -10)), 1.0, atol=1e-4)


def test_bound_grows_with_the_absolute_term():
    """The bound function uses the absolute term: more tiny weights, larger bound."""
    q, k, v, qs, ks, vs = W.random_qkv_fp8(1, 1, 64, 16, seed=43)
    Q, K, V = (oracle.dequantize_fp8(x, s) for x, s in ((q, qs), (k, ks), (v, vs)))
    full, fl = oracle.fp8_weight_error_bound(Q, K, V, 0.25, False)
    rel, rl = oracle.fp8_weight_error_bound(Q, K, V, 0.25, False, a=0.0)
    assert np.all(full >= rel) and np.all(fl >= rl) and np.any(full > rel * 1.01)
