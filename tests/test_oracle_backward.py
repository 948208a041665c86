"""The backward oracle (gradients of the forward pass) and its accuracy
contract, pinned against torch autograd and SDPA in float64, central finite
differences of the (separately pinned) forward oracle, invariants that hold
for any inputs, and a simulation of the 16-bit rounding steps."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle_pins import _randn


def _torch_grads(q, k, v, do, scale, causal, use_sdpa):
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = oracle.boundary_scale(scale)
    if use_sdpa:
        out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=s)
    else:
        S = torch.matmul(tq, tk.transpose(-1, -2)) * s
        if causal:
            n = S.shape[-1]
            S = S.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
        out = torch.matmul(torch.softmax(S, dim=-1), tv)
    out.backward(torch.tensor(do, dtype=torch.float64))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("use_sdpa", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd(causal, use_sdpa):
    q, k, v, do = (_randn(1000 + t, 2, 2, 37, 8) for t in range(4))
    dQ, dK, dV, _ = oracle.attention_backward(q, k, v, do, 0.7, causal)
    tq, tk, tv = _torch_grads(q, k, v, do, 0.7, causal, use_sdpa)
    for name, a, b in (("dQ", dQ, tq), ("dK", dK, tk), ("dV", dV, tv)):
        assert np.max(np.abs(a - b)) <= 1e-12, name


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences(causal):
    """Central differences of sum(dO * O) through attention_forward."""
    q, k, v, do = (_randn(1100 + t, 1, 1, 5, 3) for t in range(4))
    dQ, dK, dV, _ = oracle.attention_backward(q, k, v, do, 0.9, causal)
    h = 1e-6

    def f(q_, k_, v_):
        O, _ = oracle.attention_forward(q_, k_, v_, 0.9, causal)
        return float((O * do).sum())

    for name, grad, which in (("dQ", dQ, 0), ("dK", dK, 1), ("dV", dV, 2)):
        for idx in np.ndindex(q.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += h
            fp = f(*args)
            args[which][idx] -= 2 * h
            fm = f(*args)
            assert abs((fp - fm) / (2 * h) - grad[idx]) <= 1e-7, (name, idx)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    """Adding a vector to every key changes nothing: sum_j dK_j = 0.  Rows of
    P sum to one: sum_j dV_j = sum_i dO_i.  Scaling Q or K scales the scores
    alike: sum_i q_i . dQ_i = sum_j k_j . dK_j.  And D_i = sum_j P_ij dP_ij."""
    q, k, v, do = (_randn(1200 + t, 1, 2, 50, 16) for t in range(4))
    dQ, dK, dV, D = oracle.attention_backward(q, k, v, do, 0.3, causal)
    assert np.max(np.abs(dK.sum(axis=2))) <= 1e-12
    assert np.max(np.abs(dV.sum(axis=2) - do.sum(axis=2))) <= 1e-12
    lhs = (q * dQ).sum(axis=(2, 3))
    rhs = (k * dK).sum(axis=(2, 3))
    assert np.max(np.abs(lhs - rhs)) <= 1e-11
    O, _ = oracle.attention_forward(q, k, v, 0.3, causal)
    assert np.max(np.abs(D - (do * O).sum(axis=3))) <= 1e-12


def _mutant_backward(mistake):
    def bwd(q, k, v, do, scale, causal):
        Q, K, V, dO = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        s = float(np.float32(scale))
        N = Q.shape[2]
        S = np.einsum("bhid,bhjd->bhij", Q, K) * s
        if causal and mistake != "no_mask":
            S = np.where(np.triu(np.ones((N, N), bool), 1), -np.inf, S)
        P = np.exp(S - S.max(-1, keepdims=True))
        P /= P.sum(-1, keepdims=True)
        O = P @ V
        D = (dO * O).sum(-1)
        dP = dO @ np.swapaxes(V, -1, -2)
        dS = P * (dP - (0.0 if mistake == "no_D" else D[..., None]))
        dV = np.swapaxes(P, -1, -2) @ dO
        if mistake == "dV_untransposed":
            dV = P @ dO
        dQ = s * dS @ K
        dK = (1.0 if mistake == "dK_unscaled" else s) * np.swapaxes(dS, -1, -2) @ Q
        if mistake == "dQ_sign":
            dQ = -dQ
        return dQ, dK, dV
    return bwd


@pytest.mark.parametrize("mistake", ["no_mask", "no_D", "dV_untransposed", "dK_unscaled", "dQ_sign"])
def test_pins_catch_planted_backward_mistakes(mistake):
    q, k, v, do = (_randn(1300 + t, 1, 2, 20, 8) for t in range(4))
    bad = _mutant_backward(mistake)
    caught = False
    for causal in (False, True):
        tq, tk, tv = _torch_grads(q, k, v, do, 0.5, causal, True)
        gq, gk, gv = bad(q, k, v, do, 0.5, causal)
        caught |= not (np.allclose(gq, tq, atol=1e-9) and np.allclose(gk, tk, atol=1e-9)
                       and np.allclose(gv, tv, atol=1e-9))
    assert caught
    good = _mutant_backward(None)
    for causal in (False, True):
        tq, tk, tv = _torch_grads(q, k, v, do, 0.5, causal, True)
        gq, gk, gv = good(q, k, v, do, 0.5, causal)
        assert np.allclose(gq, tq, atol=1e-12) and np.allclose(gk, tk, atol=1e-12)


def _round16(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).to(torch.float64).numpy()


def _simulated_pass(q, k, v, do, scale, causal, dtype, p_rounded):
    """The 16-bit pass in float64: O handed in rounded, P rounded before
    dV = P^T dO, dS = P_in (dP - D) rounded before dQ and dK, with P_in the
    rounded P (p_rounded) or P itself."""
    s = oracle.boundary_scale(scale)
    N = q.shape[2]
    S = np.einsum("bhid,bhjd->bhij", q, k) * s
    if causal:
        S = np.where(np.triu(np.ones((N, N), bool), 1), -np.inf, S)
    P = np.exp(S - S.max(-1, keepdims=True))
    P /= P.sum(-1, keepdims=True)
    O = _round16(P @ v, dtype)
    D = (do * O).sum(-1)
    Ph = _round16(P, dtype)
    dSh = _round16((Ph if p_rounded else P) * (do @ np.swapaxes(v, -1, -2) - D[..., None]), dtype)
    return {"dV": np.swapaxes(Ph, -1, -2) @ do, "dQ": s * dSh @ k,
            "dK": s * np.swapaxes(dSh, -1, -2) @ q}


@pytest.mark.parametrize("p_rounded", [False, True])
@pytest.mark.parametrize("dtype,u", [(torch.float16, 2.0 ** -11), (torch.bfloat16, 2.0 ** -8)])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_bound_holds_for_simulated_rounding(dtype, u, causal, p_rounded):
    """Simulate the 16-bit pass, with P entering dS in fp32 (u_p = 0) or
    rounded to the input type (u_p = u, the default): the error never exceeds
    the bound and reaches a fair part of it."""
    q, k, v, do = (_round16(_randn(1400 + t, 1, 2, 64, 32), dtype) for t in range(4))
    scale = 1.0 / math.sqrt(32)
    dQ, dK, dV, _ = oracle.attention_backward(q, k, v, do, scale, causal)
    bQ, bK, bV = oracle.backward_error_bound(q, k, v, do, scale, causal, u=u,
                                             u_p=u if p_rounded else 0.0)
    sims = _simulated_pass(q, k, v, do, scale, causal, dtype, p_rounded)
    worst = 0.0
    for name, ref, b in (("dQ", dQ, bQ), ("dK", dK, bK), ("dV", dV, bV)):
        err = np.abs(sims[name] - ref)
        assert np.all(err <= b * (1 + 1e-9) + 1e-13), name
        worst = max(worst, float(np.max(err / (b + 1e-300))))
    assert worst > 0.05


@pytest.mark.parametrize("dtype,u", [(torch.float16, 2.0 ** -11), (torch.bfloat16, 2.0 ** -8)])
def test_backward_bound_needs_the_rounded_p_term(dtype, u):
    """With K the identity (N = d), dQ is scale * dS, so the dQ bound is the
    per-element bound on dS itself.  A pass that forms dS from the rounded P
    then leaves the bound without the P-rounding term (u_p = 0) and stays
    inside it with the term; a pass that forms dS from P in fp32 stays inside
    both.  Scores stay within a few units, so no weight is subnormal in the
    16-bit type (the bound treats every rounding as relative)."""
    n = 32
    rng = np.random.default_rng(11)
    q, v, do = (_round16(rng.standard_normal((1, 2, n, n)), dtype) for _ in range(3))
    k = np.broadcast_to(np.eye(n), (1, 2, n, n)).copy()
    scale = 0.5
    dQ = oracle.attention_backward(q, k, v, do, scale, False)[0]
    b_fp32_p = oracle.backward_error_bound(q, k, v, do, scale, False, u=u, u_p=0.0)[0]
    b_rounded_p = oracle.backward_error_bound(q, k, v, do, scale, False, u=u)[0]
    rounded = np.abs(_simulated_pass(q, k, v, do, scale, False, dtype, True)["dQ"] - dQ)
    fp32 = np.abs(_simulated_pass(q, k, v, do, scale, False, dtype, False)["dQ"] - dQ)
    assert np.any(rounded > b_fp32_p * (1 + 1e-6))
    assert np.all(rounded <= b_rounded_p * (1 + 1e-9) + 1e-13)
    assert np.all(fp32 <= b_fp32_p * (1 + 1e-9) + 1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_backward_is_the_full_one_restricted(causal):
    """The sampled oracle used at full size returns exactly the chosen rows
    and columns of the (torch-pinned) full gradients and bounds."""
    q, k, v, do = (_randn(1500 + t, 2, 3, 41, 16) for t in range(4))
    full = oracle.attention_backward(q, k, v, do, 0.4, causal)
    bounds = oracle.backward_error_bound(q, k, v, do, 0.4, causal, u=2.0 ** -8)
    rows, cols = np.array([0, 5, 17, 40]), np.array([1, 2, 33, 40, 39])
    got = oracle.attention_backward_sampled(q, k, v, do, 0.4, causal, [(0, 0), (1, 2), (0, 1)],
                                            rows, cols, u=2.0 ** -8)
    for (b, h), (dq, dk, dv, bq, bk, bv) in got.items():
        np.testing.assert_allclose(dq, full[0][b, h][rows], rtol=0, atol=1e-12)
        np.testing.assert_allclose(dk, full[1][b, h][cols], rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv, full[2][b, h][cols], rtol=0, atol=1e-12)
        np.testing.assert_allclose(bq, bounds[0][b, h][rows], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(bk, bounds[1][b, h][cols], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(bv, bounds[2][b, h][cols], rtol=1e-12, atol=1e-15)
