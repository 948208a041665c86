"""Checks that pin an attention-forward implementation to facts fixed by
mathematics, by a library routine or by hand derivation -- never by itself.

Every ``pin_*`` takes ``fwd(q, k, v, scale, causal, rows=None) -> (O, LSE)``
working on [B, H, N, d] float64 arrays and raises AssertionError when the
implementation disagrees.  tests/test_oracle.py runs them on the oracle;
tests/test_oracle_mutants.py runs them on copies of it with one planted
mistake each and requires every copy to fail at least one pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TIGHT = 1e-12


def _rng(seed):
    return np.random.default_rng([20251, seed])


def _randn(seed, *shape):
    return _rng(seed).standard_normal(shape)


def _visible_counts(N, causal):
    return np.arange(1, N + 1) if causal else np.full(N, N)


def _check(name, got, want, tol):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{name}: shape {got.shape} != {want.shape}"
    err = float(np.max(np.abs(got - want))) if got.size else 0.0
    assert err <= tol, f"{name}: max abs error {err:.3e} > {tol:.1e}"
    return err


# --- library routine --------------------------------------------------------

def pin_sdpa_fp64(fwd):
    """torch's scaled_dot_product_attention (an independent implementation),
    run on the CPU in float64, with its own causal mask."""
    for seed, (B, H, N, d) in enumerate([(1, 1, 1, 8), (2, 3, 5, 8),
                                         (1, 2, 64, 32), (1, 1, 129, 64),
                                         (2, 1, 200, 16)]):
        q, k, v = (_randn(10 * seed + t, B, H, N, d) for t in range(3))
        scale = 1.0 / math.sqrt(d)
        for causal in (False, True):
            O, _ = fwd(q, k, v, scale, causal)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                is_causal=causal,
                scale=float(np.float32(scale))).numpy()
            _check(f"sdpa N={N} causal={causal}", O, ref, TIGHT)


# --- brute force on tiny inputs --------------------------------------------

def _bruteforce_row(qrow, K, V, scale, n_visible):
    """Pure-Python exact-as-possible attention for one query row."""
    s = [scale * math.fsum(a * b for a, b in zip(qrow, K[j]))
         for j in range(n_visible)]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    l = math.fsum(w)
    out = [math.fsum(w[j] * V[j][c] for j in range(n_visible)) / l
           for c in range(len(V[0]))]
    return out, m + math.log(l)


def pin_bruteforce_tiny(fwd):
    """Both outputs against pure-Python loops (math.fsum) on tiny heads."""
    for seed, (N, d) in enumerate([(1, 1), (2, 3), (7, 4), (16, 5)]):
        q, k, v = (_randn(100 + 3 * seed + t, 1, 1, N, d) for t in range(3))
        scale = float(np.float32(0.7))
        for causal in (False, True):
            O, L = fwd(q, k, v, scale, causal)
            Kl, Vl = k[0, 0].tolist(), v[0, 0].tolist()
            for i in range(N):
                o_ref, l_ref = _bruteforce_row(q[0, 0, i].tolist(), Kl, Vl,
                                               scale, i + 1 if causal else N)
                _check(f"brute O row {i}", O[0, 0, i], o_ref, TIGHT)
                _check(f"brute LSE row {i}", L[0, 0, i], l_ref, TIGHT)


# --- closed forms ------------------------------------------------------------

def pin_constant_v(fwd):
    """Softmax rows sum to one, so a constant V comes back unchanged."""
    B, H, N, d = 2, 2, 70, 8
    q, k = _randn(200, B, H, N, d), _randn(201, B, H, N, d)
    for causal in (False, True):
        for c in (1.0, -2.5):
            v = np.full((B, H, N, d), c)
            O, _ = fwd(q, k, v, 0.3, causal)
            _check("constant V", O, v, 1e-13)


def pin_identical_keys(fwd):
    """All keys equal: every visible score of a row is the same, so the
    weights are uniform, O_i is the mean of the visible V rows and
    LSE_i = scale*q_i.k + ln(n_i)."""
    B, H, N, d = 1, 2, 33, 6
    q, v = _randn(210, B, H, N, d), _randn(211, B, H, N, d)
    k = np.broadcast_to(_randn(212, B, H, 1, d), (B, H, N, d)).copy()
    scale = 0.375
    for causal in (False, True):
        O, L = fwd(q, k, v, scale, causal)
        n = _visible_counts(N, causal)
        mean_v = np.cumsum(v, axis=2) / n[:, None] if causal else \
            np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
        _check("identical keys O", O, mean_v, TIGHT)
        s = scale * np.einsum("bhnd,bhd->bhn", q, k[:, :, 0])
        _check("identical keys LSE", L, s + np.log(n), TIGHT)


def pin_zero_queries(fwd):
    """Q = 0: every score is 0, weights uniform, LSE_i = ln(n_i)."""
    B, H, N, d = 1, 1, 45, 4
    k, v = _randn(220, B, H, N, d), _randn(221, B, H, N, d)
    q = np.zeros((B, H, N, d))
    for causal in (False, True):
        O, L = fwd(q, k, v, 1.7, causal)
        n = _visible_counts(N, causal)
        mean_v = np.cumsum(v, axis=2) / n[:, None] if causal else \
            np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
        _check("zero Q O", O, mean_v, TIGHT)
        _check("zero Q LSE", L, np.broadcast_to(np.log(n), L.shape), TIGHT)


def pin_single_key(fwd):
    """N = 1: the only weight is 1, so O = V and LSE = scale*q.k."""
    q, k, v = (_randn(230 + t, 3, 2, 1, 16) for t in range(3))
    for causal in (False, True):
        O, L = fwd(q, k, v, 0.25, causal)
        _check("N=1 O", O, v, 0.0)
        _check("N=1 LSE", L, 0.25 * np.sum(q * k, axis=-1), TIGHT)


def pin_dominant_key(fwd):
    """One key beats every other score of its row by a gap g >= 40: O equals
    that key's V row to within 2*(N-1)*exp(-g)*max|V| (here ~1e-15)."""
    N, d = 40, 8
    rng = _rng(240)
    q = np.zeros((1, 1, N, d))
    q[0, 0, :, 0] = 1.0
    k = rng.uniform(-1, 1, size=(1, 1, N, d))
    k[0, 0, :, 0] = rng.uniform(-1.0, 1.0, size=N)
    star = 17
    k[0, 0, star, 0] = 50.0
    v = _randn(241, 1, 1, N, d)
    O, L = fwd(q, k, v, 1.0, False)
    bound = 2 * (N - 1) * math.exp(-48.0) * np.abs(v).max() + 1e-15
    _check("dominant key O", O[0, 0], np.broadcast_to(v[0, 0, star], (N, d)), bound)
    _check("dominant key LSE", L[0, 0], np.full(N, 50.0), 1e-12)


def pin_hand_examples(fwd):
    """Closed forms derived by hand (tests/golden/hand_examples.json)."""
    with open(os.path.join(GOLDEN, "hand_examples.json")) as f:
        data = json.load(f)
    env = {name: getattr(math, name) for name in ("e", "log", "exp", "sqrt")}
    for ex in data["examples"]:
        q, k, v = (np.asarray(ex[t], dtype=np.float64)[None, None]
                   for t in ("q", "k", "v"))
        O, L = fwd(q, k, v, ex["scale"], ex["causal"])
        want_o = [[eval(e, {"__builtins__": {}}, env) for e in row]
                  for row in ex["O"]]
        want_l = [eval(e, {"__builtins__": {}}, env) for e in ex["LSE"]]
        _check(ex["name"] + " O", O[0, 0], want_o, TIGHT)
        _check(ex["name"] + " LSE", L[0, 0], want_l, TIGHT)


# --- invariants --------------------------------------------------------------

def pin_affine_in_v(fwd):
    """O(a*V + b) = a*O(V) + b for any scalar a and vector b."""
    B, H, N, d = 1, 2, 50, 6
    q, k, v = (_randn(250 + t, B, H, N, d) for t in range(3))
    a, bvec = -1.75, _randn(253, d)
    for causal in (False, True):
        O1, L1 = fwd(q, k, v, 0.4, causal)
        O2, L2 = fwd(q, k, a * v + bvec, 0.4, causal)
        _check("affine V", O2, a * O1 + bvec, 1e-12)
        _check("affine V LSE", L2, L1, 0.0)


def pin_permutations(fwd):
    """Unmasked: permuting K and V rows together changes nothing; permuting Q
    rows permutes O and LSE rows the same way."""
    B, H, N, d = 1, 1, 37, 5
    q, k, v = (_randn(260 + t, B, H, N, d) for t in range(3))
    O, L = fwd(q, k, v, 0.6, False)
    perm = _rng(263).permutation(N)
    O2, L2 = fwd(q, k[:, :, perm], v[:, :, perm], 0.6, False)
    _check("key permutation O", O2, O, 1e-13)
    _check("key permutation LSE", L2, L, 1e-13)
    O3, L3 = fwd(q[:, :, perm], k, v, 0.6, False)
    _check("query permutation O", O3, O[:, :, perm], 1e-13)
    _check("query permutation LSE", L3, L[:, :, perm], 1e-13)


def pin_key_shift(fwd):
    """Adding one vector c to every key adds scale*q_i.c to every score of
    row i: O is unchanged and LSE_i moves by exactly that amount."""
    B, H, N, d = 1, 2, 41, 7
    q, k, v = (_randn(270 + t, B, H, N, d) for t in range(3))
    c = _randn(273, d)
    for causal in (False, True):
        O1, L1 = fwd(q, k, v, 0.5, causal)
        O2, L2 = fwd(q, k + c, v, 0.5, causal)
        _check("key shift O", O2, O1, 1e-12)
        _check("key shift LSE", L2, L1 + 0.5 * (q @ c), 1e-12)


def pin_row_sampling(fwd):
    """Asking for a subset of rows returns exactly those rows of the full
    result."""
    B, H, N, d = 2, 2, 90, 8
    q, k, v = (_randn(280 + t, B, H, N, d) for t in range(3))
    rows = np.stack([np.stack([np.sort(_rng(283 + 2 * b + h).choice(N, 11, False))
                               for h in range(H)]) for b in range(B)])
    for causal in (False, True):
        O, L = fwd(q, k, v, 0.3, causal)
        Os, Ls = fwd(q, k, v, 0.3, causal, rows=rows)
        _check("sampled rows O", Os, np.take_along_axis(O, rows[..., None], 2), 1e-13)
        _check("sampled rows LSE", Ls, np.take_along_axis(L, rows, 2), 1e-13)


ALL_PINS = [pin_sdpa_fp64, pin_bruteforce_tiny, pin_constant_v,
            pin_identical_keys, pin_zero_queries, pin_single_key,
            pin_dominant_key, pin_hand_examples, pin_affine_in_v,
            pin_permutations, pin_key_shift, pin_row_sampling]
