"""The fp64 oracle with a key/value cache (K, V longer than Q) and with the
keys split into ranges, pinned against facts that do not come from the code
under test: torch's scaled_dot_product_attention with an explicit mask,
pure-Python brute force, closed forms, and the square case (itself pinned in
test_oracle.py) of which a cache query is one row.

Reading (stated with the oracle): with Nk >= Nq keys the queries are the last
Nq positions of the sequence, so a causal query i sees key j iff
j <= i + (Nk - Nq)."""
import math

import numpy as np
import pytest

import oracle
from oracle_pins import _randn


def _close(name, got, want, tol):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    err = float(np.max(np.abs(got - want))) if got.size else 0.0
    assert err <= tol, f"{name}: max abs error {err:.3e} > {tol:.1e}"


CASES = [(1, 1), (1, 9), (3, 9), (5, 5), (7, 40), (33, 100)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", CASES)
def test_cache_rows_are_rows_of_the_full_sequence(nq, nk, causal):
    """Queries for the last nq positions against all nk keys give exactly the
    last nq rows of square attention over the whole sequence."""
    qf, k, v = (_randn(500 + t, 2, 2, nk, 16) for t in range(3))
    O_full, L_full = oracle.attention_forward(qf, k, v, 0.3, causal)
    O, L = oracle.attention_forward(qf[:, :, nk - nq:], k, v, 0.3, causal)
    _close("O", O, O_full[:, :, nk - nq:], 1e-13)
    _close("LSE", L, L_full[:, :, nk - nq:], 1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", CASES)
def test_cache_against_torch_sdpa(nq, nk, causal):
    torch = pytest.importorskip("torch")
    q = _randn(600, 1, 3, nq, 8)
    k, v = _randn(601, 1, 3, nk, 8), _randn(602, 1, 3, nk, 8)
    scale = 0.7
    mask = None
    if causal:
        i = torch.arange(nq)[:, None]
        j = torch.arange(nk)[None, :]
        mask = j <= i + (nk - nq)  # True = may attend
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=mask, scale=oracle.boundary_scale(scale)).numpy()
    s = torch.matmul(tq, tk.transpose(-1, -2)) * oracle.boundary_scale(scale)
    if mask is not None:
        s = s.masked_fill(~mask, float("-inf"))
    ref_lse = torch.logsumexp(s, dim=-1).numpy()
    O, L = oracle.attention_forward(q, k, v, scale, causal)
    _close("O", O, ref, 1e-12)
    _close("LSE", L, ref_lse, 1e-12)


def test_cache_bruteforce_tiny():
    """Pure-Python scores, max, sums and weighted rows for Nq=2, Nk=5."""
    q, k, v = _randn(700, 1, 1, 2, 3), _randn(701, 1, 1, 5, 3), _randn(702, 1, 1, 5, 3)
    scale = 0.9
    s64 = float(np.float32(scale))
    for causal in (False, True):
        O, L = oracle.attention_forward(q, k, v, scale, causal)
        for i in range(2):
            n_vis = i + 1 + 3 if causal else 5
            sc = [s64 * sum(q[0, 0, i, t] * k[0, 0, j, t] for t in range(3)) for j in range(n_vis)]
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            tot = sum(w)
            for c in range(3):
                want = sum(w[j] * v[0, 0, j, c] for j in range(n_vis)) / tot
                assert abs(O[0, 0, i, c] - want) <= 1e-13
            assert abs(L[0, 0, i] - (mx + math.log(tot))) <= 1e-13


def test_cache_identical_keys_average_visible_values():
    """All keys equal: every visible key gets the same weight, so O is the
    mean of the visible V rows and LSE = s + ln(visible count)."""
    nq, nk, d = 3, 7, 4
    q = _randn(800, 1, 1, nq, d)
    k = np.broadcast_to(_randn(801, 1, 1, 1, d), (1, 1, nk, d)).copy()
    v = _randn(802, 1, 1, nk, d)
    O, L = oracle.attention_forward(q, k, v, 0.5, True)
    s64 = float(np.float32(0.5))
    for i in range(nq):
        n_vis = i + 1 + (nk - nq)
        _close(f"O[{i}]", O[0, 0, i], v[0, 0, :n_vis].mean(axis=0), 1e-14)
        s = s64 * float(q[0, 0, i] @ k[0, 0, 0])
        assert abs(L[0, 0, i] - (s + math.log(n_vis))) <= 1e-13


def test_single_cached_key():
    q, k, v = _randn(810, 1, 2, 1, 8), _randn(811, 1, 2, 1, 8), _randn(812, 1, 2, 1, 8)
    for causal in (False, True):
        O, L = oracle.attention_forward(q, k, v, 1.3, causal)
        _close("O", O, v, 0.0)
        want = float(np.float32(1.3)) * np.einsum("bhqd,bhkd->bhq", q, k)
        _close("LSE", L, want, 1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tile", [1, 4, 1000])
def test_streaming_with_cache_equals_two_pass(tile, causal):
    q, k, v = _randn(900, 1, 2, 6, 8), _randn(901, 1, 2, 23, 8), _randn(902, 1, 2, 23, 8)
    O1, L1 = oracle.attention_forward(q, k, v, 0.6, causal)
    O2, L2 = oracle.streaming_attention(q, k, v, 0.6, causal, tile=tile)
    _close("O", O2, O1, 1e-12)
    _close("LSE", L2, L1, 1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bounds", [[0, 50], [0, 1, 50], [0, 17, 18, 33, 50], [0, 0, 25, 50, 50]])
def test_split_ranges_merge_to_the_whole(bounds, causal):
    q, k, v = _randn(910, 1, 2, 9, 8), _randn(911, 1, 2, 50, 8), _randn(912, 1, 2, 50, 8)
    O1, L1 = oracle.attention_forward(q, k, v, 0.8, causal)
    O2, L2 = oracle.split_attention(q, k, v, 0.8, causal, bounds)
    _close("O", O2, O1, 1e-12)
    _close("LSE", L2, L1, 1e-12)


def test_partial_range_nobody_sees():
    """Causal rows see no key beyond i + Nk - Nq: a range past every row's
    last key gives LSE = -inf and O = 0, and merging it changes nothing."""
    q, k, v = _randn(920, 1, 1, 4, 8), _randn(921, 1, 1, 10, 8), _randn(922, 1, 1, 10, 8)
    # rows see keys up to 6, 7, 8, 9: keys 9..9 are seen by the last row only
    O, L = oracle.attention_partial(q, k, v, 0.5, True, 9, 10)
    assert np.all(np.isneginf(L[0, 0, :3])) and np.all(O[0, 0, :3] == 0.0)
    assert np.isfinite(L[0, 0, 3])
    whole = oracle.attention_forward(q, k, v, 0.5, True)
    merged = oracle.merge_partials([oracle.attention_partial(q, k, v, 0.5, True, 0, 9), (O, L)])
    _close("O", merged[0], whole[0], 1e-12)
    _close("LSE", merged[1], whole[1], 1e-12)


def test_merge_without_rescale_is_wrong():
    """Adding the ranges' normalised outputs with equal weights (no rescale by
    exp(LSE_s - M)) is a mistake the merge must not make: it differs from the
    whole by far more than rounding."""
    q, k = _randn(930, 1, 1, 8, 8), _randn(931, 1, 1, 40, 8) * 3.0
    v = _randn(932, 1, 1, 40, 8)
    parts = [oracle.attention_partial(q, k, v, 0.5, False, lo, hi) for lo, hi in ((0, 20), (20, 40))]
    O_whole, _ = oracle.attention_forward(q, k, v, 0.5, False)
    O_good, _ = oracle.merge_partials(parts)
    O_bad = (parts[0][0] + parts[1][0]) / 2
    _close("good", O_good, O_whole, 1e-12)
    assert np.max(np.abs(O_bad - O_whole)) > 1e-2


def test_cache_shape_errors():
    q, k = np.zeros((1, 1, 4, 8)), np.zeros((1, 1, 3, 8))
    with pytest.raises(ValueError):
        oracle.attention_forward(q, k, k, 1.0, True)  # fewer keys than causal queries
    with pytest.raises(ValueError):
        oracle.attention_forward(q, np.zeros((1, 1, 0, 8)), np.zeros((1, 1, 0, 8)), 1.0, False)
    with pytest.raises(ValueError):
        oracle.attention_forward(q, np.zeros((1, 2, 4, 8)), np.zeros((1, 2, 4, 8)), 1.0, False)


# Planted mistakes in the causal alignment of a cache query: each must fail
# one of the pins above (run here against a copy of the rule, on the CPU).
def _misaligned_forward(shift):
    def fwd(q, k, v, scale, causal):
        Q, K, V = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        nq, nk = Q.shape[2], K.shape[2]
        off = (nk - nq) + shift if shift != "top_left" else 0
        S = np.einsum("bhqd,bhkd->bhqk", Q, K) * float(np.float32(scale))
        if causal:
            S = np.where(np.arange(nk)[None, :] > np.arange(nq)[:, None] + off, -np.inf, S)
        m = S.max(-1, keepdims=True)
        E = np.exp(S - m)
        l = E.sum(-1, keepdims=True)
        return E / l @ V, (m + np.log(l))[..., 0]
    return fwd


@pytest.mark.parametrize("shift", ["top_left", 1, -1])
def test_pins_catch_misaligned_cache_mask(shift):
    fwd = _misaligned_forward(shift)
    q = _randn(940, 1, 2, 3, 8)
    k, v = _randn(941, 1, 2, 9, 8), _randn(942, 1, 2, 9, 8)
    O_ok, _ = oracle.attention_forward(q, k, v, 0.7, True)
    with np.errstate(all="ignore"):
        O_bad, _ = fwd(q, k, v, 0.7, True)
    # the suffix-of-square pin, restated for the mutant
    qf = _randn(943, 1, 2, 9, 8)
    O_full, _ = oracle.attention_forward(qf, k, v, 0.7, True)
    with np.errstate(all="ignore"):
        O_mut, _ = fwd(qf[:, :, 6:], k, v, 0.7, True)
    assert not np.allclose(O_mut, O_full[:, :, 6:], atol=1e-6, equal_nan=False)
    assert not np.allclose(O_bad, O_ok, atol=1e-6, equal_nan=False)
