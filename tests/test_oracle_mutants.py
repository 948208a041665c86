"""Plant one plausible mistake at a time in a copy of the oracle's arithmetic
and require the pin suite to catch every one of them.  The mistakes live here,
on the CPU, never in the product code."""
import numpy as np
import pytest

from oracle_pins import ALL_PINS


def _mutant_forward(mistake):
    def fwd(q, k, v, scale, causal, rows=None):
        Q, K, V = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, H, N, d = Q.shape
        s64 = float(np.float32(scale))
        if mistake == "scale_dropped":
            s64 = 1.0
        if mistake == "scale_squared":
            s64 = s64 * s64
        if rows is None:
            idx_all = np.broadcast_to(np.arange(N), (B, H, N))
        else:
            rows = np.asarray(rows)
            idx_all = np.broadcast_to(rows, (B, H, rows.shape[-1])) \
                if rows.ndim == 1 else rows
        if mistake == "row_offset" and rows is not None:
            idx_all = np.minimum(idx_all + 1, N - 1)
        R = idx_all.shape[-1]
        O = np.zeros((B, H, R, d))
        L = np.zeros((B, H, R))
        for b in range(B):
            for h in range(H):
                idx = idx_all[b, h]
                Kb = K[b, h]
                if mistake == "keys_reversed":
                    Kb = Kb[::-1]
                S = Q[b, h, idx] @ Kb.T * s64
                if mistake == "transposed_scores":
                    S = (Kb @ Q[b, h].T * s64)[idx, :]  # S[i, j] = k_i . q_j
                if causal:
                    j = np.arange(N)[None, :]
                    i = idx[:, None]
                    if mistake == "causal_excludes_diagonal":
                        mask = j >= i
                        mask[:, 0] = False
                    elif mistake == "causal_upper":
                        mask = j < i
                    elif mistake == "causal_off_by_one":
                        mask = j > i + 1
                    else:
                        mask = j > i
                    S = np.where(mask, -np.inf, S)
                m = S.max(axis=1, keepdims=True)
                E = np.exp(S - m)
                if mistake == "softmax_over_queries":
                    E = np.exp(S - S.max(axis=0, keepdims=True))
                    E = np.where(np.isfinite(E), E, 0.0)
                    l = E.sum(axis=0, keepdims=True)
                    P = E / l
                    l = E.sum(axis=1, keepdims=True)
                else:
                    l = E.sum(axis=1, keepdims=True)
                    P = E / l
                if mistake == "no_normalisation":
                    P = E
                Vb = V[b, h]
                if mistake == "v_rows_shifted":
                    Vb = np.roll(Vb, 1, axis=0)
                O[b, h] = P @ Vb
                lse = m[:, 0] + np.log(l[:, 0])
                if mistake == "lse_drops_max":
                    lse = np.log(l[:, 0])
                if mistake == "lse_log2":
                    lse = m[:, 0] + np.log2(l[:, 0])
                if mistake == "lse_unscaled":
                    lse = lse / s64 if s64 != 0 else lse
                L[b, h] = lse
        return O, L
    return fwd


MISTAKES = ["scale_dropped", "scale_squared", "row_offset", "keys_reversed",
            "transposed_scores", "causal_excludes_diagonal", "causal_upper",
            "causal_off_by_one", "softmax_over_queries", "no_normalisation",
            "v_rows_shifted", "lse_drops_max", "lse_log2", "lse_unscaled"]


def test_unmutated_copy_passes():
    fwd = _mutant_forward(None)
    for pin in ALL_PINS:
        pin(fwd)


@pytest.mark.parametrize("mistake", MISTAKES)
def test_pins_catch_planted_mistake(mistake):
    fwd = _mutant_forward(mistake)
    caught = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(fwd)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin detects the planted mistake {mistake!r}"
