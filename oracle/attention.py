"""fp64 CPU oracle for the exact attention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package: only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
kernels or their host library; the only thing both sides share is the seeded
input generator in ``io_aware_tiled_08_amd/workloads.py``, which holds none of
the attention arithmetic.

What it computes (sources: the explainer pages on FlashAttention):

* ``attention_forward`` is the plain definition of standard attention as the
  "FlashAttention" chapter (Chapter 15, vizuara) lays it out in its section
  "Standard vs Flash Attention": form every score of a row, take the softmax
  over the row, multiply the probabilities by V.  FlashAttention reaches this
  same result exactly (same chapter, "Key Takeaways": online softmax gives the
  exact answer, not an approximation), so the definition is the oracle.  It
  materialises the scores in fp64 (one block of rows at a time to bound host
  memory) and runs a two-pass softmax: first the row maximum and the sum of
  exponentials, then the normalised probabilities.
* ``streaming_attention`` is the tile-by-tile online softmax of "FlashAttention,
  Playable", EP 04 "The softmax puzzle", with the loop of the chapter's section
  "The Tiling Strategy": walk the keys one tile at a time, keep a running
  maximum m and running sum l per query row, and whenever a tile raises the
  maximum, scale everything accumulated so far by exp(m_old - m_new).  With
  ``rescale=False`` it is that episode's failing streamer, which updates m but
  never rescales; it exists only so the tests can show that a mistake of that
  kind is caught.

Readings where the pages are silent (each is restated in the test that pins
it):

* layout: Q, K, V are [B, H, N, d]; O is [B, H, N, d]; LSE is [B, H, N];
* the scale is an explicit argument, applied to Q K^T; the library receives it
  as a float32, so the oracle uses float64(float32(scale)) as well;
* causal means query i sees key j iff j <= i (square, diagonal included); the
  pages never treat masking;
* LSE is the natural-log log-sum-exp of the scaled, masked scores of a row;
* inputs are upcast exactly to float64 (fp16, bf16 and fp32 all embed in it).

Parity pins (tests/test_oracle.py, tests/test_oracle_mutants.py): a cross-check
against torch's scaled_dot_product_attention run on the CPU in float64, closed
forms (constant V, identical keys, zero queries, one dominant key, single key,
hand-derived two-key examples in tests/golden/), invariants (affine in V,
permutations, shift of every key), pure-Python brute force for LSE on tiny
inputs, and agreement of ``streaming_attention`` with ``attention_forward`` to
1e-12.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np


def as_f64(x) -> np.ndarray:
    """Exact upcast of a torch tensor or numpy array to a float64 ndarray."""
    if hasattr(x, "detach"):  # torch tensor (handles bfloat16, which numpy lacks)
        import torch
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def boundary_scale(scale: float) -> float:
    """The scale as the kernel sees it: rounded to float32, then widened."""
    return float(np.float64(np.float32(scale)))


def _row_index(rows, B: int, H: int, N: int) -> np.ndarray:
    if rows is None:
        return np.broadcast_to(np.arange(N, dtype=np.int64), (B, H, N))
    rows = np.asarray(rows, dtype=np.int64)
    if rows.ndim == 1:
        rows = np.broadcast_to(rows, (B, H, rows.shape[0]))
    if rows.shape[:2] != (B, H):
        raise ValueError("rows must be [R] or [B, H, R]")
    if rows.size and (rows.min() < 0 or rows.max() >= N):
        raise ValueError("row index out of range")
    return rows


def attention_forward(q, k, v, scale: float, causal: bool = False,
                      rows=None, row_block: int = 128
                      ) -> Tuple[np.ndarray, np.ndarray]:
    """Exact attention forward in float64.

    Returns ``(O, LSE)``: O is [B, H, R, d] and LSE is [B, H, R], where R = N
    when ``rows`` is None, else the number of requested query rows (``rows`` is
    [R], shared by all heads, or [B, H, R]).

    Steps per (b, h) and per block of query rows, following the standard
    attention pipeline of the chapter's "Standard vs Flash Attention" section:
      1. S = scale * Q K^T, every score of the block materialised;
      2. causal: S[i, j] = -inf for j > i;
      3. pass 1: m = max_j S[i, j] and l = sum_j exp(S[i, j] - m);
      4. pass 2: P = exp(S - m) / l;
      5. O = P V;  LSE = m + ln l.
    """
    Q, K, V = as_f64(q), as_f64(k), as_f64(v)
    if Q.ndim != 4 or K.shape != Q.shape or V.shape != Q.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    B, H, N, d = Q.shape
    s64 = boundary_scale(scale)
    idx_all = _row_index(rows, B, H, N)
    R = idx_all.shape[-1]
    O = np.zeros((B, H, R, d), dtype=np.float64)
    LSE = np.zeros((B, H, R), dtype=np.float64)
    if R == 0 or N == 0:
        return O, LSE
    for b in range(B):
        for h in range(H):
            for r0 in range(0, R, row_block):
                idx = np.asarray(idx_all[b, h, r0:r0 + row_block])
                # A causal row i sees keys 0..i only, so the block never needs
                # keys past its largest row.
                nk = int(idx.max()) + 1 if causal else N
                S = (Q[b, h, idx] @ K[b, h, :nk].T) * s64
                if causal:
                    S[np.arange(nk)[None, :] > idx[:, None]] = -np.inf
                m = S.max(axis=1, keepdims=True)
                E = np.exp(S - m)
                l = E.sum(axis=1, keepdims=True)
                P = E / l
                O[b, h, r0:r0 + len(idx)] = P @ V[b, h, :nk]
                LSE[b, h, r0:r0 + len(idx)] = m[:, 0] + np.log(l[:, 0])
    return O, LSE


def streaming_attention(q, k, v, scale: float, causal: bool = False,
                        tile: int = 64, rescale: bool = True,
                        rows: Optional[np.ndarray] = None
                        ) -> Tuple[np.ndarray, np.ndarray]:
    """Tile-by-tile online softmax, one query row at a time, in float64.

    Meant for tiny inputs: the loop over rows and tiles is plain Python.
    For each row: m = -inf, l = 0, acc = 0; for each tile of ``tile`` keys,
    take the tile's scores and their maximum t; if t > m, scale l and acc by
    exp(m - t) (skipped when ``rescale`` is False) and set m = t; then add
    exp(s_j - m) to l and exp(s_j - m) * v_j to acc.  Finally O = acc / l and
    LSE = m + ln l.  Keys a causal row may not see are left out of its tiles.
    """
    if tile < 1:
        raise ValueError("tile must be >= 1")
    Q, K, V = as_f64(q), as_f64(k), as_f64(v)
    B, H, N, d = Q.shape
    s64 = boundary_scale(scale)
    idx_all = _row_index(rows, B, H, N)
    R = idx_all.shape[-1]
    O = np.zeros((B, H, R, d), dtype=np.float64)
    LSE = np.zeros((B, H, R), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r, i in enumerate(idx_all[b, h]):
                i = int(i)
                n_visible = i + 1 if causal else N
                m = -math.inf
                l = 0.0
                acc = np.zeros(d, dtype=np.float64)
                for t0 in range(0, n_visible, tile):
                    t1 = min(t0 + tile, n_visible)
                    s = [s64 * float(np.dot(Q[b, h, i], K[b, h, j]))
                         for j in range(t0, t1)]
                    t_max = max(s)
                    if t_max > m:
                        if rescale:
                            alpha = math.exp(m - t_max)  # 0.0 on the first tile
                            l *= alpha
                            acc *= alpha
                        m = t_max
                    for j, sj in zip(range(t0, t1), s):
                        p = math.exp(sj - m)
                        l += p
                        acc += p * V[b, h, j]
                O[b, h, r] = acc / l
                LSE[b, h, r] = m + math.log(l)
    return O, LSE
