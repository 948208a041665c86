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
* ``attention_partial`` is the same definition restricted to a range of keys;
  a row that sees no key of the range gets LSE = -inf and O = 0.  It is the
  building block of ``split_attention``.
* ``merge_partials`` combines results computed over disjoint key ranges with
  the rescaling rule of EP 04 applied once per range instead of once per tile:
  with M the largest of the ranges' LSE values, each range's normalised output
  is weighted by exp(LSE_s - M), the weights are summed, and LSE = M + ln of
  that sum.  ``split_attention`` = ``attention_partial`` over each range, then
  ``merge_partials``.

Readings where the pages are silent (each is restated in the test that pins
it):

* layout: Q, K, V are [B, H, N, d]; O is [B, H, N, d]; LSE is [B, H, N];
* the scale is an explicit argument, applied to Q K^T; the library receives it
  as a float32, so the oracle uses float64(float32(scale)) as well;
* causal means query i sees key j iff j <= i (square, diagonal included); the
  pages never treat masking;
* K and V may be longer than Q (Nk >= Nq rows): the key/value cache of the
  "KV Cache: Why Generation Speeds Up" card among the related diagrams of
  "FlashAttention: Tiled & Fused" (in generation the keys and values
  of earlier tokens are stored and reused; only the newest token's are
  computed).  The Nq queries are then the last Nq
  positions of the sequence, so a causal query i sees key j iff
  j <= i + (Nk - Nq); with Nq = Nk this is the square rule above;
* LSE is the natural-log log-sum-exp of the scaled, masked scores of a row;
* inputs are upcast exactly to float64 (fp16, bf16 and fp32 all embed in it).

Parity pins (tests/test_oracle.py, tests/test_oracle_mutants.py): a cross-check
against torch's scaled_dot_product_attention run on the CPU in float64, closed
forms (constant V, identical keys, zero queries, one dominant key, single key,
hand-derived two-key examples in tests/golden/), invariants (affine in V,
permutations, shift of every key), pure-Python brute force for LSE on tiny
inputs, and agreement of ``streaming_attention`` with ``attention_forward`` to
1e-12.

The later functions carry their derivations in their docstrings and are pinned
in their own files: ``decode_e4m3``, ``dequantize_fp8`` and
``fp8_weight_error_bound`` (tests/test_oracle_fp8.py: every e4m3 code against
torch's float8_e4m3fn, fixed values, simulated weight rounding inside the
bound); ``weight_rounding_error_bound`` with 16-bit parameters and
``forward_error_bound_16`` (tests/test_oracle_bound16.py: a float64 simulation
of the 16-bit roundings stays inside the bound and reaches a good part of it);
``attention_backward`` and
``backward_error_bound`` (tests/test_oracle_backward.py: torch autograd and
SDPA in float64, central finite differences of ``attention_forward``,
invariants, planted mistakes, simulated 16-bit rounding inside the bound);
``attention_backward_sampled`` (the same file: equal to the full backward and
bound at the chosen rows and columns).
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


def _shapes(Q, K, V):
    if Q.ndim != 4 or K.ndim != 4 or V.shape != K.shape or K.shape[:2] != Q.shape[:2] \
            or K.shape[3] != Q.shape[3]:
        raise ValueError("q must be [B, H, Nq, d] and k, v one [B, H, Nk, d] shape")
    B, H, Nq, d = Q.shape
    return B, H, Nq, K.shape[2], d


def causal_offset(Nq: int, Nk: int) -> int:
    """Position of query 0 in the key sequence: the queries are its last Nq
    positions (key/value cache reading).  Causal query i sees keys
    j <= i + causal_offset(Nq, Nk)."""
    if Nk < Nq:
        raise ValueError("causal attention needs at least as many keys as queries")
    return Nk - Nq


def attention_partial(q, k, v, scale: float, causal: bool = False,
                      k_begin: int = 0, k_end: Optional[int] = None,
                      rows=None, row_block: int = 128
                      ) -> Tuple[np.ndarray, np.ndarray]:
    """Exact attention of each query row over the keys k_begin <= j < k_end,
    in float64.

    Returns ``(O, LSE)``: O is [B, H, R, d] and LSE is [B, H, R], where R = Nq
    when ``rows`` is None, else the number of requested query rows (``rows`` is
    [R], shared by all heads, or [B, H, R]).  A row that sees none of the keys
    gets O = 0 and LSE = -inf.

    Steps per (b, h) and per block of query rows, following the standard
    attention pipeline of the chapter's "Standard vs Flash Attention" section:
      1. S = scale * Q K^T over the key range, every score materialised;
      2. causal: S[i, j] = -inf for j > i + (Nk - Nq);
      3. pass 1: m = max_j S[i, j] and l = sum_j exp(S[i, j] - m);
      4. pass 2: P = exp(S - m) / l;
      5. O = P V;  LSE = m + ln l.
    """
    Q, K, V = as_f64(q), as_f64(k), as_f64(v)
    B, H, Nq, Nk, d = _shapes(Q, K, V)
    off = causal_offset(Nq, Nk) if causal else 0
    lo = max(0, int(k_begin))
    hi = Nk if k_end is None else min(Nk, int(k_end))
    s64 = boundary_scale(scale)
    idx_all = _row_index(rows, B, H, Nq)
    R = idx_all.shape[-1]
    O = np.zeros((B, H, R, d), dtype=np.float64)
    LSE = np.full((B, H, R), -np.inf, dtype=np.float64)
    if R == 0:
        return O, LSE
    for b in range(B):
        for h in range(H):
            for r0 in range(0, R, row_block):
                idx = np.asarray(idx_all[b, h, r0:r0 + row_block])
                # A causal row i sees keys up to i + off only, so the block
                # never needs keys past its largest row's last one.
                top = min(hi, int(idx.max()) + 1 + off) if causal else hi
                if top <= lo:
                    continue
                S = (Q[b, h, idx] @ K[b, h, lo:top].T) * s64
                if causal:
                    S[np.arange(lo, top)[None, :] > idx[:, None] + off] = -np.inf
                m = S.max(axis=1, keepdims=True)
                seen = np.isfinite(m)
                E = np.exp(S - np.where(seen, m, 0.0))
                l = E.sum(axis=1, keepdims=True)
                P = E / np.where(seen, l, 1.0)
                O[b, h, r0:r0 + len(idx)] = P @ V[b, h, lo:top]
                with np.errstate(divide="ignore"):
                    LSE[b, h, r0:r0 + len(idx)] = np.where(
                        seen[:, 0], m[:, 0] + np.log(l[:, 0]), -np.inf)
    return O, LSE


def attention_forward(q, k, v, scale: float, causal: bool = False,
                      rows=None, row_block: int = 128
                      ) -> Tuple[np.ndarray, np.ndarray]:
    """Exact attention forward in float64: ``attention_partial`` over every
    key.  Every query row must see at least one key."""
    O, LSE = attention_partial(q, k, v, scale, causal, 0, None, rows, row_block)
    if LSE.size and not np.all(np.isfinite(LSE)):
        raise ValueError("a query row sees no key (Nk = 0?)")
    return O, LSE


def merge_partials(parts) -> Tuple[np.ndarray, np.ndarray]:
    """Combine (O_s, LSE_s) computed over disjoint key ranges.

    The rescaling rule of the online softmax, once per range: M = max_s LSE_s,
    w_s = exp(LSE_s - M) (0 for a range the row never saw), O = sum_s w_s O_s /
    sum_s w_s, LSE = M + ln sum_s w_s.  Every row must have seen some range.
    """
    parts = list(parts)
    if not parts:
        raise ValueError("nothing to merge")
    Ls = np.stack([np.asarray(p[1], dtype=np.float64) for p in parts])
    Os = np.stack([np.asarray(p[0], dtype=np.float64) for p in parts])
    M = Ls.max(axis=0)
    if Ls[0].size and not np.all(np.isfinite(M)):
        raise ValueError("a query row saw no key in any part")
    w = np.exp(Ls - M)
    wsum = w.sum(axis=0)
    O = (w[..., None] * Os).sum(axis=0) / wsum[..., None]
    return O, M + np.log(wsum)


def split_attention(q, k, v, scale: float, causal: bool = False, bounds=None,
                    rows=None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention over the key ranges [bounds[s], bounds[s+1]) separately, then
    merged: the split-key form of the same result."""
    Nk = as_f64(k).shape[2]
    b = [0, Nk] if bounds is None else [int(x) for x in bounds]
    if b[0] != 0 or b[-1] != Nk or any(x > y for x, y in zip(b, b[1:])):
        raise ValueError("bounds must rise from 0 to Nk")
    return merge_partials(attention_partial(q, k, v, scale, causal, lo, hi, rows)
                          for lo, hi in zip(b, b[1:]))


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
    LSE = m + ln l.  Keys a causal row may not see (j > i + Nk - Nq) are left
    out of its tiles.
    """
    if tile < 1:
        raise ValueError("tile must be >= 1")
    Q, K, V = as_f64(q), as_f64(k), as_f64(v)
    B, H, Nq, Nk, d = _shapes(Q, K, V)
    off = causal_offset(Nq, Nk) if causal else 0
    s64 = boundary_scale(scale)
    idx_all = _row_index(rows, B, H, Nq)
    R = idx_all.shape[-1]
    O = np.zeros((B, H, R, d), dtype=np.float64)
    LSE = np.zeros((B, H, R), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r, i in enumerate(idx_all[b, h]):
                i = int(i)
                n_visible = i + 1 + off if causal else Nk
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


def decode_e4m3(codes) -> np.ndarray:
    """float64 value of each e4m3 code (uint8 array): sign bit 7, exponent bits
    6..3 with bias 7, mantissa bits 2..0; exponent 0 is subnormal
    (m * 2^-9); exponent 15 with mantissa 7 is NaN; no infinities."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((e == 15) & ((c & 7) == 7), np.nan, val)
    return sign * val


def dequantize_fp8(x, descale: float) -> np.ndarray:
    """Exact float64 value of an e4m3 tensor (torch float8_e4m3fn or a uint8
    code array) times float64(float32(descale))."""
    if hasattr(x, "detach"):
        import torch
        x = x.detach().cpu()
        if x.dtype != torch.uint8:
            x = x.view(torch.uint8)
        x = x.numpy()
    return decode_e4m3(x) * float(np.float64(np.float32(descale)))


def fp8_weight_error_bound(q, k, v, scale: float, causal: bool = False, rows=None,
                           u: float = 2.0 ** -4, a: float = 2.0 ** -10
                           ) -> Tuple[np.ndarray, np.ndarray]:
    """``weight_rounding_error_bound`` for weights rounded to e4m3: half a unit
    in the last place is relative 2^-4 in the normal range and absolute 2^-10
    below 2^-6 (subnormals, spacing 2^-9)."""
    return weight_rounding_error_bound(q, k, v, scale, causal, rows, u, a)


# Unit roundoff and half the subnormal spacing of the 16-bit input types, for
# weight_rounding_error_bound: fp16 has an 11-bit significand and subnormal
# spacing 2^-24; bf16 an 8-bit significand and subnormal spacing 2^-133.
ROUNDING_16 = {"f16": (2.0 ** -11, 2.0 ** -25), "bf16": (2.0 ** -8, 2.0 ** -134)}


def weight_rounding_error_bound(q, k, v, scale: float, causal: bool = False, rows=None,
                                u: float = 2.0 ** -4, a: float = 2.0 ** -10
                                ) -> Tuple[np.ndarray, np.ndarray]:
    """Bound on |O_hat - O| (per element) and |LSE_hat - LSE| (per row) for a
    forward pass that computes the scores exactly enough and rounds each
    softmax weight to a narrower type before the P V product and the row sum
    (e4m3 for the 8-bit pass, the input type for the 16-bit pass).

    Derivation.  The pass weights key j by w_j = 2^(c*s_j - m_ref) for a
    reference m_ref in [m_max - 8, m_max], rounds it to nearest-even in the
    narrow type and uses the rounded weights in both sums.  Rounding moves a
    weight by at most half a unit in the last place: relative u in the normal
    range, at most an absolute a among the subnormals.  So
    |w_hat_j - w_j| <= e_j = max(u * w_j, a).  With W = sum w_j and
    E = sum e_j,
        O_hat - O = sum_j (w_hat_j - w_j)(v_j - O) / sum_j w_hat_j
        |O_hat - O| <= sum_j e_j |v_j - O| / (W - E)
        |LSE_hat - LSE| = |ln(sum w_hat / sum w)| <= -ln(1 - E / W).
    The relative part scales with the weights and the absolute part does not,
    so the bound is largest for the smallest scale, m_ref = m_max, where the
    weights are exp(S_j - S_max) <= 1; that is the scale used here.
    Inputs are exact values (float64, already dequantized).
    """
    Q, K, V = as_f64(q), as_f64(k), as_f64(v)
    B, H, Nq, Nk, d = _shapes(Q, K, V)
    off = causal_offset(Nq, Nk) if causal else 0
    s64 = boundary_scale(scale)
    idx_all = _row_index(rows, B, H, Nq)
    R = idx_all.shape[-1]
    bO = np.zeros((B, H, R, d))
    bL = np.zeros((B, H, R))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, R, 128):
                idx = np.asarray(idx_all[b, h, r0:r0 + 128])
                top = min(Nk, int(idx.max()) + 1 + off) if causal else Nk
                S = (Q[b, h, idx] @ K[b, h, :top].T) * s64
                if causal:
                    S[np.arange(top)[None, :] > idx[:, None] + off] = -np.inf
                w = np.exp(S - S.max(axis=1, keepdims=True))
                e = np.where(np.isfinite(S), np.maximum(u * w, a), 0.0)
                W = w.sum(axis=1)
                E = e.sum(axis=1)
                O = (w @ V[b, h, :top]) / W[:, None]
                # sum_j e_j |v_jc - O_c| for every column c
                dev = np.abs(V[b, h, :top][None, :, :] - O[:, None, :])
                bO[b, h, r0:r0 + len(idx)] = np.einsum("rj,rjc->rc", e, dev) / (W - E)[:, None]
                bL[b, h, r0:r0 + len(idx)] = -np.log1p(-E / W)
    return bO, bL


def forward_error_bound_16(q, k, v, scale: float, causal: bool, dtype: str, rows=None
                           ) -> np.ndarray:
    """Per-element bound on |O_hat - O| for a 16-bit forward pass (``dtype``
    "f16" or "bf16"), first order in the unit roundoff u of that type.

    Such a pass multiplies 16-bit inputs exactly and accumulates in fp32, so
    the two roundings it adds on purpose dominate: each softmax weight is
    rounded to the input type before the P V product and the row sum (bounded
    by ``weight_rounding_error_bound`` with that type's u and subnormal floor
    a), and O itself is rounded to the input type when it is stored, which
    moves an element x by at most half its spacing, u * 2^floor(log2 |x|), or
    a below the normal range.  The value rounded is within the first term of
    O, so the spacing is taken at |O| plus that term.  The bound is the sum of
    the two.  For the unit-variance inputs and 1/sqrt(d) scale of the
    benchmark workloads it lies below the fixed tolerances; it exceeds them
    only where large scores make the softmax nearly one-hot and |O| approaches
    the largest |v| of a row (the second term alone is 2e-3 at |O| = 4 in
    fp16).
    """
    u, a = ROUNDING_16[dtype]
    bO, _ = weight_rounding_error_bound(q, k, v, scale, causal, rows, u, a)
    O, _ = attention_forward(q, k, v, scale, causal, rows=rows)
    x = np.abs(O) + bO
    with np.errstate(divide="ignore"):
        half_spacing = u * np.exp2(np.floor(np.log2(x)))
    return bO + np.maximum(half_spacing, a)


def attention_backward(q, k, v, do, scale: float, causal: bool = False):
    """(dQ, dK, dV, D) in float64 for upstream gradient dO, where
    D[i] = sum_c dO[i, c] * O[i, c] with O the exact forward output.

    Per (b, h): S = scale Q K^T (masked), P = softmax_rows(S), O = P V,
    dV = P^T dO, dP = dO V^T, dS = P * (dP - D), dQ = scale dS K,
    dK = scale dS^T Q.  Square (Nq = Nk) inputs.
    """
    Q, K, V, dO = as_f64(q), as_f64(k), as_f64(v), as_f64(do)
    if Q.shape != K.shape or V.shape != Q.shape or dO.shape != Q.shape or Q.ndim != 4:
        raise ValueError("q, k, v, do must share one [B, H, N, d] shape")
    B, H, N, d = Q.shape
    s64 = boundary_scale(scale)
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    Dm = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            S = Q[b, h] @ K[b, h].T * s64
            if causal:
                S[np.triu(np.ones((N, N), dtype=bool), 1)] = -np.inf
            m = S.max(axis=1, keepdims=True)
            E = np.exp(S - m)
            P = E / E.sum(axis=1, keepdims=True)
            O = P @ V[b, h]
            Dv = (dO[b, h] * O).sum(axis=1)
            dP = dO[b, h] @ V[b, h].T
            dS = P * (dP - Dv[:, None])
            dV[b, h] = P.T @ dO[b, h]
            dQ[b, h] = s64 * (dS @ K[b, h])
            dK[b, h] = s64 * (dS.T @ Q[b, h])
            Dm[b, h] = Dv
    return dQ, dK, dV, Dm


def backward_error_bound(q, k, v, do, scale: float, causal: bool = False, u: float = 2.0 ** -11,
                         u_o: Optional[float] = None, u_p: Optional[float] = None):
    """Per-element bounds on |dQ_hat - dQ|, |dK_hat - dK|, |dV_hat - dV| for a
    backward pass that (1) rounds P to a type with unit roundoff u before
    dV = P^T dO, (2) forms dS = P_in (dP - D) in fp32 with D = rowsum(dO * O_in),
    where O_in is the forward output rounded to unit u_o (default u) and P_in
    is P rounded to unit u_p (default u: the rounded P of step 1; 0 for P in
    fp32), and (3) rounds dS to unit u before dQ = scale dS K and
    dK = scale dS^T Q.  Inputs are exact (already in the 16-bit type);
    products of 16-bit values and fp32 sums are exact up to fp32
    accumulation, which is left to the caller's absolute slack.

    Derivation.  |P_hat - P| <= u P gives |dV_hat - dV|_jc <= u sum_i P_ij |dO_ic|.
    O_in = O (1 + e), |e| <= u_o, so |D_hat - D|_i <= u_o sum_c |dO_ic O_ic| =: dD_i.
    With P_in = P (1 + a), |a| <= u_p, and the rounding of dS (1 + b), |b| <= u,
    dS_hat = P (1 + a)(dP - D - (D_hat - D))(1 + b), so with g = (1 + u_p)(1 + u)
    it differs from dS = P (dP - D) by at most
    (g - 1) |dS_ij| + g P_ij dD_i =: e_ij  (u_p = 0: P_ij dD_i + u (|dS_ij| + P_ij dD_i)).
    Then |dQ_hat - dQ|_ic <= scale sum_j e_ij |K_jc| and
    |dK_hat - dK|_jc <= scale sum_i e_ij |Q_ic|.  A pass that forms dS from a
    less rounded P (smaller u_p) stays within the bound.
    """
    u_o = u if u_o is None else u_o
    u_p = u if u_p is None else u_p
    g = (1.0 + u_p) * (1.0 + u)
    Q, K, V, dO = as_f64(q), as_f64(k), as_f64(v), as_f64(do)
    B, H, N, d = Q.shape
    s64 = abs(boundary_scale(scale))
    bQ, bK, bV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    for b in range(B):
        for h in range(H):
            S = Q[b, h] @ K[b, h].T * boundary_scale(scale)
            if causal:
                S[np.triu(np.ones((N, N), dtype=bool), 1)] = -np.inf
            E = np.exp(S - S.max(axis=1, keepdims=True))
            P = E / E.sum(axis=1, keepdims=True)
            O = P @ V[b, h]
            Dv = (dO[b, h] * O).sum(axis=1)
            dS = P * (dO[b, h] @ V[b, h].T - Dv[:, None])
            dD = u_o * np.abs(dO[b, h] * O).sum(axis=1)
            e = (g - 1.0) * np.abs(dS) + g * P * dD[:, None]
            bV[b, h] = u * (P.T @ np.abs(dO[b, h]))
            bQ[b, h] = s64 * (e @ np.abs(K[b, h]))
            bK[b, h] = s64 * (e.T @ np.abs(Q[b, h]))
    return bQ, bK, bV


def attention_backward_sampled(q, k, v, do, scale: float, causal: bool, heads, rows, cols,
                               u: float = 2.0 ** -11, u_o: Optional[float] = None,
                               u_p: Optional[float] = None):
    """attention_backward and backward_error_bound restricted to chosen
    entries, for inputs too large to differentiate whole: for each (b, h) in
    `heads`, dQ and its bound at query rows `rows`, and dK, dV and their
    bounds at key rows `cols` (index arrays into N).

    The definitions are those of attention_backward / backward_error_bound;
    only the rows and columns of P, dP and dS that the chosen entries use are
    formed into products (P itself is needed in full per head for D, since D
    depends on every output row).  Returns {(b, h): (dQ[rows], dK[cols],
    dV[cols], bQ[rows], bK[cols], bV[cols])}.
    """
    u_o = u if u_o is None else u_o
    u_p = u if u_p is None else u_p
    g = (1.0 + u_p) * (1.0 + u)
    Q, K, V, dO = as_f64(q), as_f64(k), as_f64(v), as_f64(do)
    B, H, N, d = Q.shape
    s = boundary_scale(scale)
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    out = {}
    for (b, h) in heads:
        S = Q[b, h] @ K[b, h].T * s
        if causal:
            S[np.triu(np.ones((N, N), dtype=bool), 1)] = -np.inf
        E = np.exp(S - S.max(axis=1, keepdims=True))
        P = E / E.sum(axis=1, keepdims=True)
        O = P @ V[b, h]
        Dv = (dO[b, h] * O).sum(axis=1)
        dD = u_o * np.abs(dO[b, h] * O).sum(axis=1)
        # rows of dS (for dQ) and columns of dS (for dK); P's columns give dV
        dS_r = P[rows] * (dO[b, h][rows] @ V[b, h].T - Dv[rows, None])
        dS_c = P[:, cols] * (dO[b, h] @ V[b, h][cols].T - Dv[:, None])
        e_r = (g - 1.0) * np.abs(dS_r) + g * P[rows] * dD[rows, None]
        e_c = (g - 1.0) * np.abs(dS_c) + g * P[:, cols] * dD[:, None]
        out[(b, h)] = (s * (dS_r @ K[b, h]), s * (dS_c.T @ Q[b, h]), P[:, cols].T @ dO[b, h],
                       abs(s) * (e_r @ np.abs(K[b, h])), abs(s) * (e_c.T @ np.abs(Q[b, h])),
                       u * (P[:, cols].T @ np.abs(dO[b, h])))
    return out
