"""Seeded synthetic workloads for the attention forward pass.

This module only draws inputs and counts algorithmic work; it holds none of the
attention arithmetic.  Both the HIP path (through the tests and the benchmark)
and the fp64 CPU oracle consume the arrays it produces, so the two sides always
see bit-identical inputs.

Generation recipe (one recipe for every workload):
  * numpy PCG64, ``default_rng([seed, tensor_id])`` with tensor_id 0 = Q,
    1 = K, 2 = V, 3 = sampled query rows;
  * draws are float32 and are generated one ``[N, d]`` head slice at a time in
    (b, h) order, which bounds host memory for the long-context workloads;
  * the float32 draws are then rounded to the workload dtype with
    round-to-nearest-even (numpy ``astype(float16)`` for fp16, torch CPU
    ``.to(torch.bfloat16)`` for bf16).

The shapes mirror the workloads the FlashAttention explainer pages motivate
(long sequences, head dims 64/128, fp16/bf16 storage); the pages measure on no
dataset, so synthetic N(0,1) draws stand in for activations.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

DTYPES = {
    "f32": torch.float32,
    "f16": torch.float16,
    "bf16": torch.bfloat16,
}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_ROWS, TENSOR_DOUT = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Workload:
    """One named attention-forward workload."""

    name: str
    seed: int
    B: int
    H: int
    N: int
    d: int
    dtype: str
    causal: bool
    kind: str = "normal"          # "normal" or "rescale_stress"
    sampled_rows: Optional[int] = None  # oracle checks this many rows per head
    description: str = ""

    @property
    def scale(self) -> float:
        return default_scale(self.d)

    def flops(self) -> float:
        return metric_flops(self.B, self.H, self.N, self.d, self.causal)

    def compulsory_bytes(self) -> int:
        return compulsory_bytes(self.B, self.H, self.N, self.d, ELEM_BYTES[self.dtype])


# The five workloads: a tiny fp32 single head, a mid-size fp16 batch run both
# unmasked and causal, the fp16 d=128 headline, a bf16 running-max stress and a
# 128k-token bf16 long-context case.
WORKLOADS = {
    "single_head_f32": Workload(
        "single_head_f32", 1, 1, 1, 512, 64, "f32", False,
        description="B=1 H=1 N=512 d=64 fp32, N(0,1), non-causal"),
    "batch_f16_d64": Workload(
        "batch_f16_d64", 2, 4, 8, 2048, 64, "f16", False,
        description="B=4 H=8 N=2048 d=64 fp16, N(0,1), non-causal"),
    "batch_f16_d64_causal": Workload(
        "batch_f16_d64_causal", 2, 4, 8, 2048, 64, "f16", True,
        description="B=4 H=8 N=2048 d=64 fp16, N(0,1), causal (same inputs)"),
    "headline_f16_d128": Workload(
        "headline_f16_d128", 3, 2, 16, 4096, 128, "f16", False,
        description="B=2 H=16 N=4096 d=128 fp16, N(0,1), non-causal"),
    "rescale_stress_bf16": Workload(
        "rescale_stress_bf16", 4, 1, 16, 32768, 128, "bf16", True,
        kind="rescale_stress",
        description="B=1 H=16 N=32768 d=128 bf16, causal; K row j scaled by "
                    "1+3j/N, V~U(-1,1)"),
    "long_context_bf16": Workload(
        "long_context_bf16", 5, 1, 8, 131072, 128, "bf16", True,
        sampled_rows=256,
        description="B=1 H=8 N=131072 d=128 bf16, N(0,1), causal; oracle on "
                    "256 sampled rows per head"),
}
HEADLINE = "headline_f16_d128"


@dataclasses.dataclass(frozen=True)
class CacheWorkload:
    """New queries against a key/value cache: Q is [B, H, Nq, d], K and V
    [B, H, Nk, d]; causal queries are the last Nq of Nk positions."""

    name: str
    seed: int
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str
    causal: bool
    description: str = ""

    @property
    def scale(self) -> float:
        return default_scale(self.d)

    def visible_keys(self) -> int:
        """Query-key pairs of one head that the mask lets through."""
        if not self.causal:
            return self.Nq * self.Nk
        off = self.Nk - self.Nq
        return sum(min(self.Nk, i + 1 + off) for i in range(self.Nq))

    def flops(self) -> float:
        """Matrix-product FLOPs: 4*d per visible query-key pair."""
        return 4.0 * self.B * self.H * self.visible_keys() * self.d

    def compulsory_bytes(self) -> int:
        """Read Q, K, V once, write O and the fp32 LSE once."""
        e = ELEM_BYTES[self.dtype]
        return (2 * self.B * self.H * self.Nq * self.d * e + 2 * self.B * self.H * self.Nk * self.d * e
                + 4 * self.B * self.H * self.Nq)


# Decode against a cache: a batch of single-token queries over an 8k cache, and
# a 16-token causal step (e.g. speculative decoding) over a 128k-token cache at
# batch 1.  Bound by reading K and V from HBM.
CACHE_WORKLOADS = {
    "decode_f16_d128": CacheWorkload(
        "decode_f16_d128", 6, 16, 16, 1, 8192, 128, "f16", False,
        description="B=16 H=16 Nq=1 Nk=8192 d=128 fp16, N(0,1)"),
    "decode_long_bf16": CacheWorkload(
        "decode_long_bf16", 7, 1, 8, 16, 131072, 128, "bf16", True,
        description="B=1 H=8 Nq=16 Nk=131072 d=128 bf16, N(0,1), causal "
                    "(queries are the last 16 positions)"),
}


def random_cache_inputs(B: int, H: int, Nq: int, Nk: int, d: int, dtype: str, seed: int):
    """Q [B, H, Nq, d] and K, V [B, H, Nk, d], iid N(0,1), same recipe as
    random_qkv (tensor ids 0, 1, 2)."""
    def normal(n):
        return lambda rng, b, h: rng.standard_normal((n, d), dtype=np.float32)

    q = _draw(seed, TENSOR_Q, B, H, Nq, d, dtype, normal(Nq))
    k = _draw(seed, TENSOR_K, B, H, Nk, d, dtype, normal(Nk))
    v = _draw(seed, TENSOR_V, B, H, Nk, d, dtype, normal(Nk))
    return q, k, v


def cache_workload_inputs(w: CacheWorkload):
    return random_cache_inputs(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.seed)


def default_scale(d: int) -> float:
    """1/sqrt(d), rounded to float32: the value the kernel receives."""
    return float(np.float32(1.0 / math.sqrt(d)))


def metric_flops(B: int, H: int, N: int, d: int, causal: bool) -> float:
    """Matrix-product FLOPs the metric counts: 2*N*N*d for Q K^T plus
    2*N*N*d for P V per head, halved under the causal mask."""
    f = 4.0 * B * H * N * N * d
    return f / 2.0 if causal else f


def compulsory_bytes(B: int, H: int, N: int, d: int, elem: int) -> int:
    """Bytes that must cross HBM once: read Q, K, V, write O, write fp32 LSE."""
    return 4 * B * H * N * d * elem + 4 * B * H * N


def naive_score_bytes(N: int, elem: int) -> int:
    """Size of one head's materialised N x N score matrix."""
    return N * N * elem


def naive_score_round_trip_bytes(N: int, elem: int) -> int:
    """Write plus read-back of one head's N x N score matrix."""
    return 2 * N * N * elem


def roofline_ridge(peak_flops: float, peak_bytes_per_s: float) -> float:
    """FLOPs per byte at which a kernel stops being bandwidth bound."""
    return peak_flops / peak_bytes_per_s


def _round_to(x32: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    if dtype == "f16":
        return torch.from_numpy(x32.astype(np.float16))
    if dtype == "bf16":
        return torch.from_numpy(x32).to(torch.bfloat16)
    raise ValueError(f"unknown dtype {dtype!r}")


def _draw(seed: int, tensor_id: int, B: int, H: int, N: int, d: int, dtype: str,
          sampler) -> torch.Tensor:
    rng = np.random.default_rng([seed, tensor_id])
    out = torch.empty((B, H, N, d), dtype=DTYPES[dtype])
    for b in range(B):
        for h in range(H):
            out[b, h] = _round_to(sampler(rng, b, h), dtype)
    return out


def random_qkv(B: int, H: int, N: int, d: int, dtype: str, seed: int,
               kind: str = "normal"):
    """Q, K, V as contiguous CPU tensors of ``dtype`` with shape [B, H, N, d].

    kind="normal": all three iid N(0,1).
    kind="rescale_stress": Q iid N(0,1); K row j iid N(0,1) multiplied in
    float32 by (1 + 3*j/N) before rounding, so score maxima keep growing
    along the sequence; V iid U(-1, 1).
    """
    def normal(rng, b, h):
        return rng.standard_normal((N, d), dtype=np.float32)

    if kind == "normal":
        q = _draw(seed, TENSOR_Q, B, H, N, d, dtype, normal)
        k = _draw(seed, TENSOR_K, B, H, N, d, dtype, normal)
        v = _draw(seed, TENSOR_V, B, H, N, d, dtype, normal)
    elif kind == "rescale_stress":
        growth = (np.float32(1.0) + np.float32(3.0)
                  * (np.arange(N, dtype=np.float32) / np.float32(N)))[:, None]

        def scaled_normal(rng, b, h):
            return rng.standard_normal((N, d), dtype=np.float32) * growth

        def uniform(rng, b, h):
            return rng.uniform(-1.0, 1.0, size=(N, d)).astype(np.float32)

        q = _draw(seed, TENSOR_Q, B, H, N, d, dtype, normal)
        k = _draw(seed, TENSOR_K, B, H, N, d, dtype, scaled_normal)
        v = _draw(seed, TENSOR_V, B, H, N, d, dtype, uniform)
    else:
        raise ValueError(f"unknown input kind {kind!r}")
    return q, k, v


def sample_rows(seed: int, B: int, H: int, N: int, count: int) -> np.ndarray:
    """[B, H, count] sorted distinct query indices per head, drawn uniformly
    without replacement."""
    rng = np.random.default_rng([seed, TENSOR_ROWS])
    count = min(count, N)
    rows = np.empty((B, H, count), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            rows[b, h] = np.sort(rng.choice(N, size=count, replace=False))
    return rows


def workload_inputs(w: Workload):
    """(q, k, v) CPU tensors for a named workload."""
    return random_qkv(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.kind)


E4M3_MAX = 448.0  # largest finite e4m3 value


def quantize_e4m3(x32: np.ndarray):
    """Per-tensor scaled e4m3 quantization: descale = float32(amax / 448),
    codes = round-to-nearest-even of x / descale (float32 division), as a
    torch float8_e4m3fn tensor.  Returns (codes, descale)."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    amax = float(t.abs().max()) if t.numel() else 0.0
    descale = float(np.float32(amax / E4M3_MAX)) if amax > 0 else 1.0
    codes = (t / np.float32(descale)).to(torch.float8_e4m3fn)
    return codes, descale


def random_qkv_fp8(B: int, H: int, N: int, d: int, seed: int, Nk: Optional[int] = None):
    """Q [B, H, N, d] and K, V [B, H, Nk, d] as e4m3 tensors with per-tensor
    descale factors: the float32 N(0,1) draws of random_qkv (same seeds and
    tensor ids, one head slice at a time), each tensor quantized with
    quantize_e4m3.  Returns (q, k, v, q_descale, k_descale, v_descale)."""
    Nk = N if Nk is None else Nk

    def draw(tensor_id, n):
        rng = np.random.default_rng([seed, tensor_id])
        out = np.empty((B, H, n, d), dtype=np.float32)
        for b in range(B):
            for h in range(H):
                out[b, h] = rng.standard_normal((n, d), dtype=np.float32)
        return out

    q, qs = quantize_e4m3(draw(TENSOR_Q, N))
    k, ks = quantize_e4m3(draw(TENSOR_K, Nk))
    v, vs = quantize_e4m3(draw(TENSOR_V, Nk))
    return q, k, v, qs, ks, vs


@dataclasses.dataclass(frozen=True)
class Fp8Workload:
    """The 8-bit forward pass: e4m3 Q, K, V ([B, H, N, d], per-tensor
    descales), bf16 O."""

    name: str
    seed: int
    B: int
    H: int
    N: int
    d: int
    causal: bool
    dtype: str = "fp8_e4m3"
    description: str = ""

    @property
    def scale(self) -> float:
        return default_scale(self.d)

    def flops(self) -> float:
        return metric_flops(self.B, self.H, self.N, self.d, self.causal)

    def compulsory_bytes(self) -> int:
        """Read 1-byte Q, K, V; write 2-byte O and 4-byte LSE."""
        n = self.B * self.H * self.N * self.d
        return 3 * n + 2 * n + 4 * self.B * self.H * self.N


# The headline shape with 8-bit inputs (same seed as the fp16 headline draws).
FP8_WORKLOADS = {
    "headline_fp8_d128": Fp8Workload(
        "headline_fp8_d128", 3, 2, 16, 4096, 128, False,
        description="B=2 H=16 N=4096 d=128, N(0,1) drawn in fp32 and quantized to e4m3 "
                    "with per-tensor descale amax/448, bf16 O, non-causal"),
}


def fp8_workload_inputs(w: Fp8Workload):
    return random_qkv_fp8(w.B, w.H, w.N, w.d, w.seed)


def random_dout(B: int, H: int, N: int, d: int, dtype: str, seed: int) -> torch.Tensor:
    """Upstream gradient dO [B, H, N, d], iid N(0,1), same recipe as
    random_qkv with tensor id 4."""
    return _draw(seed, TENSOR_DOUT, B, H, N, d, dtype,
                 lambda rng, b, h: rng.standard_normal((N, d), dtype=np.float32))


@dataclasses.dataclass(frozen=True)
class BwdWorkload:
    """The backward pass on a square workload: gradients of Q, K, V."""

    name: str
    seed: int
    B: int
    H: int
    N: int
    d: int
    dtype: str
    causal: bool
    description: str = ""

    @property
    def scale(self) -> float:
        return default_scale(self.d)

    def flops(self) -> float:
        """Algorithmic matrix-product FLOPs of the gradient: 2*N*N*d for each
        of S = Q K^T, dV = P^T dO, dP = dO V^T, dQ = dS K and dK = dS^T Q per
        head (2.5x the forward's count), halved under the causal mask.  The
        kernels recompute S and dP once more (7 products instead of 5)."""
        return 2.5 * metric_flops(self.B, self.H, self.N, self.d, self.causal)

    def compulsory_bytes(self) -> int:
        """Read Q, K, V, O, dO and LSE; write dQ, dK, dV (and D in and out)."""
        e = ELEM_BYTES[self.dtype]
        n = self.B * self.H * self.N
        return 8 * n * self.d * e + 4 * n + 8 * n


BWD_WORKLOADS = {
    "headline_bwd_f16_d128": BwdWorkload(
        "headline_bwd_f16_d128", 3, 2, 16, 4096, 128, "f16", False,
        description="backward of B=2 H=16 N=4096 d=128 fp16, N(0,1) inputs and dO, non-causal"),
    "causal_bwd_bf16_d128": BwdWorkload(
        "causal_bwd_bf16_d128", 6, 1, 16, 8192, 128, "bf16", True,
        description="backward of B=1 H=16 N=8192 d=128 bf16, N(0,1) inputs and dO, causal"),
}
