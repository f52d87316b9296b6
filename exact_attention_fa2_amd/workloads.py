"""The five synthetic workloads the path is checked and measured on.

No dataset is involved anywhere: every workload is iid N(0,1) Q/K/V drawn by
``inputs.qkv`` from the seed given here.  Shapes come from the pages:

  * single-head f32, Nq = Nk = 4096, D = 64 ("Flash attention, f32": the size
    its benchmark runs at), plus a 256-row version small enough for the oracle
    to finish instantly;
  * multi-head B = 4, H = 12, M = N in {512, 1024, 2048}, D = 64, in fp16 and in
    bf16 (the FlashAttention-2 README's Benchmarks and Accuracy sections);
  * Z = 1, H = 2, N_CTX = 1024, D = 64, scale 0.5, causal and not, with the
    per-row log-sum-exp ("06: Fused attention", the check);
  * flash-decoding, batch 8, 32 heads, one query row, KV length 32768, D = 128,
    fp16 and bf16 ("Flash decoding": one query row per (batch, head)).

Seeds: 0 everywhere except the causal workload, which uses 20 (the fused
attention tutorial seeds its check with 20).  Inputs are N(0,1) throughout,
including the causal workload, whose tutorial check drew std 0.5.
"""
from __future__ import annotations

import dataclasses
import math


@dataclasses.dataclass(frozen=True)
class Prefill:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    D: int
    dtype: str
    scale: float
    causal: bool
    seed: int

    @property
    def flops(self) -> float:
        """4 * B * H * Nq * Nk * D, halved when causal (the work actually done
        counts only the lower triangle)."""
        f = 4.0 * self.B * self.H * self.Nq * self.Nk * self.D
        return f / 2.0 if self.causal else f


@dataclasses.dataclass(frozen=True)
class Decode:
    name: str
    B: int
    H: int
    N: int
    D: int
    dtype: str
    scale: float
    seed: int

    @property
    def kv_bytes(self) -> int:
        """Algorithmic bytes: K and V read once, q read once, O written once."""
        esz = 4 if self.dtype == "f32" else 2
        return esz * self.B * self.H * (2 * self.N * self.D + 2 * self.D)


TINY_F32 = Prefill("single-head f32 256x256 D64", 1, 1, 256, 256, 64, "f32", 1 / 8.0, False, 0)
HEADLINE_F32 = Prefill("single-head f32 Nq=Nk=4096 D64", 1, 1, 4096, 4096, 64, "f32", 1 / 8.0,
                       False, 0)


def multihead(n: int, dtype: str) -> Prefill:
    return Prefill("B4 H12 M=N=%d D64 %s" % (n, dtype), 4, 12, n, n, 64, dtype, 1 / 8.0,
                   False, 0)


def causal_lse(causal: bool = True) -> Prefill:
    return Prefill("Z1 H2 N1024 D64 f16 scale0.5 %s" % ("causal" if causal else "full"),
                   1, 2, 1024, 1024, 64, "f16", 0.5, causal, 20)


def decode(dtype: str = "f16") -> Decode:
    return Decode("decode B8 H32 N32768 D128 %s" % dtype, 8, 32, 32768, 128, dtype,
                  1.0 / math.sqrt(128.0), 0)
