"""The five workload definitions (shapes, types, value scales, seeds).

Shapes and value distributions follow the attention workloads this library is
measured on: self-attention with L_q = L_k = L, tensors laid out (B, H, L, d).
Seeds are the workload index (0..4); streams 0/1/2 are Q/K/V.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    B: int
    H: int
    L: int
    d: int
    dtype: int          # 0 = f32, 1 = f16, 2 = bf16 (storage of Q, K, V and O)
    causal: int
    scale: float
    seed: int
    sigma_q: float = 1.0
    sigma_k: float = 1.0
    sigma_v: float = 1.0
    # number of query rows per (b, h) that the parity check compares against
    # the oracle; None means every row
    check_rows: int | None = None
    notes: str = field(default="", compare=False)

    @property
    def flops(self) -> int:
        """Metric FLOPs: 4*B*H*L^2*d, halved when causal."""
        f = 4 * self.B * self.H * self.L * self.L * self.d
        return f // 2 if self.causal else f

    @property
    def algorithmic_bytes(self) -> int:
        """Q, K, V read once, O written once, lse (fp32) written once."""
        eb = 4 if self.dtype == 0 else 2
        n = self.B * self.H * self.L * self.d
        return 4 * n * eb + 4 * self.B * self.H * self.L


CONFIGS = [
    Config(0, "single-head fp32 L256 d64", 1, 1, 256, 64, 0, 0, 1.0 / 8.0, 0,
           notes="fp32 Q/K/V ~ N(0,1); tolerance 1e-5 relative"),
    Config(1, "bf16 B4 H16 L1024 d64", 4, 16, 1024, 64, 2, 0, 1.0 / 8.0, 1),
    Config(2, "bf16 causal B2 H32 L4096 d128", 2, 32, 4096, 128, 2, 1, 1.0 / math.sqrt(128.0), 2),
    Config(3, "bf16 peaked B1 H32 L8192 d128", 1, 32, 8192, 128, 2, 0, 1.0 / math.sqrt(128.0), 3,
           sigma_q=3.0, sigma_k=3.0,
           notes="Q, K ~ 3*N(0,1): score sigma ~ 9, peaked softmax"),
    Config(4, "fp16 causal B1 H16 L16384 d64", 1, 16, 16384, 64, 1, 1, 1.0 / 8.0, 4,
           check_rows=64, notes="oracle checked on 64 sampled query rows per head"),
]


def config(index: int) -> Config:
    return CONFIGS[index]


@dataclass(frozen=True)
class DecodeConfig:
    """A decoding shape for the split-K/V path: Lq query rows per (b, h)
    against a cache of Lk keys (no mask)."""
    name: str
    B: int
    H: int
    Lq: int
    Lk: int
    d: int
    dtype: int
    scale: float
    seed: int
    sigma_q: float = 1.0
    sigma_k: float = 1.0
    sigma_v: float = 1.0

    @property
    def flops(self) -> int:
        """4*B*H*Lq*Lk*d (both products)."""
        return 4 * self.B * self.H * self.Lq * self.Lk * self.d

    @property
    def algorithmic_bytes(self) -> int:
        """Q, K, V read once, O written once, lse (fp32) written once."""
        eb = 4 if self.dtype == 0 else 2
        bh = self.B * self.H
        return bh * (2 * self.Lq + 2 * self.Lk) * self.d * eb + 4 * bh * self.Lq


# Decoding with a long K/V cache: one new query row per (batch, head), 1 GiB
# of K/V in bf16.  Seed 10; streams 0/1/2 are Q/K/V.
DECODE = DecodeConfig("decode bf16 B8 H32 Lq1 Lk16384 d128", 8, 32, 1, 16384, 128, 2,
                      1.0 / math.sqrt(128.0), 10)


@dataclass(frozen=True)
class BwdConfig:
    """A backward-pass shape: Q, K, V and the upstream gradient dO, (B, H, L, d)."""
    name: str
    B: int
    H: int
    L: int
    d: int
    dtype: int
    causal: int
    scale: float
    seed: int

    @property
    def flops(self) -> int:
        """10*B*H*L^2*d: the five L x L x d products of the backward pass
        (S, dP, dV, dK, dQ), halved when causal."""
        f = 10 * self.B * self.H * self.L * self.L * self.d
        return f // 2 if self.causal else f

    @property
    def algorithmic_bytes(self) -> int:
        """Bytes one backward call must move: Q, K, V, O, dO and the float32 lse
        read once, dQ, dK, dV written once (16-bit storage)."""
        n = self.B * self.H * self.L
        return 8 * n * self.d * 2 + 4 * n


# Backward shapes.  Seeds 20/21; streams 0/1/2/3 are Q/K/V/dO.
BWD = [
    BwdConfig("bwd bf16 B1 H32 L8192 d128", 1, 32, 8192, 128, 2, 0, 1.0 / math.sqrt(128.0), 20),
    BwdConfig("bwd bf16 causal B2 H32 L4096 d128", 2, 32, 4096, 128, 2, 1, 1.0 / math.sqrt(128.0), 21),
]


@dataclass(frozen=True)
class Fp8Config:
    """An FP8 forward shape: Q and K block-quantised to E4M3 (blocks of
    block_q / block_k rows of a head), V and O in `dtype`.  The inputs are
    those of the 16-bit workload with the same seed and value scales."""
    name: str
    B: int
    H: int
    L: int
    d: int
    dtype: int
    causal: int
    scale: float
    seed: int
    sigma_q: float
    sigma_k: float
    sigma_v: float
    block_q: int
    block_k: int

    @property
    def flops(self) -> int:
        """Metric FLOPs as for the 16-bit forward: 4*B*H*L^2*d, halved when causal."""
        f = 4 * self.B * self.H * self.L * self.L * self.d
        return f // 2 if self.causal else f

    @property
    def algorithmic_bytes(self) -> int:
        """Bytes the attention kernel must move: the E4M3 codes of Q and K (one
        byte each), V and O (two bytes each), lse, and the float32 block scales
        of Q and K, each read or written once."""
        n = self.B * self.H * self.L
        nbq = -(-self.L // self.block_q)
        nbk = -(-self.L // self.block_k)
        return n * self.d * (1 + 1 + 2 + 2) + 4 * n + 4 * self.B * self.H * (nbq + nbk)


# FP8 shapes: the peaked B1 H32 L8192 d128 workload (seed 3) and the causal
# B2 H32 L4096 d128 one (seed 2), quantised in blocks of 128 rows.
FP8 = [
    Fp8Config("fp8 e4m3 q/k, bf16 v, peaked B1 H32 L8192 d128", 1, 32, 8192, 128, 2, 0, 1.0 / math.sqrt(128.0),
              3, 3.0, 3.0, 1.0, 128, 128),
    Fp8Config("fp8 e4m3 q/k, bf16 v, causal B2 H32 L4096 d128", 2, 32, 4096, 128, 2, 1, 1.0 / math.sqrt(128.0),
              2, 1.0, 1.0, 1.0, 128, 128),
]
