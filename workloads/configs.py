"""Problem shapes.

Five decode workloads shaped like the KPA and TPA pages' model scales, plus
the head-split shapes the KPA page ablates ([KPA] §3.3, App. D; d1 = d2 = 8,
R_K = R_V = 2).

[KPA] "Kronecker Product Attention: Memory-Efficient KV Compression via
Structured Factorization" (arXiv 2610.12657).
"""
from __future__ import annotations

import dataclasses
import math


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    p1: int
    p2: int
    q1: int
    q2: int
    r_k: int
    r_v: int
    dtype: str          # "f32" or "bf16" (cached factors)
    batch: int
    ctx: int            # cached tokens per sequence attended by the decode
    n_q: int = 1        # queries per sequence (multi-query decode when > 1)
    sigma_a: float = 0.0
    sigma_b: float = 0.0
    rope_base: float = 10000.0

    @property
    def h(self) -> int:
        return self.p1 * self.p2

    @property
    def d_h(self) -> int:
        return self.q1 * self.q2

    @property
    def bytes_per_elem(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def numbers_per_token(self) -> int:
        """(R_K + R_V)(p1 q1 + p2 q2) -- [KPA] §2.5."""
        return (self.r_k + self.r_v) * (self.p1 * self.q1 + self.p2 * self.q2)

    @property
    def bytes_per_token(self) -> int:
        return self.numbers_per_token * self.bytes_per_elem

    @property
    def capacity(self) -> int:
        return self.ctx

    def scaled(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


def _sig(q: int) -> float:
    return 1.0 / math.sqrt(q)


CONFIGS = {
    # Tiny KPA decode, fp32.  Factors ~ N(0, sd 1/4).
    "tiny_f32": Config("tiny_f32", 2, 2, 4, 4, 2, 2, "f32", batch=1, ctx=256,
                       sigma_a=0.25, sigma_b=0.25),
    # TPA degenerate split: A_r is h x 1, B_r is 1 x d_h.  Factors ~ N(0, sd 1/8).
    "tpa_degenerate": Config("tpa_degenerate", 12, 1, 1, 64, 2, 2, "bf16", batch=16, ctx=4096,
                             sigma_a=0.125, sigma_b=0.125),
    # KPA non-degenerate h = 4x4, d_h = 8x16, 32 sequences of 32768 tokens.
    "kpa_32k": Config("kpa_32k", 4, 4, 8, 16, 2, 2, "bf16", batch=32, ctx=32768,
                      sigma_a=_sig(8), sigma_b=_sig(16)),
    # Long context: one sequence of 2^19 tokens, h = 8x4, R_K = 2, R_V = 4.
    "long_512k": Config("long_512k", 8, 4, 8, 16, 2, 4, "bf16", batch=1, ctx=524288,
                        sigma_a=_sig(8), sigma_b=_sig(16)),
    # Multi-query (chunked / speculative) decode: 8 sequences, 16384 cached
    # tokens + 16 new tokens appended, 16 causal queries per sequence.
    "multiq_16": Config("multiq_16", 4, 8, 16, 8, 4, 4, "bf16", batch=8, ctx=16384 + 16, n_q=16,
                        sigma_a=_sig(16), sigma_b=_sig(8)),
}

# Head splits ablated on the KPA page (d1 = d2 = 8, R_K = R_V = 2).
SWEEP_SHAPES = [
    (8, 2), (4, 4), (2, 8),            # 353M, h = 16
    (10, 2), (4, 5), (2, 10),          # 773M, h = 20
    (5, 5),                            # 1.5B, h = 25
    (6, 2), (4, 3), (3, 4), (2, 6),    # 125M, h = 12
]


# FlashTPA decoding benchmark shapes ("Tensor Product Attention Is All You
# Need", summary page: d_model 1024 / 2048 / 3072, d_h = 64, R_K = R_V = 1,
# sequence lengths 2^12 .. 2^19, batch 1 .. 16), as TPA's degenerate split of
# KPA: A_r is h x 1, B_r is 1 x 64.  The pages give no factor distribution;
# the TPA config's sd 1/8 is used.
FLASHTPA_HEADS = (16, 32, 48)
FLASHTPA_SEQS = tuple(1 << k for k in range(12, 20))
FLASHTPA_BATCHES = (1, 2, 4, 8, 16)
FLASHTPA_RQ = 16  # the benchmark's factored-query rank


def headsplit_config(p1: int, p2: int, batch: int, ctx: int) -> Config:
    """A head split of the KPA page's ablation: h = p1 x p2 heads, d1 = d2 = 8
    (d_h = 64), R_K = R_V = 2, bf16 factors with sd 1/sqrt(8) per axis."""
    s = 1.0 / math.sqrt(8)
    return Config(f"split_{p1}x{p2}_b{batch}_s{ctx}", p1, p2, 8, 8, 2, 2, "bf16", batch=batch, ctx=ctx,
                  sigma_a=s, sigma_b=s)


def flashtpa_config(h: int, batch: int, ctx: int) -> Config:
    return Config(f"flashtpa_h{h}_b{batch}_s{ctx}", h, 1, 1, 64, 1, 1, "bf16", batch=batch, ctx=ctx,
                  sigma_a=0.125, sigma_b=0.125)

