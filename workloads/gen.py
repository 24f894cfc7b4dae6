"""Seeded synthetic inputs (torch CPU generator).

Recipe (the same for every consumer):
  * generator: ``torch.Generator().manual_seed(seed)``;
  * draw order: A^K, B^K, A^V, B^V (each [batch][ctx][R][p][q], normal with the
    config's standard deviation, drawn in float32 and then rounded to the
    cache dtype), then the dense query q ([batch][n_q][h][d_h], N(0, 1) times
    ``q_scale``, float32);
  * positions: slot s of every sequence holds position s;
  * query positions: the n_q newest slots, ctx_len - n_q + n;
  * ``ragged``: per-sequence context lengths drawn uniformly in [n_q, ctx] with a
    second generator seeded ``seed + 1``.
The factors are the unrotated ones the caller hands to the cache append.

Factored queries (``make_query_factors``): their own generator seeded
``seed + 2``; A^Q [batch][n_q][R_Q][p1][q1] with the config's A deviation,
then B^Q [batch][n_q][R_Q][p2][q2] with its B deviation, both scaled so that
the expanded query has unit-variance elements like the dense one, float32.
"""
from __future__ import annotations

import dataclasses

import torch

from .configs import Config


@dataclasses.dataclass
class Inputs:
    cfg: Config
    a_k: torch.Tensor
    b_k: torch.Tensor
    a_v: torch.Tensor
    b_v: torch.Tensor
    positions: torch.Tensor  # int32 [B][S]
    ctx_len: torch.Tensor    # int32 [B]
    q: torch.Tensor          # float32 [B][n_q][h][d_h]
    q_pos: torch.Tensor      # int32 [B][n_q]

    @property
    def batch(self) -> int:
        return self.a_k.shape[0]

    @property
    def slots(self) -> int:
        return self.a_k.shape[1]


def _draw(gen, shape, sigma, dtype):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    x.mul_(sigma)
    return x.to(dtype)


def make_inputs(cfg: Config, seed: int = 0, *, batch: int | None = None, ctx: int | None = None,
                n_q: int | None = None, q_scale: float = 1.0, ragged: bool = False,
                pos_offset: int = 0) -> Inputs:
    nb = cfg.batch if batch is None else batch
    s = cfg.ctx if ctx is None else ctx
    nq = cfg.n_q if n_q is None else n_q
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    g = torch.Generator().manual_seed(seed)
    a_k = _draw(g, (nb, s, cfg.r_k, cfg.p1, cfg.q1), cfg.sigma_a, dt)
    b_k = _draw(g, (nb, s, cfg.r_k, cfg.p2, cfg.q2), cfg.sigma_b, dt)
    a_v = _draw(g, (nb, s, cfg.r_v, cfg.p1, cfg.q1), cfg.sigma_a, dt)
    b_v = _draw(g, (nb, s, cfg.r_v, cfg.p2, cfg.q2), cfg.sigma_b, dt)
    q = torch.randn((nb, nq, cfg.h, cfg.d_h), generator=g, dtype=torch.float32)
    if q_scale != 1.0:
        q.mul_(q_scale)
    positions = (torch.arange(s, dtype=torch.int32) + pos_offset).repeat(nb, 1).contiguous()
    if ragged:
        g2 = torch.Generator().manual_seed(seed + 1)
        ctx_len = torch.randint(min(nq, s), s + 1, (nb,), generator=g2, dtype=torch.int32)
    else:
        ctx_len = torch.full((nb,), s, dtype=torch.int32)
    q_pos = (ctx_len.view(-1, 1) - nq + torch.arange(nq, dtype=torch.int32).view(1, -1)
             + pos_offset).to(torch.int32).contiguous()
    return Inputs(cfg, a_k, b_k, a_v, b_v, positions, ctx_len, q, q_pos)


def make_query_factors(cfg: Config, r_q: int, seed: int = 0, *, batch: int | None = None,
                       n_q: int | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """Random factors of a factored query (see the module docstring)."""
    nb = cfg.batch if batch is None else batch
    nq = cfg.n_q if n_q is None else n_q
    g = torch.Generator().manual_seed(seed + 2)
    # an element of (1/R) sum_r a_r b_r has variance sa^2 sb^2 / R: scale it to 1
    s = (r_q ** 0.5) ** 0.5
    a_q = torch.randn((nb, nq, r_q, cfg.p1, cfg.q1), generator=g, dtype=torch.float32).mul_(s)
    b_q = torch.randn((nb, nq, r_q, cfg.p2, cfg.q2), generator=g, dtype=torch.float32).mul_(s)
    return a_q, b_q
