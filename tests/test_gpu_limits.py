"""Decode at the limits the C ABI accepts (KPA_MAX_NQ, KPA_MAX_RANK,
KPA_MAX_HEADS, KPA_MAX_HEAD_DIM, KPA_MAX_HD in include/kpa.h) and at the
method's degenerate shapes (one head, one rotary pair per row, unequal key
and value ranks, many short sequences), every output element against the
float64 oracle.  Whichever kernel path the library picks for a shape
(matrix cores or the vector-ALU kernel) must meet the same tolerance."""
import math

import numpy as np
import pytest

import factorized_kv_cache_kpa_amd as kpa
from oracle import kpa_oracle
from tests.kpa_testutil import assert_close, dims_of, fill_cache, run_decode, scale_of, score_scale
from workloads import Config, make_inputs

pytestmark = pytest.mark.gpu


def _cfg(name, p1, p2, q1, q2, r_k, r_v, dtype="bf16"):
    return Config(name, p1, p2, q1, q2, r_k, r_v, dtype, batch=1, ctx=1,
                  sigma_a=1 / math.sqrt(q1), sigma_b=1 / math.sqrt(q2))


CASES = [
    # config, batch, ctx, n_q, ragged
    (_cfg("max_nq", 4, 4, 8, 16, 2, 2), 2, 150, kpa.KPA_MAX_NQ, True),
    (_cfg("max_nq_multiq_shape", 4, 8, 16, 8, 4, 4), 1, 300, kpa.KPA_MAX_NQ, False),
    (_cfg("max_rank", 2, 2, 4, 4, kpa.KPA_MAX_RANK, kpa.KPA_MAX_RANK), 2, 130, 1, True),
    (_cfg("max_rank_f32", 2, 2, 4, 4, kpa.KPA_MAX_RANK, kpa.KPA_MAX_RANK, "f32"), 2, 70, 3, False),
    (_cfg("max_heads", 16, 8, 8, 8, 1, 1), 1, 100, 1, False),          # h = 128, h d_h = 8192
    (_cfg("max_head_dim", 4, 8, 16, 16, 2, 2), 2, 90, 1, True),        # d_h = 256, h d_h = 8192
    (_cfg("one_head", 1, 1, 8, 16, 2, 2), 3, 200, 1, True),
    (_cfg("one_pair_per_row", 4, 4, 64, 2, 2, 2), 2, 160, 1, False),   # q2 = 2
    (_cfg("ranks_1_3", 4, 4, 8, 16, 1, 3), 2, 140, 2, True),
    (_cfg("wide_rotary", 2, 2, 1, 128, 1, 2), 2, 75, 1, True),         # q2 = 128: the per-token append
]


@pytest.mark.parametrize("cfg,batch,ctx,n_q,ragged", CASES, ids=[c[0].name for c in CASES])
def test_limits_and_degenerate_shapes(gpu_lib, cfg, batch, ctx, n_q, ragged):
    inp = make_inputs(cfg, seed=31, batch=batch, ctx=ctx, n_q=n_q, ragged=ragged)
    dims = dims_of(cfg)
    assert kpa.kpa_decode_path(dims, n_q) != ""
    cache, cap = fill_cache(inp, dims)
    go, gl = run_decode(inp, dims, cache, cap)
    ro, rl = kpa_oracle.decode(inp.a_k, inp.b_k, inp.a_v, inp.b_v, inp.positions, inp.ctx_len,
                               inp.q, inp.q_pos, causal=True)
    assert_close(go, gl, ro, rl, cfg.dtype, f"{cfg.name} ({kpa.kpa_decode_path(dims, n_q)})", scale=scale_of(inp),
                 path=kpa.kpa_decode_path(dims, n_q))


def test_many_short_sequences(gpu_lib):
    """batch * n_q near its bound with contexts of 1 .. 40 slots (most of
    them shorter than one tile)."""
    cfg = _cfg("many_sequences", 4, 4, 8, 16, 2, 2)
    inp = make_inputs(cfg, seed=32, batch=3000, ctx=40, n_q=1, ragged=True)
    dims = dims_of(cfg)
    cache, cap = fill_cache(inp, dims)
    go, gl = run_decode(inp, dims, cache, cap)
    rng = np.random.default_rng(3)
    rows = np.sort(rng.choice(inp.batch, size=64, replace=False))
    sub = lambda t: t[rows]
    ro, rl = kpa_oracle.decode(sub(inp.a_k), sub(inp.b_k), sub(inp.a_v), sub(inp.b_v), sub(inp.positions),
                               sub(inp.ctx_len), sub(inp.q), sub(inp.q_pos), causal=True)
    assert_close(go[rows], gl[rows], ro, rl, cfg.dtype, "many short sequences",
                 scale=score_scale(sub(inp.a_k), sub(inp.b_k), sub(inp.ctx_len), sub(inp.q)))
