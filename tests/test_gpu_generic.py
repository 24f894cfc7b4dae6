"""Matrix-core decode of shapes without an exact instantiation (the generic
families: head split, G-side feature dimension, ranks and orientation read
at launch) against the float64 oracle, through the C ABI.  Each shape has a
feature dimension of 8, 16, 32 or 64 and ranks up to 4; together they cover
every family (F width 8/16/32/64; rows up to 32, 64 and 128; rank caps 2
and 4; one and several queries; F = A and F = B; G feature dimensions 1, 2,
4, 8, 16 and 32).  Ragged contexts over several chunks, automatic and forced
chunk counts."""
import math

import numpy as np
import pytest
import torch

import factorized_kv_cache_kpa_amd as kpa
from oracle import kpa_oracle, kpa_ref
from tests.kpa_testutil import assert_close, dims_of, fill_cache, run_decode, scale_of
from workloads import Config, make_inputs, make_query_factors

pytestmark = pytest.mark.gpu

# (p1, p2, q1, q2, r_k, r_v)
SHAPES = [
    (3, 2, 8, 8, 1, 1),      # F width 8, 24 rows
    (6, 3, 8, 8, 3, 2),      # 48 rows, rank cap 4
    (16, 2, 8, 8, 2, 2),     # 128 rows
    (2, 16, 8, 8, 1, 1),     # F = A, 128 rows
    (4, 2, 4, 16, 1, 3),     # F width 16, G width 4
    (3, 3, 8, 16, 2, 2),
    (8, 2, 16, 16, 2, 2),    # d_h 256, G width 16, 128 rows
    (4, 2, 2, 32, 2, 2),     # F width 32, G width 2
    (4, 4, 4, 32, 4, 1),
    (2, 2, 8, 32, 3, 3),
    (20, 1, 1, 64, 2, 2),    # TPA split with 20 heads (G width 1)
    (7, 1, 1, 64, 1, 1),     # 7 rows (rank one)
    (8, 2, 2, 64, 1, 2),
    (6, 1, 4, 64, 3, 3),
    (2, 2, 32, 8, 2, 2),     # G width 32
    (3, 4, 16, 2, 2, 2),     # only q1 qualifies: F = A, G width 2
    (4, 4, 8, 16, 4, 4),     # kpa_32k's split at rank 4
]


def _cfg(shape, batch, ctx, n_q):
    p1, p2, q1, q2, rk, rv = shape
    return Config(f"gen_{p1}x{p2}_{q1}x{q2}_r{rk}{rv}", p1, p2, q1, q2, rk, rv, "bf16", batch=batch, ctx=ctx,
                  n_q=n_q, sigma_a=1 / math.sqrt(q1), sigma_b=1 / math.sqrt(q2))


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("n_q", [1, 5])
def test_generic_shapes_match_oracle(gpu_lib, shape, n_q):
    cfg = _cfg(shape, 3, 420, n_q)
    inp = make_inputs(cfg, seed=40 + n_q, ragged=True, q_scale=2.0)
    inp.ctx_len[0] = 420
    dims = dims_of(cfg)
    assert kpa.kpa_decode_path(dims, n_q) == "mfma_bf16"
    cache, cap = fill_cache(inp, dims)
    ro, rl = kpa_oracle.decode(inp.a_k, inp.b_k, inp.a_v, inp.b_v, inp.positions, inp.ctx_len, inp.q, inp.q_pos)
    for s in (0, 4):
        go, gl = run_decode(inp, dims, cache, cap, num_splits=s)
        assert_close(go, gl, ro, rl, cfg.dtype, f"{cfg.name} n_q={n_q} splits={s}", scale=scale_of(inp))


def test_generic_fused_step_equals_append_then_decode(gpu_lib):
    """kpa_append_decode on a generic family (the single-query kernels write
    the step's token themselves): same cache bytes and outputs as the two
    calls."""
    cfg = _cfg((6, 3, 8, 8, 3, 2), 2, 300, 1)
    inp = make_inputs(cfg, seed=47)
    dims = dims_of(cfg)
    h, dh = cfg.h, cfg.d_h
    res = []
    for fused in (False, True):
        pre = make_inputs(cfg, seed=47)
        pre.a_k, pre.b_k, pre.a_v, pre.b_v = (t[:, :299].contiguous() for t in (inp.a_k, inp.b_k, inp.a_v, inp.b_v))
        pre.positions = inp.positions[:, :299].contiguous()
        cache, cap = fill_cache(pre, dims, capacity=300)
        new = [t[:, 299:].contiguous().cuda() for t in (inp.a_k, inp.b_k, inp.a_v, inp.b_v, inp.positions)]
        slot0 = torch.full((2,), 299, dtype=torch.int32, device="cuda")
        out = torch.empty((2, h, dh), device="cuda")
        lse = torch.empty((2, h), device="cuda")
        ws = kpa.alloc_workspace(dims, 2, 300, 1, 3)
        ctx = inp.ctx_len.cuda()
        q, qp = inp.q.cuda().view(2, h, dh), inp.q_pos.cuda().view(2)
        if fused:
            kpa.kpa_append_decode(dims, cache, 2, cap, *new[:5], slot0, ctx, 300, 1, 1, q.view(2, 1, h, dh),
                                  qp.view(2, 1), out.view(2, 1, h, dh), lse.view(2, 1, h), ws, 3, n_new=1)
        else:
            kpa.kpa_cache_append(dims, cache, 2, cap, *new[:5], slot0, n_new=1)
            kpa.kpa_decode(dims, cache, 2, cap, ctx, 300, q, qp, out, lse, ws, 3)
        torch.cuda.synchronize()
        res.append((cache.cpu().numpy().copy(), out.cpu().numpy(), lse.cpu().numpy()))
    assert np.array_equal(res[0][0], res[1][0]), "cache bytes differ"
    assert np.array_equal(res[0][1], res[1][1]) and np.array_equal(res[0][2], res[1][2]), "outputs differ"
    ro, rl = kpa_oracle.decode(inp.a_k, inp.b_k, inp.a_v, inp.b_v, inp.positions, inp.ctx_len, inp.q, inp.q_pos)
    assert_close(res[1][1][:, None].astype(np.float64), res[1][2][:, None].astype(np.float64), ro, rl, cfg.dtype,
                 "generic fused step", scale=scale_of(inp))


@pytest.mark.parametrize("shape", [(6, 3, 8, 8, 3, 2), (3, 4, 16, 2, 2, 2), (20, 1, 1, 64, 2, 2)],
                         ids=lambda s: "x".join(map(str, s)))
def test_generic_factored_query_matches_oracle(gpu_lib, shape):
    cfg = _cfg(shape, 2, 300, 3)
    inp = make_inputs(cfg, seed=48, ragged=True)
    a_q, b_q = make_query_factors(cfg, 4, seed=48)
    dims = dims_of(cfg)
    cache, cap = fill_cache(inp, dims)
    h, dh = cfg.h, cfg.d_h
    mc = int(inp.ctx_len.max())
    out = torch.empty((2, 3, h, dh), device="cuda")
    lse = torch.empty((2, 3, h), device="cuda")
    ws = kpa.alloc_workspace(dims, 2, mc, 3)
    kpa.kpa_decode_factored(dims, 4, cache, 2, cap, inp.ctx_len.cuda(), mc, 3, 1, a_q.cuda(), b_q.cuda(),
                            inp.q_pos.cuda(), out, lse, ws)
    torch.cuda.synchronize()
    q = kpa_ref.query_from_factors(a_q.numpy(), b_q.numpy())
    ro, rl = kpa_oracle.decode(inp.a_k, inp.b_k, inp.a_v, inp.b_v, inp.positions, inp.ctx_len, q, inp.q_pos)
    assert_close(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl, cfg.dtype,
                 f"{cfg.name} factored", scale=scale_of(inp, q=q))
