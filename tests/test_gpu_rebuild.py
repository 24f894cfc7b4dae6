"""The multi-query decode that rebuilds K and V per tile on the matrix cores
(kpa_decode_path "mfma_rebuild") against the float64 oracle, through the C
ABI.

K_s and V_s are rebuilt from their factors ([KPA] Eqs. (3)-(4), Def. 2.1)
and attended with the dense query.  Cases span the kernel's family: B head
counts 2 / 4 / 6 / 8 (one wave each), A head counts 1 / 3 / 4 (one
workgroup each), ranks 1..4 for keys and values independently, 8..64
queries (one or several groups of 16 per sequence), causal and non-causal,
ragged contexts over several tiles with a ragged tail, one chunk (direct
output) and several (the merge), sharp softmaxes, a factored query, NaN
bytes past the context, and an empty sequence.  The same kernel with the
factors' roles swapped serves q1 = 8, q2 = 16 with p1 = 8 (long_512k's
split): its cases span B head counts 1 / 3 / 4 (the kernel's A role) and
12..40 queries.  Every output element is compared.
"""
import numpy as np
import pytest
import torch

import factorized_kv_cache_kpa_amd as kpa
from oracle import kpa_oracle, kpa_ref
from tests.kpa_testutil import assert_close, dims_of, fill_cache, run_decode, scale_of
from workloads import CONFIGS, make_inputs, make_query_factors

pytestmark = pytest.mark.gpu

BASE = CONFIGS["multiq_16"]
SWAPPED = CONFIGS["long_512k"]  # q1 = 8, q2 = 16, p1 = 8


def _cfg(p1, p2, r_k, r_v, base=BASE):
    return base.scaled(name=f"rebuild_{p1}x{p2}_q{base.q1}x{base.q2}_r{r_k}{r_v}", p1=p1, p2=p2, r_k=r_k, r_v=r_v)


def _oracle(inp, causal=True, q=None):
    return kpa_oracle.decode(inp.a_k, inp.b_k, inp.a_v, inp.b_v, inp.positions, inp.ctx_len,
                             inp.q if q is None else q, inp.q_pos, causal=causal)


CASES = [
    # p1, p2, r_k, r_v, batch, ctx, n_q, ragged, causal, q_scale, num_splits
    (4, 8, 4, 4, 2, 700, 16, True, True, 1.0, 0),
    (4, 8, 4, 4, 2, 700, 16, True, True, 1.0, 1),     # one chunk: the kernel writes the output
    (4, 8, 4, 4, 3, 333, 8, True, True, 4.0, 5),      # sharp softmax, 8 queries (half a group)
    (4, 8, 4, 4, 2, 400, 20, False, True, 1.0, 0),    # two query groups, the second 4 wide
    (4, 8, 4, 4, 1, 260, 64, False, True, 1.0, 3),    # KPA_MAX_NQ: four groups
    (4, 8, 4, 4, 2, 500, 12, True, False, 1.0, 0),    # non-causal
    (1, 8, 1, 1, 2, 321, 16, True, True, 2.0, 0),     # rank one, one A head
    (3, 8, 2, 3, 2, 450, 16, True, True, 1.0, 4),     # mixed ranks, three A heads
    (4, 2, 4, 1, 2, 390, 9, True, True, 1.0, 0),      # two B heads (two waves)
    (3, 4, 3, 2, 2, 515, 16, True, True, 1.0, 6),     # four B heads
    (2, 6, 2, 4, 2, 610, 16, True, True, 1.0, 0),     # six B heads
]


SWAPPED_CASES = [
    # p1, p2, r_k, r_v, batch, ctx, n_q, ragged, causal, q_scale, num_splits  (q1 = 8, q2 = 16)
    (8, 4, 2, 4, 2, 520, 16, True, True, 1.0, 0),     # long_512k's split
    (8, 4, 2, 4, 2, 520, 16, True, True, 1.0, 1),     # one chunk: the kernel writes the output
    (8, 4, 2, 4, 1, 300, 40, False, True, 2.0, 3),    # three query groups, the last 8 wide
    (8, 3, 1, 3, 2, 333, 12, True, True, 4.0, 5),     # three B heads, sharp softmax
    (8, 1, 4, 1, 2, 410, 13, True, False, 1.0, 0),    # one B head, non-causal
]


def _check_rebuild(case, base):
    p1, p2, r_k, r_v, batch, ctx, n_q, ragged, causal, q_scale, ns = case
    cfg = _cfg(p1, p2, r_k, r_v, base)
    dims = dims_of(cfg)
    assert kpa.kpa_decode_path(dims, n_q) == "mfma_rebuild"
    inp = make_inputs(cfg, seed=41, batch=batch, ctx=ctx, n_q=n_q, ragged=ragged, q_scale=q_scale)
    cache, cap = fill_cache(inp, dims)
    go, gl = run_decode(inp, dims, cache, cap, num_splits=ns, causal=causal)
    ro, rl = _oracle(inp, causal=causal)
    assert_close(go, gl, ro, rl, cfg.dtype, cfg.name, scale=scale_of(inp), path="mfma_rebuild")


_IDS = lambda c: "p{}x{}_r{}{}_b{}_s{}_q{}_{}_{}_x{}_ns{}".format(*c)


@pytest.mark.parametrize("case", CASES, ids=_IDS)
def test_rebuild_matches_oracle(gpu_lib, case):
    _check_rebuild(case, BASE)


@pytest.mark.parametrize("case", SWAPPED_CASES, ids=_IDS)
def test_rebuild_swapped_matches_oracle(gpu_lib, case):
    _check_rebuild(case, SWAPPED)


@pytest.mark.parametrize("base", [BASE, SWAPPED], ids=["q16x8", "q8x16"])
def test_rebuild_factored_query(gpu_lib, base):
    cfg = base
    dims = dims_of(cfg)
    assert kpa.kpa_decode_path(dims, 16) == "mfma_rebuild"
    inp = make_inputs(cfg, seed=42, batch=2, ctx=480, n_q=16, ragged=True)
    a_q, b_q = make_query_factors(cfg, 6, seed=42, batch=2, n_q=16)
    cache, cap = fill_cache(inp, dims)
    nb, nq, h, dh = 2, 16, dims.h, dims.d_h
    mc = int(inp.ctx_len.max().item())
    out = torch.full((nb, nq, h, dh), float("nan"), device="cuda")
    lse = torch.full((nb, nq, h), float("nan"), device="cuda")
    ws = kpa.alloc_workspace(dims, nb, mc, nq)
    kpa.kpa_decode_factored(dims, 6, cache, nb, cap, inp.ctx_len.cuda(), mc, nq, 1, a_q.cuda().contiguous(),
                            b_q.cuda().contiguous(), inp.q_pos.cuda().contiguous(), out, lse, ws)
    torch.cuda.synchronize()
    q = kpa_ref.query_from_factors(a_q.numpy(), b_q.numpy())
    ro, rl = _oracle(inp, q=q)
    assert_close(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl, cfg.dtype,
                 "factored query", scale=scale_of(inp, q=q), path="mfma_rebuild")


@pytest.mark.parametrize("base", [BASE, SWAPPED], ids=["q16x8", "q8x16"])
def test_rebuild_ignores_nan_bytes_past_the_context(gpu_lib, base):
    cfg = base
    dims = dims_of(cfg)
    assert kpa.kpa_decode_path(dims, 16) == "mfma_rebuild"
    inp = make_inputs(cfg, seed=43, batch=2, ctx=150, n_q=16)
    inp.ctx_len[1] = 90                       # a ragged tail inside a tile
    inp.q_pos[1] = 90 - 16 + torch.arange(16, dtype=torch.int32)
    cap = 192
    cache = kpa.alloc_cache(dims, 2, cap)
    cache.fill_(0xFF)                         # NaN bit patterns everywhere
    kpa.kpa_cache_append(dims, cache, 2, cap, inp.a_k.cuda(), inp.b_k.cuda(), inp.a_v.cuda(), inp.b_v.cuda(),
                         inp.positions.cuda(), torch.zeros(2, dtype=torch.int32, device="cuda"), n_new=150)
    torch.cuda.synchronize()
    for ns in (1, 0):
        go, gl = run_decode(inp, dims, cache, cap, max_ctx=cap, num_splits=ns)
        ro, rl = _oracle(inp)
        assert_close(go, gl, ro, rl, cfg.dtype, f"NaN past the context, splits={ns}", scale=scale_of(inp),
                     path="mfma_rebuild")


def test_rebuild_empty_and_short_sequences(gpu_lib):
    # a sequence with no slots gives 0 / -inf; others shorter than a tile
    cfg = BASE
    dims = dims_of(cfg)
    inp = make_inputs(cfg, seed=44, batch=3, ctx=100, n_q=16, ragged=True)
    inp.ctx_len[:] = torch.tensor([0, 17, 100], dtype=torch.int32)
    inp.q_pos.copy_((inp.ctx_len.view(-1, 1) - 16 + torch.arange(16, dtype=torch.int32)).clamp(min=0))
    cache, cap = fill_cache(inp, dims)
    go, gl = run_decode(inp, dims, cache, cap, causal=False)
    ro, rl = _oracle(inp, causal=False)
    assert np.all(go[0] == 0) and np.all(np.isneginf(gl[0]))
    assert_close(go[1:], gl[1:], ro[1:], rl[1:], cfg.dtype, "short", scale=scale_of(inp)[1:], path="mfma_rebuild")


def test_rebuild_two_level_merge(gpu_lib):
    """More than 1024 forced chunks: the partials go through the two-level
    merge (arrival counters cleared by the decode kernel's first chunk)."""
    cfg = BASE
    dims = dims_of(cfg)
    inp = make_inputs(cfg, seed=45, batch=1, ctx=35200, n_q=8)
    cache, cap = fill_cache(inp, dims)
    for ns in (1100, 70):
        go, gl = run_decode(inp, dims, cache, cap, num_splits=ns)
        ro, rl = _oracle(inp)
        assert_close(go, gl, ro, rl, cfg.dtype, f"splits={ns}", scale=scale_of(inp), path="mfma_rebuild")


def test_rebuild_ctx_len_above_max_ctx_is_flagged(gpu_lib):
    cfg = BASE
    dims = dims_of(cfg)
    inp = make_inputs(cfg, seed=46, batch=2, ctx=64, n_q=16)
    cache, cap = fill_cache(inp, dims)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    nb, nq, h, dh = 2, 16, dims.h, dims.d_h
    out = torch.empty((nb, nq, h, dh), device="cuda")
    lse = torch.empty((nb, nq, h), device="cuda")
    ctx = torch.tensor([64, 40], dtype=torch.int32, device="cuda")
    ws = kpa.alloc_workspace(dims, nb, 40, nq)
    kpa.kpa_decode_multiq(dims, cache, nb, cap, ctx, 40, nq, 1, inp.q.cuda(), inp.q_pos.cuda(), out, lse, ws,
                          dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == kpa.KPA_DEV_CTX_OUT_OF_RANGE
    # zero sequences: nothing to do, no error
    kpa.kpa_decode_multiq(dims, cache, 0, cap, ctx, 40, nq, 1, inp.q.cuda(), inp.q_pos.cuda(), out, lse, ws,
                          dev_status=status)
    torch.cuda.synchronize()
