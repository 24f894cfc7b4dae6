"""GPU decode parity against the float64 oracle, through the C ABI.

Small cases compare every output element with the oracle; they span several
32-slot tiles, a ragged tail, ragged per-sequence contexts and several KV
chunks.  Full-size cases (every config at its real shape, in the launch
configuration the benchmark times) compare every (sequence, query, head)
row with the streaming oracle.
"""
import numpy as np
import pytest
import torch

import factorized_kv_cache_kpa_amd as kpa
from oracle import kpa_oracle
from tests.kpa_testutil import assert_close, dims_of, fill_cache, rel_err, run_decode, scale_of
from workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu


def _oracle(inp, causal=True, items=None):
    return kpa_oracle.decode(inp.a_k, inp.b_k, inp.a_v, inp.b_v, inp.positions, inp.ctx_len,
                             inp.q, inp.q_pos, causal=causal, items=items)


SMALL = [
    # name, batch, ctx, n_q, ragged, q_scale
    ("tiny_f32", 1, 256, 1, False, 1.0),
    ("tiny_f32", 3, 301, 1, True, 4.0),
    ("tpa_degenerate", 4, 1000, 1, True, 1.0),
    ("kpa_32k", 3, 2000, 1, True, 1.0),
    ("kpa_32k", 2, 777, 1, False, 8.0),      # sharp softmax
    ("long_512k", 1, 3000, 1, False, 1.0),
    ("multiq_16", 2, 600, 16, True, 1.0),
    ("multiq_16", 1, 16, 16, False, 2.0),    # the chunk is the whole context
    ("multiq_16", 2, 500, 1, True, 3.0),     # one query on the multi-query shape (F = A orientation)
    ("long_512k", 2, 45, 1, True, 1.0),      # contexts shorter than two tiles
]


def test_decode_rank_one_kpa(gpu_lib):
    cfg = CONFIGS["kpa_32k"].scaled(r_k=1, r_v=1)
    inp = make_inputs(cfg, seed=12, batch=2, ctx=333, ragged=True, q_scale=2.0)
    dims = dims_of(cfg)
    cache, cap = fill_cache(inp, dims)
    go, gl = run_decode(inp, dims, cache, cap)
    ro, rl = _oracle(inp)
    assert_close(go, gl, ro, rl, cfg.dtype, "rank one", scale=scale_of(inp))


def _headsplit(p1, p2):
    from workloads import headsplit_config
    return headsplit_config(p1, p2, 2, 256)


NAN_CASES = [
    # config, ctx (the last tile holds ctx % 32 slots), n_q, forced chunks
    ("kpa_32k", 100, 1, 0),
    ("long_512k", 101, 1, 0),    # strided chunks, the weights folded on the matrix cores
    ("long_512k", 197, 1, 2),    # ... two strided chunks: tiles 0, 2, 4 and 1, 3, 5
    ("tpa_degenerate", 99, 1, 0),  # the weights folded on the vector ALU (G feature dimension 1)
    ("split_5x5", 71, 1, 0),     # 8-wide F, padded rows
    ("split_4x5", 125, 1, 3),
    ("multiq_16", 77, 3, 0),     # several queries per workgroup (factor-space kernel)
]


@pytest.mark.parametrize("name,ctx,n_q,num_splits", NAN_CASES)
def test_garbage_past_the_context_is_ignored(gpu_lib, name, ctx, n_q, num_splits):
    # slots past ctx_len hold NaN bit patterns; the result must not see them
    cfg = _headsplit(*(int(x) for x in name[6:].split("x"))) if name.startswith("split_") else CONFIGS[name]
    inp = make_inputs(cfg, seed=13, batch=2, ctx=ctx, n_q=n_q)
    dims = dims_of(cfg)
    cap = (ctx + 31) // 32 * 32 + 32
    nan_cache = kpa.alloc_cache(dims, 2, cap)
    nan_cache.fill_(0xFF)
    kpa.kpa_cache_append(dims, nan_cache, 2, cap, inp.a_k.cuda(), inp.b_k.cuda(), inp.a_v.cuda(), inp.b_v.cuda(),
                         inp.positions.cuda(), torch.zeros(2, dtype=torch.int32, device="cuda"), n_new=ctx)
    torch.cuda.synchronize()
    go, gl = run_decode(inp, dims, nan_cache, cap, max_ctx=cap, num_splits=num_splits)
    ro, rl = _oracle(inp)
    assert_close(go, gl, ro, rl, cfg.dtype, f"{name}: NaN past the context", scale=scale_of(inp),
                 path=kpa.kpa_decode_path(dims, n_q))


@pytest.mark.parametrize("name,batch,ctx,n_q,ragged,q_scale", SMALL)
def test_decode_matches_oracle_small(gpu_lib, name, batch, ctx, n_q, ragged, q_scale):
    cfg = CONFIGS[name]
    inp = make_inputs(cfg, seed=11, batch=batch, ctx=ctx, n_q=n_q, ragged=ragged, q_scale=q_scale)
    dims = dims_of(cfg)
    cache, cap = fill_cache(inp, dims)
    go, gl = run_decode(inp, dims, cache, cap)
    ro, rl = _oracle(inp)
    assert_close(go, gl, ro, rl, cfg.dtype, f"{name} b{batch} ctx{ctx}", scale=scale_of(inp),
                 path=kpa.kpa_decode_path(dims, n_q))


@pytest.mark.parametrize("name", ["tiny_f32", "kpa_32k", "multiq_16"])
def test_split_count_invariance(gpu_lib, name):
    cfg = CONFIGS[name]
    inp = make_inputs(cfg, seed=5, batch=2, ctx=900, ragged=True)
    dims = dims_of(cfg)
    cache, cap = fill_cache(inp, dims)
    # the matrix-core path rounds the weighted value operand to bf16 against each
    # chunk's own running max, so chunkings agree to that rounding (at most 2^-8
    # relative per term in each of the two results)
    path = kpa.kpa_decode_path(dims, inp.q.shape[1])
    tol = 1e-5 if path == "valu" else 1e-2
    ro, rl = _oracle(inp)
    base_o, base_l = run_decode(inp, dims, cache, cap, num_splits=1)
    for s in (2, 7, 29, 0):
        o, l = run_decode(inp, dims, cache, cap, num_splits=s)
        assert rel_err(o, base_o).max() <= tol, s
        assert np.allclose(l, base_l, atol=1e-5), s
        assert_close(o, l, ro, rl, cfg.dtype, f"splits={s}", scale=scale_of(inp), path=path)


def test_non_causal_multi_query(gpu_lib):
    cfg = CONFIGS["multiq_16"]
    inp = make_inputs(cfg, seed=6, batch=2, ctx=300, n_q=5)
    dims = dims_of(cfg)
    cache, cap = fill_cache(inp, dims)
    go, gl = run_decode(inp, dims, cache, cap, causal=False)
    ro, rl = _oracle(inp, causal=False)
    assert_close(go, gl, ro, rl, cfg.dtype, "non-causal", scale=scale_of(inp))


MULTI_CASES = [
    # config (its shape), batch, ctx, n_q, ragged, causal, forced chunks
    ("kpa_32k", 3, 700, 2, True, True, 0),
    ("kpa_32k", 2, 1000, 5, False, True, 7),
    ("kpa_32k", 2, 530, 16, True, True, 0),
    ("kpa_32k", 2, 300, 9, False, False, 0),
    ("long_512k", 2, 650, 3, True, True, 0),
    ("long_512k", 1, 1100, 16, False, True, 5),
    ("long_512k", 2, 260, 6, True, False, 0),
    ("long_512k", 2, 400, 9, True, True, 0),
    ("long_512k", 2, 480, 12, True, False, 3),
]


@pytest.mark.parametrize("name,batch,ctx,n_q,ragged,causal,num_splits", MULTI_CASES)
def test_multi_query_on_the_single_query_shapes(gpu_lib, name, batch, ctx, n_q, ragged, causal, num_splits):
    """Several queries per sequence on kpa_32k's and long_512k's head and
    feature splits (tuned multi-query matrix-core kernels; on long_512k's
    split K and V rebuilt per tile from 12 queries): every output element
    against the oracle, query counts that leave a query group partly filled,
    causal and not, automatic and forced chunk counts."""
    cfg = CONFIGS[name]
    inp = make_inputs(cfg, seed=31, batch=batch, ctx=ctx, n_q=n_q, ragged=ragged)
    dims = dims_of(cfg)
    path = kpa.kpa_decode_path(dims, n_q)
    assert path == ("mfma_rebuild" if name == "long_512k" and n_q >= 12 else "mfma_bf16")
    cache, cap = fill_cache(inp, dims)
    go, gl = run_decode(inp, dims, cache, cap, causal=causal, num_splits=num_splits)
    ro, rl = _oracle(inp, causal=causal)
    assert_close(go, gl, ro, rl, cfg.dtype, f"{name} n_q={n_q}", scale=scale_of(inp), path=path)


def test_multi_query_row_equals_truncated_single_query(gpu_lib):
    cfg = CONFIGS["multiq_16"]
    inp = make_inputs(cfg, seed=8, batch=2, ctx=200, n_q=4)
    dims = dims_of(cfg)
    cache, cap = fill_cache(inp, dims)
    go, gl = run_decode(inp, dims, cache, cap)
    for n in range(4):
        sub = make_inputs(cfg, seed=8, batch=2, ctx=200, n_q=4)
        sub.q = inp.q[:, n:n + 1].contiguous()
        sub.q_pos = inp.q_pos[:, n:n + 1].contiguous()
        sub.ctx_len = inp.ctx_len - 4 + n + 1
        o1, l1 = run_decode(sub, dims, cache, cap)
        # the two calls may take different kernel paths; the matrix-core path
        # rounds the weighted value operand to bf16 (2^-8 relative per term)
        paths = {kpa.kpa_decode_path(dims, 4), kpa.kpa_decode_path(dims, 1)}
        tol = 1e-5 if paths == {"valu"} else 1e-2
        assert rel_err(go[:, n], o1[:, 0]).max() <= tol


def test_empty_context_and_zero_batch(gpu_lib):
    cfg = CONFIGS["kpa_32k"]
    inp = make_inputs(cfg, seed=9, batch=3, ctx=100)
    dims = dims_of(cfg)
    cache, cap = fill_cache(inp, dims)
    inp.ctx_len[1] = 0
    go, gl = run_decode(inp, dims, cache, cap, num_splits=3)
    assert np.all(go[1] == 0) and np.all(np.isneginf(gl[1]))
    ro, rl = _oracle(inp)
    assert_close(go, gl, ro, rl, cfg.dtype, "ragged with empty", scale=scale_of(inp))
    # every sequence empty, max_ctx = 0
    inp.ctx_len[:] = 0
    go, gl = run_decode(inp, dims, cache, cap, max_ctx=0)
    assert np.all(go == 0) and np.all(np.isneginf(gl))


def test_ctx_len_above_max_ctx_is_flagged(gpu_lib):
    cfg = CONFIGS["kpa_32k"]
    inp = make_inputs(cfg, seed=10, batch=2, ctx=64)
    dims = dims_of(cfg)
    cache, cap = fill_cache(inp, dims)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.empty((2, dims.h, dims.d_h), device="cuda")
    ctx = torch.tensor([64, 40], dtype=torch.int32, device="cuda")
    ws = kpa.alloc_workspace(dims, 2, 40)
    kpa.kpa_decode(dims, cache, 2, cap, ctx, 40, inp.q.cuda().view(2, dims.h, dims.d_h),
                   inp.q_pos.cuda().view(2), out, None, ws, dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == kpa.KPA_DEV_CTX_OUT_OF_RANGE


@pytest.mark.parametrize("name", ["tpa_degenerate", "kpa_32k", "long_512k", "multiq_16"])
def test_decode_full_size_every_row(gpu_lib, name):
    """Every config at its real shape, with the automatic chunk count the
    benchmark uses: every (sequence, query, head) row against the streaming
    float64 oracle."""
    cfg = CONFIGS[name]
    inp = make_inputs(cfg, seed=0)
    dims = dims_of(cfg)
    cache, cap = fill_cache(inp, dims)
    go, gl = run_decode(inp, dims, cache, cap)
    del cache
    ro, rl = _oracle(inp)
    assert_close(go, gl, ro, rl, cfg.dtype, f"{name} full size", scale=scale_of(inp),
                 path=kpa.kpa_decode_path(dims, inp.q.shape[1]))


def test_kernel_timing_hook_brackets_the_decode_kernel(gpu_lib):
    """The measurement hook records its events around the split-KV kernel
    only: that interval is positive and no longer than the whole call's, and
    the results do not change."""
    cfg = CONFIGS["kpa_32k"]
    inp = make_inputs(cfg, seed=11, batch=2, ctx=4096)
    dims = dims_of(cfg)
    cache, cap = fill_cache(inp, dims)
    ref_o, ref_l = run_decode(inp, dims, cache, cap, num_splits=8)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record()
    kpa.kpa_time_next_decode_kernel(ev[1], ev[2])
    go, gl = run_decode(inp, dims, cache, cap, num_splits=8)
    ev[3].record()
    torch.cuda.synchronize()
    t_kernel = ev[1].elapsed_time(ev[2])
    t_call = ev[0].elapsed_time(ev[3])
    assert 0.0 < t_kernel <= t_call
    assert np.array_equal(go, ref_o) and np.array_equal(gl, ref_l)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_odd_shape_and_two_level_merge(gpu_lib, dtype):
    """A shape no matrix-core kernel covers (d_h = 18, not a multiple of 4;
    ranks 3 and 1) on the general kernel, with chunk counts that take the
    single-level merge and the two-level merge (more than 64 chunks)."""
    cfg = CONFIGS["tiny_f32"].scaled(name="odd", p1=3, p2=5, q1=3, q2=6, r_k=3, r_v=1, dtype=dtype,
                                     sigma_a=0.3, sigma_b=0.3)
    inp = make_inputs(cfg, seed=12, batch=2, ctx=2400, ragged=True)
    inp.ctx_len[0] = 2400  # at least 75 tiles in one sequence
    dims = dims_of(cfg)
    cache, cap = fill_cache(inp, dims)
    ro, rl = _oracle(inp)
    for s in (1, 9, 75):
        go, gl = run_decode(inp, dims, cache, cap, num_splits=s)
        assert_close(go, gl, ro, rl, dtype, f"odd shape, splits={s}", scale=scale_of(inp))


@pytest.mark.parametrize("name,batch,ctx", [("kpa_32k", 32, 8192), ("long_512k", 1, 40000)])
def test_garbage_workspace_and_repeated_calls(gpu_lib, name, batch, ctx):
    """The workspace is caller scratch: fill it with random bytes, use it for
    several calls in a row with the automatic chunk count, and check every
    call against the oracle (ragged contexts, one of them empty)."""
    cfg = CONFIGS[name]
    inp = make_inputs(cfg, seed=13, batch=batch, ctx=ctx, ragged=True)
    inp.ctx_len[0] = ctx
    if batch > 2:
        inp.ctx_len[1] = 0
        inp.ctx_len[2] = 33
    dims = dims_of(cfg)
    cache, cap = fill_cache(inp, dims)
    ro, rl = _oracle(inp)
    h, dh = dims.h, dims.d_h
    ws = kpa.alloc_workspace(dims, batch, ctx)
    g = torch.Generator(device="cuda").manual_seed(3)
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda", generator=g))
    q = inp.q.cuda().view(batch, h, dh)
    qp = inp.q_pos.cuda().view(batch)
    cl = inp.ctx_len.cuda()
    for call in range(3):
        out = torch.full((batch, h, dh), float("nan"), device="cuda")
        lse = torch.full((batch, h), float("nan"), device="cuda")
        kpa.kpa_decode(dims, cache, batch, cap, cl, ctx, q, qp, out, lse, ws)
        torch.cuda.synchronize()
        go = out.cpu().numpy().astype(np.float64)[:, None]
        gl = lse.cpu().numpy().astype(np.float64)[:, None]
        assert_close(go, gl, ro, rl, cfg.dtype, f"{name} call {call}", scale=scale_of(inp))


@pytest.mark.parametrize("p1,p2", [(8, 2), (4, 4), (2, 8), (10, 2), (4, 5), (2, 10), (5, 5),
                                   (6, 2), (4, 3), (3, 4), (2, 6)])
def test_head_split_shapes_match_oracle(gpu_lib, p1, p2):
    """The head splits the KPA page ablates (d1 = d2 = 8, R_K = R_V = 2), on
    the matrix cores (8-wide contraction): ragged contexts over several
    chunks, automatic and forced chunk counts."""
    from workloads import SWEEP_SHAPES, headsplit_config
    assert (p1, p2) in SWEEP_SHAPES
    cfg = headsplit_config(p1, p2, 3, 330)
    inp = make_inputs(cfg, seed=20, ragged=True)  # lengths 274, 94, 127
    dims = dims_of(cfg)
    assert kpa.kpa_decode_path(dims, 1) == "mfma_bf16"
    cache, cap = fill_cache(inp, dims)
    ro, rl = _oracle(inp)
    for s in (0, 3):
        go, gl = run_decode(inp, dims, cache, cap, num_splits=s)
        assert_close(go, gl, ro, rl, cfg.dtype, f"split {p1}x{p2} splits={s}", scale=scale_of(inp))


@pytest.mark.parametrize("h", [16, 32, 48])
def test_flashtpa_shapes_match_oracle(gpu_lib, h):
    """FlashTPA's benchmark shapes (TPA split, d_h = 64, R_K = R_V = 1) on their
    matrix-core instantiations: ragged contexts over several chunks."""
    from workloads import flashtpa_config
    cfg = flashtpa_config(h, 3, 2100)
    inp = make_inputs(cfg, seed=14, ragged=True)
    dims = dims_of(cfg)
    assert kpa.kpa_decode_path(dims, 1) == "mfma_bf16"
    cache, cap = fill_cache(inp, dims)
    ro, rl = _oracle(inp)
    for s in (0, 5):
        go, gl = run_decode(inp, dims, cache, cap, num_splits=s)
        assert_close(go, gl, ro, rl, cfg.dtype, f"flashtpa h={h} splits={s}", scale=scale_of(inp))
