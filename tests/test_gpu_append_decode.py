"""kpa_append_decode: one decode step (append the step's tokens, then decode)
through the C ABI.

The fused step must leave the same cache bytes and give the same outputs,
bit for bit, as kpa_cache_append followed by kpa_decode_multiq on the same
inputs; and, with the step's tokens in place, the decode must match the
float64 oracle.  Before the step the new tokens' slots hold other tokens'
factors, so a step that skipped or misplaced its append would read them.
Cases cover every kernel shape (head splits included), new tokens in the first tile of a KV chunk
(one-tile chunks), tokens straddling two chunks, ragged contexts, the
vector-ALU path (append kernel launched first), an out-of-range slot,
n_new = 0, more new tokens than queries, and new tokens written past the
context (stored, but not read by this step's decode).
"""
import numpy as np
import pytest
import torch

import factorized_kv_cache_kpa_amd as kpa
from oracle import kpa_oracle
from tests.kpa_testutil import assert_close, dims_of, fill_cache, scale_of
from workloads import CONFIGS, flashtpa_config, headsplit_config, make_inputs

pytestmark = pytest.mark.gpu


def _new_tokens(inp, n_new, dev="cuda"):
    """The last n_new tokens of each sequence's context: factors, positions, slot0."""
    slot0 = (inp.ctx_len - n_new).to(torch.int32)
    idx = slot0.view(-1, 1).long() + torch.arange(n_new).view(1, -1)
    pick = lambda t: torch.stack([t[b, idx[b]] for b in range(inp.batch)]).contiguous().to(dev)
    return (pick(inp.a_k), pick(inp.b_k), pick(inp.a_v), pick(inp.b_v), pick(inp.positions),
            slot0.contiguous().to(dev))


def _stale_copy(inp, dims, cap, n_new, seed):
    """Two caches holding every slot of inp except the step's tokens, whose
    slots hold another seed's factors at the same positions."""
    cache, _ = fill_cache(inp, dims, capacity=cap)
    cfg = inp.cfg
    junk = make_inputs(cfg, seed=seed + 100, batch=inp.batch, ctx=inp.slots)
    jt = _new_tokens(junk, n_new)
    ak, bk, av, bv, _, _ = jt
    pos, slot0 = _new_tokens(inp, n_new)[4:]
    kpa.kpa_cache_append(dims, cache, inp.batch, cap, ak, bk, av, bv, pos, slot0, n_new=n_new)
    torch.cuda.synchronize()
    return cache, cache.clone()


def _step(inp, dims, cache, cap, n_new, fused, num_splits=0, causal=True, status=None, slot0=None, new=None):
    """One step: append n_new tokens (by default the last n_new of each
    context, else `new` = (a_k, b_k, a_v, b_v, positions, slot0)), then decode
    inp's queries over inp.ctx_len; fused or as two calls."""
    nb, nq = inp.batch, inp.q.shape[1]
    h, dh = dims.h, dims.d_h
    mc = int(inp.ctx_len.max().item())
    ak, bk, av, bv, pos, s0 = _new_tokens(inp, n_new) if new is None else new
    if slot0 is not None:
        s0 = slot0
    q = inp.q.cuda().contiguous()
    qp = inp.q_pos.cuda().contiguous()
    ctx = inp.ctx_len.cuda().contiguous()
    out = torch.full((nb, nq, h, dh), float("nan"), device="cuda")
    lse = torch.full((nb, nq, h), float("nan"), device="cuda")
    ws = kpa.alloc_workspace(dims, nb, mc, nq, num_splits)
    if fused:
        kpa.kpa_append_decode(dims, cache, nb, cap, ak, bk, av, bv, pos, s0, ctx, mc, nq, causal, q, qp, out, lse,
                              ws, num_splits, n_new=n_new, dev_status=status)
    else:
        kpa.kpa_cache_append(dims, cache, nb, cap, ak, bk, av, bv, pos, s0, n_new=n_new, dev_status=status)
        kpa.kpa_decode_multiq(dims, cache, nb, cap, ctx, mc, nq, causal, q, qp, out, lse, ws, num_splits,
                              dev_status=status)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


CASES = [
    # name, batch, ctx, n_q, ragged, num_splits
    ("kpa_32k", 3, 2000, 1, True, 0),
    ("kpa_32k", 2, 777, 1, False, 25),     # one-tile chunks: the new token opens its chunk
    ("long_512k", 1, 3000, 1, False, 0),
    ("long_512k", 2, 1025, 1, True, 33),
    ("multiq_16", 2, 600, 16, True, 0),
    ("multiq_16", 2, 590, 16, False, 19),  # the 16 new tokens straddle two one-tile chunks
    ("multiq_16", 2, 500, 1, True, 0),     # one query on the multi-query shape
    ("tpa_degenerate", 4, 1000, 1, True, 0),
    ("tiny_f32", 2, 301, 1, True, 0),      # vector-ALU path: append kernel, then decode
    ("flashtpa_h32", 2, 4100, 1, True, 0),
    ("split_8x2", 3, 1000, 1, True, 0),    # the KPA page's head splits: 8-wide contraction
    ("split_10x2", 3, 900, 1, True, 0),    # two waves per F head
    ("split_6x2", 2, 777, 1, False, 25),   # two waves per F head, one-tile chunks
    ("split_4x5", 2, 1100, 1, True, 0),    # F = A, rows not a multiple of 32
]


def _cfg(name):
    if name == "flashtpa_h32":
        return flashtpa_config(32, 2, 4100)
    if name.startswith("split_"):
        p1, p2 = (int(x) for x in name[len("split_"):].split("x"))
        return headsplit_config(p1, p2, 2, 1024)
    return CONFIGS[name]


@pytest.mark.parametrize("name,batch,ctx,n_q,ragged,num_splits", CASES)
def test_fused_step_equals_append_then_decode(gpu_lib, name, batch, ctx, n_q, ragged, num_splits):
    cfg = _cfg(name)
    inp = make_inputs(cfg, seed=21, batch=batch, ctx=ctx, n_q=n_q, ragged=ragged)
    dims = dims_of(cfg)
    n_new = n_q
    cache_seq, cache_fused = _stale_copy(inp, dims, ctx, n_new, seed=21)
    so, sl = _step(inp, dims, cache_seq, ctx, n_new, fused=False, num_splits=num_splits)
    fo, fl = _step(inp, dims, cache_fused, ctx, n_new, fused=True, num_splits=num_splits)
    assert torch.equal(cache_seq, cache_fused), "cache bytes differ"
    assert np.array_equal(so, fo) and np.array_equal(sl, fl, equal_nan=True), "outputs differ"
    ro, rl = kpa_oracle.decode(inp.a_k, inp.b_k, inp.a_v, inp.b_v, inp.positions, inp.ctx_len,
                               inp.q, inp.q_pos, causal=True)
    assert_close(fo.astype(np.float64), fl.astype(np.float64), ro, rl, cfg.dtype, f"{name} fused step",
                 scale=scale_of(inp), path=kpa.kpa_decode_path(dims, inp.q.shape[1]))


def test_fused_step_without_new_tokens_is_the_decode(gpu_lib):
    cfg = CONFIGS["kpa_32k"]
    inp = make_inputs(cfg, seed=22, batch=2, ctx=300, ragged=True)
    dims = dims_of(cfg)
    cache, cap = fill_cache(inp, dims)
    before = cache.clone()
    nb, h, dh = inp.batch, dims.h, dims.d_h
    q = inp.q.cuda().contiguous()
    qp = inp.q_pos.cuda().contiguous()
    ctx = inp.ctx_len.cuda()
    outs = []
    for fused in (False, True):
        out = torch.empty((nb, 1, h, dh), device="cuda")
        lse = torch.empty((nb, 1, h), device="cuda")
        ws = kpa.alloc_workspace(dims, nb, cap, 1)
        if fused:
            kpa.kpa_append_decode(dims, cache, nb, cap, None, None, None, None, None, None, ctx, cap, 1, 1, q, qp,
                                  out, lse, ws, n_new=0)
        else:
            kpa.kpa_decode(dims, cache, nb, cap, ctx, cap, q.view(nb, h, dh), qp.view(nb), out.view(nb, h, dh),
                           lse.view(nb, h), ws)
        torch.cuda.synchronize()
        outs.append((out.cpu(), lse.cpu()))
    assert torch.equal(cache, before)
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_fused_step_flags_an_out_of_range_slot_like_the_append(gpu_lib):
    # sequence 1's new token points past the capacity: skipped and flagged,
    # the decode still runs over what the cache holds
    cfg = CONFIGS["kpa_32k"]
    inp = make_inputs(cfg, seed=23, batch=2, ctx=400)
    dims = dims_of(cfg)
    cache_seq, cache_fused = _stale_copy(inp, dims, 400, 1, seed=23)
    bad = torch.tensor([399, 400], dtype=torch.int32, device="cuda")
    res = []
    for cache, fused in ((cache_seq, False), (cache_fused, True)):
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        res.append(_step(inp, dims, cache, 400, 1, fused, status=status, slot0=bad) + (int(status.item()),))
    assert torch.equal(cache_seq, cache_fused)
    assert res[0][2] == res[1][2] == 1  # KPA_DEV_SLOT_OUT_OF_RANGE
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])


@pytest.mark.parametrize("name", ["kpa_32k", "multiq_16"])
def test_fused_step_full_size_equals_append_then_decode(gpu_lib, name):
    """At the configuration's real size, in the launch configuration the
    benchmark times: bit-identical outputs and cache bytes."""
    cfg = CONFIGS[name]
    inp = make_inputs(cfg, seed=24)
    dims = dims_of(cfg)
    n_new = cfg.n_q
    cache_seq, cache_fused = _stale_copy(inp, dims, cfg.ctx, n_new, seed=24)
    so, sl = _step(inp, dims, cache_seq, cfg.ctx, n_new, fused=False)
    fo, fl = _step(inp, dims, cache_fused, cfg.ctx, n_new, fused=True)
    assert np.all(np.isfinite(fo))
    assert torch.equal(cache_seq, cache_fused), "cache bytes differ"
    assert np.array_equal(so, fo) and np.array_equal(sl, fl), "outputs differ"


MORE_CASES = [
    # name, batch, ctx, n_new, ragged, num_splits  (one query)
    ("kpa_32k", 2, 770, 3, False, 25),          # slots 767 .. 769: one-tile chunks 23 and 24
    ("tpa_degenerate", 2, 642, 5, False, 21),   # slots 637 .. 641 straddle chunks 19 and 20
    ("long_512k", 2, 1000, 40, True, 0),
    ("multiq_16", 2, 530, 9, True, 0),
]


@pytest.mark.parametrize("name,batch,ctx,n_new,ragged,num_splits", MORE_CASES)
def test_fused_step_with_more_new_tokens_than_queries(gpu_lib, name, batch, ctx, n_new, ragged, num_splits):
    cfg = _cfg(name)
    inp = make_inputs(cfg, seed=25, batch=batch, ctx=ctx, n_q=1, ragged=ragged)
    if ragged:  # every context holds the step's tokens
        inp.ctx_len.clamp_(min=n_new)
        inp.q_pos.copy_(inp.ctx_len.view(-1, 1) - 1)
    dims = dims_of(cfg)
    cache_seq, cache_fused = _stale_copy(inp, dims, ctx, n_new, seed=25)
    so, sl = _step(inp, dims, cache_seq, ctx, n_new, fused=False, num_splits=num_splits)
    fo, fl = _step(inp, dims, cache_fused, ctx, n_new, fused=True, num_splits=num_splits)
    assert torch.equal(cache_seq, cache_fused), "cache bytes differ"
    assert np.array_equal(so, fo) and np.array_equal(sl, fl, equal_nan=True), "outputs differ"
    ro, rl = kpa_oracle.decode(inp.a_k, inp.b_k, inp.a_v, inp.b_v, inp.positions, inp.ctx_len,
                               inp.q, inp.q_pos, causal=True)
    assert_close(fo.astype(np.float64), fl.astype(np.float64), ro, rl, cfg.dtype, f"{name} fused step",
                 scale=scale_of(inp), path=kpa.kpa_decode_path(dims, inp.q.shape[1]))


PAST_CASES = [
    # name, batch, ctx, n_new, gap past the context, extra capacity, ragged, num_splits
    ("kpa_32k", 2, 700, 1, 0, 64, True, 0),       # right after the context, same tile or the next
    ("kpa_32k", 2, 704, 2, 0, 64, False, 22),     # one-tile chunks: slot 704 is past the last chunk
    ("kpa_32k", 2, 704, 1, 50, 96, False, 0),     # far past the context
    ("long_512k", 2, 1500, 3, 7, 64, True, 0),
    ("tpa_degenerate", 3, 400, 2, 31, 80, True, 13),
]


@pytest.mark.parametrize("name,batch,ctx,n_new,gap,extra,ragged,num_splits", PAST_CASES)
def test_fused_step_writes_tokens_past_the_context(gpu_lib, name, batch, ctx, n_new, gap, extra, ragged, num_splits):
    """New tokens at slots ctx_len + gap ..: the step stores them like the
    append does, and its decode, over ctx_len slots, does not read them."""
    cfg = _cfg(name)
    inp = make_inputs(cfg, seed=26, batch=batch, ctx=ctx, n_q=1, ragged=ragged)
    dims = dims_of(cfg)
    cap = ctx + extra
    cache_seq, _ = fill_cache(inp, dims, capacity=cap)
    cache_fused = cache_seq.clone()
    junk = make_inputs(cfg, seed=126, batch=batch, ctx=n_new)
    slot0 = (inp.ctx_len + gap).to(torch.int32)
    assert int(slot0.max()) + n_new <= cap
    new = tuple(t.contiguous().cuda() for t in (junk.a_k, junk.b_k, junk.a_v, junk.b_v))
    new += ((slot0.view(-1, 1) + torch.arange(n_new, dtype=torch.int32).view(1, -1)).contiguous().cuda(),
            slot0.contiguous().cuda())
    res = []
    for cache, fused in ((cache_seq, False), (cache_fused, True)):
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        res.append(_step(inp, dims, cache, cap, n_new, fused, num_splits=num_splits, status=status, new=new)
                   + (int(status.item()),))
    assert res[0][2] == res[1][2] == 0
    assert torch.equal(cache_seq, cache_fused), "cache bytes differ"
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1]), "outputs differ"
    ro, rl = kpa_oracle.decode(inp.a_k, inp.b_k, inp.a_v, inp.b_v, inp.positions, inp.ctx_len,
                               inp.q, inp.q_pos, causal=True)
    assert_close(res[1][0].astype(np.float64), res[1][1].astype(np.float64), ro, rl, cfg.dtype,
                 f"{name} step with tokens past the context", scale=scale_of(inp),
                 path=kpa.kpa_decode_path(dims, inp.q.shape[1]))


def test_fused_step_flags_a_slot_near_the_int32_limit_like_the_append(gpu_lib):
    # sequence 0's four new tokens start 2 slots below 2^31 (the last two
    # slots past the int32 range): all skipped and flagged on both paths
    cfg = CONFIGS["kpa_32k"]
    inp = make_inputs(cfg, seed=29, batch=2, ctx=400)
    dims = dims_of(cfg)
    cache_seq, cache_fused = _stale_copy(inp, dims, 400, 4, seed=29)
    bad = torch.tensor([2 ** 31 - 2, 396], dtype=torch.int32, device="cuda")
    res = []
    for cache, fused in ((cache_seq, False), (cache_fused, True)):
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        res.append(_step(inp, dims, cache, 400, 4, fused, status=status, slot0=bad) + (int(status.item()),))
    assert torch.equal(cache_seq, cache_fused)
    assert res[0][2] == res[1][2] == 1  # KPA_DEV_SLOT_OUT_OF_RANGE
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
