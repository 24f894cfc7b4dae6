"""kpa_project_append on the GPU: the factor projection of hidden states
([KPA] Eq. (5), one stacked weight) written straight into the cache, against
the float64 oracle's projection and rotation.

Decode-step token counts run the small kernel (32 x 32 tiles); from 1024
tokens on, the LDS-tiled one.  Each stored value must lie within half a unit
in the last place of the cache type (bf16: 8 significant bits) plus the
float32 accumulation bound
d_model * 2^-24 * sum_c |w x| of the exact float64 value.  Slots the call does
not own stay untouched, positions are recorded, and an out-of-range slot is
flagged and skipped.  An end-to-end case decodes over a projected cache and
compares with the oracle's decode of the unrounded projected factors.
"""
import numpy as np
import pytest
import torch

import factorized_kv_cache_kpa_amd as kpa
from oracle import kpa_oracle, kpa_ref
from tests.kpa_testutil import assert_close, dims_of, score_scale
from tests.test_gpu_append import unpack
from workloads import CONFIGS, flashtpa_config

pytestmark = pytest.mark.gpu


def _inputs(cfg, batch, n_new, d_model, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((batch, n_new, d_model), generator=g).to(torch.bfloat16)
    n_feat = (cfg.r_k + cfg.r_v) * (cfg.p1 * cfg.q1 + cfg.p2 * cfg.q2)
    w = (torch.randn((n_feat, d_model), generator=g) / d_model ** 0.5).to(torch.bfloat16)
    return x, w


def _bf16_ulp(v):
    a = np.maximum(np.abs(v), 1e-30)
    return np.exp2(np.floor(np.log2(a)) - 7)


def _check_set(got, want, bound, dtype, what):
    if dtype == "f32":
        tol = bound + np.abs(want) * 2.0 ** -24
    else:
        tol = 0.5 * _bf16_ulp(np.maximum(np.abs(want), np.abs(got))) + bound
    err = np.abs(got - want)
    assert np.all(err <= tol * (1 + 1e-12) + 1e-30), f"{what}: max excess {(err - tol).max():.3e}"


def _to_f64(raw, dtype):
    if dtype == "f32":
        return raw.astype(np.float64)
    return (raw.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


SHAPES = [
    # name, batch, n_new, d_model, capacity
    ("kpa_32k", 32, 1, 2048, 64),
    ("kpa_32k", 3, 40, 256, 128),       # several row and token blocks, ragged token tail
    ("long_512k", 2, 5, 4096, 40),
    ("multiq_16", 8, 16, 4096, 48),
    ("tpa_degenerate", 16, 1, 768, 32),  # 304 factor rows: a partial row block
    ("tiny_f32", 2, 7, 64, 16),          # float32 cache
    ("flashtpa_h48", 3, 2, 3072, 36),
    # from 1024 tokens on, the LDS-tiled kernel (128 rows x 128 tokens per workgroup)
    ("kpa_32k", 4, 600, 2048, 640),      # 2400 tokens: a ragged token tile
    ("tpa_degenerate", 3, 700, 768, 704),  # F = 304: a partial row tile
    ("tiny_f32", 2, 600, 64, 640),       # float32 cache, one d_model step, F = 64
    ("long_512k", 1, 1024, 4096, 1024),  # exactly the threshold
    ("multiq_16", 1, 1030, 4096, 1040),
]


def _cfg(name):
    return flashtpa_config(48, 3, 36) if name == "flashtpa_h48" else CONFIGS[name]


@pytest.mark.parametrize("name,batch,n_new,d_model,cap", SHAPES)
def test_projected_factors_match_oracle(gpu_lib, name, batch, n_new, d_model, cap):
    cfg = _cfg(name)
    dims = dims_of(cfg)
    x, w = _inputs(cfg, batch, n_new, d_model, seed=41)
    g = torch.Generator().manual_seed(42)
    slot0 = torch.randint(0, cap - n_new + 1, (batch,), generator=g, dtype=torch.int32)
    positions = (slot0.view(-1, 1) + torch.arange(n_new, dtype=torch.int32).view(1, -1) + 1000).to(torch.int32)
    cache = kpa.alloc_cache(dims, batch, cap)
    cache.random_(0, 256, generator=None)  # garbage everywhere the call does not write
    before = cache.cpu().numpy().copy()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    kpa.kpa_project_append(dims, cache, batch, cap, x.cuda(), w.cuda(), positions.cuda(), slot0.cuda(),
                           n_new=n_new, dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    after = cache.cpu().numpy()
    lay = kpa.kpa_cache_layout(dims, batch, cap)
    sets, pos = unpack(after, lay, dims, batch, cap)

    xs = x.to(torch.float64).numpy().reshape(batch * n_new, d_model)
    ws = w.to(torch.float64).numpy()
    ps = positions.numpy().reshape(-1)
    want = kpa_ref.projected_cache_values(xs, ws, ps, cfg.r_k, cfg.r_v, cfg.p1, cfg.q1, cfg.p2, cfg.q2,
                                          cfg.rope_base)
    # float32 accumulation bound per projected value, in the same layout
    mag = kpa_ref.project_factors(np.abs(xs), np.abs(ws), cfg.r_k, cfg.r_v, cfg.p1, cfg.q1, cfg.p2, cfg.q2)
    gam = [m * d_model * 2.0 ** -24 for m in mag]
    # a rotated pair mixes both members' errors
    gk = gam[1].reshape(batch * n_new, -1, 2).sum(-1, keepdims=True)
    gam[1] = np.broadcast_to(gk, gk.shape[:-1] + (2,)).reshape(gam[1].shape)
    touched = np.zeros((batch, cap), bool)
    for b in range(batch):
        for n in range(n_new):
            t, s = b * n_new + n, int(slot0[b]) + n
            touched[b, s] = True
            assert pos[b, s] == ps[t]
            for c in range(4):
                got = _to_f64(sets[c][b, s], cfg.dtype)
                _check_set(got, want[c][t].reshape(-1), gam[c][t].reshape(-1), cfg.dtype, f"{name} set {c} token {t}")
    # every slot the call does not own keeps its bytes
    untouched_sets, untouched_pos = unpack(before, lay, dims, batch, cap)
    for c in range(4):  # raw bits (random float32 bytes include NaNs)
        bits = lambda a: np.ascontiguousarray(a[~touched]).view(np.uint8)
        assert np.array_equal(bits(sets[c]), bits(untouched_sets[c])), f"set {c} changed outside the new slots"
    assert np.array_equal(pos[~touched], untouched_pos[~touched])


def test_out_of_range_slot_is_flagged_and_skipped(gpu_lib):
    cfg = CONFIGS["kpa_32k"]
    dims = dims_of(cfg)
    x, w = _inputs(cfg, 2, 1, 256, seed=43)
    cache = kpa.alloc_cache(dims, 2, 32)
    before = cache.clone()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    kpa.kpa_project_append(dims, cache, 2, 32, x.cuda(), w.cuda(), torch.tensor([[5], [-1]], dtype=torch.int32).cuda(),
                           torch.tensor([32, 3], dtype=torch.int32).cuda(), n_new=1, dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 1 | 2  # slot out of range (sequence 0), negative position (sequence 1)
    assert torch.equal(cache, before)


def test_slot_near_the_int32_limit_is_flagged_not_wrapped(gpu_lib):
    # sequence 0's three tokens start 2 slots below 2^31 (the third past the
    # int32 range): skipped and flagged; sequence 1's tokens are written
    cfg = CONFIGS["kpa_32k"]
    dims = dims_of(cfg)
    x, w = _inputs(cfg, 2, 3, 256, seed=44)
    cache = kpa.alloc_cache(dims, 2, 32)
    before = cache.clone()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    pos = torch.tensor([[0, 1, 2], [7, 8, 9]], dtype=torch.int32).cuda()
    kpa.kpa_project_append(dims, cache, 2, 32, x.cuda(), w.cuda(), pos,
                           torch.tensor([2 ** 31 - 2, 5], dtype=torch.int32).cuda(), n_new=3, dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 1  # KPA_DEV_SLOT_OUT_OF_RANGE
    lay = kpa.kpa_cache_layout(dims, 2, 32)
    tb = lay["tile_bytes"]
    assert torch.equal(cache[:tb], before[:tb])  # sequence 0's one tile
    p = cache[lay["positions_offset"]:].cpu().numpy().view(np.int32).reshape(2, 32)
    assert not np.any(p[0]) and list(p[1, 5:8]) == [7, 8, 9]


@pytest.mark.parametrize("ctx", [300, 600])  # 600 tokens, 1200 in all: the tiled kernel
def test_decode_over_a_projected_cache_matches_oracle(gpu_lib, ctx):
    """End to end: every context token projected from its hidden state into
    the cache, then the decode; the oracle decodes the float64 projected
    factors (the cache rounds them once to bf16, 2^-8 relative)."""
    cfg = CONFIGS["kpa_32k"]
    dims = dims_of(cfg)
    batch, d_model = 2, 512
    x, w = _inputs(cfg, batch, ctx, d_model, seed=44)
    positions = torch.arange(ctx, dtype=torch.int32).repeat(batch, 1).contiguous()
    cache = kpa.alloc_cache(dims, batch, ctx)
    kpa.kpa_project_append(dims, cache, batch, ctx, x.cuda(), w.cuda(), positions.cuda(),
                           torch.zeros(batch, dtype=torch.int32).cuda(), n_new=ctx)
    g = torch.Generator().manual_seed(45)
    q = torch.randn((batch, 1, cfg.h, cfg.d_h), generator=g)
    ctx_len = torch.tensor([ctx, ctx - 83], dtype=torch.int32)
    q_pos = (ctx_len - 1).view(batch, 1).to(torch.int32)
    out = torch.empty((batch, cfg.h, cfg.d_h), device="cuda")
    lse = torch.empty((batch, cfg.h), device="cuda")
    ws = kpa.alloc_workspace(dims, batch, ctx)
    kpa.kpa_decode(dims, cache, batch, ctx, ctx_len.cuda(), ctx, q.view(batch, cfg.h, cfg.d_h).cuda(),
                   q_pos.view(batch).cuda(), out, lse, ws)
    torch.cuda.synchronize()
    xs = x.to(torch.float64).numpy()
    ws_ = w.to(torch.float64).numpy()
    a_k, b_k, a_v, b_v = kpa_ref.project_factors(xs, ws_, cfg.r_k, cfg.r_v, cfg.p1, cfg.q1, cfg.p2, cfg.q2)
    ro, rl = kpa_oracle.decode(a_k, b_k, a_v, b_v, positions.numpy(), ctx_len.numpy(), q.numpy(), q_pos.numpy(),
                               causal=True)
    go = out.cpu().numpy().astype(np.float64).reshape(batch, 1, cfg.h, cfg.d_h)
    gl = lse.cpu().numpy().astype(np.float64).reshape(batch, 1, cfg.h)
    # both key factors are rounded from their float64 projections here (the
    # seeded-input tests round only B~^K), so the score error is up to twice
    # the one the lse bound assumes
    assert_close(go, gl, ro, rl, cfg.dtype, "decode over projected cache",
                 scale=2.0 * score_scale(a_k, b_k, ctx_len, q))
