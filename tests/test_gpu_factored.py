"""GPU decode with a factored query (kpa_decode_factored) against the float64
oracle: the oracle expands the query from its factors with the Kronecker
product ([KPA] Eq. (5), Def. 2.1) and runs the dense decode; the GPU expands
the elements each workgroup needs in its prologue.  Small cases on every
kernel shape (general kernel, both matrix-core orientations, the TPA split,
one and several queries), ranks R_Q = 1, 3, 6, ragged contexts, and the
full-size kpa_32k shape on every row."""
import numpy as np
import pytest
import torch

import factorized_kv_cache_kpa_amd as kpa
from oracle import kpa_oracle, kpa_ref
from tests.kpa_testutil import assert_close, dims_of, fill_cache, scale_of
from workloads import CONFIGS, make_inputs, make_query_factors

pytestmark = pytest.mark.gpu


def _run(inp, dims, cache, cap, a_q, b_q, *, causal=True, num_splits=0):
    nb, nq = inp.batch, a_q.shape[1]
    h, dh = dims.h, dims.d_h
    mc = int(inp.ctx_len.max().item())
    out = torch.full((nb, nq, h, dh), float("nan"), device="cuda")
    lse = torch.full((nb, nq, h), float("nan"), device="cuda")
    ws = kpa.alloc_workspace(dims, nb, mc, nq, num_splits)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    kpa.kpa_decode_factored(dims, a_q.shape[2], cache, nb, cap, inp.ctx_len.cuda(), mc, nq, causal,
                            a_q.cuda().contiguous(), b_q.cuda().contiguous(), inp.q_pos.cuda().contiguous(),
                            out, lse, ws, num_splits, dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


CASES = [
    # name, batch, ctx, n_q, r_q, ragged
    ("tiny_f32", 2, 300, 1, 3, True),
    ("kpa_32k", 3, 1500, 1, 6, True),
    ("long_512k", 1, 2000, 1, 1, False),
    ("tpa_degenerate", 3, 700, 1, 2, True),
    ("multiq_16", 2, 500, 16, 3, True),
    ("multiq_16", 2, 400, 1, 6, False),
]


@pytest.mark.parametrize("name,batch,ctx,n_q,r_q,ragged", CASES)
def test_factored_query_matches_oracle(gpu_lib, name, batch, ctx, n_q, r_q, ragged):
    cfg = CONFIGS[name]
    inp = make_inputs(cfg, seed=31, batch=batch, ctx=ctx, n_q=n_q, ragged=ragged)
    a_q, b_q = make_query_factors(cfg, r_q, seed=31, batch=batch, n_q=n_q)
    dims = dims_of(cfg)
    cache, cap = fill_cache(inp, dims)
    go, gl = _run(inp, dims, cache, cap, a_q, b_q)
    q = kpa_ref.query_from_factors(a_q.numpy(), b_q.numpy())
    ro, rl = kpa_oracle.decode(inp.a_k, inp.b_k, inp.a_v, inp.b_v, inp.positions, inp.ctx_len, q, inp.q_pos)
    assert_close(go, gl, ro, rl, cfg.dtype, f"{name} factored R_Q={r_q}", scale=scale_of(inp, q=q),
                 path=kpa.kpa_decode_path(dims, n_q))


def test_factored_query_equals_dense_decode_of_its_expansion(gpu_lib):
    """Same result as kpa_decode on the expanded query (the expansion is the
    only difference between the two entry points)."""
    cfg = CONFIGS["kpa_32k"]
    inp = make_inputs(cfg, seed=32, batch=2, ctx=1000)
    a_q, b_q = make_query_factors(cfg, 2, seed=32, batch=2, n_q=1)
    dims = dims_of(cfg)
    cache, cap = fill_cache(inp, dims)
    go, gl = _run(inp, dims, cache, cap, a_q, b_q, num_splits=4)
    q = torch.from_numpy(kpa_ref.query_from_factors(a_q.numpy(), b_q.numpy()).astype(np.float32)).cuda()
    out = torch.empty((2, dims.h, dims.d_h), device="cuda")
    lse = torch.empty((2, dims.h), device="cuda")
    ws = kpa.alloc_workspace(dims, 2, 1000, 1, 4)
    kpa.kpa_decode(dims, cache, 2, cap, inp.ctx_len.cuda(), 1000, q.view(2, dims.h, dims.d_h),
                   inp.q_pos.cuda().view(2), out, lse, ws, 4)
    torch.cuda.synchronize()
    d = np.abs(go[:, 0] - out.cpu().numpy()).max() / np.abs(out.cpu().numpy()).max()
    assert d < 1e-3, d


def test_factored_query_full_size_every_row(gpu_lib):
    cfg = CONFIGS["kpa_32k"]
    inp = make_inputs(cfg, seed=0)
    a_q, b_q = make_query_factors(cfg, 6, seed=0)
    dims = dims_of(cfg)
    cache, cap = fill_cache(inp, dims, chunk=8192)
    go, gl = _run(inp, dims, cache, cap, a_q, b_q)
    del cache
    q = kpa_ref.query_from_factors(a_q.numpy(), b_q.numpy())
    ro, rl = kpa_oracle.decode(inp.a_k, inp.b_k, inp.a_v, inp.b_v, inp.positions, inp.ctx_len, q, inp.q_pos)
    assert_close(go, gl, ro, rl, cfg.dtype, "kpa_32k factored full size", scale=scale_of(inp, q=q))


@pytest.mark.parametrize("h", [16, 32, 48])
def test_flashtpa_shapes_with_a_rank_16_factored_query(gpu_lib, h):
    """FlashTPA's decoding benchmark as the TPA summary page states it: TPA
    split, d_h = 64, R_K = R_V = 1 and a factored query of rank R_Q = 16
    (batches of ragged contexts over several chunks)."""
    from workloads import FLASHTPA_RQ, flashtpa_config
    cfg = flashtpa_config(h, 3, 2500)
    inp = make_inputs(cfg, seed=33, ragged=True)
    a_q, b_q = make_query_factors(cfg, FLASHTPA_RQ, seed=33, n_q=1)
    dims = dims_of(cfg)
    assert kpa.kpa_decode_path(dims, 1) == "mfma_bf16"
    cache, cap = fill_cache(inp, dims)
    q = kpa_ref.query_from_factors(a_q.numpy(), b_q.numpy())
    ro, rl = kpa_oracle.decode(inp.a_k, inp.b_k, inp.a_v, inp.b_v, inp.positions, inp.ctx_len, q, inp.q_pos)
    for s in (0, 6):
        go, gl = _run(inp, dims, cache, cap, a_q, b_q, num_splits=s)
        assert_close(go, gl, ro, rl, cfg.dtype, f"flashtpa h={h} R_Q={FLASHTPA_RQ} splits={s}", scale=scale_of(inp, q=q))
