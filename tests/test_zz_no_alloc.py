"""kpa_append_decode_noalloc (the entry point for callers that cannot
allocate) against kpa_append_decode with a caller workspace, through the C
ABI: the same cache bytes and outputs, bit for bit, on two calls in a row
(the second with a smaller input, so the shared scratch holds the first
call's partials), and both within the parity tolerances of the float64
oracle."""
import numpy as np
import pytest
import torch

import factorized_kv_cache_kpa_amd as kpa
from oracle import kpa_oracle
from tests.kpa_testutil import assert_close, dims_of, fill_cache, scale_of
from workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu


def _step(inp, dims, n_new, noalloc, num_splits):
    """Cache with all but the step's n_new tokens, then one step (append of
    those tokens + decode).  Returns (cache bytes, out, lse)."""
    nb, nq = inp.batch, inp.q.shape[1]
    s = inp.slots
    pre = make_inputs(inp.cfg, seed=0, batch=nb, ctx=s - n_new, n_q=nq)
    pre.a_k, pre.b_k, pre.a_v, pre.b_v = (t[:, :s - n_new].contiguous() for t in (inp.a_k, inp.b_k, inp.a_v, inp.b_v))
    pre.positions = inp.positions[:, :s - n_new].contiguous()
    cache, cap = fill_cache(pre, dims, capacity=s)
    new = [t[:, s - n_new:].contiguous().cuda() for t in (inp.a_k, inp.b_k, inp.a_v, inp.b_v, inp.positions)]
    slot0 = torch.full((nb,), s - n_new, dtype=torch.int32, device="cuda")
    h, dh = dims.h, dims.d_h
    out = torch.full((nb, nq, h, dh), float("nan"), device="cuda")
    lse = torch.full((nb, nq, h), float("nan"), device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    args = (dims, cache, nb, cap, *new, slot0, inp.ctx_len.cuda(), s, nq, 1, inp.q.cuda(), inp.q_pos.cuda(), out, lse)
    if noalloc:
        kpa.kpa_append_decode_noalloc(*args, num_splits=num_splits, n_new=n_new, dev_status=status)
    else:
        ws = kpa.alloc_workspace(dims, nb, s, nq, num_splits)
        kpa.kpa_append_decode(*args, workspace=ws, num_splits=num_splits, n_new=n_new, dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return cache.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("name,cases", [
    # (batch, ctx, n_q, n_new, num_splits): the second call smaller than the first
    ("kpa_32k", [(4, 3000, 1, 1, 0), (2, 700, 1, 1, 5)]),
    ("multiq_16", [(3, 1200, 16, 16, 0), (1, 400, 16, 16, 3)]),
    ("long_512k", [(1, 40000, 1, 1, 0), (1, 2000, 1, 1, 0)]),
])
def test_noalloc_step_equals_workspace_step(gpu_lib, name, cases):
    cfg = CONFIGS[name]
    dims = dims_of(cfg)
    for k, (nb, ctx, nq, n_new, ns) in enumerate(cases):
        inp = make_inputs(cfg, seed=60 + k, batch=nb, ctx=ctx, n_q=nq)
        ref = _step(inp, dims, n_new, False, ns)
        got = _step(inp, dims, n_new, True, ns)
        assert np.array_equal(ref[0], got[0]), f"{name} call {k}: cache bytes differ"
        assert np.array_equal(ref[1], got[1]) and np.array_equal(ref[2], got[2]), f"{name} call {k}: outputs differ"
        ro, rl = kpa_oracle.decode(inp.a_k, inp.b_k, inp.a_v, inp.b_v, inp.positions, inp.ctx_len, inp.q, inp.q_pos)
        assert_close(got[1].astype(np.float64), got[2].astype(np.float64), ro, rl, cfg.dtype, f"{name} call {k}",
                     scale=scale_of(inp), path=kpa.kpa_decode_path(dims, nq))


def test_noalloc_refuses_a_call_beyond_the_scratch(gpu_lib):
    cfg = CONFIGS["kpa_32k"]
    dims = dims_of(cfg)
    need = kpa.kpa_decode_workspace_bytes(dims, 256, 65536, 1, 64)
    assert need > kpa.KPA_NOALLOC_SCRATCH_BYTES
    cache = torch.zeros(16, dtype=torch.uint8, device="cuda")
    z = torch.zeros(256, dtype=torch.int32, device="cuda")
    q = torch.zeros((256, 1, cfg.h, cfg.d_h), device="cuda")
    with pytest.raises(kpa.KpaError) as e:
        kpa.kpa_append_decode_noalloc(dims, cache, 256, 65536, None, None, None, None, None, None, z, 65536, 1, 1,
                                      q, z.view(256, 1), q, None, num_splits=64, n_new=0)
    assert e.value.status == -4
