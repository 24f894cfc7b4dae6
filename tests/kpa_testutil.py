"""Helpers shared by the GPU tests: move seeded inputs to the device, fill a
cache through kpa_cache_append, run the decode through the C ABI, and compare
with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import factorized_kv_cache_kpa_amd as kpa

# Tolerances (max relative error per (sequence, query, head), norm-wise:
# max_j |gpu - ref| / max_j |ref|).
TOL = {"f32": 1e-5, "bf16": 2e-2}


def dims_of(cfg):
    return kpa.make_dims(cfg.p1, cfg.p2, cfg.q1, cfg.q2, cfg.r_k, cfg.r_v, dtype=cfg.dtype,
                         rope_base=cfg.rope_base)


def fill_cache(inp, dims, capacity=None, chunk=None, dev="cuda"):
    """Append every slot of `inp` (slot s gets position inp.positions[b, s])."""
    nb, s = inp.batch, inp.slots
    cap = s if capacity is None else capacity
    cache = kpa.alloc_cache(dims, nb, cap, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    step = s if chunk is None else chunk
    for s0 in range(0, s, step):
        s1 = min(s, s0 + step)
        sl = slice(s0, s1)
        kpa.kpa_cache_append(
            dims, cache, nb, cap,
            inp.a_k[:, sl].contiguous().to(dev), inp.b_k[:, sl].contiguous().to(dev),
            inp.a_v[:, sl].contiguous().to(dev), inp.b_v[:, sl].contiguous().to(dev),
            inp.positions[:, sl].contiguous().to(dev),
            torch.full((nb,), s0, dtype=torch.int32, device=dev), n_new=s1 - s0, dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return cache, cap


def run_decode(inp, dims, cache, cap, *, num_splits=0, causal=True, max_ctx=None, dev="cuda"):
    nb, nq = inp.batch, inp.q.shape[1]
    h, dh = dims.h, dims.d_h
    mc = int(inp.ctx_len.max().item()) if max_ctx is None else max_ctx
    q = inp.q.to(dev).contiguous()
    qp = inp.q_pos.to(dev).contiguous()
    ctx = inp.ctx_len.to(dev).contiguous()
    out = torch.full((nb, nq, h, dh), float("nan"), device=dev)
    lse = torch.full((nb, nq, h), float("nan"), device=dev)
    ws = kpa.alloc_workspace(dims, nb, mc, nq, num_splits, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    if nq == 1 and causal:
        kpa.kpa_decode(dims, cache, nb, cap, ctx, mc, q.view(nb, h, dh), qp.view(nb), out.view(nb, h, dh),
                       lse.view(nb, h), ws, num_splits, dev_status=status)
    else:
        kpa.kpa_decode_multiq(dims, cache, nb, cap, ctx, mc, nq, causal, q, qp, out, lse, ws, num_splits,
                              dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    """Norm-wise relative error per leading index: max|g - r| / max|r| over the last axis."""
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-30)
    return num / den


def assert_close(got_o, got_l, ref_o, ref_l, dtype, what=""):
    tol = TOL[dtype]
    err = rel_err(got_o, ref_o)
    assert np.all(np.isfinite(got_o)), f"{what}: non-finite output"
    assert err.max() <= tol, f"{what}: max rel err {err.max():.3e} > {tol} at {np.unravel_index(err.argmax(), err.shape)}"
    finite = np.isfinite(ref_l)
    assert np.array_equal(finite, np.isfinite(got_l)), f"{what}: lse finiteness differs"
    lerr = np.abs(got_l[finite] - ref_l[finite]).max() if finite.any() else 0.0
    assert lerr <= 10 * tol, f"{what}: lse abs err {lerr:.3e}"
    return float(err.max())
