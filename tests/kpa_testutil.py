"""Helpers shared by the GPU tests: move seeded inputs to the device, fill a
cache through kpa_cache_append, run the decode through the C ABI, and compare
with the oracle."""
from __future__ import annotations

import math

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


def score_scale(a_k, b_k, ctx_len, q, items=None):
    """Per (sequence, query, head): an upper bound of the absolute score sum
    S = max_s sum_{r,j} |q'_j| |A_r[s, i1, j1]| |B~_r[s, i2, j2]| / (R_K sqrt(d_h))
    over the sequence's slots s < ctx_len[b]:
      S <= ||q_i|| max_s sum_r ||A_r[s, i1, :]|| ||B_r[s, i2, :]|| / (R_K sqrt(d_h))
    (Cauchy-Schwarz per rank; the rotations keep every norm).  a_k [B][S][R][p1][q1],
    b_k [B][S][R][p2][q2], q [B][n_q][h][d_h] (torch or numpy).  Returns
    [B][n_q][h], or [n] for the (b, n, head) rows of `items`."""
    a = torch.as_tensor(a_k).to(torch.float64)
    b = torch.as_tensor(b_k).to(torch.float64)
    qq = torch.as_tensor(q).to(torch.float64)
    nb, ns, r, p1, q1 = a.shape
    p2, q2 = b.shape[3], b.shape[4]
    na = a.norm(dim=-1)                                   # [B][S][R][p1]
    nbn = b.norm(dim=-1)                                  # [B][S][R][p2]
    t = torch.einsum("bsri,bsrj->bsij", na, nbn).reshape(nb, ns, p1 * p2)
    ctx = torch.as_tensor(ctx_len).to(torch.int64).clamp(0, ns)
    live = torch.arange(ns).view(1, ns, 1) < ctx.view(nb, 1, 1)
    t = torch.where(live, t, torch.zeros((), dtype=t.dtype)).amax(dim=1)  # [B][h]
    sc = qq.norm(dim=-1) * t[:, None, :] / (r * math.sqrt(q1 * q2))       # [B][n_q][h]
    sc = sc.numpy()
    if items is not None:
        it = np.asarray(items).reshape(-1, 3)
        sc = sc[it[:, 0], it[:, 1], it[:, 2]]
    return sc


def scale_of(inp, q=None, items=None):
    """score_scale of a seeded input set (its own dense query unless `q` is given)."""
    return score_scale(inp.a_k, inp.b_k, inp.ctx_len, inp.q if q is None else q, items)


# lse bound of the bf16 paths.  Each score differs from the float64 one by at
# most (2^-8 + 2^-15) S: B~^K is rounded once to bf16 (relative 2^-8, round
# to nearest with an 8-bit significand), the query is carried as bf16 hi + lo
# (2^-16) and float32 accumulation over at most d_h + R_K q terms adds less
# than 2^-16 more.  lse is 1-Lipschitz in the max-norm of the scores.  2^-12
# covers the float32 summation of the softmax normaliser (a few thousand
# terms at most in any one chain) and the exp2/log2 units, 2^-21 |lse| the
# final rounding.
LSE_SCORE_COEF = 2.0 ** -7
LSE_ABS = 2.0 ** -12
LSE_REL = 2.0 ** -21
# The rebuild path ("mfma_rebuild") also rounds every rebuilt key element
# (1/R_K) sum_r A_r B~_r to bf16 before the score product (relative 2^-8 of
# that element, at most 2^-8 (1/R_K) sum_r |A_r| |B~_r|) and carries the
# rotated query in bf16 (relative 2^-8 per element): each adds 2^-8 S, so its
# scores are off by at most (3 * 2^-8 + 2^-16) S, and twice that for headroom
# is 3 * 2^-7 S.
LSE_SCORE_COEF_REBUILD = 3 * 2.0 ** -7


def assert_close(got_o, got_l, ref_o, ref_l, dtype, what="", *, scale, path=None):
    """Outputs: norm-wise relative error per row <= TOL[dtype].  lse: relative
    error |dlse| / max(|lse|, 1) <= TOL[dtype], and for bf16 caches also the
    derived bound |dlse| <= c S + 2^-12 + 2^-21 |lse| with S = score_scale
    of the same rows (`scale`, shaped like the lse arrays) and c = 2^-7, or
    3 * 2^-7 for the kernel path (`path`, kpa_decode_path) "mfma_rebuild"."""
    tol = TOL[dtype]
    err = rel_err(got_o, ref_o)
    assert np.all(np.isfinite(got_o)), f"{what}: non-finite output"
    assert err.max() <= tol, f"{what}: max rel err {err.max():.3e} > {tol} at {np.unravel_index(err.argmax(), err.shape)}"
    finite = np.isfinite(ref_l)
    assert np.array_equal(finite, np.isfinite(got_l)), f"{what}: lse finiteness differs"
    if finite.any():
        d = np.abs(got_l[finite] - ref_l[finite])
        r = np.abs(ref_l[finite])
        lrel = d / np.maximum(r, 1.0)
        assert lrel.max() <= tol, f"{what}: lse rel err {lrel.max():.3e} > {tol}"
        if dtype == "bf16":
            sc = np.broadcast_to(np.asarray(scale, np.float64), np.shape(ref_l))[finite]
            coef = LSE_SCORE_COEF_REBUILD if path == "mfma_rebuild" else LSE_SCORE_COEF
            bound = coef * sc + LSE_ABS + LSE_REL * r
            k = int(np.argmax(d - bound))
            assert np.all(d <= bound), f"{what}: lse err {d[k]:.3e} above the derived bound {bound[k]:.3e}"
    return float(err.max())
