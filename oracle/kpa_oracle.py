"""ctypes wrapper and build step for the streaming C oracle (``kpa_oracle.c``).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kpa_oracle.c")
_LIB = os.path.join(_HERE, "libkpa_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile kpa_oracle.c with gcc (-O2, OpenMP) into oracle/libkpa_oracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = f"{_LIB}.{os.getpid()}.tmp"  # per process: concurrent builds do not collide
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i = ctypes.c_int
        lib.kpa_oracle_decode.argtypes = [i, i, i, i, i, i, ctypes.c_double,
                                          i, i, i, p, p, p, p, p, p, i, i, p, p, p, i,
                                          p, p, i]
        lib.kpa_oracle_decode.restype = i
        lib.kpa_oracle_max_threads.restype = i
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().kpa_oracle_max_threads())


def _as_factor_array(x):
    """Return (contiguous array, elem_kind): float32 -> 0, bfloat16 bits -> 1."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), 1
            return x.to(torch.float32).numpy(), 0
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, 1
    return np.ascontiguousarray(x, dtype=np.float32), 0


def _np(x, dtype):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x), dtype=dtype)


def decode(a_k, b_k, a_v, b_v, positions, ctx_len, q, q_pos, *, causal=True,
           base=10000.0, items=None, n_threads=0):
    """Float64 decode, same arguments and meaning as ``kpa_ref.decode``.

    Factor arrays are [B][S][R][p][q] in float32 or bfloat16 (torch tensors or
    NumPy arrays; bfloat16 may be passed as uint16 bit patterns).  ``items``:
    optional int array [n][3] of (b, n, head) rows to compute; then the
    result is (out [n][d_h], lse [n]), else (out [B][n_q][h][d_h], lse [B][n_q][h]).
    """
    lib = _load()
    ak, kind = _as_factor_array(a_k)
    bk, kind_b = _as_factor_array(b_k)
    av, kind_c = _as_factor_array(a_v)
    bv, kind_d = _as_factor_array(b_v)
    if len({kind, kind_b, kind_c, kind_d}) != 1:
        raise ValueError("all factor arrays must share one element type")
    nb, stride_s, r_k, p1, q1 = ak.shape
    r_v = av.shape[2]
    p2, q2 = bk.shape[3], bk.shape[4]
    pos = _np(positions, np.int32)
    ctx = _np(ctx_len, np.int32)
    qq = _np(q, np.float32)
    qp = _np(q_pos, np.int32)
    n_q = qq.shape[1]
    h, d_h = p1 * p2, q1 * q2
    if items is not None:
        it = _np(items, np.int32).reshape(-1, 3)
        n_items = it.shape[0]
        out = np.zeros((n_items, d_h))
        lse = np.zeros(n_items)
        it_ptr = it.ctypes.data
    else:
        it = None
        n_items = nb * n_q * h
        out = np.zeros((nb, n_q, h, d_h))
        lse = np.zeros((nb, n_q, h))
        it_ptr = None
    rc = lib.kpa_oracle_decode(p1, p2, q1, q2, r_k, r_v, float(base), nb, stride_s, kind,
                               ak.ctypes.data, bk.ctypes.data, av.ctypes.data, bv.ctypes.data,
                               pos.ctypes.data, ctx.ctypes.data, n_q, int(bool(causal)),
                               qq.ctypes.data, qp.ctypes.data, it_ptr, n_items,
                               out.ctypes.data, lse.ctypes.data, int(n_threads))
    if rc != 0:
        raise RuntimeError(f"kpa_oracle_decode failed ({rc})")
    return out, lse
