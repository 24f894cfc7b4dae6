"""Python binding of libkpa (KPA factor-cache decode on MI355X / gfx950).

Argument marshalling only: every function forwards torch tensors' device
pointers and the current HIP stream to the C entry point of the same name in
``include/kpa.h``; every step of the computation runs in the HIP kernels.
There is no fallback: if ``libkpa.so`` is missing or fails to load, every
call raises.

Build the library with ``python -m factorized_kv_cache_kpa_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkpa.so")

KPA_F32 = 0
KPA_BF16 = 1
KPA_DEV_SLOT_OUT_OF_RANGE = 1
KPA_DEV_NEGATIVE_POSITION = 2
KPA_DEV_CTX_OUT_OF_RANGE = 4
# build limits (include/kpa.h)
KPA_MAX_HEADS = 128
KPA_MAX_HEAD_DIM = 256
KPA_MAX_RANK = 16
KPA_MAX_HD = 8192
KPA_MAX_NQ = 64
KPA_MAX_CAPACITY = 1 << 30
TILE_SLOTS = 32

_lib = None


class KpaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({kpa_status_string(status)})")


class kpa_dims(ctypes.Structure):
    _fields_ = [("p1", ctypes.c_int32), ("p2", ctypes.c_int32), ("q1", ctypes.c_int32),
                ("q2", ctypes.c_int32), ("r_k", ctypes.c_int32), ("r_v", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("rope_base", ctypes.c_float)]

    @property
    def h(self):
        return self.p1 * self.p2

    @property
    def d_h(self):
        return self.q1 * self.q2

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == KPA_F32 else torch.bfloat16


class kpa_layout_info(ctypes.Structure):
    _fields_ = [("version", ctypes.c_int32), ("tile_slots", ctypes.c_int32),
                ("elem_bytes", ctypes.c_int32), ("n_tiles", ctypes.c_int32),
                ("tile_bytes", ctypes.c_int64), ("comp_offset", ctypes.c_int64 * 4),
                ("comp_elems", ctypes.c_int64 * 4), ("positions_offset", ctypes.c_int64),
                ("total_bytes", ctypes.c_int64)]


def load():
    """Load libkpa.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run python -m factorized_kv_cache_kpa_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I32 = ctypes.c_int32
    DP = ctypes.POINTER(kpa_dims)
    lib.kpa_cache_layout.argtypes = [DP, I32, I32, ctypes.POINTER(kpa_layout_info)]
    lib.kpa_cache_layout.restype = ctypes.c_int
    lib.kpa_cache_bytes.argtypes = [DP, I32, I32]
    lib.kpa_cache_bytes.restype = ctypes.c_size_t
    lib.kpa_cache_append.argtypes = [DP, P, I32, I32, P, P, P, P, P, P, I32, P, P]
    lib.kpa_cache_append.restype = ctypes.c_int
    lib.kpa_decode_workspace_bytes.argtypes = [DP, I32, I32, I32, I32]
    lib.kpa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.kpa_decode.argtypes = [DP, P, I32, I32, P, I32, P, P, P, P, P, ctypes.c_size_t, I32, P, P]
    lib.kpa_decode.restype = ctypes.c_int
    lib.kpa_decode_multiq.argtypes = [DP, P, I32, I32, P, I32, I32, I32, P, P, P, P, P,
                                      ctypes.c_size_t, I32, P, P]
    lib.kpa_decode_multiq.restype = ctypes.c_int
    lib.kpa_decode_factored.argtypes = [DP, I32, P, I32, I32, P, I32, I32, I32, P, P, P, P, P, P,
                                        ctypes.c_size_t, I32, P, P]
    lib.kpa_decode_factored.restype = ctypes.c_int
    lib.kpa_project_append.argtypes = [DP, P, I32, I32, P, I32, P, P, P, I32, P, P]
    lib.kpa_project_append.restype = ctypes.c_int
    lib.kpa_append_decode.argtypes = [DP, P, I32, I32, P, P, P, P, P, P, I32, P, I32, I32, I32, P, P, P, P, P,
                                      ctypes.c_size_t, I32, P, P]
    lib.kpa_append_decode.restype = ctypes.c_int
    lib.kpa_append_decode_noalloc.argtypes = [DP, P, I32, I32, P, P, P, P, P, P, I32, P, I32, I32, I32, P, P, P, P,
                                              I32, P, P]
    lib.kpa_append_decode_noalloc.restype = ctypes.c_int
    lib.kpa_status_string.argtypes = [ctypes.c_int]
    lib.kpa_status_string.restype = ctypes.c_char_p
    lib.kpa_decode_path.argtypes = [DP, I32]
    lib.kpa_decode_path.restype = ctypes.c_char_p
    lib.kpa_time_next_decode_kernel.argtypes = [P, P]
    lib.kpa_stream_xor.argtypes = [P, ctypes.c_size_t, P, I32, P]
    lib.kpa_stream_xor.restype = ctypes.c_int
    lib.kpa_time_next_decode_kernel.restype = ctypes.c_int
    _lib = lib
    return lib


def make_dims(p1, p2, q1, q2, r_k, r_v, dtype="bf16", rope_base=10000.0) -> kpa_dims:
    dt = {"f32": KPA_F32, "bf16": KPA_BF16, KPA_F32: KPA_F32, KPA_BF16: KPA_BF16}[dtype]
    return kpa_dims(p1, p2, q1, q2, r_k, r_v, dt, rope_base)


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream, on):
    """HIP stream handle: the given stream, else the current stream of the
    device that tensor `on` lives on (read without building a Stream object,
    which costs microseconds per call)."""
    if stream is None:
        if on is None:
            return torch.cuda.current_stream().cuda_stream
        return torch._C._cuda_getCurrentRawStream(on.device.index)
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(fn, status):
    if status != 0:
        raise KpaError(fn, status)


def kpa_status_string(status: int) -> str:
    return load().kpa_status_string(int(status)).decode()


def kpa_decode_path(dims: kpa_dims, n_q: int = 1) -> str:
    return load().kpa_decode_path(ctypes.byref(dims), n_q).decode()


def kpa_cache_layout(dims: kpa_dims, batch: int, capacity: int) -> dict:
    info = kpa_layout_info()
    _check("kpa_cache_layout", load().kpa_cache_layout(ctypes.byref(dims), batch, capacity, ctypes.byref(info)))
    return {"version": info.version, "tile_slots": info.tile_slots, "elem_bytes": info.elem_bytes,
            "n_tiles": info.n_tiles, "tile_bytes": info.tile_bytes,
            "comp_offset": list(info.comp_offset), "comp_elems": list(info.comp_elems),
            "positions_offset": info.positions_offset, "total_bytes": info.total_bytes}


def kpa_cache_bytes(dims: kpa_dims, batch: int, capacity: int) -> int:
    return int(load().kpa_cache_bytes(ctypes.byref(dims), batch, capacity))


def kpa_cache_append(dims, cache, batch, capacity, a_k, b_k, a_v, b_v, positions, slot0,
                     n_new=None, dev_status=None, stream=None):
    dt = dims.torch_dtype
    if n_new is None:
        n_new = a_k.shape[1] if a_k.dim() > 1 else 0
    st = load().kpa_cache_append(
        ctypes.byref(dims), _ptr(cache, torch.uint8, "cache"), batch, capacity,
        _ptr(a_k, dt, "a_k"), _ptr(b_k, dt, "b_k"), _ptr(a_v, dt, "a_v"), _ptr(b_v, dt, "b_v"),
        _ptr(positions, torch.int32, "positions"), _ptr(slot0, torch.int32, "slot0"), int(n_new),
        _ptr(dev_status, torch.int32, "dev_status"), _stream(stream, cache))
    _check("kpa_cache_append", st)


def kpa_project_append(dims, cache, batch, capacity, x, w, positions, slot0, n_new=None, dev_status=None,
                       stream=None):
    """x [batch][n_new][d_model] bf16, w [F][d_model] bf16 (rows B^K, A^K, A^V, B^V)."""
    if n_new is None:
        n_new = x.shape[1] if x.dim() > 2 else 0
    st = load().kpa_project_append(
        ctypes.byref(dims), _ptr(cache, torch.uint8, "cache"), batch, capacity, _ptr(x, torch.bfloat16, "x"),
        int(x.shape[-1]), _ptr(w, torch.bfloat16, "w"), _ptr(positions, torch.int32, "positions"),
        _ptr(slot0, torch.int32, "slot0"), int(n_new), _ptr(dev_status, torch.int32, "dev_status"),
        _stream(stream, cache))
    _check("kpa_project_append", st)


def kpa_stream_xor(buf, partial, n_blocks=None, nbytes=None, stream=None):
    """Streaming read of `buf` (any contiguous device tensor; the first
    `nbytes` bytes, default all): partial[w] = XOR of the 32-bit words of
    workgroup w's contiguous share.  partial: int32 [n_blocks]."""
    if n_blocks is None:
        n_blocks = partial.numel()
    if partial.numel() < n_blocks:
        raise ValueError("partial holds fewer than n_blocks words")
    if nbytes is None:
        nbytes = buf.numel() * buf.element_size()
    st = load().kpa_stream_xor(_ptr(buf, None, "buf"), int(nbytes), _ptr(partial, torch.int32, "partial"),
                               int(n_blocks), _stream(stream, buf))
    _check("kpa_stream_xor", st)


def kpa_decode_workspace_bytes(dims, batch, max_ctx, n_q=1, num_splits=0) -> int:
    return int(load().kpa_decode_workspace_bytes(ctypes.byref(dims), batch, max_ctx, n_q, num_splits))


def kpa_decode(dims, cache, batch, capacity, ctx_len, max_ctx, q, q_pos, out, lse=None,
               workspace=None, num_splits=0, dev_status=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().kpa_decode(
        ctypes.byref(dims), _ptr(cache, torch.uint8, "cache"), batch, capacity,
        _ptr(ctx_len, torch.int32, "ctx_len"), max_ctx, _ptr(q, torch.float32, "q"),
        _ptr(q_pos, torch.int32, "q_pos"), _ptr(out, torch.float32, "out"),
        _ptr(lse, torch.float32, "lse"), _ptr(workspace, None, "workspace"), ws_bytes, num_splits,
        _ptr(dev_status, torch.int32, "dev_status"), _stream(stream, cache))
    _check("kpa_decode", st)


def kpa_decode_multiq(dims, cache, batch, capacity, ctx_len, max_ctx, n_q, causal, q, q_pos, out,
                      lse=None, workspace=None, num_splits=0, dev_status=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().kpa_decode_multiq(
        ctypes.byref(dims), _ptr(cache, torch.uint8, "cache"), batch, capacity,
        _ptr(ctx_len, torch.int32, "ctx_len"), max_ctx, n_q, int(bool(causal)),
        _ptr(q, torch.float32, "q"), _ptr(q_pos, torch.int32, "q_pos"),
        _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"),
        _ptr(workspace, None, "workspace"), ws_bytes, num_splits,
        _ptr(dev_status, torch.int32, "dev_status"), _stream(stream, cache))
    _check("kpa_decode_multiq", st)


def kpa_decode_factored(dims, r_q, cache, batch, capacity, ctx_len, max_ctx, n_q, causal, a_q, b_q, q_pos,
                        out, lse=None, workspace=None, num_splits=0, dev_status=None, stream=None):
    """a_q [batch][n_q][r_q][p1][q1], b_q [batch][n_q][r_q][p2][q2] float32 (unrotated)."""
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().kpa_decode_factored(
        ctypes.byref(dims), r_q, _ptr(cache, torch.uint8, "cache"), batch, capacity,
        _ptr(ctx_len, torch.int32, "ctx_len"), max_ctx, n_q, int(bool(causal)),
        _ptr(a_q, torch.float32, "a_q"), _ptr(b_q, torch.float32, "b_q"), _ptr(q_pos, torch.int32, "q_pos"),
        _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"),
        _ptr(workspace, None, "workspace"), ws_bytes, num_splits,
        _ptr(dev_status, torch.int32, "dev_status"), _stream(stream, cache))
    _check("kpa_decode_factored", st)


def kpa_append_decode(dims, cache, batch, capacity, a_k, b_k, a_v, b_v, positions, slot0, ctx_len, max_ctx,
                      n_q, causal, q, q_pos, out, lse=None, workspace=None, num_splits=0, n_new=None,
                      dev_status=None, stream=None):
    """kpa_cache_append of the new tokens, then kpa_decode_multiq, as one call
    (fused into the decode kernel where the matrix-core path runs)."""
    dt = dims.torch_dtype
    if n_new is None:
        n_new = a_k.shape[1] if a_k is not None and a_k.dim() > 1 else 0
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().kpa_append_decode(
        ctypes.byref(dims), _ptr(cache, torch.uint8, "cache"), batch, capacity,
        _ptr(a_k, dt, "a_k"), _ptr(b_k, dt, "b_k"), _ptr(a_v, dt, "a_v"), _ptr(b_v, dt, "b_v"),
        _ptr(positions, torch.int32, "positions"), _ptr(slot0, torch.int32, "slot0"), int(n_new),
        _ptr(ctx_len, torch.int32, "ctx_len"), max_ctx, n_q, int(bool(causal)),
        _ptr(q, torch.float32, "q"), _ptr(q_pos, torch.int32, "q_pos"),
        _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"),
        _ptr(workspace, None, "workspace"), ws_bytes, num_splits,
        _ptr(dev_status, torch.int32, "dev_status"), _stream(stream, cache))
    _check("kpa_append_decode", st)


def kpa_append_decode_noalloc(dims, cache, batch, capacity, a_k, b_k, a_v, b_v, positions, slot0, ctx_len,
                              max_ctx, n_q, causal, q, q_pos, out, lse=None, num_splits=0, n_new=None,
                              dev_status=None, stream=None):
    """kpa_append_decode without a workspace argument: the partials go to the
    library's static per-device scratch (no device allocation in the call)."""
    dt = dims.torch_dtype
    if n_new is None:
        n_new = a_k.shape[1] if a_k is not None and a_k.dim() > 1 else 0
    st = load().kpa_append_decode_noalloc(
        ctypes.byref(dims), _ptr(cache, torch.uint8, "cache"), batch, capacity,
        _ptr(a_k, dt, "a_k"), _ptr(b_k, dt, "b_k"), _ptr(a_v, dt, "a_v"), _ptr(b_v, dt, "b_v"),
        _ptr(positions, torch.int32, "positions"), _ptr(slot0, torch.int32, "slot0"), int(n_new),
        _ptr(ctx_len, torch.int32, "ctx_len"), max_ctx, n_q, int(bool(causal)),
        _ptr(q, torch.float32, "q"), _ptr(q_pos, torch.int32, "q_pos"),
        _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"), num_splits,
        _ptr(dev_status, torch.int32, "dev_status"), _stream(stream, cache))
    _check("kpa_append_decode_noalloc", st)


KPA_NOALLOC_SCRATCH_BYTES = 32 << 20


# --------------------------------------------------------------------------
# Allocation conveniences (torch does the allocating; no computation here)
# --------------------------------------------------------------------------
def kpa_time_next_decode_kernel(start_event, stop_event):
    """Have the next decode call on this thread record the two events (torch
    timing events, or None to cancel) around its split-KV decode kernel."""
    def handle(ev):
        if ev is None:
            return None
        if not isinstance(ev, torch.cuda.Event):
            raise TypeError("events must be torch.cuda.Event")
        if not ev.cuda_event:  # torch creates the HIP event on its first record
            ev.record()
        return ev.cuda_event
    _check("kpa_time_next_decode_kernel", load().kpa_time_next_decode_kernel(handle(start_event), handle(stop_event)))


def alloc_cache(dims, batch, capacity, device="cuda"):
    n = kpa_cache_bytes(dims, batch, capacity)
    if n == 0 and batch > 0:
        raise KpaError("kpa_cache_bytes", -1)
    return torch.zeros(max(n, 1), dtype=torch.uint8, device=device)


def alloc_workspace(dims, batch, max_ctx, n_q=1, num_splits=0, device="cuda"):
    n = kpa_decode_workspace_bytes(dims, batch, max_ctx, n_q, num_splits)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device) if n > 0 else None
