"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/kpa.h declares, reports the documented cache
layout, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

import factorized_kv_cache_kpa_amd as kpa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # non-null, aligned; only reached by calls that must fail before any launch


def _declared_symbols():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names.update(re.findall(r"\b(kpa_\w+)\s*\(", text))
    return names


def test_library_exports_every_declared_entry_point():
    lib = kpa.load()
    declared = _declared_symbols()
    assert {"kpa_cache_append", "kpa_decode", "kpa_decode_multiq"} <= declared
    for name in sorted(declared):
        assert hasattr(lib, name), name


def _layout_by_hand(p1, p2, q1, q2, r_k, r_v, es, batch, capacity):
    """The cache layout written out from its description in kpa.h."""
    T = 32
    elems = [r_k * p1 * q1, r_k * p2 * q2, r_v * p1 * q1, r_v * p2 * q2]
    sizes = [-(-elems[0] * es // 16) * 16 * T, -(-elems[1] * es // 16) * 16 * T,
             elems[2] * es * T, elems[3] * es * T]
    offs = [0, sizes[0], sizes[0] + sizes[1], sizes[0] + sizes[1] + sizes[2]]
    tile = -(-sum(sizes) // 128) * 128
    n_tiles = -(-capacity // T)
    pos_off = batch * n_tiles * tile
    return dict(tile_bytes=tile, comp_offset=offs, comp_elems=elems, n_tiles=n_tiles,
                positions_offset=pos_off, total_bytes=pos_off + batch * n_tiles * T * 4)


@pytest.mark.parametrize("shape", [(2, 2, 4, 4, 2, 2, "f32"), (12, 1, 1, 64, 2, 2, "bf16"),
                                   (4, 4, 8, 16, 2, 2, "bf16"), (8, 4, 8, 16, 2, 4, "bf16"),
                                   (4, 8, 16, 8, 4, 4, "bf16"), (3, 5, 3, 6, 3, 1, "bf16")])
@pytest.mark.parametrize("batch,capacity", [(1, 256), (3, 1000), (2, 31), (1, 0)])
def test_layout_matches_description(shape, batch, capacity):
    *dd, dt = shape
    dims = kpa.make_dims(*dd, dtype=dt)
    got = kpa.kpa_cache_layout(dims, batch, capacity)
    want = _layout_by_hand(*dd, 4 if dt == "f32" else 2, batch, capacity)
    for k, v in want.items():
        assert got[k] == v, (k, got[k], v)
    assert got["version"] == 1 and got["tile_slots"] == 32
    assert kpa.kpa_cache_bytes(dims, batch, capacity) == want["total_bytes"]
    # per-token factor bytes without padding: (R_K + R_V)(p1 q1 + p2 q2) * elem bytes
    p1, p2, q1, q2, r_k, r_v = dd
    assert sum(got["comp_elems"]) == (r_k + r_v) * (p1 * q1 + p2 * q2)


def test_layout_has_no_per_token_padding_for_the_configs():
    from workloads import CONFIGS
    for cfg in CONFIGS.values():
        dims = kpa.make_dims(cfg.p1, cfg.p2, cfg.q1, cfg.q2, cfg.r_k, cfg.r_v, dtype=cfg.dtype)
        lay = kpa.kpa_cache_layout(dims, 1, 32)
        assert lay["tile_bytes"] == 32 * cfg.bytes_per_token, cfg.name


@pytest.mark.parametrize("bad,code", [
    (dict(q2=5), -1), (dict(p1=0), -1), (dict(r_k=0), -1), (dict(r_v=17), -1),
    (dict(p1=16, p2=16), -1), (dict(q1=32, q2=16), -1), (dict(rope_base=0.0), -1), (dict(dtype=7), -3),
])
def test_invalid_dims_rejected(bad, code):
    base = dict(p1=4, p2=4, q1=8, q2=16, r_k=2, r_v=2, dtype=1, rope_base=10000.0)
    base.update(bad)
    dims = kpa.kpa_dims(**base)
    lib = kpa.load()
    info = kpa.kpa_layout_info()
    assert lib.kpa_cache_layout(ctypes.byref(dims), 1, 64, ctypes.byref(info)) == code
    assert lib.kpa_cache_bytes(ctypes.byref(dims), 1, 64) == 0
    assert lib.kpa_cache_append(ctypes.byref(dims), FAKE, 1, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                1, None, None) == code
    assert lib.kpa_decode(ctypes.byref(dims), FAKE, 1, 64, FAKE, 64, FAKE, FAKE, FAKE, None,
                          FAKE, 1 << 30, 0, None, None) == code
    assert kpa.kpa_decode_path(dims) == ""


def test_null_and_range_errors_return_before_launch():
    lib = kpa.load()
    dims = kpa.make_dims(4, 4, 8, 16, 2, 2)
    d = ctypes.byref(dims)
    assert lib.kpa_cache_layout(None, 1, 1, None) == -2
    assert lib.kpa_cache_append(d, None, 1, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None, None) == -2
    assert lib.kpa_cache_append(d, FAKE, -1, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None, None) == -7
    assert lib.kpa_cache_append(d, FAKE + 4, 1, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None, None) == -7
    # nothing to do: OK without touching any pointer
    assert lib.kpa_cache_append(d, None, 0, 64, None, None, None, None, None, None, 1, None, None) == 0
    assert lib.kpa_cache_append(d, None, 1, 64, None, None, None, None, None, None, 0, None, None) == 0
    # decode: null pointers, max_ctx beyond capacity, bad n_q, workspace too small
    assert lib.kpa_decode(d, None, 1, 64, FAKE, 64, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, 0, None, None) == -2
    assert lib.kpa_decode(d, FAKE, 1, 64, FAKE, 65, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, 0, None, None) == -7
    assert lib.kpa_decode_multiq(d, FAKE, 1, 64, FAKE, 64, 0, 1, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, 0,
                                 None, None) == -7
    assert lib.kpa_decode_multiq(d, FAKE, 1, 64, FAKE, 64, 65, 1, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, 0,
                                 None, None) == -7
    need = lib.kpa_decode_workspace_bytes(d, 4, 4096, 1, 8)
    assert need > 0
    assert lib.kpa_decode(d, FAKE, 4, 4096, FAKE, 4096, FAKE, FAKE, FAKE, None, FAKE, need - 1, 8,
                          None, None) == -4
    assert lib.kpa_decode(d, FAKE, 4, 4096, FAKE, 4096, FAKE, FAKE, FAKE, None, None, need, 8,
                          None, None) == -4
    assert lib.kpa_decode(d, None, 0, 4096, None, 4096, None, None, None, None, None, 0, 0, None, None) == 0
    # factored query: rank out of range, missing factor, nothing to do
    fq = lib.kpa_decode_factored
    assert fq(d, 0, FAKE, 1, 64, FAKE, 64, 1, 0, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, 0, None, None) == -1
    assert fq(d, 17, FAKE, 1, 64, FAKE, 64, 1, 0, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, 0, None, None) == -1
    assert fq(d, 2, FAKE, 1, 64, FAKE, 64, 1, 0, FAKE, None, FAKE, FAKE, None, FAKE, 1 << 30, 0, None, None) == -2
    assert fq(d, 2, FAKE, 1, 64, FAKE, 64, 1, 0, None, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, 0, None, None) == -2
    assert fq(d, 2, None, 0, 64, None, 64, 1, 0, None, None, None, None, None, None, 0, 0, None, None) == 0
    # projection + append: d_model a positive multiple of 64, pointers, nothing to do
    pa = lib.kpa_project_append
    assert pa(d, FAKE, 1, 64, FAKE, 100, FAKE, FAKE, FAKE, 1, None, None) == -7
    assert pa(d, FAKE, 1, 64, FAKE, 0, FAKE, FAKE, FAKE, 1, None, None) == -7
    assert pa(d, FAKE, 1, 64, None, 128, FAKE, FAKE, FAKE, 1, None, None) == -2
    assert pa(d, FAKE, 1, 64, FAKE, 128, FAKE, FAKE, None, 1, None, None) == -2
    assert pa(d, FAKE + 2, 1, 64, FAKE, 128, FAKE, FAKE, FAKE, 1, None, None) == -7
    assert pa(d, None, 0, 64, None, 128, None, None, None, 1, None, None) == 0
    assert pa(d, None, 1, 64, None, 128, None, None, None, 0, None, None) == 0
    # append + decode: the append arguments are checked first, then the decode's
    ad = lib.kpa_append_decode
    big = 1 << 30
    assert ad(d, FAKE, 1, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -1, FAKE, 64, 1, 0, FAKE, FAKE, FAKE, None,
              FAKE, big, 0, None, None) == -7
    assert ad(d, FAKE, 1, 64, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, 64, 1, 0, FAKE, FAKE, FAKE, None,
              FAKE, big, 0, None, None) == -2
    assert ad(d, FAKE, 1, 64, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, FAKE, 64, 1, 0, FAKE, FAKE, FAKE, None,
              FAKE, big, 0, None, None) == -2
    # n_new = 0 needs no append input; the decode's own checks still apply
    assert ad(d, None, 1, 64, None, None, None, None, None, None, 0, FAKE, 64, 1, 0, FAKE, FAKE, FAKE, None,
              FAKE, big, 0, None, None) == -2
    assert ad(d, FAKE, 1, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, 65, 1, 0, FAKE, FAKE, FAKE, None,
              FAKE, big, 0, None, None) == -7
    assert ad(d, None, 0, 64, None, None, None, None, None, None, 1, None, 64, 1, 0, None, None, None, None,
              None, 0, 0, None, None) == 0
    # streaming read (measurement aid): pointers, sizes, alignment, block count
    sx = lib.kpa_stream_xor
    assert sx(None, 1024, FAKE, 4, None) == -2
    assert sx(FAKE, 1024, None, 4, None) == -2
    assert sx(FAKE, 0, FAKE, 4, None) == -7
    assert sx(FAKE, 1000, FAKE, 4, None) == -7
    assert sx(FAKE + 8, 1024, FAKE, 4, None) == -7
    assert sx(FAKE, 1024, FAKE, 0, None) == -7
    assert sx(FAKE, 1024, FAKE, 65536, None) == -7


def test_workspace_sizes_follow_the_split_count():
    dims = kpa.make_dims(4, 4, 8, 16, 2, 2)
    h, dh = 16, 128
    assert kpa.kpa_decode_workspace_bytes(dims, 2, 4096, 1, 1) == 0
    assert kpa.kpa_decode_workspace_bytes(dims, 2, 4096, 1, 8) == 2 * 8 * h * (dh + 2) * 4
    # a forced count above the number of 32-slot tiles is clamped
    assert kpa.kpa_decode_workspace_bytes(dims, 1, 64, 1, 99) == 1 * 2 * h * (dh + 2) * 4


def test_status_strings():
    for code in range(-7, 1):
        assert kpa.kpa_status_string(code)
    assert kpa.kpa_status_string(-99) == "unknown status"


def test_kernel_timing_hook_needs_both_events_or_none():
    lib = kpa.load()
    assert lib.kpa_time_next_decode_kernel(FAKE, None) == -2  # KPA_ERR_NULL_PTR
    assert lib.kpa_time_next_decode_kernel(None, FAKE) == -2
    # both NULL cancels; a pending pair is dropped by the next decode call even
    # when that call fails its checks, so no later call touches FAKE handles
    assert lib.kpa_time_next_decode_kernel(None, None) == 0
    assert lib.kpa_time_next_decode_kernel(FAKE, FAKE) == 0
    dims = kpa.make_dims(4, 4, 8, 16, 2, 2)
    st = lib.kpa_decode(ctypes.byref(dims), FAKE, 1, 64, FAKE, 128, FAKE, FAKE, FAKE, None, None, 0, 0, None, None)
    assert st != 0
    assert lib.kpa_time_next_decode_kernel(None, None) == 0


def test_binding_constants_match_the_header():
    import os
    import re
    text = open(os.path.join(os.path.dirname(__file__), "..", "include", "kpa.h")).read()
    defines = dict(re.findall(r"#define (KPA_\w+) (\d+)u?", text))
    for name in ("KPA_MAX_HEADS", "KPA_MAX_HEAD_DIM", "KPA_MAX_RANK", "KPA_MAX_HD", "KPA_MAX_NQ",
                 "KPA_DEV_SLOT_OUT_OF_RANGE", "KPA_DEV_NEGATIVE_POSITION", "KPA_DEV_CTX_OUT_OF_RANGE"):
        assert int(defines[name]) == getattr(kpa, name), name


def test_limits_are_enforced():
    lib = kpa.load()
    ok = kpa.make_dims(4, 8, 16, 16, kpa.KPA_MAX_RANK, kpa.KPA_MAX_RANK)  # h d_h = 8192 exactly
    assert lib.kpa_cache_layout(ctypes.byref(ok), 1, 32, None) == -2  # dims accepted; then the NULL output
    for bad in (kpa.make_dims(4, 8, 16, 16, kpa.KPA_MAX_RANK + 1, 1),   # rank
                kpa.make_dims(16, 9, 8, 8, 1, 1),                        # h = 144 > 128
                kpa.make_dims(2, 2, 32, 16, 1, 1),                       # d_h = 512 > 256
                kpa.make_dims(8, 8, 16, 16, 1, 1)):                      # h d_h = 16384 > 8192
        assert lib.kpa_cache_layout(ctypes.byref(bad), 1, 32, None) == -1
    d = ctypes.byref(kpa.make_dims(4, 4, 8, 16, 2, 2))
    big = 1 << 30
    assert lib.kpa_decode_multiq(d, FAKE, 1, 64, FAKE, 64, kpa.KPA_MAX_NQ + 1, 1, FAKE, FAKE, FAKE, None, FAKE,
                                 big, 0, None, None) == -7
    assert lib.kpa_decode_multiq(d, FAKE, 1025, 64, FAKE, 64, 64, 1, FAKE, FAKE, FAKE, None, FAKE,
                                 big, 0, None, None) == -7  # batch * n_q > 65535


def test_capacity_limit():
    lib = kpa.load()
    d = kpa.make_dims(4, 4, 8, 16, 2, 2)
    info = kpa.kpa_cache_layout(d, 1, kpa.KPA_MAX_CAPACITY)
    assert info["n_tiles"] == kpa.KPA_MAX_CAPACITY // 32
    dp = ctypes.byref(d)
    for cap in (kpa.KPA_MAX_CAPACITY + 1, 2 ** 31 - 1):
        assert lib.kpa_cache_bytes(dp, 1, cap) == 0
        assert lib.kpa_cache_append(dp, FAKE, 1, cap, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None, None) == -7
        assert lib.kpa_project_append(dp, FAKE, 1, cap, FAKE, 256, FAKE, FAKE, FAKE, 1, None, None) == -7
        assert lib.kpa_decode(dp, FAKE, 1, cap, FAKE, 64, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, 0, None,
                              None) == -7


# Which shapes the matrix-core kernels take (host-side path choice; no GPU).
# bf16 caches with a feature dimension of 8, 16, 32 or 64 contracted on the
# matrix cores, the other a power of two up to 32, ranks up to 4, within the
# row, wave and LDS caps include/kpa.h states; everything else on the
# vector ALUs.
MATRIX_CORE_SHAPES = [
    # the workload configurations and the KPA page's head splits (d1 = d2 = 8, R = 2)
    (12, 1, 1, 64, 2, 2), (4, 4, 8, 16, 2, 2), (8, 4, 8, 16, 2, 4), (4, 8, 16, 8, 4, 4),
    (8, 2, 8, 8, 2, 2), (4, 4, 8, 8, 2, 2), (2, 8, 8, 8, 2, 2), (10, 2, 8, 8, 2, 2), (4, 5, 8, 8, 2, 2),
    (2, 10, 8, 8, 2, 2), (5, 5, 8, 8, 2, 2), (6, 2, 8, 8, 2, 2), (4, 3, 8, 8, 2, 2), (3, 4, 8, 8, 2, 2),
    (2, 6, 8, 8, 2, 2),
    # FlashTPA's shapes
    (16, 1, 1, 64, 1, 1), (32, 1, 1, 64, 1, 1), (48, 1, 1, 64, 1, 1),
    # generic families
    (3, 2, 8, 8, 1, 1), (6, 3, 8, 8, 3, 2), (16, 2, 8, 8, 2, 2), (2, 16, 8, 8, 1, 1), (4, 2, 4, 16, 1, 3),
    (3, 3, 8, 16, 2, 2), (8, 2, 16, 16, 2, 2), (4, 2, 2, 32, 2, 2), (4, 4, 4, 32, 4, 1), (2, 2, 8, 32, 3, 3),
    (20, 1, 1, 64, 2, 2), (7, 1, 1, 64, 1, 1), (8, 2, 2, 64, 1, 2), (6, 1, 4, 64, 3, 3), (2, 2, 32, 8, 2, 2),
    (3, 4, 16, 2, 2, 2), (4, 4, 8, 16, 4, 4), (4, 4, 8, 16, 3, 1), (2, 4, 16, 8, 1, 4),
]
VECTOR_ALU_SHAPES = [
    (3, 5, 3, 6, 2, 2),     # no feature dimension of 8, 16, 32 or 64
    (3, 3, 6, 8, 2, 2),     # the other feature dimension (6) not a power of two
    (4, 4, 8, 16, 5, 2),    # rank above 4
    (7, 1, 1, 64, 2, 2),    # 7 rows with two key ranks
    (2, 2, 4, 4, 2, 2),     # feature dimensions 4 and 4
]


@pytest.mark.parametrize("shape", MATRIX_CORE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_matrix_core_path_for_shapes_in_the_family(shape):
    dims = kpa.make_dims(*shape)
    assert kpa.kpa_decode_path(dims, 1) == "mfma_bf16"


@pytest.mark.parametrize("shape", VECTOR_ALU_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_vector_alu_path_outside_the_family(shape):
    dims = kpa.make_dims(*shape)
    assert kpa.kpa_decode_path(dims, 1) == "valu"
    # float32 caches always take the vector ALUs
    assert kpa.kpa_decode_path(kpa.make_dims(4, 4, 8, 16, 2, 2, dtype="f32"), 1) == "valu"


@pytest.mark.parametrize("shape", [(4, 8, 16, 8, 4, 4), (6, 3, 8, 8, 3, 2), (20, 1, 1, 64, 2, 2),
                                   (8, 2, 16, 16, 2, 2), (3, 4, 16, 2, 2, 2)], ids=lambda s: "x".join(map(str, s)))
def test_matrix_core_path_for_several_queries(shape):
    dims = kpa.make_dims(*shape)
    # q1 = 16, q2 = 8 with an even p2 <= 8 rebuilds K and V per tile
    rebuild = shape[2] == 16 and shape[3] == 8 and shape[1] in (2, 4, 6, 8)
    assert kpa.kpa_decode_path(dims, 16) == ("mfma_rebuild" if rebuild else "mfma_bf16")
    assert kpa.kpa_decode_path(dims, 7) == "mfma_bf16"


def test_noalloc_scratch_limit_matches_binding_and_is_enforced_before_launch():
    text = open(os.path.join(ROOT, "include", "kpa.h")).read()
    m = re.search(r"#define KPA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == kpa.KPA_NOALLOC_SCRATCH_BYTES
    lib = kpa.load()
    d = ctypes.byref(kpa.make_dims(4, 4, 8, 16, 2, 2))
    # 256 sequences x 64 chunks of partials (136 MB) exceed the scratch: refused before anything runs
    need = lib.kpa_decode_workspace_bytes(d, 256, 65536, 1, 64)
    assert need > kpa.KPA_NOALLOC_SCRATCH_BYTES
    st = lib.kpa_append_decode_noalloc(d, FAKE, 256, 65536, None, None, None, None, None, None, 0, FAKE, 65536, 1,
                                       1, FAKE, FAKE, FAKE, None, 64, None, None)
    assert st == -4  # KPA_ERR_WORKSPACE
    # argument errors come first, as for kpa_append_decode
    st = lib.kpa_append_decode_noalloc(d, FAKE, 1, 64, None, None, None, None, None, None, 0, FAKE, 65, 1,
                                       1, FAKE, FAKE, FAKE, None, 0, None, None)
    assert st == -7  # KPA_ERR_INVALID_ARG (max_ctx > capacity)
