"""The kernel path the library picks for a shape (`kpa_decode_path`, host
only) against the rule `include/kpa.h` states for it, on seeded random
shapes within the kpa_dims limits.

The rule is restated here from that header's text, independently of the
kernel tables: a bf16 shape runs on the matrix cores when it is one of the
tuned shapes, or when one factor F has a contracted feature dimension of 8,
16, 32 or 64 and the other factor G meets the row, rank, head-count and LDS
conditions of a generic family; everything else (and every float32 cache)
runs on the vector ALUs.  Several queries per sequence (8 or more) on
shapes with q1 = 16, q2 = 8, an even p2 up to 8 and ranks up to 4 -- or,
from 12 queries, q1 = 8, q2 = 16 and p1 = 8 -- rebuild K and V per tile on
the matrix cores instead.
"""
import random

import pytest

import factorized_kv_cache_kpa_amd as kpa

# The tuned shapes (p1, p2, q1, q2, r_k, r_v), any query count: the workload
# configurations, the KPA page's head splits and FlashTPA's shapes.
TUNED = {
    (4, 4, 8, 16, 2, 2), (4, 4, 8, 16, 1, 1), (8, 4, 8, 16, 2, 4), (4, 8, 16, 8, 4, 4),
    (12, 1, 1, 64, 2, 2), (16, 1, 1, 64, 1, 1), (32, 1, 1, 64, 1, 1), (48, 1, 1, 64, 1, 1),
    (8, 2, 8, 8, 2, 2), (4, 4, 8, 8, 2, 2), (2, 8, 8, 8, 2, 2), (10, 2, 8, 8, 2, 2), (4, 5, 8, 8, 2, 2),
    (2, 10, 8, 8, 2, 2), (5, 5, 8, 8, 2, 2), (6, 2, 8, 8, 2, 2), (4, 3, 8, 8, 2, 2), (3, 4, 8, 8, 2, 2),
    (2, 6, 8, 8, 2, 2),
}
# tuned shapes with a multi-query kernel of their own
TUNED_MULTI = {(4, 8, 16, 8, 4, 4), (4, 4, 8, 16, 2, 2), (8, 4, 8, 16, 2, 4)}

LDS_BYTES = 160 * 1024


def _pow2_ceil(x):
    p = 1
    while p < x:
        p *= 2
    return p


def _generic_lds(pg, qg, pf, r_k, r_v, multi):
    """LDS of a generic launch: two buffers of the tile's G factors (key set in
    16-byte chunks of 8 elements, 512 B per chunk for 32 slots; value set 64 B
    per element row; each set padded to whole 1 KB blocks), the rotary table
    (32 angle pairs per query of the workgroup) and per-wave score rows."""
    m = pg * qg
    gk = (r_k * m + 7) // 8 * 512
    gv = r_v * m * 64
    blocks = (gk + 1023) // 1024 + (gv + 1023) // 1024
    nqw = 2 if multi else 1
    rows_p = max(2, _pow2_ceil(nqw * pg))
    return 2 * blocks * 1024 + nqw * 32 * 2 * 4 + pf * rows_p * (36 + 3) * 4


def _generic_ok(pf, qf, pg, qg, r_k, r_v, multi):
    """One orientation (F = the factor with feature dimension qf, pf heads)."""
    if qf not in (8, 16, 32, 64) or qg not in (1, 2, 4, 8, 16, 32):
        return False
    if r_k > 4 or r_v > 4:
        return False
    m = pg * qg
    if qf <= 16:
        max_rows = 128
    else:
        max_rows = 32 if multi else 64
    if m > max_rows or (m % 4 != 0 and r_k != 1):
        return False
    if multi:
        if pf > 4 or 2 * pg > 64:
            return False
    else:
        if pg > 64:
            return False
        cap = 4 if (m > 64 or r_k > 2 or r_v > 2 or qf >= 32) else 8
        if pf > cap:
            return False
    return _generic_lds(pg, qg, pf, r_k, r_v, multi) <= LDS_BYTES


def documented_path(p1, p2, q1, q2, r_k, r_v, n_q):
    multi = n_q > 1
    shape = (p1, p2, q1, q2, r_k, r_v)
    if r_k <= 4 and r_v <= 4 and (
            (n_q >= 8 and q1 == 16 and q2 == 8 and p2 in (2, 4, 6, 8))
            or (n_q >= 12 and q1 == 8 and q2 == 16 and p1 == 8)):
        return "mfma_rebuild"
    if shape in TUNED and (not multi or shape in TUNED_MULTI):
        return "mfma_bf16"
    if _generic_ok(p2, q2, p1, q1, r_k, r_v, multi) or _generic_ok(p1, q1, p2, q2, r_k, r_v, multi):
        return "mfma_bf16"
    return "valu"


def _random_shapes(n, seed):
    rng = random.Random(seed)
    qs = [1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 64]
    out = []
    while len(out) < n:
        p1, p2 = rng.choice([1, 2, 3, 4, 5, 6, 8, 10, 12, 16, 24, 32]), rng.choice([1, 2, 3, 4, 5, 6, 8, 10, 16])
        q1, q2 = rng.choice(qs), rng.choice([2, 4, 6, 8, 12, 16, 32, 64])  # RoPE pairs: q2 even
        if rng.random() < 0.15:
            # many heads on one side with a feature dimension of 1 (the TPA split and its kin)
            p1, p2, q1 = rng.choice([40, 48, 64, 72, 96, 128]), rng.choice([1, 2]), 1
        r_k, r_v = rng.randint(1, 5), rng.randint(1, 5)
        h, dh = p1 * p2, q1 * q2
        if h > 128 or dh > 256 or h * dh > 8192:
            continue
        out.append((p1, p2, q1, q2, r_k, r_v))
    return out


SHAPES = _random_shapes(400, seed=2024)


@pytest.mark.parametrize("n_q", [1, 4, 16])
def test_library_path_matches_the_documented_rule(n_q):
    mismatches = []
    for shape in SHAPES:
        dims = kpa.make_dims(*shape)
        got = kpa.kpa_decode_path(dims, n_q)
        want = documented_path(*shape, n_q)
        if got != want:
            mismatches.append((shape, got, want))
    assert not mismatches, f"{len(mismatches)} of {len(SHAPES)} differ, e.g. {mismatches[:5]}"
    # the sample covers both paths
    paths = {kpa.kpa_decode_path(kpa.make_dims(*s), n_q) for s in SHAPES + REBUILD_SHAPES}
    assert paths == ({"mfma_bf16", "valu", "mfma_rebuild"} if n_q >= 8 else {"mfma_bf16", "valu"})


# shapes of the rebuild family and its edges (q1 = 16, q2 = 8, and swapped)
REBUILD_SHAPES = [(p1, p2, 16, 8, rk, rv) for p1 in (1, 3, 4) for p2 in (1, 2, 3, 4, 6, 8, 10)
                  for rk, rv in ((1, 1), (4, 4), (2, 3), (5, 2))]
REBUILD_SHAPES += [(p1, p2, 8, 16, rk, rv) for p1 in (1, 2, 3, 4, 6, 8, 10) for p2 in (1, 3, 4)
                   for rk, rv in ((1, 1), (4, 4), (2, 3), (2, 5))]


@pytest.mark.parametrize("n_q", [1, 7, 8, 11, 12, 16, 64])
def test_rebuild_family_matches_the_documented_rule(n_q):
    for shape in REBUILD_SHAPES:
        assert kpa.kpa_decode_path(kpa.make_dims(*shape), n_q) == documented_path(*shape, n_q), shape


def test_float32_caches_take_the_vector_alus():
    for shape in SHAPES[:50]:
        assert kpa.kpa_decode_path(kpa.make_dims(*shape, dtype="f32"), 1) == "valu"
