"""Decode parity on seeded random shapes within the kpa_dims limits: whatever
kernel the library picks (a tuned matrix-core shape, a generic matrix-core
family in either orientation, or the vector-ALU kernel), every output row
matches the float64 oracle.  Small ragged contexts over several tiles, one
and three queries, bf16 and (for a few shapes) float32 caches."""
import math

import pytest

import factorized_kv_cache_kpa_amd as kpa
from oracle import kpa_oracle
from tests.kpa_testutil import assert_close, dims_of, fill_cache, run_decode, scale_of
from tests.test_path_rule import SHAPES
from workloads import make_inputs
from workloads.configs import Config

pytestmark = pytest.mark.gpu

# from the host test's sample: the first 30 shapes on the matrix cores and the
# first 20 on the vector ALUs (for one query)
def _cases():
    try:
        path = [kpa.kpa_decode_path(kpa.make_dims(*sh), 1) for sh in SHAPES]
    except (OSError, RuntimeError):  # library not built: the tests then fail when they load it
        return SHAPES[:50]
    return ([sh for sh, p in zip(SHAPES, path) if p == "mfma_bf16"][:30]
            + [sh for sh, p in zip(SHAPES, path) if p == "valu"][:20])


CASES = _cases()


@pytest.mark.parametrize("idx", range(len(CASES)), ids=lambda i: "x".join(map(str, CASES[i])))
@pytest.mark.parametrize("n_q", [1, 3])
def test_random_shape_matches_oracle(gpu_lib, idx, n_q):
    p1, p2, q1, q2, r_k, r_v = CASES[idx]
    dtype = "f32" if idx % 7 == 3 else "bf16"
    cfg = Config(f"rand_{idx}", p1, p2, q1, q2, r_k, r_v, dtype, batch=2, ctx=200 + 37 * idx % 300,
                 n_q=n_q, sigma_a=1 / math.sqrt(q1), sigma_b=1 / math.sqrt(q2))
    inp = make_inputs(cfg, seed=300 + idx, ragged=True, q_scale=2.0)
    dims = dims_of(cfg)
    path = kpa.kpa_decode_path(dims, n_q)
    assert path in ("mfma_bf16", "valu")
    cache, cap = fill_cache(inp, dims)
    ro, rl = kpa_oracle.decode(inp.a_k, inp.b_k, inp.a_v, inp.b_v, inp.positions, inp.ctx_len, inp.q, inp.q_pos)
    go, gl = run_decode(inp, dims, cache, cap)
    assert_close(go, gl, ro, rl, cfg.dtype, f"{cfg.name} {CASES[idx]} n_q={n_q} {path}", scale=scale_of(inp))
