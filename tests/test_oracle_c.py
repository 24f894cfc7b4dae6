"""The streaming C oracle equals the literal NumPy oracle.

The C oracle is what the full-size parity checks and the CPU baseline use, so
it is pinned here to ``kpa_ref`` (itself pinned in test_oracle_pins.py) on
random small shapes covering every structural case: non-degenerate splits,
the TPA split, d1 = 1, unequal ranks, ragged and empty contexts, causal and
non-causal multi-query, float32 and bfloat16 inputs, and row selection.
"""
import numpy as np
import pytest
import torch

from oracle import kpa_oracle, kpa_ref
from workloads import CONFIGS, make_inputs


def setup_module(module):
    kpa_oracle.build(force=True)


SHAPES = [
    # p1, p2, q1, q2, r_k, r_v
    (2, 2, 4, 4, 2, 2),
    (12, 1, 1, 64, 2, 2),   # TPA degenerate split
    (3, 2, 1, 6, 1, 3),     # d1 = 1
    (2, 3, 3, 2, 3, 1),
    (1, 1, 2, 2, 1, 1),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("n_q,causal", [(1, True), (3, True), (2, False)])
def test_c_oracle_equals_numpy_oracle(shape, n_q, causal):
    p1, p2, q1, q2, r_k, r_v = shape
    cfg = CONFIGS["tiny_f32"].scaled(p1=p1, p2=p2, q1=q1, q2=q2, r_k=r_k, r_v=r_v)
    inp = make_inputs(cfg, seed=sum(shape) + n_q, batch=3, ctx=13, n_q=n_q, ragged=True, q_scale=3.0)
    args = (inp.a_k, inp.b_k, inp.a_v, inp.b_v, inp.positions, inp.ctx_len, inp.q, inp.q_pos)
    o_ref, l_ref = kpa_ref.decode(*[a.numpy() for a in args], causal=causal)
    o_c, l_c = kpa_oracle.decode(*args, causal=causal)
    np.testing.assert_allclose(o_c, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_c, l_ref, rtol=0, atol=1e-12)


def test_c_oracle_bf16_inputs_and_row_selection():
    cfg = CONFIGS["kpa_32k"]
    inp = make_inputs(cfg, seed=5, batch=2, ctx=40)
    args = (inp.a_k, inp.b_k, inp.a_v, inp.b_v, inp.positions, inp.ctx_len, inp.q, inp.q_pos)
    f64 = [a.to(torch.float64).numpy() if a.is_floating_point() else a.numpy() for a in args]
    o_ref, l_ref = kpa_ref.decode(*f64)
    o_c, l_c = kpa_oracle.decode(*args)
    np.testing.assert_allclose(o_c, o_ref, rtol=0, atol=1e-12)
    items = np.array([[1, 0, 15], [0, 0, 3], [1, 0, 0]])
    o_s, l_s = kpa_oracle.decode(*args, items=items)
    for k, (b, n, hd) in enumerate(items):
        np.testing.assert_array_equal(o_s[k], o_c[b, n, hd])
        assert l_s[k] == l_c[b, n, hd]


def test_c_oracle_empty_context():
    cfg = CONFIGS["tiny_f32"]
    inp = make_inputs(cfg, seed=1, batch=2, ctx=8)
    inp.ctx_len[:] = 0
    o, l = kpa_oracle.decode(inp.a_k, inp.b_k, inp.a_v, inp.b_v, inp.positions, inp.ctx_len,
                             inp.q, inp.q_pos, causal=False)
    assert np.all(o == 0) and np.all(np.isneginf(l))
