"""Pins of the NumPy oracle to what the pages and the mathematics fix.

Sources:
  [KPA] "Kronecker Product Attention: Memory-Efficient KV Compression via
        Structured Factorization" (arXiv 2610.12657)
  [TPA] "Tensor Product Attention Is All You Need" (arXiv 2501.06425),
        architecture-summary page
Each test names the passage it pins.  None of them re-calls the oracle
function it checks as its own expected value.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import kpa_ref as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _rand(*shape):
    return RNG.standard_normal(shape)


# --------------------------------------------------------------------------
# Kronecker product and factorised K/V  ([KPA] Def. 2.1, Eq. (1), Eqs. (3)-(4))
# --------------------------------------------------------------------------
@pytest.mark.parametrize("shapes", [((2, 3), (4, 5)), ((1, 1), (3, 2)), ((3, 1), (1, 4)), ((4, 4), (4, 4))])
def test_kron_reconstruct_matches_block_definition(shapes):
    (m1, n1), (m2, n2) = shapes
    a, b = _rand(1, m1, n1), _rand(1, m2, n2)
    np.testing.assert_allclose(ref.kron_reconstruct(a, b), ref.kron_block(a[0], b[0]), rtol=0, atol=1e-15)


def test_kron_entry_index_convention():
    # head i = i1*p2 + i2, feature j = j1*q2 + j2: entry is a[i1,j1] * b[i2,j2]  ([KPA] Def. 2.1)
    p1, q1, p2, q2 = 3, 2, 2, 4
    a, b = _rand(1, p1, q1), _rand(1, p2, q2)
    k = ref.kron_reconstruct(a, b)
    for i1 in range(p1):
        for i2 in range(p2):
            for j1 in range(q1):
                for j2 in range(q2):
                    assert k[i1 * p2 + i2, j1 * q2 + j2] == pytest.approx(a[0, i1, j1] * b[0, i2, j2], abs=1e-15)


def test_kron_sum_is_normalised_by_rank():
    # (1/R) sum_r: R identical terms reconstruct the single term  ([KPA] Eqs. (3)-(4))
    a, b = _rand(1, 2, 3), _rand(1, 4, 2)
    a3, b3 = np.repeat(a, 3, axis=0), np.repeat(b, 3, axis=0)
    np.testing.assert_allclose(ref.kron_reconstruct(a3, b3), ref.kron_block(a[0], b[0]), atol=1e-14)


def test_mixed_product_identity():
    # (M (x) N)(P (x) Q) = (MP) (x) (NQ)  ([KPA] Eq. (1))
    m, n, p, q = _rand(2, 3), _rand(4, 2), _rand(3, 5), _rand(2, 3)
    lhs = ref.kron_block(m, n) @ ref.kron_block(p, q)
    rhs = ref.kron_block(m @ p, n @ q)
    np.testing.assert_allclose(lhs, rhs, atol=1e-12)


def test_tpa_degenerate_split_is_outer_product():
    # h1 = h, d1 = 1, h2 = 1, d2 = d_h: each term is the outer product a b^T  ([KPA] §2.2;
    # [TPA] summary, (a (x) b)_ij = a_i b_j)
    h, d_h, r = 7, 6, 3
    a, b = _rand(r, h, 1), _rand(r, 1, d_h)
    expect = sum(np.outer(a[k, :, 0], b[k, 0, :]) for k in range(r)) / r
    np.testing.assert_allclose(ref.kron_reconstruct(a, b), expect, atol=1e-14)


# --------------------------------------------------------------------------
# Cache size  ([KPA] Eq. (10)/(11), printed ratios; [TPA] printed sizes)
# --------------------------------------------------------------------------
def test_compression_factor_reproduces_printed_values():
    cases = json.load(open(os.path.join(GOLDEN, "kpa_compression.json")))["cases"]
    for c in cases:
        got = ref.compression_factor(c["p1"], c["p2"], c["q1"], c["q2"], c["r_k"], c["r_v"])
        assert round(got, c["digits"]) == pytest.approx(c["printed"]), c
        # the same ratio from the numbers one token's factor arrays really hold
        ak = np.zeros((c["r_k"], c["p1"], c["q1"]))
        bk = np.zeros((c["r_k"], c["p2"], c["q2"]))
        av = np.zeros((c["r_v"], c["p1"], c["q1"]))
        bv = np.zeros((c["r_v"], c["p2"], c["q2"]))
        h, d_h = c["p1"] * c["p2"], c["q1"] * c["q2"]
        counted = ref.mha_numbers_per_token(h, d_h) / ref.cached_numbers_per_token(ak, bk, av, bv)
        assert counted == pytest.approx(got, rel=1e-15)


def test_tpa_cache_numbers_reproduce_printed_values():
    g = json.load(open(os.path.join(GOLDEN, "tpa_cache_numbers.json")))
    for c in g["tpa_cases"]:
        h, d_h = c["h"], c["d_h"]
        # TPA is the degenerate KPA split (p1 = h, q1 = 1, p2 = 1, q2 = d_h)
        ak, bk = np.zeros((c["r_k"], h, 1)), np.zeros((c["r_k"], 1, d_h))
        av, bv = np.zeros((c["r_v"], h, 1)), np.zeros((c["r_v"], 1, d_h))
        n = ref.cached_numbers_per_token(ak, bk, av, bv)
        assert n == c["numbers"], c
        if "ratio_vs_mha" in c:
            assert round(n / ref.mha_numbers_per_token(h, d_h), c["ratio_digits"]) == pytest.approx(c["ratio_vs_mha"])
    for c in g["mha_cases"]:
        assert ref.mha_numbers_per_token(c["h"], c["d_h"]) == c["numbers"]
        if "bytes_half" in c:
            assert 2 * ref.mha_numbers_per_token(c["h"], c["d_h"]) == c["bytes_half"]


# --------------------------------------------------------------------------
# Kronecker-separable RoPE  ([KPA] Def. 2.3, Thm. 2.4, App. A.2)
# --------------------------------------------------------------------------
def test_rope_convention_sign_pairs_and_frequencies():
    # pair m turns by pos*theta_m with theta_0 = 1 and theta_m = base^(-2m/d2):
    # at pos = pi/(2 theta_m) the rotation maps e_{2m} to e_{2m+1} (counter-clockwise)
    q2, base = 8, 10000.0
    for m in range(q2 // 2):
        theta_m = base ** (-(2.0 * m) / q2)
        rot = ref.rope_block(math.pi / (2 * theta_m), q2, base)
        e = np.zeros(q2)
        e[2 * m] = 1.0
        out = rot @ e
        want = np.zeros(q2)
        want[2 * m + 1] = 1.0
        np.testing.assert_allclose(out, want, atol=1e-9)
    # theta_0 = 1: position pi is a half turn of the first pair
    rot = ref.rope_block(math.pi, q2, base)
    np.testing.assert_allclose(rot[:2, :2], -np.eye(2), atol=1e-12)


def test_rope_matches_complex_multiplication_form():
    # RoFormer's complex form: (x_{2m} + i x_{2m+1}) * exp(i pos theta_m)
    q2, pos = 16, 12345
    x = _rand(q2)
    theta = 10000.0 ** (-np.arange(0, q2, 2) / q2)
    z = (x[0::2] + 1j * x[1::2]) * np.exp(1j * pos * theta)
    want = np.empty(q2)
    want[0::2], want[1::2] = z.real, z.imag
    np.testing.assert_allclose(ref.rope_block(pos, q2) @ x, want, atol=1e-12)


@pytest.mark.parametrize("t,s", [(0, 5), (17, 3), (40000, 524287)])
def test_rope_relative_position_property(t, s):
    # R(t)^T R(s) = R(s - t)  ([KPA] App. A.2)
    q2 = 16
    lhs = ref.rope_block(t, q2).T @ ref.rope_block(s, q2)
    np.testing.assert_allclose(lhs, ref.rope_block(s - t, q2), atol=1e-9)


def test_rope_kpa_rotates_only_the_b_factor():
    # (I_{d1} (x) R(t)) (a (x) b) = a (x) R(t) b  ([KPA] Thm. 2.4, Eqs. (7)-(8))
    q1, q2, t = 4, 8, 321
    a, b = _rand(q1), _rand(q2)
    lhs = ref.rope_kpa(t, q1, q2) @ np.kron(a, b)
    rhs = np.kron(a, ref.rope_block(t, q2) @ b)
    np.testing.assert_allclose(lhs, rhs, atol=1e-12)
    # and it is not R(t) (x) I (the other Kronecker order)
    assert not np.allclose(ref.rope_kpa(t, q1, q2), np.kron(ref.rope_block(t, q2), np.eye(q1)))


def test_rope_with_d1_one_is_ordinary_rope_over_d_h():
    # d1 = 1: R_KPA = R^(2) over the whole head dimension  ([KPA] Def. 2.3)
    np.testing.assert_allclose(ref.rope_kpa(77, 1, 12), ref.rope_block(77, 12), atol=0)


def test_append_rotate_equals_rotating_full_key():
    # caching R(t) B^K and rebuilding K equals rotating every row of K  ([KPA] Eq. (8), §2.4 (i))
    r, p1, q1, p2, q2, t = 3, 2, 3, 4, 8, 999
    a, b = _rand(r, p1, q1), _rand(r, p2, q2)
    k_pre = ref.kron_reconstruct(a, ref.append_rotate(b, t))
    k_rot = ref.kron_reconstruct(a, b) @ ref.rope_kpa(t, q1, q2).T
    np.testing.assert_allclose(k_pre, k_rot, atol=1e-12)


# --------------------------------------------------------------------------
# Factored score and relative position  ([KPA] Prop. 2.2 / Eq. (6), Eq. (9))
# --------------------------------------------------------------------------
def test_dense_score_equals_factored_score():
    rq, rk, p1, q1, p2, q2 = 3, 2, 2, 3, 3, 4
    aq, bq, ak, bk = _rand(rq, p1, q1), _rand(rq, p2, q2), _rand(rk, p1, q1), _rand(rk, p2, q2)
    qm, km = ref.kron_reconstruct(aq, bq), ref.kron_reconstruct(ak, bk)
    for i1 in range(p1):
        for i2 in range(p2):
            i = i1 * p2 + i2
            assert float(qm[i] @ km[i]) == pytest.approx(ref.factored_score(aq, bq, ak, bk, i1, i2), abs=1e-12)


def test_score_depends_only_on_relative_position():
    # Eq. (9): rotating q at t and the key factors at s equals rotating B^K by s - t
    rq, rk, p1, q1, p2, q2 = 2, 2, 2, 2, 2, 8
    aq, bq, ak, bk = _rand(rq, p1, q1), _rand(rq, p2, q2), _rand(rk, p1, q1), _rand(rk, p2, q2)
    t, s = 1000, 37
    qm = ref.kron_reconstruct(aq, bq) @ ref.rope_kpa(t, q1, q2).T
    km = ref.kron_reconstruct(ak, bk) @ ref.rope_kpa(s, q1, q2).T
    rel = np.einsum("ab,rib->ria", ref.rope_block(s - t, q2), bk)
    for i1 in range(p1):
        for i2 in range(p2):
            i = i1 * p2 + i2
            assert float(qm[i] @ km[i]) == pytest.approx(ref.factored_score(aq, bq, ak, rel, i1, i2), abs=1e-12)


def _small_problem(p1=2, p2=3, q1=2, q2=4, r_k=2, r_v=3, nb=2, s=9, n_q=1, seed=0):
    rng = np.random.default_rng(seed)
    ak = rng.standard_normal((nb, s, r_k, p1, q1))
    bk = rng.standard_normal((nb, s, r_k, p2, q2))
    av = rng.standard_normal((nb, s, r_v, p1, q1))
    bv = rng.standard_normal((nb, s, r_v, p2, q2))
    pos = np.tile(np.arange(s), (nb, 1))
    ctx = np.full(nb, s)
    q = rng.standard_normal((nb, n_q, p1 * p2, q1 * q2))
    qp = ctx[:, None] - n_q + np.arange(n_q)[None, :]
    return ak, bk, av, bv, pos, ctx, q, qp


def test_decode_is_invariant_to_a_common_position_shift():
    ak, bk, av, bv, pos, ctx, q, qp = _small_problem(n_q=3)
    o1, l1 = ref.decode(ak, bk, av, bv, pos, ctx, q, qp)
    o2, l2 = ref.decode(ak, bk, av, bv, pos + 70000, ctx, q, qp + 70000)
    np.testing.assert_allclose(o1, o2, atol=1e-10)
    np.testing.assert_allclose(l1, l2, atol=1e-10)


# --------------------------------------------------------------------------
# Softmax special cases and MHA / MQA / GQA as non-contextual TPA
# ([TPA] summary page, "Expressing MHA, MQA, and GQA as Non-Contextual TPA")
# --------------------------------------------------------------------------
def test_zero_query_gives_mean_of_values():
    ak, bk, av, bv, pos, ctx, q, qp = _small_problem()
    q[:] = 0.0
    out, lse = ref.decode(ak, bk, av, bv, pos, ctx, q, qp)
    for b in range(out.shape[0]):
        r_v = av.shape[2]
        values = [sum(ref.kron_block(av[b, s, r], bv[b, s, r]) for r in range(r_v)) / r_v
                  for s in range(ctx[b])]
        mean_v = np.mean(values, axis=0)
        np.testing.assert_allclose(out[b, 0], mean_v, atol=1e-12)
        np.testing.assert_allclose(lse[b, 0], np.log(ctx[b]), atol=1e-12)


def test_single_token_context_returns_its_value():
    ak, bk, av, bv, pos, ctx, q, qp = _small_problem(s=1)
    out, _ = ref.decode(ak, bk, av, bv, pos, ctx, q, qp)
    for b in range(out.shape[0]):
        v0 = sum(ref.kron_block(av[b, 0, r], bv[b, 0, r]) for r in range(av.shape[2])) / av.shape[2]
        np.testing.assert_allclose(out[b, 0], v0, atol=1e-12)


def test_empty_context():
    ak, bk, av, bv, pos, ctx, q, qp = _small_problem()
    ctx[:] = 0
    out, lse = ref.decode(ak, bk, av, bv, pos, ctx, q, qp, causal=False)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def _textbook_rope(x, pos, base=10000.0):
    """Ordinary RoPE over the last axis in RoFormer's complex form (torch)."""
    d = x.shape[-1]
    theta = base ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
    ang = torch.as_tensor(pos, dtype=torch.float64)[..., None] * theta
    xc = torch.view_as_complex(x.reshape(*x.shape[:-1], d // 2, 2).contiguous())
    return torch.view_as_real(xc * torch.polar(torch.ones_like(ang), ang)).reshape(x.shape)


def _sdpa_decode(k_heads, v_heads, q_heads, pos, q_pos):
    """Textbook attention of one query per head: torch SDPA in float64 on CPU.
    k_heads, v_heads: [S][h][d]; q_heads: [h][d]."""
    k = _textbook_rope(torch.as_tensor(k_heads).permute(1, 0, 2), torch.as_tensor(pos)[None, :])
    q = _textbook_rope(torch.as_tensor(q_heads)[:, None, :], torch.as_tensor([q_pos])[None, :])
    v = torch.as_tensor(v_heads).permute(1, 0, 2)
    out = torch.nn.functional.scaled_dot_product_attention(q, k.contiguous(), v.contiguous())
    return out[:, 0, :].numpy()


@pytest.mark.parametrize("kind", ["mha", "mqa", "gqa"])
def test_non_contextual_tpa_reduces_to_textbook_attention(kind):
    h, d_h, s = 4, 8, 11
    rng = np.random.default_rng(7)
    groups = {"mha": h, "mqa": 1, "gqa": 2}[kind]
    r = groups
    # head factors: h e_i (MHA), 1_h (MQA), G mask_j (GQA)
    a = np.zeros((r, h, 1))
    for j in range(r):
        members = [i for i in range(h) if i * groups // h == j]
        a[j, members, 0] = r
    b_k = rng.standard_normal((1, s, r, 1, d_h))
    b_v = rng.standard_normal((1, s, r, 1, d_h))
    a_k = np.broadcast_to(a, (1, s, r, h, 1)).copy()
    q = rng.standard_normal((1, 1, h, d_h))
    pos = np.arange(s)[None, :]
    out, _ = ref.decode(a_k, b_k, a_k.copy(), b_v, pos, np.array([s]), q, np.array([[s - 1]]))
    # textbook: head i uses its group's key/value vectors directly
    grp = [i * groups // h for i in range(h)]
    k_heads = np.stack([b_k[0, :, grp[i], 0, :] for i in range(h)], axis=1)
    v_heads = np.stack([b_v[0, :, grp[i], 0, :] for i in range(h)], axis=1)
    want = _sdpa_decode(k_heads, v_heads, q[0, 0], np.arange(s), s - 1)
    np.testing.assert_allclose(out[0, 0], want, atol=1e-12)


def test_causal_multi_query_row_equals_truncated_single_query():
    n_q = 4
    ak, bk, av, bv, pos, ctx, q, qp = _small_problem(n_q=n_q, s=10)
    out, lse = ref.decode(ak, bk, av, bv, pos, ctx, q, qp, causal=True)
    for n in range(n_q):
        trunc = ctx - n_q + n + 1
        o1, l1 = ref.decode(ak, bk, av, bv, pos, trunc, q[:, n:n + 1], qp[:, n:n + 1], causal=True)
        np.testing.assert_allclose(out[:, n], o1[:, 0], atol=1e-14)
        np.testing.assert_allclose(lse[:, n], l1[:, 0], atol=1e-14)


def test_causal_first_query_sees_only_its_own_token():
    # a chunk of n_q new tokens over an empty prior context: query 0 attends to slot 0 alone
    ak, bk, av, bv, pos, ctx, q, qp = _small_problem(n_q=5, s=5)
    out, lse = ref.decode(ak, bk, av, bv, pos, ctx, q, qp, causal=True)
    for b in range(out.shape[0]):
        v0 = sum(ref.kron_block(av[b, 0, r], bv[b, 0, r]) for r in range(av.shape[2])) / av.shape[2]
        np.testing.assert_allclose(out[b, 0], v0, atol=1e-12)


# ---------------------------------------------------------------------------
# Factored query ([KPA] Eqs. (5)-(6), Prop. 2.2)
# ---------------------------------------------------------------------------
def test_query_from_factors_matches_element_formula():
    rng = np.random.default_rng(21)
    r_q, p1, q1, p2, q2 = 3, 2, 3, 4, 2
    a_q = rng.normal(size=(2, 2, r_q, p1, q1))
    b_q = rng.normal(size=(2, 2, r_q, p2, q2))
    q = ref.query_from_factors(a_q, b_q)
    for b in range(2):
        for n in range(2):
            for i1 in range(p1):
                for i2 in range(p2):
                    for j1 in range(q1):
                        for j2 in range(q2):
                            want = sum(a_q[b, n, r, i1, j1] * b_q[b, n, r, i2, j2] for r in range(r_q)) / r_q
                            assert abs(q[b, n, i1 * p2 + i2, j1 * q2 + j2] - want) < 1e-14


def test_factored_query_decode_equals_attention_from_factored_scores():
    """Decode with the expanded query equals attention built from Eq. (6)
    scores of the factors alone, with RoPE applied to B^Q and B^K rows
    (Thm. 2.4) and V rebuilt from its factors (Eq. (4))."""
    rng = np.random.default_rng(22)
    r_q, r_k, r_v, p1, q1, p2, q2 = 2, 2, 3, 2, 2, 2, 4
    ctx, nq, base = 7, 2, 10000.0
    a_k = rng.normal(size=(1, ctx, r_k, p1, q1))
    b_k = rng.normal(size=(1, ctx, r_k, p2, q2))
    a_v = rng.normal(size=(1, ctx, r_v, p1, q1))
    b_v = rng.normal(size=(1, ctx, r_v, p2, q2))
    a_q = rng.normal(size=(1, nq, r_q, p1, q1))
    b_q = rng.normal(size=(1, nq, r_q, p2, q2))
    positions = np.arange(ctx)[None] * 3 + 5
    q_pos = np.array([[positions[0, ctx - 2], positions[0, ctx - 1]]])
    got, got_lse = ref.decode(a_k, b_k, a_v, b_v, positions, np.array([ctx]), ref.query_from_factors(a_q, b_q),
                              q_pos, causal=True, base=base)
    h, d_h = p1 * p2, q1 * q2
    for n in range(nq):
        vis = ctx - nq + n + 1
        bq_rot = ref.append_rotate(b_q[0, n], q_pos[0, n], base)
        for i1 in range(p1):
            for i2 in range(p2):
                z = np.array([ref.factored_score(a_q[0, n], bq_rot, a_k[0, s],
                                                 ref.append_rotate(b_k[0, s], positions[0, s], base), i1, i2)
                              for s in range(vis)]) / math.sqrt(d_h)
                w = np.exp(z - z.max())
                v = np.stack([ref.kron_reconstruct(a_v[0, s], b_v[0, s])[i1 * p2 + i2] for s in range(vis)])
                want = (w[:, None] * v).sum(0) / w.sum()
                assert np.allclose(got[0, n, i1 * p2 + i2], want, atol=1e-12, rtol=1e-12)
                assert abs(got_lse[0, n, i1 * p2 + i2] - (z.max() + math.log(w.sum()))) < 1e-12


# ---------------------------------------------------------------------------
# Factor projection from hidden states ([KPA] Eq. (5), the merged form after it)
# ---------------------------------------------------------------------------
PROJ = dict(r_k=2, r_v=3, p1=2, q1=3, p2=4, q2=2)


def _proj_sizes(r_k, r_v, p1, q1, p2, q2):
    return [("b_k", r_k, p2, q2), ("a_k", r_k, p1, q1), ("a_v", r_v, p1, q1), ("b_v", r_v, p2, q2)]


def test_projection_of_unit_vectors_reads_weight_columns_in_the_stated_order():
    """x = e_c returns column c of w: rows in the order W^{B^K}, W^{A^K},
    W^{A^V}, W^{B^V}, each block read row-major as [R][p][q]."""
    rng = np.random.default_rng(31)
    sizes = _proj_sizes(**PROJ)
    n_rows = sum(r * p * q for _, r, p, q in sizes)
    d_model = 5
    w = rng.normal(size=(n_rows, d_model))
    for c in range(d_model):
        x = np.zeros(d_model)
        x[c] = 1.0
        got = dict(zip(("a_k", "b_k", "a_v", "b_v"), ref.project_factors(x, w, **PROJ)))
        row = 0
        for name, r_n, p, q in sizes:
            for r in range(r_n):
                for i in range(p):
                    for j in range(q):
                        assert got[name][r, i, j] == w[row, c], (name, r, i, j)
                        row += 1


def test_projection_is_linear_and_keys_are_quadratic_in_the_hidden_state():
    """Each factor is a linear map of x (Eq. (5)), so K_t = (1/R) sum A_r(x) (x) B_r(x)
    scales with the square of x and the factors add."""
    rng = np.random.default_rng(32)
    sizes = _proj_sizes(**PROJ)
    n_rows = sum(r * p * q for _, r, p, q in sizes)
    w = rng.normal(size=(n_rows, 7))
    x1, x2 = rng.normal(size=7), rng.normal(size=7)
    f1, f2 = ref.project_factors(x1, w, **PROJ), ref.project_factors(x2, w, **PROJ)
    f12 = ref.project_factors(x1 + 2.5 * x2, w, **PROJ)
    for a, b, c in zip(f1, f2, f12):
        assert np.allclose(c, a + 2.5 * b, atol=1e-12)
    a_k, b_k, _, _ = f1
    a_k3, b_k3, _, _ = ref.project_factors(3.0 * x1, w, **PROJ)
    assert np.allclose(ref.kron_reconstruct(a_k3, b_k3), 9.0 * ref.kron_reconstruct(a_k, b_k), atol=1e-10)


def test_projected_cache_values_rotate_only_the_key_b_factor():
    rng = np.random.default_rng(34)
    sizes = _proj_sizes(**PROJ)
    n_rows = sum(r * p * q for _, r, p, q in sizes)
    w = rng.normal(size=(n_rows, 6))
    x = rng.normal(size=(3, 6))
    pos = np.array([0, 5, 1000])
    a_k, b_k, a_v, b_v = ref.project_factors(x, w, **PROJ)
    ca_k, cb_k, ca_v, cb_v = ref.projected_cache_values(x, w, pos, **PROJ)
    assert np.array_equal(ca_k, a_k) and np.array_equal(ca_v, a_v) and np.array_equal(cb_v, b_v)
    assert np.allclose(cb_k[0], b_k[0], atol=1e-15)  # position 0: no rotation
    for t in range(3):
        # each rotated row keeps its norm per rotation pair
        n0 = (b_k[t].reshape(-1, 2) ** 2).sum(-1)
        n1 = (cb_k[t].reshape(-1, 2) ** 2).sum(-1)
        assert np.allclose(n0, n1, atol=1e-12)


def test_projected_cache_values_equal_the_rotated_full_key():
    """The cached key factors of a projected token t, rebuilt into K, equal the
    full projected key rotated by R_KPA at that token's own position
    ([KPA] Thm. 2.4, Eqs. (7)-(8): (I (x) R(x)) (A (x) B) = A (x) (R(x) B)),
    at positions that are not the token indices and are not in order."""
    rng = np.random.default_rng(35)
    sizes = _proj_sizes(**PROJ)
    n_rows = sum(r * p * q for _, r, p, q in sizes)
    w = rng.normal(size=(n_rows, 9))
    x = rng.normal(size=(4, 9))
    pos = np.array([7, 123457, 3, 524287])
    a_k, b_k, _, _ = ref.project_factors(x, w, **PROJ)
    ca_k, cb_k, _, _ = ref.projected_cache_values(x, w, pos, **PROJ)
    q1, q2 = PROJ["q1"], PROJ["q2"]
    for t in range(4):
        # full-K route: rebuild K from the unrotated factors, then rotate every head row
        k_full = ref.kron_block(a_k[t, 0], b_k[t, 0]) + ref.kron_block(a_k[t, 1], b_k[t, 1])
        k_full /= 2.0
        rot = np.kron(np.eye(q1), ref.rope_block(float(pos[t]), q2))
        want = k_full @ rot.T
        got = sum(ref.kron_block(ca_k[t, r], cb_k[t, r]) for r in range(2)) / 2.0
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
