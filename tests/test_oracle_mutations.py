"""Planted mistakes in the oracle (on the CPU) are caught by its pins.

Each case swaps one oracle function for a plausible wrong variant -- a
transposed Kronecker order, a dropped 1/R, a flipped rotation sign, the
other Kronecker order of the rotary operator, the wrong softmax scale, a
causal off-by-one, a factored query expanded with its factors' roles
transposed, a projected key rotated by its token index instead of its
position -- and checks that at least one pin fails.
"""
import numpy as np
import pytest

from oracle import kpa_ref as ref
import tests.test_oracle_pins as pins


def _kron_swapped(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return sum(np.kron(b[k], a[k]).reshape(a.shape[1] * b.shape[1], a.shape[2] * b.shape[2])
               for k in range(a.shape[0])) / a.shape[0]


def _kron_no_norm(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return sum(np.kron(a[k], b[k]) for k in range(a.shape[0]))


_orig_rope_block = ref.rope_block


def _rope_flipped(pos, q2, base=10000.0):
    return _orig_rope_block(-pos, q2, base)


def _rope_wrong_order(pos, q1, q2, base=10000.0):
    return np.kron(_orig_rope_block(pos, q2, base), np.eye(q1))


_orig_attention = ref.attention_one_query


def _attention_wrong_scale(q_rot, k_rot, v):
    # 1/sqrt(d2)-like scale: use a quarter of d_h
    return _orig_attention(q_rot * np.sqrt(4.0), k_rot, v)


_orig_decode = ref.decode


def _decode_causal_off_by_one(a_k, b_k, a_v, b_v, positions, ctx_len, q, q_pos, *, causal=True, base=10000.0):
    if not causal:
        return _orig_decode(a_k, b_k, a_v, b_v, positions, ctx_len, q, q_pos, causal=False, base=base)
    # every query misses its own token
    n_q = np.asarray(q).shape[1]
    outs, lses = [], []
    for n in range(n_q):
        vis = np.asarray(ctx_len) - n_q + n
        o, l = _orig_decode(a_k, b_k, a_v, b_v, positions, vis, np.asarray(q)[:, n:n + 1],
                            np.asarray(q_pos)[:, n:n + 1], causal=False, base=base)
        outs.append(o[:, 0])
        lses.append(l[:, 0])
    return np.stack(outs, 1), np.stack(lses, 1)


_orig_query_from_factors = ref.query_from_factors


def _query_factors_swapped(a_q, b_q):
    # the roles of the head and feature factors exchanged in the expansion
    a_q, b_q = np.asarray(a_q, np.float64), np.asarray(b_q, np.float64)
    nb, nq, r = a_q.shape[:3]
    out = np.zeros((nb, nq, a_q.shape[3] * b_q.shape[3], a_q.shape[4] * b_q.shape[4]))
    for b in range(nb):
        for n in range(nq):
            out[b, n] = sum(np.kron(b_q[b, n, k], a_q[b, n, k]) for k in range(r)) / r
    return out


_orig_project_factors = ref.project_factors


def _project_sets_swapped(x, w, r_k, r_v, p1, q1, p2, q2):
    # the W^{A^K} and W^{B^K} blocks read in the other order
    n_b, n_a = r_k * p2 * q2, r_k * p1 * q1
    w = np.asarray(w, np.float64)
    w2 = np.concatenate([w[n_b:n_b + n_a], w[:n_b], w[n_b + n_a:]]) if n_a == n_b else w[::-1]
    return _orig_project_factors(x, w2, r_k, r_v, p1, q1, p2, q2)


_orig_projected_cache_values = ref.projected_cache_values


def _projected_rotated_by_index(x, w, positions, r_k, r_v, p1, q1, p2, q2, base=10000.0):
    # token t rotated by its index t instead of its position
    idx = np.arange(np.asarray(positions).shape[0])
    return _orig_projected_cache_values(x, w, idx, r_k, r_v, p1, q1, p2, q2, base)


MUTATIONS = [
    ("kron_reconstruct", _kron_swapped, [pins.test_kron_entry_index_convention]),
    ("kron_reconstruct", _kron_no_norm, [pins.test_kron_sum_is_normalised_by_rank,
                                         lambda: pins.test_non_contextual_tpa_reduces_to_textbook_attention("mha")]),
    ("rope_block", _rope_flipped, [pins.test_rope_convention_sign_pairs_and_frequencies,
                                   pins.test_rope_matches_complex_multiplication_form]),
    ("rope_kpa", _rope_wrong_order, [pins.test_rope_kpa_rotates_only_the_b_factor]),
    ("attention_one_query", _attention_wrong_scale,
     [lambda: pins.test_non_contextual_tpa_reduces_to_textbook_attention("gqa")]),
    ("decode", _decode_causal_off_by_one, [pins.test_causal_first_query_sees_only_its_own_token]),
    ("query_from_factors", _query_factors_swapped, [pins.test_query_from_factors_matches_element_formula,
                                                    pins.test_factored_query_decode_equals_attention_from_factored_scores]),
    ("project_factors", _project_sets_swapped,
     [pins.test_projection_of_unit_vectors_reads_weight_columns_in_the_stated_order]),
    ("projected_cache_values", _projected_rotated_by_index,
     [pins.test_projected_cache_values_equal_the_rotated_full_key]),
]


@pytest.mark.parametrize("name,bad,checks", MUTATIONS, ids=[m[1].__name__ for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, bad, checks):
    monkeypatch.setattr(ref, name, bad)
    for check in checks:
        with pytest.raises(AssertionError):
            check()
