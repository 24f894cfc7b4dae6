"""Literal float64 definitions of KPA factor-cache decode (NumPy).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Every function below
writes one definition out as plainly as possible; nothing is blocked, fused or
reordered beyond what the cited definition states.

Index conventions (the block order of the Kronecker product, [KPA] Def. 2.1):
  head    i = i1 * p2 + i2      (i1 < p1 = h1, i2 < p2 = h2)
  feature j = j1 * q2 + j2      (j1 < q1 = d1, j2 < q2 = d2)
A factor A_r is p1 x q1 (head-partition factor), B_r is p2 x q2 (within-head
factor); K_t = (1/R_K) sum_r A_r (x) B_r is h x d_h ([KPA] §2.2, Eqs. (3)-(4)).

Readings of points the pages leave open (each is listed in the design doc):
  * the query is dense (h x d_h) and unrotated, with its own position -- the
    "KV-only" form ([TPA] Appendix G, TPA-KVonly); no 1/R_Q is involved;
  * rotary pairs are consecutive features (2m, 2m+1) inside each d2 block,
    theta_m = base^(-2m/d2), m = 0..d2/2-1 ([KPA] Def. 2.3; [TPA] summary
    page, "RoPE Compatibility and Acceleration"), rotation
    (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos);
  * the score is scaled by 1/sqrt(d_h), d_h = d1*d2 ([KPA] §2.3);
  * V is never rotated ([KPA] Fig. 1 caption);
  * an empty context gives output 0 and log-sum-exp -inf;
  * the factor projection ([KPA] Eq. (5)) takes one stacked weight matrix,
    rows W^{B^K}, W^{A^K}, W^{A^V}, W^{B^V} (the pages merge the ranks of each
    factor type; stacking the four types is this build's choice), and each
    product block is reshaped row-major to [R][p][q].
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "kron_block",
    "kron_reconstruct",
    "rope_theta",
    "rope_block",
    "rope_kpa",
    "append_rotate",
    "cached_numbers_per_token",
    "mha_numbers_per_token",
    "compression_factor",
    "attention_one_query",
    "decode",
    "factored_score",
    "project_factors",
    "projected_cache_values",
]


# ---------------------------------------------------------------------------
# Kronecker product and the factorised K/V ([KPA] Def. 2.1, §2.2)
# ---------------------------------------------------------------------------
def kron_block(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """A (x) B written from the block definition: block (i1, j1) is a[i1, j1] * B.

    [KPA] Def. 2.1.  Used by the tests to pin ``np.kron`` (the library routine
    that ``kron_reconstruct`` calls) to the definition on the pages.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    m1, n1 = a.shape
    m2, n2 = b.shape
    out = np.zeros((m1 * m2, n1 * n2))
    for i1 in range(m1):
        for j1 in range(n1):
            out[i1 * m2:(i1 + 1) * m2, j1 * n2:(j1 + 1) * n2] = a[i1, j1] * b
    return out


def kron_reconstruct(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """(1/R) sum_r A_r (x) B_r for one token.

    a: [R][p1][q1], b: [R][p2][q2]  ->  [p1*p2][q1*q2]   ([KPA] Eqs. (3)-(4)).
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    r = a.shape[0]
    assert b.shape[0] == r
    acc = np.zeros((a.shape[1] * b.shape[1], a.shape[2] * b.shape[2]))
    for k in range(r):
        acc += np.kron(a[k], b[k])
    return acc / r


# ---------------------------------------------------------------------------
# Kronecker-separable RoPE ([KPA] Def. 2.3, Thm. 2.4)
# ---------------------------------------------------------------------------
def rope_theta(q2: int, base: float = 10000.0) -> np.ndarray:
    """theta_m = base^(-2m/d2), m = 0 .. d2/2-1 ([KPA] Def. 2.3)."""
    if q2 % 2:
        raise ValueError("d2 must be even for RoPE")
    m = np.arange(q2 // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * m / q2)


def rope_block(pos: float, q2: int, base: float = 10000.0) -> np.ndarray:
    """R^(2)_theta(pos): the d2 x d2 RoPE matrix, 2x2 rotations on consecutive pairs."""
    th = rope_theta(q2, base)
    out = np.zeros((q2, q2))
    for m in range(q2 // 2):
        ang = float(pos) * th[m]
        c, s = np.cos(ang), np.sin(ang)
        out[2 * m, 2 * m] = c
        out[2 * m, 2 * m + 1] = -s
        out[2 * m + 1, 2 * m] = s
        out[2 * m + 1, 2 * m + 1] = c
    return out


def rope_kpa(pos: float, q1: int, q2: int, base: float = 10000.0) -> np.ndarray:
    """R_KPA(pos) = I_{d1} (x) R^(2)_theta(pos), a d_h x d_h matrix ([KPA] Def. 2.3)."""
    return np.kron(np.eye(q1), rope_block(pos, q2, base))


def append_rotate(b_k: np.ndarray, pos: float, base: float = 10000.0) -> np.ndarray:
    """Pre-rotated key factor: every row (B_r)_{i2} becomes R^(2)(pos) (B_r)_{i2}.

    b_k: [R][p2][q2].  Only B^K is rotated; A^K, A^V, B^V are cached as they
    are ([KPA] Thm. 2.4, Eq. (8), and consequence (i) after it; §2.5).
    """
    b_k = np.asarray(b_k, dtype=np.float64)
    rot = rope_block(pos, b_k.shape[-1], base)
    return np.einsum("ab,rib->ria", rot, b_k)


# ---------------------------------------------------------------------------
# Cache size ([KPA] §2.5 Eq. (10), App. B Eq. (11); [TPA] cache table)
# ---------------------------------------------------------------------------
def cached_numbers_per_token(a_k, b_k, a_v, b_v) -> int:
    """Numbers cached for one token: the sizes of its four factor sets.

    Arguments are one token's factors ([R][p][q] each).  [KPA] §2.5: the cache
    holds {A^K_r, B^K_r} for r <= R_K and {A^V_r, B^V_r} for r <= R_V.
    """
    return int(np.size(a_k) + np.size(b_k) + np.size(a_v) + np.size(b_v))


def mha_numbers_per_token(h: int, d_h: int) -> int:
    """MHA caches K_t and V_t, 2 h d_h numbers ([KPA] §2.5)."""
    return 2 * h * d_h


def compression_factor(p1: int, p2: int, q1: int, q2: int, r_k: int, r_v: int) -> float:
    """C_KPA = 2 h1 h2 d1 d2 / ((R_K + R_V)(h1 d1 + h2 d2))  ([KPA] Eq. (10))."""
    return 2.0 * p1 * p2 * q1 * q2 / ((r_k + r_v) * (p1 * q1 + p2 * q2))


# ---------------------------------------------------------------------------
# Attention ([KPA] §2.3; textbook softmax attention)
# ---------------------------------------------------------------------------
def attention_one_query(q_rot: np.ndarray, k_rot: np.ndarray, v: np.ndarray):
    """Textbook softmax attention of one (already rotated) query over n keys.

    q_rot: [h][d_h]; k_rot, v: [n][h][d_h].  Per head i:
      z_s = q_i . k_{s,i} / sqrt(d_h),  p = softmax(z),  o_i = sum_s p_s v_{s,i},
      lse_i = log sum_s exp(z_s).
    n = 0 gives o = 0 and lse = -inf.
    """
    h, d_h = q_rot.shape
    n = k_rot.shape[0]
    if n == 0:
        return np.zeros((h, d_h)), np.full(h, -np.inf)
    z = np.einsum("ij,sij->is", q_rot, k_rot) / np.sqrt(d_h)  # [h][n]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    o = np.einsum("is,sij->ij", p, v)
    lse = (m + np.log(l))[:, 0]
    return o, lse


def decode(a_k, b_k, a_v, b_v, positions, ctx_len, q, q_pos, *, causal=True,
           base=10000.0):
    """KPA decode from the UNROTATED factors, float64.

    a_k: [B][S][R_K][p1][q1]   b_k: [B][S][R_K][p2][q2]
    a_v: [B][S][R_V][p1][q1]   b_v: [B][S][R_V][p2][q2]
    positions: [B][S] int      ctx_len: [B] int
    q: [B][n_q][h][d_h]        q_pos: [B][n_q] int
    Returns out [B][n_q][h][d_h], lse [B][n_q][h].

    Query n of sequence b sees slots s < ctx_len[b] - n_q + n + 1 when
    ``causal`` (the n_q newest slots are the queries' own tokens), otherwise
    every slot s < ctx_len[b].  For each visible slot, K_s and V_s are rebuilt
    with the Kronecker product (Eqs. (3)-(4)); every head row of K_s and of the
    query is rotated with R_KPA at its own position (Def. 2.3, Eqs. (7)-(9));
    then textbook softmax attention.
    """
    a_k = np.asarray(a_k, np.float64)
    b_k = np.asarray(b_k, np.float64)
    a_v = np.asarray(a_v, np.float64)
    b_v = np.asarray(b_v, np.float64)
    q = np.asarray(q, np.float64)
    nb, _, _, p1, q1 = a_k.shape
    p2, q2 = b_k.shape[3], b_k.shape[4]
    n_q = q.shape[1]
    h, d_h = p1 * p2, q1 * q2
    out = np.zeros((nb, n_q, h, d_h))
    lse = np.zeros((nb, n_q, h))
    for b in range(nb):
        ctx = int(ctx_len[b])
        k_rot = np.zeros((ctx, h, d_h))
        v = np.zeros((ctx, h, d_h))
        for s in range(ctx):
            k_s = kron_reconstruct(a_k[b, s], b_k[b, s])
            rot = rope_kpa(positions[b][s], q1, q2, base)
            k_rot[s] = k_s @ rot.T          # row i  ->  R_KPA k_i
            v[s] = kron_reconstruct(a_v[b, s], b_v[b, s])
        for n in range(n_q):
            visible = ctx - n_q + n + 1 if causal else ctx
            visible = max(0, min(visible, ctx))
            rot_q = rope_kpa(q_pos[b][n], q1, q2, base)
            q_rot = q[b, n] @ rot_q.T
            out[b, n], lse[b, n] = attention_one_query(q_rot, k_rot[:visible], v[:visible])
    return out, lse


def query_from_factors(a_q, b_q) -> np.ndarray:
    """Dense queries of factored ones: for every (sequence, query) row,
    (1/R_Q) sum_r A^Q_r (x) B^Q_r ([KPA] Eq. (5) with Def. 2.1, the keys' form).

    a_q: [B][n_q][R_Q][p1][q1], b_q: [B][n_q][R_Q][p2][q2] -> [B][n_q][h][d_h].
    """
    a_q = np.asarray(a_q, np.float64)
    b_q = np.asarray(b_q, np.float64)
    nb, nq = a_q.shape[0], a_q.shape[1]
    out = np.zeros((nb, nq, a_q.shape[3] * b_q.shape[3], a_q.shape[4] * b_q.shape[4]))
    for b in range(nb):
        for n in range(nq):
            out[b, n] = kron_reconstruct(a_q[b, n], b_q[b, n])
    return out


def factored_score(a_q, b_q, a_k, b_k, i1: int, i2: int) -> float:
    """Prop. 2.2 / Eq. (6): the score of head (i1, i2) from the factors alone.

    a_q: [R_Q][p1][q1], b_q: [R_Q][p2][q2], a_k: [R_K][p1][q1], b_k: [R_K][p2][q2]
    (one query token t and one key token s; unscaled, i.e. before 1/sqrt(d_h)).
    score = 1/(R_Q R_K) sum_{r, r'} [(A^Q_r)_{i1} . (A^K_r')_{i1}] [(B^Q_r)_{i2} . (B^K_r')_{i2}]
    """
    a_q = np.asarray(a_q, np.float64)
    b_q = np.asarray(b_q, np.float64)
    a_k = np.asarray(a_k, np.float64)
    b_k = np.asarray(b_k, np.float64)
    total = 0.0
    for r in range(a_q.shape[0]):
        for rp in range(a_k.shape[0]):
            head_level = float(np.dot(a_q[r, i1], a_k[rp, i1]))
            feature_level = float(np.dot(b_q[r, i2], b_k[rp, i2]))
            total += head_level * feature_level
    return total / (a_q.shape[0] * a_k.shape[0])


# ---------------------------------------------------------------------------
# Factor projection from hidden states ([KPA] Eq. (5) and the merged form
# after it)
# ---------------------------------------------------------------------------
def project_factors(x, w, r_k: int, r_v: int, p1: int, q1: int, p2: int, q2: int):
    """The four factor sets of tokens x from one merged weight matrix.

    [KPA] Eq. (5): A^K_r(x) = W^{A^K}_r x, B^K_r(x) = W^{B^K}_r x, W^{A^K}_r of
    shape (h1 d1) x d_model; the ranks are merged into one matrix per factor
    type, (R_K h1 d1) x d_model, whose product is reshaped to R_K x h1 x d1
    (read: row-major, row r h1 d1 + i1 d1 + j1 -> [r][i1][j1]).  Here the four
    merged matrices are stacked into one w of F rows in the order
    W^{B^K}, W^{A^K}, W^{A^V}, W^{B^V}.

    x: [..., d_model]; w: [F][d_model].  Returns (a_k, b_k, a_v, b_v), float64,
    shapes [..., R][p][q], unrotated.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    sizes = [r_k * p2 * q2, r_k * p1 * q1, r_v * p1 * q1, r_v * p2 * q2]
    if w.shape[0] != sum(sizes) or w.shape[1] != x.shape[-1]:
        raise ValueError("w must be F x d_model with F = (R_K + R_V)(p1 q1 + p2 q2)")
    y = x @ w.T  # [..., F]
    lead = x.shape[:-1]
    parts = []
    o = 0
    for n in sizes:
        parts.append(y[..., o:o + n])
        o += n
    b_k = parts[0].reshape(*lead, r_k, p2, q2)
    a_k = parts[1].reshape(*lead, r_k, p1, q1)
    a_v = parts[2].reshape(*lead, r_v, p1, q1)
    b_v = parts[3].reshape(*lead, r_v, p2, q2)
    return a_k, b_k, a_v, b_v


def projected_cache_values(x, w, positions, r_k: int, r_v: int, p1: int, q1: int, p2: int, q2: int,
                           base: float = 10000.0):
    """What the cache holds for tokens x after projection and append, before
    the final rounding to the cache type: A^K, A^V, B^V as projected, and
    B~^K = R^(2)(pos) B^K ([KPA] Thm. 2.4, Eq. (8)), all float64.

    x: [T][d_model], positions: [T].  Returns (a_k, b_k_rotated, a_v, b_v).
    """
    a_k, b_k, a_v, b_v = project_factors(x, w, r_k, r_v, p1, q1, p2, q2)
    b_rot = np.stack([append_rotate(b_k[t], float(positions[t]), base) for t in range(b_k.shape[0])])
    return a_k, b_rot, a_v, b_v
