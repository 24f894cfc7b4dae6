"""Host checks of the parity helpers (no GPU): the score scale that bounds
the lse tolerance is an upper bound of the absolute score sums, computed by
brute force from the float64 oracle's rotated keys and queries."""
import numpy as np

from oracle import kpa_ref as ref
from tests.kpa_testutil import score_scale
from workloads import CONFIGS, make_inputs


def test_score_scale_bounds_the_absolute_score_sum():
    for name, ragged in (("kpa_32k", True), ("multiq_16", False), ("tpa_degenerate", True)):
        cfg = CONFIGS[name]
        inp = make_inputs(cfg, seed=3, batch=2, ctx=9, n_q=min(cfg.n_q, 3), ragged=ragged, q_scale=2.0)
        sc = score_scale(inp.a_k, inp.b_k, inp.ctx_len, inp.q)
        a_k = inp.a_k.double().numpy()
        b_k = inp.b_k.double().numpy()
        q = inp.q.double().numpy()
        p2, q1, q2 = cfg.p2, cfg.q1, cfg.q2
        for b in range(inp.batch):
            for n in range(q.shape[1]):
                qrot = q[b, n] @ ref.rope_kpa(int(inp.q_pos[b, n]), q1, q2).T
                for i in range(cfg.h):
                    i1, i2 = divmod(i, p2)
                    best = 0.0
                    for s in range(int(inp.ctx_len[b])):
                        brot = ref.append_rotate(b_k[b, s], int(inp.positions[b, s]))
                        kabs = sum(np.kron(np.abs(a_k[b, s, r, i1])[None], np.abs(brot[r, i2])[None])[0]
                                   for r in range(cfg.r_k)) / cfg.r_k
                        kk = ref.kron_reconstruct(a_k[b, s], b_k[b, s])[i] @ ref.rope_kpa(
                            int(inp.positions[b, s]), q1, q2).T
                        z = abs(qrot[i] @ kk) / np.sqrt(cfg.d_h)
                        tot = np.abs(qrot[i]) @ kabs / np.sqrt(cfg.d_h)
                        assert z <= tot + 1e-12
                        best = max(best, tot)
                    assert best <= sc[b, n, i] * (1 + 1e-12), (name, b, n, i)
