// Matrix-core decode: the exact-shape instantiations and the choice of
// kernel for a shape (exact first, else a generic family).  The kernel
// itself is in decode_mfma.hpp.
#include "decode_mfma.hpp"

namespace kpa {
namespace mfma {

// Shapes with an exact instantiation.  Cfg arguments: PG, QG, PF, QF (F = the
// factor whose feature dimension is contracted on the matrix cores: B for
// most, A for the multi-query shape and some head splits), R_K, R_V, F is B,
// queries per wave, query subgroups, waves/SIMD[, waves per F head[, percent
// of the resident-workgroup slots the planner fills[, strided chunks]]].
const MfmaKernel* exact_kernels(int* count) {
    static const MfmaKernel tab[] = {
        KPA_MFMA_ENTRY(4, 4, 8, 16, 2, 2, false, 4, 8, 4, 16, 2, 2, true, 1, 1, 3),
        KPA_MFMA_ENTRY(4, 4, 8, 16, 1, 1, false, 4, 8, 4, 16, 1, 1, true, 1, 1, 2),
        // long_512k's shape: 48 KB tiles, two workgroups per CU.  One
        // sequence of 2^19 tokens runs fastest with ~90% of the slots filled
        // (456 chunks against 512: 136.1 -> 131.3 us per call) and strided
        // chunks (-> 128.9 us; 136.9 -> 128.5-130.3 us for the two together,
        // A/B on one box)
        KPA_MFMA_ENTRY(8, 4, 8, 16, 2, 4, false, 8, 8, 4, 16, 2, 4, true, 1, 1, 2, 1, 90, true),
        // several queries per sequence on kpa_32k's and long_512k's shapes
        // (the generic family they fell to runs one 2-query workgroup per CU;
        // 8 x 16400 tokens, A/B): kpa_32k's with 4 queries per wave, 16
        // queries 985 -> 110-119 us, 4 queries 138 -> 41 us, 2 queries 78 ->
        // 38 us; long_512k's with 2 queries per wave and 2 query subgroups
        // (4 sequences for 4 queries), 16 queries 2250 -> 274-283 us, 4
        // queries 170 -> 52 us
        KPA_MFMA_ENTRY(4, 4, 8, 16, 2, 2, true, 4, 8, 4, 16, 2, 2, true, 4, 1, 2),
        KPA_MFMA_ENTRY(8, 4, 8, 16, 2, 4, true, 8, 8, 4, 16, 2, 4, true, 2, 2, 1),
        KPA_MFMA_ENTRY(4, 8, 16, 8, 4, 4, false, 8, 8, 4, 16, 4, 4, false, 1, 1, 1),
        KPA_MFMA_ENTRY(4, 8, 16, 8, 4, 4, true, 8, 8, 4, 16, 4, 4, false, 2, 2, 2),
        // TPA split (A: h x 1, B: 1 x d_h): G = A with feature dimension 1, F = B
        KPA_MFMA_ENTRY(12, 1, 1, 64, 2, 2, false, 12, 1, 1, 64, 2, 2, true, 1, 1, 1),
        // FlashTPA's benchmark shapes: d_h = 64, R_K = R_V = 1, h = 16 / 32 / 48
        // (strided chunks for h = 32 and 48: 0.9-2.1% faster at batch 1, 4
        // and 16, A/B; h = 16 within 0.5%)
        KPA_MFMA_ENTRY(16, 1, 1, 64, 1, 1, false, 16, 1, 1, 64, 1, 1, true, 1, 1, 2),
        KPA_MFMA_ENTRY(32, 1, 1, 64, 1, 1, false, 32, 1, 1, 64, 1, 1, true, 1, 1, 2, 1, 100, true),
        KPA_MFMA_ENTRY(48, 1, 1, 64, 1, 1, false, 48, 1, 1, 64, 1, 1, true, 1, 1, 1, 1, 100, true),
        // The KPA page's head splits (d1 = d2 = 8, R_K = R_V = 2).  F is the
        // factor with fewer heads (fewer waves, more rows per wave), except for
        // 4 x 5, where four waves per workgroup (F = A) spread evenly over a
        // CU's four SIMDs (five waves: 46% -> 62% of 8 TB/s measured), with
        // registers for three waves per SIMD (61.6 -> 59.6 us).  10 x 2, 2 x 10
        // and 6 x 2 split each F head's G heads over two waves, so a CU runs 8
        // (10 x 2: LDS held it to three 2-wave workgroups) and 12 waves instead
        // of 6 and 8 (75.2 -> 69.4, 75.9 -> 72.2, 48.1 -> 47.0 us at 16 x 32768
        // tokens, A/B).
        KPA_MFMA_ENTRY(8, 2, 8, 8, 2, 2, false, 8, 8, 2, 8, 2, 2, true, 1, 1, 2),
        KPA_MFMA_ENTRY(4, 4, 8, 8, 2, 2, false, 4, 8, 4, 8, 2, 2, true, 1, 1, 3),
        KPA_MFMA_ENTRY(2, 8, 8, 8, 2, 2, false, 8, 8, 2, 8, 2, 2, false, 1, 1, 2),
        KPA_MFMA_ENTRY(10, 2, 8, 8, 2, 2, false, 10, 8, 2, 8, 2, 2, true, 1, 1, 2, 2),
        KPA_MFMA_ENTRY(4, 5, 8, 8, 2, 2, false, 5, 8, 4, 8, 2, 2, false, 1, 1, 3),
        KPA_MFMA_ENTRY(2, 10, 8, 8, 2, 2, false, 10, 8, 2, 8, 2, 2, false, 1, 1, 2, 2),
        KPA_MFMA_ENTRY(5, 5, 8, 8, 2, 2, false, 5, 8, 5, 8, 2, 2, true, 1, 1, 3),
        KPA_MFMA_ENTRY(6, 2, 8, 8, 2, 2, false, 6, 8, 2, 8, 2, 2, true, 1, 1, 3, 2),
        KPA_MFMA_ENTRY(4, 3, 8, 8, 2, 2, false, 4, 8, 3, 8, 2, 2, true, 1, 1, 3),
        KPA_MFMA_ENTRY(3, 4, 8, 8, 2, 2, false, 4, 8, 3, 8, 2, 2, false, 1, 1, 3),
        KPA_MFMA_ENTRY(2, 6, 8, 8, 2, 2, false, 6, 8, 2, 8, 2, 2, false, 1, 1, 2),
    };
    *count = (int)(sizeof(tab) / sizeof(tab[0]));
    return tab;
}

}  // namespace mfma

namespace {

using mfma::MfmaKernel;

struct Choice {
    const MfmaKernel* k = nullptr;
    int f_is_b = 1;
};

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// The generic family that runs (d, n_q) with F = B (fb = 1) or F = A, and
// the cost of that choice (lower is better), or nullptr.  Rules, checked
// here so the kernel need not: F feature dimension 8/16/32/64; G feature
// dimension a power of two up to 32; rows M = PG*QG within the family's row
// cap and a multiple of 4 (or R_K = 1); ranks within its caps; NQW*PG
// softmax rows within a wave's 64 lanes; waves within the family's cap; LDS
// within a CU's.
const MfmaKernel* generic_for(const kpa_dims& d, int n_q, int fb, int* cost) {
    const int QF = fb ? d.q2 : d.q1, QG = fb ? d.q1 : d.q2;
    const int PG = fb ? d.p1 : d.p2, PF = fb ? d.p2 : d.p1;
    if (!(QF == 8 || QF == 16 || QF == 32 || QF == 64)) return nullptr;
    if (!pow2(QG) || QG > 32) return nullptr;
    const int M = PG * QG;
    // a lane reads four consecutive key-set G elements r*M + R0 (R0 a
    // multiple of 4) as 8 bytes: aligned for every rank when M is a multiple
    // of 4, for the only rank otherwise
    if (M % 4 != 0 && d.r_k > 1) return nullptr;
    const bool multi = n_q > 1;
    const MfmaKernel* best = nullptr;
    auto consider = [&](const MfmaKernel* tab, int count) {
        for (int i = 0; i < count; ++i) {
            const MfmaKernel& k = tab[i];
            if (!k.generic || k.multi != multi || k.qf != QF || k.rkc < d.r_k || k.rvc < d.r_v || k.m_max < M) continue;
            if (k.queries_per_wave * PG > 64 || PF * k.query_subgroups > k.waves_max) continue;
            if (k.lds_bytes(d, fb) > mfma::kLdsBytes) continue;
            // the tightest fit: fewest rows, then smallest rank caps
            if (!best || k.m_max < best->m_max || (k.m_max == best->m_max && k.rkc + k.rvc < best->rkc + best->rvc))
                best = &k;
        }
    };
    int na = 0, nb = 0;
    const MfmaKernel* ta = mfma::generic_kernels_a(&na);
    const MfmaKernel* tb = mfma::generic_kernels_b(&nb);
    consider(ta, na);
    consider(tb, nb);
    if (best) {
        // waves spread evenly over a CU's four SIMDs first, then fewer padded
        // rows, then fewer waves
        const bool even = PF == 1 || PF == 2 || PF == 4 || PF == 8;
        *cost = (even ? 0 : 1 << 20) + (best->m_max - M) * 64 + PF;
    }
    return best;
}

Choice find_kernel(const kpa_dims& d, int n_q) {
    Choice c;
    if (d.dtype != KPA_BF16) return c;
    const bool multi = n_q > 1;
    int ne = 0;
    const MfmaKernel* te = mfma::exact_kernels(&ne);
    for (int i = 0; i < ne; ++i) {
        const MfmaKernel& k = te[i];
        if (k.multi == multi && k.p1 == d.p1 && k.p2 == d.p2 && k.q1 == d.q1 && k.q2 == d.q2 && k.r_k == d.r_k &&
            k.r_v == d.r_v) {
            c.k = &k;
            return c;
        }
    }
    int cost_b = 0, cost_a = 0;
    const MfmaKernel* kb = generic_for(d, n_q, 1, &cost_b);
    const MfmaKernel* ka = generic_for(d, n_q, 0, &cost_a);
    if (kb && (!ka || cost_b <= cost_a)) {
        c.k = kb;
        c.f_is_b = 1;
    } else if (ka) {
        c.k = ka;
        c.f_is_b = 0;
    }
    return c;
}

}  // namespace

bool decode_mfma_supported(const kpa_dims& d, int n_q) { return find_kernel(d, n_q).k != nullptr; }

int decode_mfma_blocks_per_cu(const kpa_dims& d, int n_q) {
    const Choice c = find_kernel(d, n_q);
    return c.k ? c.k->blocks_per_cu(d, c.f_is_b) : 1;
}

int decode_mfma_fill_pct(const kpa_dims& d, int n_q) {
    const Choice c = find_kernel(d, n_q);
    return c.k ? c.k->fill_pct : 100;
}

// Workgroups one KV chunk needs (one per group of queries).
int decode_mfma_query_groups(const kpa_dims& d, int n_q) {
    const Choice c = find_kernel(d, n_q);
    const int qpg = c.k ? c.k->queries_per_wave * c.k->query_subgroups : 1;
    return (n_q + qpg - 1) / qpg;
}

hipError_t launch_decode_mfma(const DecodeParams& P, hipStream_t s, const KernelEvents& ev) {
    const Choice c = find_kernel(P.d, P.n_q);
    if (!c.k) return hipErrorInvalidValue;
    DecodeParams Q = P;
    Q.f_is_b = c.f_is_b;
    return c.k->launch(Q, s, ev);
}

}  // namespace kpa
