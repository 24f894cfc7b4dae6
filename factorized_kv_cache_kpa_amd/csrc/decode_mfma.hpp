// Split-KV decode on the bf16 matrix cores (gfx950 MFMA), one query or a
// causal chunk of queries per sequence: the kernel template, shared by the
// translation units that instantiate it (decode_mfma*.hip).
//
// Math ([KPA] = "Kronecker Product Attention: Memory-Efficient KV Compression
// via Structured Factorization"; [TPA] = "Tensor Product Attention Is All You
// Need", summary page):
//   K_s = (1/R_K) sum_r A^K_r (x) B~^K_r, V_s likewise      ([KPA] Eqs. (3)-(4))
//   z_{i,s} = q'_i . k_{s,i} / sqrt(d_h), q' = R_KPA(q_pos) q  ([KPA] §2.3, Def. 2.3)
// Written with the two factors of a head: call F the factor whose feature
// dimension is contracted on the matrix cores (8, 16, 32 or 64 wide) and G
// the other one.  Head i = (iG, iF), feature j = (jG, jF) in the block order
// of the Kronecker product ([KPA] Def. 2.1).  Then, per query n, rank r and
// cached slot s,
//   W_r[(n,iG,jG), s] = sum_jF q'[n,iG,iF,jG,jF] F_r[s,iF,jF]   (MFMA 32x32x16:
//        M = (n,iG,jG), N = 32 slots, K = jF -- the queries are the
//        stationary operand, as a grouped-query decode shares K across heads)
//   z[n,iG,iF,s] = sum_r sum_jG G_r[s,iG,jG] W_r[(n,iG,jG),s]   (VALU, in lane)
// which is [KPA] Prop. 2.2 / Eq. (6) with a dense query: contract with one
// factor, then the other; K is never rebuilt.  The value side, per iF,
//   O[(n,iG,jG), jF] += sum_{r,s} (p[n,iG,iF,s] G^V_r[s,iG,jG]) F^V_r[s,iF,jF]
// is a GEMM over slots (MFMA 16x16x32: M = (iG,jG), N = jF, K = 32 slots),
// with the softmax weight folded into the G factor: by 4x4x4 matrix
// instructions (A = diag of four weights, B = four slots of G^V) where four
// consecutive rows (iG, jG) share a head, else on the VALU.  The online
// softmax (running max and sum per (query, head), rescaling O when the max
// grows) is the blocked online log-sum-exp of FlashTPA decoding ([TPA]).
//
// Work split: a workgroup owns one KV chunk of one sequence for a group of
// queries; its waves are (iF, part of the G heads, query subgroup) -- a tuned
// shape may split an F head's G heads over two waves.  The G factors of a tile are
// shared by every wave of the workgroup: they go HBM -> LDS by direct DMA,
// one tile ahead, double-buffered.  Each wave's F slice goes HBM ->
// registers, one tile ahead.  No cross-wave reduction: the (query, head)
// rows of a wave are its own.  With several query groups per chunk, the
// workgroups of one chunk are placed on the same XCD so the tile is fetched
// from HBM once and shared through that XCD's L2.
//
// Two kinds of instantiation share this code:
//   * exact (Cfg): every dimension of the shape is a compile-time constant
//     (the tuned kernels of the workload shapes);
//   * generic (GenCfg): only the F feature dimension, caps on the ranks and
//     on the (iG, jG) rows, and the queries per wave are compile-time; the
//     head split, the G feature dimension (a power of two up to 32), the
//     ranks and which factor is F are read from the launch parameters, and
//     the LDS is sized per launch.
//
// Precision: bf16 factors exactly; the rotated, scaled query is split into
// bf16 hi + lo parts (two MFMAs, or one with the two parts in the two K
// halves when F is 8 wide) so it carries ~16 bits; the value operand
// p * G^V is rounded to bf16 (relative 2^-8 per term, unbiased) -- formed in
// fp32 on the VALU, or, on the matrix cores, from p rounded to bf16 first
// (the product of two bf16 is exact in fp32: 2 * 2^-8 per term); the
// normaliser sums the fp32 weights; all accumulation is fp32.  Because each KV chunk rounds against its own running max, results
// for different chunk counts agree to that bf16 rounding, not bit for bit.
#pragma once

#include <atomic>
#include <climits>
#include <mutex>
#include <type_traits>

#include "kpa_append.hpp"
#include "kpa_common.hpp"
#include "kpa_mfma.hpp"

namespace kpa {
namespace mfma {

constexpr int kXcds = 8;        // workgroups are dealt to the 8 XCDs round-robin
constexpr int kLdsBytes = 160 * 1024;  // LDS per CU (gfx950)

constexpr int pow2_at_least(int x) { return x <= 1 ? 1 : 2 * pow2_at_least((x + 1) / 2); }
__host__ __device__ __forceinline__ int pow2_ceil(int x) {
    int p = 1;
    while (p < x) p *= 2;
    return p;
}
__host__ __device__ __forceinline__ int ilog2(int x) {
    int l = 0;
    while ((1 << l) < x) ++l;
    return l;
}

// Exact shape: G factor PG x QG, F factor PF x QF, ranks RK, RV; F_IS_B: F
// is B (else A); NQW queries per wave, NQG query subgroups per workgroup; MW
// waves per SIMD the registers must allow; RS waves share one F head, each
// taking PG / RS of the G heads (the tile's G factors in LDS serve them all);
// FILL: percent of the resident-workgroup slots the split-KV planner fills;
// STRIDED: a chunk is every n_split-th tile (one query per workgroup only)
// rather than consecutive tiles.
template <int PG, int QG, int PF, int QF, int RK, int RV, bool F_IS_B, int NQW, int NQG, int MW, int RS = 1,
          int FILL = 100, bool STRIDED = false>
struct Cfg {
    static constexpr bool GEN = false;
    static constexpr int PG_ = PG, QG_ = QG, PF_ = PF, QF_ = QF, RK_ = RK, RV_ = RV;
    static constexpr int RS_ = RS, PGW_ = PG / RS;    // G heads per wave
    static constexpr int FILL_ = FILL;
    static constexpr bool STRIDED_ = STRIDED;
    static constexpr bool F_IS_B_ = F_IS_B;
    static constexpr int RKC = RK, RVC = RV;          // register arrays per rank
    // Kernels with one query per workgroup serve single-query decode, where a
    // tile's bytes are read once per step: their cache loads carry the
    // nontemporal hint (kpa_32k's kernel: 140 -> 126 us).  The multi-query
    // kernels' query groups share each tile through L2: no hint there (it
    // cost multiq_16 2%).
    static constexpr bool NT_ = NQW * NQG == 1;
    static constexpr int NQW_ = NQW;                 // queries per wave
    static constexpr int NQG_ = NQG;                 // query subgroups per workgroup
    static constexpr int QPW = NQW * NQG;            // queries per workgroup
    static constexpr int WAVES = PF * RS * NQG;
    static constexpr int WAVES_MAX = WAVES;
    static constexpr int MIN_WAVES = MW;
    static constexpr int M = PG * QG;                // rows (iG, jG) per query in a tile's G factors
    static constexpr int MR = PGW_ * QG;             // rows of one wave
    static constexpr int MB32 = (MR + 31) / 32;      // score MFMA row blocks (rows past MR are zero)
    static constexpr int MB16 = (MR + 15) / 16;      // value MFMA row blocks
    // An 8-wide F feature dimension takes one 16-wide K step: the bf16 hi part
    // of the query in the lower K half, its lo part in the upper half, and the
    // F factor in both (so one MFMA forms (hi + lo) . F).
    static constexpr bool K8 = QF == 8;
    static constexpr int KC = K8 ? 1 : QF / 16;      // score MFMA K steps = value MFMA column blocks
    static constexpr int H = PG * PF;
    static constexpr int DH = QG * QF;
    // G factors of one tile: key set R_K*M elements in 16-byte chunks of 8
    // (512 B per chunk for 32 slots), value set R_V*M elements x 32 slots; in
    // LDS each set is padded to whole 1 KB DMA blocks
    static constexpr int GK_BYTES = (RK * M + 7) / 8 * 512;
    static constexpr int GV_BYTES = RV * M * 64;
    static constexpr int GK_BLOCKS = (GK_BYTES + 1023) / 1024;
    static constexpr int GV_BLOCKS = (GV_BYTES + 1023) / 1024;
    static constexpr int G_BLOCKS = GK_BLOCKS + GV_BLOCKS;
    // softmax: NQW*PGW_ (query, head) rows per wave, padded to a power of
    // two, spread over 64 lanes
    static constexpr int ROWS = NQW * PGW_;
    static constexpr int ROWS_P = pow2_at_least(ROWS);
    static constexpr int GROUPS = 64 / ROWS_P;       // lanes per row
    static constexpr int TPG = 32 / GROUPS;          // slots per lane
    // row stride of the per-wave score scratch, padded so that the softmax's
    // reads (TPG consecutive floats per lane, rows = lane % ROWS_P) fall in
    // distinct LDS banks
    static constexpr int ZS = 32 + (ROWS_P >= 8 ? 4 : ROWS_P == 4 ? 8 : 16);
    static_assert(QF == 8 || QF == 16 || QF == 32 || QF == 64, "the MFMA-side feature dimension must be 8, 16, 32 or 64");
    static_assert(QG == 1 || QG == 2 || QG == 4 || QG == 8 || QG == 16 || QG == 32,
                  "G-side feature dimension 1, 2, 4, 8, 16 or 32");
    static_assert(PG % RS == 0, "the G heads split evenly over a head's waves");
    static_assert(MR % 4 == 0, "rows (iG, jG) come in groups of four");
    static_assert(ROWS_P <= 64 && ROWS_P >= 2, "query-head rows of a wave must fit 64 lanes");
    static_assert((F_IS_B ? QF : QG) <= 64, "rotary table holds 32 pairs");
    static_assert(RK <= 4 && RV <= 4, "ranks up to 4");
    static_assert(WAVES * 64 <= 1024, "at most 16 waves per workgroup");
    static_assert(!STRIDED || NQW * NQG == 1, "strided chunks for one query per workgroup");
};

// Generic family: F feature dimension QF, at most RKC key and RVC value
// ranks, at most 32*MB32 rows (iG, jG), NQW queries per wave, NQG query
// subgroups; everything else from the launch parameters (checked on the
// host: M = PG*QG <= 32*MB32 and a multiple of 4 unless R_K = 1, QG a power
// of two <= 32,
// NQW*PG <= 64 softmax rows per wave, PF*NQG <= WMAX waves).
template <int QF, int RKC_, int RVC_, int MB32_, int NQW, int NQG, int MW, int WMAX>
struct GenCfg {
    static constexpr bool GEN = true;
    static constexpr int QF_ = QF, RKC = RKC_, RVC = RVC_;
    static constexpr bool NT_ = NQW * NQG == 1;
    static constexpr int NQW_ = NQW, NQG_ = NQG, QPW = NQW * NQG;
    // at most WMAX waves (4 or 8): the workgroup size bounds the registers a
    // wave may hold (8 waves: 256 per lane; 4 waves: 512, AGPRs included)
    static constexpr int WAVES_MAX = WMAX;
    static constexpr int MIN_WAVES = MW;
    static constexpr int MB32 = MB32_, MB16 = 2 * MB32_;
    static constexpr bool K8 = QF == 8;
    static constexpr int KC = K8 ? 1 : QF / 16;
    static constexpr int ZS = 36;  // score scratch row stride (floats)
    // placeholders of the exact-only names (never read on the generic path)
    static constexpr int PG_ = 0, QG_ = 0, PF_ = 0, RK_ = 0, RV_ = 0, TPG = 1, ROWS_P = 2, WAVES = 0;
    static constexpr int RS_ = 1, PGW_ = 0, FILL_ = 100;
    static constexpr bool STRIDED_ = false;
    static constexpr int GK_BYTES = 0, GV_BYTES = 0, GK_BLOCKS = 0, G_BLOCKS = 0;
    static constexpr bool F_IS_B_ = true;
    static_assert(QF == 8 || QF == 16 || QF == 32 || QF == 64, "the MFMA-side feature dimension must be 8, 16, 32 or 64");
    static_assert(RKC <= 4 && RVC <= 4, "ranks up to 4");
};

// Geometry of one launch: constants of the exact configuration, or the
// values read from the launch parameters for a generic one.
struct Geo {
    int pg, pf, qg, lqg, m, h, rk, rv;
    int rs, pgw, mr;  // waves per F head, G heads and rows per wave
    bool fb;      // F is B
    int qrot;     // feature dimension of B (the rotary pairs)
    int gk_bytes, gv_bytes, gkb, gb;  // G key/value sets per tile; 1 KB blocks (key, total)
    int set_gk, set_fk, set_gv, set_fv;
    int waves, rows, rows_p, groups, tpg;
    __host__ __device__ __forceinline__ int head(int iG, int iF) const { return fb ? iG * pf + iF : iF * pg + iG; }
};

template <class S>
__host__ __device__ __forceinline__ Geo make_geo(const kpa_dims& d, int f_is_b) {
    Geo g{};
    if constexpr (!S::GEN) {
        g.pg = S::PG_;
        g.pf = S::PF_;
        g.qg = S::QG_;
        g.rk = S::RK_;
        g.rv = S::RV_;
        g.fb = S::F_IS_B_;
        g.lqg = ilog2(S::QG_);
        g.rows_p = S::ROWS_P;
        g.rs = S::RS_;
        g.pgw = S::PGW_;
    } else {
        g.fb = f_is_b != 0;
        g.pg = g.fb ? d.p1 : d.p2;
        g.pf = g.fb ? d.p2 : d.p1;
        g.qg = g.fb ? d.q1 : d.q2;
        g.rk = d.r_k;
        g.rv = d.r_v;
        g.lqg = ilog2(g.qg);
        g.rows_p = pow2_ceil(S::NQW_ * g.pg);
        if (g.rows_p < 2) g.rows_p = 2;
        g.rs = 1;
        g.pgw = g.pg;
    }
    g.m = g.pg * g.qg;
    g.mr = g.pgw * g.qg;
    g.h = g.pg * g.pf;
    g.qrot = g.fb ? S::QF_ : g.qg;
    g.gk_bytes = (g.rk * g.m + 7) / 8 * 512;
    g.gv_bytes = g.rv * g.m * 64;
    g.gkb = (g.gk_bytes + 1023) / 1024;
    g.gb = g.gkb + (g.gv_bytes + 1023) / 1024;
    g.set_gk = g.fb ? 0 : 1;
    g.set_fk = g.fb ? 1 : 0;
    g.set_gv = g.fb ? 2 : 3;
    g.set_fv = g.fb ? 3 : 2;
    g.waves = g.pf * g.rs * S::NQG_;
    g.rows = S::NQW_ * g.pgw;
    g.groups = 64 / g.rows_p;
    g.tpg = 32 / g.groups;
    return g;
}

template <class S>
__host__ __device__ __forceinline__ int feat(const Geo& g, int jG, int jF) {
    return g.fb ? jG * S::QF_ + jF : jF * g.qg + jG;
}

// Per-wave LDS scratch of the exact kernels: scores, overwritten in place by
// the softmax weights.
template <class S>
struct alignas(16) WaveScratch {
    float zp[S::ROWS_P][S::ZS];
    float alpha[S::ROWS_P];
    float m_fin[S::ROWS_P];
    float l_fin[S::ROWS_P];
};

// Dynamic LDS of a generic launch: two G buffers, the rotary table, then
// each wave's score scratch (rows_p x ZS scores, alpha, m, l).
template <class S>
struct GenLds {
    int gbuf_bytes, cs_off, scratch_off, wave_floats, total;
};
template <class S>
__host__ __device__ __forceinline__ GenLds<S> gen_lds(const Geo& g) {
    GenLds<S> l{};
    l.gbuf_bytes = g.gb * 1024;
    l.cs_off = 2 * l.gbuf_bytes;
    l.scratch_off = l.cs_off + S::QPW * 32 * 2 * 4;
    l.wave_floats = g.rows_p * (S::ZS + 3);
    l.total = l.scratch_off + g.waves * l.wave_floats * 4;
    return l;
}

// The G blocks of one tile, HBM -> LDS by DMA: 1 KB blocks of the key set,
// then of the value set, dealt to the waves round-robin.  A set's last block
// may be partial: only lanes inside the set copy.  Value set: 16-byte chunk q
// of element row e lands at chunk q ^ ((e >> 1) & 3) of its 64-byte row, so
// the value phase's reads of 16 rows x 4 chunks hit distinct LDS banks; a
// DMA lane writes a fixed LDS position, so it fetches the chunk that belongs
// there.
template <class S>
__device__ __forceinline__ void dma_g_blocks(const Geo& g, const uint8_t* gk, const uint8_t* gv, uint8_t* gdst, int wave,
                                             int lane) {
    constexpr int KB = S::GEN ? 0 : S::GK_BLOCKS, NBLK = S::GEN ? 0 : S::G_BLOCKS;
    const int kb_n = S::GEN ? g.gkb : KB, nblk = S::GEN ? g.gb : NBLK;
#pragma unroll
    for (int k = wave; k < nblk; k += (S::GEN ? g.waves : S::WAVES_MAX)) {
        const bool key = k < kb_n;
        const int kb = key ? k : k - kb_n;
        const int left = (key ? g.gk_bytes : g.gv_bytes) - kb * 1024;
        const int vchunk = (lane & ~3) | ((lane & 3) ^ ((lane >> 3) & 3));
        const uint8_t* src = (key ? gk : gv) + kb * 1024 + (key ? lane : vchunk) * 16;
        bool whole = false;
        if constexpr (!S::GEN) whole = S::GK_BYTES % 1024 == 0 && S::GV_BYTES % 1024 == 0;
        if (whole || lane * 16 < left) dma_to_lds16<S::NT_>(src, lds_addr(gdst + k * 1024));
    }
}

// One wave's F factor bytes, HBM -> registers.
template <class S>
__device__ __forceinline__ bf16x8 ld_f(const uint8_t* p) {
    if constexpr (S::NT_) return ld16_nt<bf16x8>(p);
    else return ld16<bf16x8>(p);
}

// One wave's F factors of one tile in registers: key set (R_K ranks) and
// value set (R_V ranks), KC 16-byte groups each.  With an 8-wide F feature
// dimension both halves of the wave hold the same key chunk, and the value
// lanes of columns 8 .. 15 hold zeros.  Ranks past the launch's own (generic
// kernels) are not loaded.
template <class S>
struct FRegs {
    bf16x8 fk[S::RKC][S::KC];
    bf16x8 fv[S::RVC][S::KC];
};

// The F slice of wave iF: key-set lane (slot s, half) takes 8 features of
// each 16-feature group (both halves the same 8 when F is 8 wide);
// value-set lane (row l16, slot group g16) takes 8 slots of one feature row.
template <class S>
__device__ __forceinline__ void load_f_regs(const Geo& g, const uint8_t* tile, int64_t offFK, int64_t offFV, int iF,
                                            int half, int s, int l16, int g16, FRegs<S>& f) {
    constexpr int QF = S::QF_;
#pragma unroll
    for (int r = 0; r < S::RKC; ++r) {
        if (r >= g.rk) continue;
#pragma unroll
        for (int kc = 0; kc < S::KC; ++kc)
            f.fk[r][kc] = ld_f<S>(tile + offFK + (int64_t)((r * g.pf + iF) * (QF / 8) + (S::K8 ? 0 : 2 * kc + half)) * 512 +
                                  s * 16);
    }
#pragma unroll
    for (int r = 0; r < S::RVC; ++r) {
        if (r >= g.rv) continue;
#pragma unroll
        for (int nb = 0; nb < S::KC; ++nb) {
            if (S::K8 && l16 >= 8)
                f.fv[r][nb] = bf16x8{};
            else
                f.fv[r][nb] = ld_f<S>(tile + offFV + ((int64_t)((r * g.pf + iF) * QF + 16 * nb + l16) * 32 + 8 * g16) * 2);
        }
    }
}

// Query elements (iG, iF, jG, jF0 .. jF0 + 7) of row `row`, unrotated.  Dense:
// two 16-byte loads when F = B (8 contiguous features).  Factored ((1/R_Q)
// sum_r A^Q_r (x) B^Q_r): per rank one element of the G-side factor times 8
// consecutive elements of the F-side factor -- its feature dimension is the
// contracted one, so the 8 are contiguous.
template <class S>
__device__ __forceinline__ void query_group8(const Geo& g, const DecodeParams& P, int64_t row, int iG, int iF, int jG,
                                             int jF0, float* out) {
    constexpr int QF = S::QF_;
    const int dh = g.qg * QF;
    if (P.a_q == nullptr) {
        const float* src = P.q + (row * g.h + g.head(iG, iF)) * dh;
        if (g.fb) {  // feat(jG, jF) = jG * QF + jF: contiguous in jF
            const f32x4 lo = *reinterpret_cast<const f32x4*>(src + feat<S>(g, jG, jF0));
            const f32x4 hi = *reinterpret_cast<const f32x4*>(src + feat<S>(g, jG, jF0) + 4);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                out[k] = lo[k];
                out[4 + k] = hi[k];
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) out[k] = src[feat<S>(g, jG, jF0 + k)];
        }
        return;
    }
    // F = B: A^Q_r[iG][jG] * B^Q_r[iF][jF];  F = A: A^Q_r[iF][jF] * B^Q_r[iG][jG]
    const int F_SET = g.pf * QF, G_SET = g.pg * g.qg;
    const float* fs = g.fb ? P.b_q : P.a_q;  // the F side's factor (8 contiguous)
    const float* gs = g.fb ? P.a_q : P.b_q;  // the G side's factor (one element)
    const float* f = fs + row * P.r_q * F_SET + iF * QF + jF0;
    const float* gp = gs + row * P.r_q * G_SET + iG * g.qg + jG;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // four ranks per round: their loads are all issued before the first
    // multiply-add, so a rank-16 query costs four memory round trips, not 16
    constexpr int RB = 4;
    for (int r0 = 0; r0 < P.r_q; r0 += RB) {
        float gv[RB];
        f32x4 lo[RB], hi[RB];
#pragma unroll
        for (int t = 0; t < RB; ++t) {
            const int r = min(r0 + t, P.r_q - 1);  // past the last rank: reloads it, weight 0 below
            gv[t] = gp[(int64_t)r * G_SET];
            lo[t] = *reinterpret_cast<const f32x4*>(f + (int64_t)r * F_SET);
            hi[t] = *reinterpret_cast<const f32x4*>(f + (int64_t)r * F_SET + 4);
        }
#pragma unroll
        for (int t = 0; t < RB; ++t) {
            const float w = r0 + t < P.r_q ? gv[t] : 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                acc[k] = fmaf(w, lo[t][k], acc[k]);
                acc[4 + k] = fmaf(w, hi[t][k], acc[4 + k]);
            }
        }
    }
    const float inv = 1.f / (float)P.r_q;
#pragma unroll
    for (int k = 0; k < 8; ++k) out[k] = acc[k] * inv;
}

template <class S>
__global__ void __launch_bounds__(S::WAVES_MAX * 64, S::MIN_WAVES) decode_mfma_kernel(DecodeParams P) {
    constexpr int QF = S::QF_, MB32 = S::MB32, MB16 = S::MB16, NQW = S::NQW_, KC = S::KC, ZS = S::ZS;
    constexpr int RKC = S::RKC, RVC = S::RVC;
    const Geo G = make_geo<S>(P.d, P.f_is_b);
    // whole row blocks: the bounds checks on rows vanish at compile time
    constexpr bool kFull32 = !S::GEN && S::PGW_ * S::QG_ % 32 == 0, kFull16 = !S::GEN && S::PGW_ * S::QG_ % 16 == 0;
    // M, PG: this wave's rows and G heads; MT: rows of the tile's G factors
    const int M = G.mr, PG = G.pgw, QG = G.qg, MT = G.m;

    // LDS: static arrays for the exact kernels, one dynamic region for the
    // generic ones
    uint8_t *gbuf_a, *gbuf_b;
    float* cs_base;     // [QPW][32][2]
    float* zp0;         // this wave's scores [rows_p][ZS]
    float *alpha_s, *m_fin, *l_fin;
    const int lane = threadIdx.x & 63;
    const int wave = S::WAVES_MAX == 1 ? 0 : (int)(threadIdx.x >> 6);
    if constexpr (!S::GEN) {
        __shared__ WaveScratch<S> scratch[S::WAVES];
        __shared__ float cs_tab[S::QPW][32][2];
        // two separate LDS objects (not one 2-D array) so the compiler can tell
        // the buffer being filled by DMA from the one being read
        __shared__ __attribute__((aligned(1024))) uint8_t gbuf_sa[S::G_BLOCKS * 1024];
        __shared__ __attribute__((aligned(1024))) uint8_t gbuf_sb[S::G_BLOCKS * 1024];
        gbuf_a = gbuf_sa;
        gbuf_b = gbuf_sb;
        cs_base = &cs_tab[0][0][0];
        zp0 = &scratch[wave].zp[0][0];
        alpha_s = scratch[wave].alpha;
        m_fin = scratch[wave].m_fin;
        l_fin = scratch[wave].l_fin;
    } else {
        extern __shared__ __attribute__((aligned(1024))) uint8_t dyn_lds[];
        const GenLds<S> lay = gen_lds<S>(G);
        gbuf_a = dyn_lds;
        gbuf_b = dyn_lds + lay.gbuf_bytes;
        cs_base = reinterpret_cast<float*>(dyn_lds + lay.cs_off);
        zp0 = reinterpret_cast<float*>(dyn_lds + lay.scratch_off) + wave * lay.wave_floats;
        alpha_s = zp0 + G.rows_p * ZS;
        m_fin = alpha_s + G.rows_p;
        l_fin = m_fin + G.rows_p;
    }
    auto cs_at = [&](int nq, int m, int k) -> float& { return cs_base[(nq * 32 + m) * 2 + k]; };

    const int iF = wave % G.pf;
    const int rsub = (wave / G.pf) % G.rs;  // which G heads of F head iF
    const int qsub = wave / (G.pf * G.rs);
    const int iG0 = rsub * PG, m0 = rsub * M;  // first G head, first tile row of this wave
    const int half = lane >> 5;
    const int s = lane & 31;       // slot within the tile for the score side
    const int l16 = lane & 15;
    const int g16 = lane >> 4;     // 8-slot group for the value side
    const int b = blockIdx.y;
    // workgroup -> (chunk, query group): the query groups of a chunk share an
    // XCD (blockIdx.x mod 8 -- the row's part of the linear index is a
    // multiple of 8); chunk k of sequence b goes to XCD (b n_split + k) mod
    // 8, so that when n_split is not a multiple of 8 the grid's padding
    // spreads over the XCDs instead of idling the same ones in every row
    const int qwg_count = (P.n_q + S::QPW - 1) / S::QPW;
    const int bx = blockIdx.x;
    const int xcd_off = (int)(((int64_t)b * P.n_split) % kXcds);
    const int split = (bx / (kXcds * qwg_count)) * kXcds + (bx % kXcds - xcd_off + kXcds) % kXcds;
    const int qwg = (bx / kXcds) % qwg_count;
    if (split >= P.n_split) return;  // padding of the grid to a multiple of the XCD count
    const Layout& L = P.L;
    const int n0 = qwg * S::QPW + qsub * NQW;  // first query of this wave

    // slot of the first new token of a fused append (single-query kernels),
    // read now so that its latency overlaps the prologue.  A vector load:
    // scalar loads complete out of order, so waiting on this one would also
    // hold up every kernel-argument load issued after it.
    int app_slot0_v = 0;
    if (NQW == 1 && P.app.n_new > 0) {
        int lane_zero = 0;
        asm volatile("" : "+v"(lane_zero));
        app_slot0_v = P.app.slot0[b + lane_zero];
    }

    // One query per wave: the first tile goes in flight before the query is
    // prepared (its latency hides the rotation's float64 arithmetic): its G
    // blocks land in gbuf_a by DMA, its F slice in fa.  A dense query's
    // elements (8 contiguous per lane and K step when F = B; exact kernels)
    // and the query positions are requested just before.  Loads complete in
    // order, so the prologue's wait for them need not cover the F loads; it
    // still covers the G blocks, whose inline-asm DMA the compiler's wait
    // counts cannot see.
    FRegs<S> fa, fb;
    constexpr bool kEarly = NQW == 1;
    constexpr bool kQPre = kEarly && !S::GEN && S::F_IS_B_;
    f32x4 q_pre[kQPre ? MB32 : 1][KC][2];
    int qpos_pre = 0;  // this thread's first rotary angle's query position
    if constexpr (kEarly) {
        const int e = threadIdx.x;
        if (e < S::QPW * (G.qrot / 2))
            qpos_pre = P.q_pos[(int64_t)b * P.n_q + min(qwg * S::QPW + e / (G.qrot / 2), P.n_q - 1)];
    }
    if constexpr (kQPre) {
        if (P.a_q == nullptr) {
            const int64_t qrow = (int64_t)b * P.n_q + min(n0, P.n_q - 1);
#pragma unroll
            for (int mb = 0; mb < MB32; ++mb) {
                const int R = mb * 32 + s;
                const bool row_ok = kFull32 || R < M;
                const int iG = iG0 + (row_ok ? R / QG : 0), jG = row_ok ? R % QG : 0;
                const float* src = P.q + (qrow * G.h + G.head(iG, iF)) * (QG * QF) + feat<S>(G, jG, S::K8 ? 0 : 8 * half);
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    q_pre[mb][kc][0] = *reinterpret_cast<const f32x4*>(src + 16 * kc);
                    q_pre[mb][kc][1] = *reinterpret_cast<const f32x4*>(src + 16 * kc + 4);
                }
            }
        }
    }
    const int64_t offFK = L.off[G.set_fk], offGK = L.off[G.set_gk];
    const int64_t offFV = L.off[G.set_fv], offGV = L.off[G.set_gv];
    // The tiles of a chunk: chunk_tiles consecutive tiles, or (STRIDED)
    // tiles split, split + n_split, split + 2 n_split, ..., so that the
    // chunks' workgroups sweep one sequence side by side and at any time read
    // one contiguous stretch of it.
    constexpr bool kStrided = S::STRIDED_;
    const int chunk_first = kStrided ? split * kTileSlots : split * P.chunk_tiles * kTileSlots;
    const int chunk_end = kStrided ? INT_MAX : chunk_first + P.chunk_tiles * kTileSlots;
    const int t_step = kStrided ? P.n_split : 1;  // tiles from one tile of the chunk to the next
    int early_first = 0, early_last = 0;
    if constexpr (kEarly) {
        int vis_e = 0;
        for (int n = qwg * S::QPW; n < min(P.n_q, (qwg + 1) * S::QPW); ++n) vis_e = max(vis_e, visible_slots(P, b, n));
        early_first = chunk_first;
        early_last = min(chunk_end, vis_e);
        if (early_first < early_last) {
            const uint8_t* tile = P.cache + (int64_t)b * L.n_tiles * L.tile_bytes +
                                  (int64_t)(early_first / kTileSlots) * L.tile_bytes;
            dma_g_blocks<S>(G, tile + offGK, tile + offGV, gbuf_a, wave, lane);
            load_f_regs<S>(G, tile, offFK, offFV, iF, half, s, l16, g16, fa);
        }
    }

    // ---- rotated, scaled queries as MFMA A operands (hi + lo bf16) ----------
    for (int e = threadIdx.x; e < S::QPW * (G.qrot / 2); e += G.waves * 64) {
        const int nq = e / (G.qrot / 2), m = e % (G.qrot / 2);
        const int n = min(qwg * S::QPW + nq, P.n_q - 1);
        const double theta = exp2(-(2.0 * m / G.qrot) * log2((double)P.d.rope_base));
        double sn, c;
        const int qp = kEarly && e == (int)threadIdx.x ? qpos_pre : P.q_pos[(int64_t)b * P.n_q + n];
        sincos((double)qp * theta, &sn, &c);
        cs_at(nq, m, 0) = (float)c;
        cs_at(nq, m, 1) = (float)sn;
    }
    for (int n = 0; n < S::QPW; ++n)  // every thread takes part: the clear strides over heads
        if (qwg * S::QPW + n < P.n_q) clear_merge_counters(P, (int64_t)b * P.n_q + qwg * S::QPW + n, split);
    __syncthreads();
    bf16x8 q_hi[NQW][MB32][KC], q_lo[NQW][MB32][KC];
#pragma unroll
    for (int u = 0; u < NQW; ++u) {
        const int n = min(n0 + u, P.n_q - 1);  // queries past n_q compute and are discarded
        const int64_t qrow = (int64_t)b * P.n_q + n;
        const int nq = qsub * NQW + u;
#pragma unroll
        for (int mb = 0; mb < MB32; ++mb) {
            const int R = mb * 32 + s;
            const bool row_ok = kFull32 || R < M;  // padding rows of the last block are zero
            const int iG = iG0 + (row_ok ? R >> G.lqg : 0), jG = row_ok ? R & (QG - 1) : 0;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                // the 8 query elements (jG, jF0 .. jF0 + 7) of this lane and
                // their rotary partners: (jG, jF ^ 1) when F = B (inside the
                // same 8), (jG ^ 1, jF) when F = A
                const int jF0 = S::K8 ? 0 : 16 * kc + 8 * half;
                float xs[8], ys[8];
                if (kQPre && P.a_q == nullptr) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        xs[k] = q_pre[kQPre ? mb : 0][kc][0][k];
                        xs[4 + k] = q_pre[kQPre ? mb : 0][kc][1][k];
                    }
                } else {
                    query_group8<S>(G, P, qrow, iG, iF, jG, jF0, xs);
                }
                if (!G.fb) query_group8<S>(G, P, qrow, iG, iF, jG ^ 1, jF0, ys);
                float v[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int jF = jF0 + k;
                    float x, y;  // this element and its rotary partner
                    int m, first;
                    if (G.fb) {
                        x = xs[k];
                        y = xs[k ^ 1];
                        m = jF >> 1;
                        first = !(jF & 1);
                    } else {
                        x = xs[k];
                        y = ys[k];
                        m = jG >> 1;
                        first = !(jG & 1);
                    }
                    const float c = cs_at(nq, m, 0), sn = cs_at(nq, m, 1);
                    // (x0, x1) -> (x0 c - x1 s, x0 s + x1 c)
                    const float rot = first ? (x * c - y * sn) : (y * sn + x * c);
                    v[k] = row_ok ? rot * P.q_scale : 0.f;
                }
                if constexpr (S::K8) {
                    // lower K half: hi; upper K half: lo (the F operand repeats)
                    bf16x8 hi, lo;
                    split_bf16x8(v, hi, lo);
                    q_hi[u][mb][kc] = half ? lo : hi;
                } else {
                    split_bf16x8(v, q_hi[u][mb][kc], q_lo[u][mb][kc]);
                }
            }
        }
    }

    f32x4 o_acc[NQW][MB16][KC];
#pragma unroll
    for (int u = 0; u < NQW; ++u)
#pragma unroll
        for (int k = 0; k < MB16; ++k)
#pragma unroll
            for (int nb = 0; nb < KC; ++nb) o_acc[u][k][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int rows_p = G.rows_p;
    // padding rows of the softmax scratch never receive scores: keep them at -inf
    for (int e = lane; e < (rows_p - G.rows) * 32; e += 64) zp0[(G.rows + e / 32) * ZS + e % 32] = -INFINITY;
    // softmax state for row sm_row = (query u, head iG) of this wave; l is this
    // lane's partial sum over its slots
    const int sm_row = lane % rows_p, sm_g = lane / rows_p;
    float m_run = -INFINITY, l_run = 0.f;

    // visible slots: per query (causal), and the workgroup's furthest
    int vis[NQW];
#pragma unroll
    for (int u = 0; u < NQW; ++u) vis[u] = n0 + u < P.n_q ? visible_slots(P, b, n0 + u) : 0;
    int vis_wg = 0;
    for (int n = qwg * S::QPW; n < min(P.n_q, (qwg + 1) * S::QPW); ++n) vis_wg = max(vis_wg, visible_slots(P, b, n));
    const int first = chunk_first;
    const int last = min(chunk_end, vis_wg);  // the chunk's slots lie in [first, last)
    const int step = t_step * kTileSlots;     // slots from one tile of the chunk to the next
    const int64_t tstep = (int64_t)t_step * L.tile_bytes;
    const uint8_t* seq = P.cache + (int64_t)b * L.n_tiles * L.tile_bytes;

    // Pipeline, one tile ahead for every byte:
    //  * G factors (shared by the workgroup's waves): HBM -> LDS by direct DMA
    //    (global_load_lds_dwordx4), double-buffered, each wave copying 1 KB
    //    blocks.  The DMA is issued from inline asm so the compiler does not
    //    make every LDS read wait for it; the explicit vmcnt(0) below is the
    //    only wait it needs;
    //  * the wave's own F slice: HBM -> registers, double-buffered.
    // At the top of each tile one wait for everything issued a tile earlier
    // and one barrier (all G blocks landed; the other buffer is free).
    using FR = kpa::mfma::FRegs<S>;
    auto load_f = [&](const uint8_t* tile, FR& f) __attribute__((always_inline)) {
        load_f_regs<S>(G, tile, offFK, offFV, iF, half, s, l16, g16, f);
    };
    auto issue = [&](const uint8_t* tile, uint8_t* gdst, FR& f) __attribute__((always_inline)) {
        dma_g_blocks<S>(G, tile + offGK, tile + offGV, gdst, wave, lane);
        load_f(tile, f);
    };

    // Exact kernels whose G feature dimension is a multiple of 4 (so each
    // group of four rows is one head) fold the softmax weights into the
    // value factor on the matrix cores; the others on the vector ALU.
    constexpr bool kMxFold = !S::GEN && S::QG_ % 4 == 0;
    // v_perm_b32 selectors that place the low bf16 of a dword at element i4
    // of a zeroed 4-element operand: dword 0, dword 1
    const int i4 = lane & 3;
    uint32_t psel[2];
    {
        constexpr uint32_t kZ = 0x0c0c0c0cu;  // every byte 0
        constexpr uint32_t kLo = 0x0c0c0100u, kHi = 0x01000c0cu;  // the low bf16 to the low / high half
        psel[0] = i4 == 0 ? kLo : i4 == 1 ? kHi : kZ;
        psel[1] = i4 == 2 ? kLo : i4 == 3 ? kHi : kZ;
    }

    auto process = [&](int s0, const uint8_t* gcur, FR& f) __attribute__((always_inline)) {
        const int valid = min(kTileSlots, last - s0);
        // ---- scores: W = q' F (MFMA), z = sum G W (VALU) --------------------
        // This lane holds rows R = mb*32 + 8a + 4half + b (b = 0..3) of W for slot s.
#pragma unroll
        for (int mb = 0; mb < MB32; ++mb) {
            if (S::GEN && mb * 32 >= M) continue;
            // [query][a][b]: sums over the rank, per row b (G feature dimension 1:
            // every row is a head; generic kernels: every row), per pair of rows
            // (dimension 2) or already summed over the in-lane jG
            constexpr int ZB = S::GEN ? 4 : S::QG_ == 1 ? 4 : S::QG_ == 2 ? 2 : 1;
            float zp[NQW][4][ZB];
#pragma unroll
            for (int u = 0; u < NQW; ++u)
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int bb = 0; bb < ZB; ++bb) zp[u][a][bb] = 0.f;
#pragma unroll
            for (int r = 0; r < RKC; ++r) {
                if (r >= G.rk) continue;
                // this lane's G values for its rows, shared by every query:
                // element e0 = r*MT + m0 + mb*32 + 8a + 4half, four
                // consecutive ones in one 16-byte chunk (m0 is a multiple of
                // 4); the lane's part of the address is per rank, the (mb, a)
                // part a constant offset
                const int e_lane = r * MT + m0 + 4 * half;
                const uint8_t* gk_lane = gcur + (e_lane >> 3) * 512 + s * 16 + (e_lane & 7) * 2;
                float gx[4][4];
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int R0 = mb * 32 + 8 * a + 4 * half;
                    if (kFull32 || R0 < M) {
                        const uint2 gk = *reinterpret_cast<const uint2*>(gk_lane + (mb * 4 + a) * 512);
                        unpack_bf16x4(gk, gx[a][0], gx[a][1], gx[a][2], gx[a][3]);
                    } else {
                        gx[a][0] = gx[a][1] = gx[a][2] = gx[a][3] = 0.f;
                    }
                }
#pragma unroll
                for (int u = 0; u < NQW; ++u) {
                    f32x16 w = f32x16{};
#pragma unroll
                    for (int kc = 0; kc < KC; ++kc) {
                        w = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q_hi[u][mb][kc], f.fk[r][kc], w, 0, 0, 0);
                        if constexpr (!S::K8)
                            w = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q_lo[u][mb][kc], f.fk[r][kc], w, 0, 0, 0);
                    }
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        // row groups past M (the last block of a partial M): nothing to add
                        if (!kFull32 && mb * 32 + 8 * a >= M) continue;
                        if constexpr (ZB == 4) {
#pragma unroll
                            for (int bb = 0; bb < 4; ++bb) zp[u][a][bb] += w[a * 4 + bb] * gx[a][bb];
                        } else if constexpr (ZB == 2) {
#pragma unroll
                            for (int bb = 0; bb < 4; ++bb)
                                zp[u][a][bb >> 1] = fmaf(w[a * 4 + bb], gx[a][bb], zp[u][a][bb >> 1]);
                        } else {
                            // a chain of fused multiply-adds into the running sum
#pragma unroll
                            for (int bb = 0; bb < 4; ++bb) zp[u][a][0] = fmaf(w[a * 4 + bb], gx[a][bb], zp[u][a][0]);
                        }
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < NQW; ++u) {
                const bool ok = s0 + s < vis[u] && s < valid;  // causal mask per query
                float* zrow = zp0 + (u * PG) * ZS;
                if constexpr (S::GEN) {
                    // rows -> heads by the G feature dimension (a power of two)
                    if (QG == 1) {
#pragma unroll
                        for (int a = 0; a < 4; ++a)
#pragma unroll
                            for (int bb = 0; bb < 4; ++bb) {
                                const int R = mb * 32 + 8 * a + 4 * half + bb;
                                if (R < M) zrow[R * ZS + s] = ok ? zp[u][a][bb] : -INFINITY;
                            }
                    } else if (QG == 2) {
#pragma unroll
                        for (int a = 0; a < 4; ++a)
#pragma unroll
                            for (int c = 0; c < 2; ++c) {
                                const int R = mb * 32 + 8 * a + 4 * half + 2 * c;
                                if (R < M) zrow[(R >> 1) * ZS + s] = ok ? zp[u][a][2 * c] + zp[u][a][2 * c + 1] : -INFINITY;
                            }
                    } else {
                        float z4[4];
#pragma unroll
                        for (int a = 0; a < 4; ++a) z4[a] = (zp[u][a][0] + zp[u][a][1]) + (zp[u][a][2] + zp[u][a][3]);
                        if (QG == 4) {
#pragma unroll
                            for (int a = 0; a < 4; ++a) {
                                const int R0 = mb * 32 + 8 * a + 4 * half;
                                if (R0 < M) zrow[(R0 >> 2) * ZS + s] = ok ? z4[a] : -INFINITY;
                            }
                        } else if (QG == 8) {
#pragma unroll
                            for (int a = 0; a < 4; ++a) z4[a] = sum_halves(z4[a]);
#pragma unroll
                            for (int a = 0; a < 4; ++a)
                                if ((a >> 1) == half && mb * 32 + 8 * a < M) zrow[(mb * 4 + a) * ZS + s] = ok ? z4[a] : -INFINITY;
                        } else if (QG == 16) {
                            const float z0 = sum_halves(z4[0] + z4[1]), z1 = sum_halves(z4[2] + z4[3]);
                            if (mb * 32 + 16 * half < M) zrow[(mb * 2 + half) * ZS + s] = ok ? (half ? z1 : z0) : -INFINITY;
                        } else {  // QG == 32: the whole row block is head mb
                            const float z = sum_halves((z4[0] + z4[1]) + (z4[2] + z4[3]));
                            if (half == 0) zrow[mb * ZS + s] = ok ? z : -INFINITY;
                        }
                    }
                } else if constexpr (ZB == 4) {
                    // every row is a head
#pragma unroll
                    for (int a = 0; a < 4; ++a)
#pragma unroll
                        for (int bb = 0; bb < ZB; ++bb) {
                            const int R = mb * 32 + 8 * a + 4 * half + bb;
                            if (kFull32 || R < M) zrow[R * ZS + s] = ok ? zp[u][a][bb] : -INFINITY;
                        }
                } else if constexpr (ZB == 2) {
                    // rows 8a + 4half + 2c + {0, 1} form head mb*16 + 4a + 2half + c
#pragma unroll
                    for (int a = 0; a < 4; ++a)
#pragma unroll
                        for (int c = 0; c < 2; ++c) {
                            const int R = mb * 32 + 8 * a + 4 * half + 2 * c;
                            if (kFull32 || R < M) zrow[(R >> 1) * ZS + s] = ok ? zp[u][a][c] : -INFINITY;
                        }
                } else {
                    constexpr int QGc = S::QG_;
                    float z4[4];
#pragma unroll
                    for (int a = 0; a < 4; ++a) z4[a] = zp[u][a][0];
                    if constexpr (QGc == 4) {
                        // rows 8a + 4half + b: iG = mb*8 + 2a + half, jG = b -- complete in lane
#pragma unroll
                        for (int a = 0; a < 4; ++a)
                            if (kFull32 || mb * 32 + 8 * a + 4 * half < M) zrow[(mb * 8 + 2 * a + half) * ZS + s] = ok ? z4[a] : -INFINITY;
                    } else if constexpr (QGc == 8) {
                        // iG = mb*4 + a, jG = 4half + b: add the other half
#pragma unroll
                        for (int a = 0; a < 4; ++a) z4[a] = sum_halves(z4[a]);
                        // selects, not a lane-dependent array index (which would go to scratch)
                        const float za = half ? z4[2] : z4[0];
                        const float zb = half ? z4[3] : z4[1];
                        if (kFull32 || mb * 32 + 16 * half < M) zrow[(mb * 4 + 2 * half + 0) * ZS + s] = ok ? za : -INFINITY;
                        if (kFull32 || mb * 32 + 16 * half + 8 < M) zrow[(mb * 4 + 2 * half + 1) * ZS + s] = ok ? zb : -INFINITY;
                    } else if constexpr (QGc == 16) {
                        // iG = mb*2 + a/2, jG = 8(a%2) + 4half + b
                        float z0 = z4[0] + z4[1], z1 = z4[2] + z4[3];
                        z0 = sum_halves(z0);
                        z1 = sum_halves(z1);
                        if (kFull32 || mb * 32 + 16 * half < M) zrow[(mb * 2 + half) * ZS + s] = ok ? (half ? z1 : z0) : -INFINITY;
                    } else {
                        // QG == 32: the whole row block is head mb
                        const float z = sum_halves((z4[0] + z4[1]) + (z4[2] + z4[3]));
                        if (half == 0 && (kFull32 || mb * 32 < M)) zrow[mb * ZS + s] = ok ? z : -INFINITY;
                    }
                }
            }
            // KPA_SCHED_MB
        }
        wave_lds_sync();

        // ---- online softmax for the wave's (query, head) rows -----------------
        if constexpr (!S::GEN) {
            float zl[S::TPG];
            float mt = -INFINITY;
#pragma unroll
            for (int t = 0; t < S::TPG; ++t) {
                zl[t] = zp0[sm_row * ZS + sm_g * S::TPG + t];
                mt = fmaxf(mt, zl[t]);
            }
#pragma unroll
            for (int x = S::ROWS_P; x < 64; x <<= 1) mt = fmaxf(mt, __shfl_xor(mt, x));
            const float m_new = fmaxf(m_run, mt);
            // with no slot seen yet (m = -inf) every weight is 0 and alpha 1
            const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_ref);
            float lsum = 0.f;
#pragma unroll
            for (int t = 0; t < S::TPG; ++t) {
                const float p = fast_exp2(zl[t] - m_ref);  // masked slots: 2^-inf = 0
                zp0[sm_row * ZS + sm_g * S::TPG + t] = p;
                lsum += p;
            }
            l_run = l_run * alpha + lsum;
            m_run = m_new;
            if (sm_g == 0) alpha_s[sm_row] = alpha;
        } else {
            // the same, with the row layout read from the launch: two passes
            // over the LDS row (no register array of run-time length)
            const int tpg = G.tpg;
            float* zr = zp0 + sm_row * ZS + sm_g * tpg;
            float mt = -INFINITY;
            for (int t = 0; t < tpg; ++t) mt = fmaxf(mt, zr[t]);
            for (int x = rows_p; x < 64; x <<= 1) mt = fmaxf(mt, __shfl_xor(mt, x));
            const float m_new = fmaxf(m_run, mt);
            const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_ref);
            float lsum = 0.f;
            for (int t = 0; t < tpg; ++t) {
                const float p = fast_exp2(zr[t] - m_ref);
                zr[t] = p;
                lsum += p;
            }
            l_run = l_run * alpha + lsum;
            m_run = m_new;
            if (sm_g == 0) alpha_s[sm_row] = alpha;
        }
        wave_lds_sync();

        // ---- values: O = alpha O + (p G^V) F^V (MFMA over slots) -------------
        const uint8_t* gvbase = gcur + (S::GEN ? G.gkb : S::GK_BLOCKS) * 1024;
        auto values = [&](auto partial_tag) __attribute__((always_inline)) {
            constexpr bool kPartial = decltype(partial_tag)::value;
            if constexpr (kPartial) {
                // slots past the end: zero both operands (the cache may hold NaNs there)
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (8 * g16 + k >= valid)
#pragma unroll
                        for (int r = 0; r < RVC; ++r)
#pragma unroll
                            for (int nb = 0; nb < KC; ++nb) f.fv[r][nb][k] = (__bf16)0.f;
            }
#pragma unroll
            for (int mb = 0; mb < MB16; ++mb) {
                if (S::GEN && mb * 16 >= M) continue;
                const int R_row = mb * 16 + l16;               // row of this lane's A operand
                const bool row_ok = kFull16 || R_row < M;
                const int iG_row = row_ok ? R_row >> G.lqg : 0;
                float p[NQW][kMxFold ? 2 : 8];
#pragma unroll
                for (int u = 0; u < NQW; ++u) {
                    // rows of this lane's accumulators: mb*16 + 4*g16 + c
                    if (QG % 4 == 0) {
                        // the four rows share one head
                        const float a = alpha_s[u * PG + ((mb * 16 + 4 * g16) >> G.lqg)];
#pragma unroll
                        for (int nb = 0; nb < KC; ++nb)
#pragma unroll
                            for (int c = 0; c < 4; ++c) o_acc[u][mb][nb][c] *= a;
                    } else {
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const int R_out = mb * 16 + 4 * g16 + c;
                            const float a = alpha_s[u * PG + (kFull16 || R_out < M ? R_out >> G.lqg : 0)];
#pragma unroll
                            for (int nb = 0; nb < KC; ++nb) o_acc[u][mb][nb][c] *= a;
                        }
                    }
                    if constexpr (kMxFold) {
                        // two weights: slots 8 g16 + i4 and 8 g16 + 4 + i4
                        const float* pz = &zp0[(u * PG + iG_row) * ZS + 8 * g16 + i4];
                        p[u][0] = row_ok ? pz[0] : 0.f;
                        p[u][1] = row_ok ? pz[4] : 0.f;
                    } else {
                        ld_lds32(&zp0[(u * PG + iG_row) * ZS + 8 * g16], p[u]);
                        if (!row_ok)
#pragma unroll
                            for (int k = 0; k < 8; ++k) p[u][k] = 0.f;
                    }
                }
                if constexpr (kMxFold) {
                    // p * G^V on the matrix cores.  One 4x4x4 block per (four
                    // rows of one head, four slots): A = diag(p of the four
                    // slots), B = G^V of the rows at those slots, so D holds
                    // p * G^V with each lane's own row in its column -- the
                    // four slots of the value MFMA's A operand, in order.
                    // Lane (4 blk + i) gives A's row i: its weight at k = i.
                    s16x4 pa[NQW][2];
#pragma unroll
                    for (int u = 0; u < NQW; ++u) {
                        // the weight in the low half of a packed pair, the other
                        // weight in the high half (not read)
                        const uint32_t pk0 = pack2_bf16(p[u][0], p[u][1]), pk1 = pack2_bf16(p[u][1], p[u][0]);
                        pa[u][0] = __builtin_bit_cast(s16x4, uint2{__builtin_amdgcn_perm(pk0, pk0, psel[0]),
                                                                     __builtin_amdgcn_perm(pk0, pk0, psel[1])});
                        pa[u][1] = __builtin_bit_cast(s16x4, uint2{__builtin_amdgcn_perm(pk1, pk1, psel[0]),
                                                                     __builtin_amdgcn_perm(pk1, pk1, psel[1])});
                    }
#pragma unroll
                    for (int r = 0; r < RVC; ++r) {
                        uint4 graw = uint4{0u, 0u, 0u, 0u};
                        if (row_ok) {
                            const int e_lane = r * MT + m0 + l16;
                            const uint8_t* gv_lane = gvbase + e_lane * 64 + ((g16 ^ ((e_lane >> 1) & 3)) * 16);
                            graw = *reinterpret_cast<const uint4*>(gv_lane + mb * 1024);
                        }
                        if constexpr (kPartial) {
                            // slots past the end hold arbitrary bytes: 0 * NaN
                            // would reach every output of the block
                            const int left = valid - 8 * g16;  // slots of this lane's 8 that are valid
                            graw.x = left >= 2 ? graw.x : left >= 1 ? (graw.x & 0xffffu) : 0u;
                            graw.y = left >= 4 ? graw.y : left >= 3 ? (graw.y & 0xffffu) : 0u;
                            graw.z = left >= 6 ? graw.z : left >= 5 ? (graw.z & 0xffffu) : 0u;
                            graw.w = left >= 8 ? graw.w : left >= 7 ? (graw.w & 0xffffu) : 0u;
                        }
                        const s16x4 gb0 = __builtin_bit_cast(s16x4, uint2{graw.x, graw.y});
                        const s16x4 gb1 = __builtin_bit_cast(s16x4, uint2{graw.z, graw.w});
#pragma unroll
                        for (int u = 0; u < NQW; ++u) {
                            const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
                            const f32x4 d0 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(pa[u][0], gb0, zero4, 0, 0, 0);
                            const f32x4 d1 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(pa[u][1], gb1, zero4, 0, 0, 0);
                            const bf16x8 ga = __builtin_bit_cast(
                                bf16x8, u32x4{pack2_bf16(d0[0], d0[1]), pack2_bf16(d0[2], d0[3]),
                                              pack2_bf16(d1[0], d1[1]), pack2_bf16(d1[2], d1[3])});
#pragma unroll
                            for (int nb = 0; nb < KC; ++nb)
                                o_acc[u][mb][nb] =
                                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(ga, f.fv[r][nb], o_acc[u][mb][nb], 0, 0, 0);
                        }
                    }
                    continue;
                }
#pragma unroll
                for (int r = 0; r < RVC; ++r) {
                    if (r >= G.rv) continue;
                    float gvf[8];
                    if (row_ok) {
                        // element row e = r*MT + m0 + mb*16 + l16 of the value
                        // set; its chunk swizzle depends on bits 1-2 of e, which
                        // mb*16 leaves alone: a per-rank lane address plus mb KB
                        const int e_lane = r * MT + m0 + l16;
                        const uint8_t* gv_lane = gvbase + e_lane * 64 + ((g16 ^ ((e_lane >> 1) & 3)) * 16);
                        unpack_bf16x8(*reinterpret_cast<const bf16x8*>(gv_lane + mb * 1024), gvf);
                    } else {
#pragma unroll
                        for (int k = 0; k < 8; ++k) gvf[k] = 0.f;
                    }
                    if constexpr (kPartial)
#pragma unroll
                        for (int k = 0; k < 8; ++k) gvf[k] = (8 * g16 + k >= valid) ? 0.f : gvf[k];
#pragma unroll
                    for (int u = 0; u < NQW; ++u) {
                        float prod[8];
#pragma unroll
                        for (int k = 0; k < 8; ++k) prod[k] = p[u][k] * gvf[k];
                        const bf16x8 ga = pack_bf16x8(prod);
#pragma unroll
                        for (int nb = 0; nb < KC; ++nb)
                            o_acc[u][mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ga, f.fv[r][nb], o_acc[u][mb][nb], 0, 0, 0);
                    }
                }
            }
        };
        if (valid < kTileSlots) values(std::true_type{});
        else values(std::false_type{});
    };

    const uint8_t* t0 = seq + (int64_t)(first / kTileSlots) * L.tile_bytes;
    if constexpr (!kEarly) {
        if (first < last) issue(t0, gbuf_a, fa);
    }
    // Fused append (kpa_append_decode, single-query kernels; the host runs
    // the append kernel first for the others): each new token is written by
    // the workgroup of the chunk whose tiles hold it before it reads it.  The
    // slot0 value arrives behind the first tile's G blocks (loads complete in
    // order), so workgroups owning no token wait here for what the tile
    // loop's first wait would wait for anyway.
    // The owner writes its tokens and waits for the stores, all before the
    // next tile's loads are issued; for a token in the first tile it fetches
    // that tile again (the loop's first wait covers it).
    if (kEarly && P.app.n_new > 0) {
        // keeps the wait for slot0 (and the loads ahead of it) after the
        // first tile's loads have been issued
        asm volatile("" : "+v"(app_slot0_v)::"memory");
        const int app_slot0 = __builtin_amdgcn_readfirstlane(app_slot0_v);
        const int span = P.chunk_tiles * kTileSlots;
        bool owned = false, in_first = false;
        for (int n = 0; n < P.app.n_new; ++n) {
            const int j = slot_add(app_slot0, n);
            // (a slot past every contiguous chunk: the last chunk)
            const int owner = j < 0 ? 0 : kStrided ? (j / kTileSlots) % P.n_split : min(j / span, P.n_split - 1);
            if (owner != split) continue;
            append_token<false>(P.d, L, P.cache_w, P.capacity, P.app, P.dev_status, b, n, threadIdx.x,
                                G.waves * 64);
            owned = true;
            if (j >= first && j < first + kTileSlots) in_first = true;
        }
        if (owned) {
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's stores are done
            __syncthreads();                     // ... and every other wave's
            if (in_first && first < last) {
                dma_g_blocks<S>(G, t0 + offGK, t0 + offGV, gbuf_a, wave, lane);
                load_f(t0, fa);
            }
        }
    }
    for (int s0 = first; s0 < last; s0 += 2 * step) {
        // tile s0: data in gbuf_a and fa
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the DMA and loads issued one tile ago
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const uint8_t* tile = seq + (int64_t)(s0 / kTileSlots) * L.tile_bytes;
        if (s0 + step < last) issue(tile + tstep, gbuf_b, fb);
        process(s0, gbuf_a, fa);
        if (s0 + step >= last) break;
        // the chunk's next tile: data in gbuf_b and fb
        __builtin_amdgcn_s_waitcnt(0x0f70);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (s0 + 2 * step < last) issue(tile + 2 * tstep, gbuf_a, fa);
        process(s0 + step, gbuf_b, fb);
    }

    // ---- finish: full sums per row, then write --------------------------------
    for (int x = rows_p; x < 64; x <<= 1) l_run += __shfl_xor(l_run, x);
    if (sm_g == 0) {
        m_fin[sm_row] = m_run;
        l_fin[sm_row] = l_run;
    }
    wave_lds_sync();
    const int H = G.h, DH = QG * QF;
#pragma unroll
    for (int u = 0; u < NQW; ++u) {
        if (n0 + u >= P.n_q) continue;
        const int64_t row = (int64_t)b * P.n_q + n0 + u;
#pragma unroll
        for (int mb = 0; mb < MB16; ++mb) {
            if (S::GEN && mb * 16 >= M) continue;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int R = mb * 16 + 4 * g16 + c;
                if (R >= M) continue;
                const int iG = R >> G.lqg, jG = R & (QG - 1);
                const int i = G.head(iG0 + iG, iF);
                const float l = l_fin[u * PG + iG];
#pragma unroll
                for (int nb = 0; nb < KC; ++nb) {
                    if (S::K8 && l16 >= 8) continue;  // the zero columns of an 8-wide F
                    const int j = feat<S>(G, jG, 16 * nb + l16);
                    const float v = o_acc[u][mb][nb][c] * P.v_scale;
                    if (P.n_split == 1)
                        P.out[(row * H + i) * DH + j] = l > 0.f ? v / l : 0.f;
                    else
                        P.part_o[((row * P.n_split + split) * H + i) * DH + j] = v;
                }
            }
        }
        if (lane < PG) {
            const int i = G.head(iG0 + lane, iF);
            const float m = m_fin[u * PG + lane], l = l_fin[u * PG + lane];
            if (P.n_split == 1) {
                if (P.lse) P.lse[row * H + i] = l > 0.f ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
            } else {
                float* ml = P.part_ml + ((row * P.n_split + split) * H + i) * 2;
                ml[0] = m;
                ml[1] = l;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
// A matrix-core instantiation: an exact shape (p1, p2, q1, q2, r_k, r_v), or
// a generic family (qf = F feature dimension, rank caps, row cap).
struct MfmaKernel {
    bool generic;
    int p1, p2, q1, q2, r_k, r_v;  // exact shape
    int qf, rkc, rvc, m_max;       // generic family
    bool multi;                    // kernel for n_q > 1
    int queries_per_wave, query_subgroups;
    int waves_max;                 // waves per workgroup the kernel allows
    int fill_pct;                  // percent of the resident-workgroup slots to fill
    hipError_t (*launch)(const DecodeParams&, hipStream_t, const KernelEvents&);
    int (*blocks_per_cu)(const kpa_dims&, int f_is_b);
    int (*lds_bytes)(const kpa_dims&, int f_is_b);
};

template <class C>
struct Entry {
    static int lds(const kpa_dims& d, int fb) {
        if constexpr (C::GEN) return gen_lds<C>(make_geo<C>(d, fb)).total;
        else return 0;
    }
    static int block_threads(const kpa_dims& d, int fb) { return make_geo<C>(d, fb).waves * 64; }
    static hipError_t launch(const DecodeParams& P, hipStream_t s, const KernelEvents& ev) {
        const int qwg = (P.n_q + C::QPW - 1) / C::QPW;
        const int split_pad = (P.n_split + kXcds - 1) / kXcds * kXcds;
        dim3 grid(split_pad * qwg, P.batch);
        const int smem = lds(P.d, P.f_is_b);
        if constexpr (C::GEN) {
            // dynamic LDS above the default limit needs the attribute once
            static std::once_flag once;
            std::call_once(once, [] {
                (void)hipFuncSetAttribute(reinterpret_cast<const void*>(decode_mfma_kernel<C>),
                                          hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
            });
        }
        hipExtLaunchKernelGGL(decode_mfma_kernel<C>, grid, dim3(block_threads(P.d, P.f_is_b)), smem, s, ev.start,
                              ev.stop, 0, P);
        return hipGetLastError();
    }
    // Workgroups of this kernel one CU holds at once (registers and LDS), as
    // the runtime reports it for this launch's block size and LDS.
    static int blocks_per_cu(const kpa_dims& d, int fb) {
        if constexpr (!C::GEN) {
            static std::atomic<int> cached{0};
            int v = cached.load(std::memory_order_relaxed);
            if (v > 0) return v;
            int n = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_mfma_kernel<C>, C::WAVES * 64, 0) !=
                    hipSuccess ||
                n <= 0)
                n = 1;
            cached.store(n, std::memory_order_relaxed);
            return n;
        } else {
            // a few recent (block size, LDS) answers
            static std::mutex mu;
            static int keys[8][2], vals[8], used = 0;
            const int bt = block_threads(d, fb), sm = lds(d, fb);
            std::lock_guard<std::mutex> lock(mu);
            for (int k = 0; k < used; ++k)
                if (keys[k][0] == bt && keys[k][1] == sm) return vals[k];
            int n = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_mfma_kernel<C>, bt, sm) != hipSuccess || n <= 0)
                n = 1;
            const int slot = used < 8 ? used++ : (bt + sm) % 8;
            keys[slot][0] = bt;
            keys[slot][1] = sm;
            vals[slot] = n;
            return n;
        }
    }
};

}  // namespace mfma
}  // namespace kpa

#define KPA_MFMA_ENTRY(p1, p2, q1, q2, rk, rv, multi, ...)                                                        \
    {false, p1, p2, q1, q2, rk, rv, 0, 0, 0, 0, multi, ::kpa::mfma::Cfg<__VA_ARGS__>::NQW_,                       \
     ::kpa::mfma::Cfg<__VA_ARGS__>::NQG_, ::kpa::mfma::Cfg<__VA_ARGS__>::WAVES_MAX,                                 \
     ::kpa::mfma::Cfg<__VA_ARGS__>::FILL_,                                                                          \
     ::kpa::mfma::Entry<::kpa::mfma::Cfg<__VA_ARGS__>>::launch,                                                    \
     ::kpa::mfma::Entry<::kpa::mfma::Cfg<__VA_ARGS__>>::blocks_per_cu,                                             \
     ::kpa::mfma::Entry<::kpa::mfma::Cfg<__VA_ARGS__>>::lds}

// Generic family: QF, rank caps (key, value), row-block cap MB32, queries per
// wave, query subgroups, waves per SIMD, waves per workgroup cap.
#define KPA_MFMA_GENERIC(multi, QF, RKC, RVC, MB32, NQW, NQG, MW, WMAX)                                       \
    {true, 0, 0, 0, 0, 0, 0, QF, RKC, RVC, 32 * (MB32), multi, NQW, NQG, WMAX, 100,                              \
     ::kpa::mfma::Entry<::kpa::mfma::GenCfg<QF, RKC, RVC, MB32, NQW, NQG, MW, WMAX>>::launch,                    \
     ::kpa::mfma::Entry<::kpa::mfma::GenCfg<QF, RKC, RVC, MB32, NQW, NQG, MW, WMAX>>::blocks_per_cu,             \
     ::kpa::mfma::Entry<::kpa::mfma::GenCfg<QF, RKC, RVC, MB32, NQW, NQG, MW, WMAX>>::lds}

namespace kpa {
namespace mfma {
// The instantiation tables (one per translation unit, so they compile in
// parallel; host functions, so the device compilation leaves them out).
const MfmaKernel* exact_kernels(int* count);
const MfmaKernel* generic_kernels_a(int* count);
const MfmaKernel* generic_kernels_b(int* count);
}  // namespace mfma
}  // namespace kpa
