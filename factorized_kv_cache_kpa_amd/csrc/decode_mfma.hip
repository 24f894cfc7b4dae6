// Split-KV decode on the bf16 matrix cores (gfx950 MFMA), one query or a
// causal chunk of queries per sequence.
//
// Math ([KPA] = "Kronecker Product Attention: Memory-Efficient KV Compression
// via Structured Factorization"; [TPA] = "Tensor Product Attention Is All You
// Need", summary page):
//   K_s = (1/R_K) sum_r A^K_r (x) B~^K_r, V_s likewise      ([KPA] Eqs. (3)-(4))
//   z_{i,s} = q'_i . k_{s,i} / sqrt(d_h), q' = R_KPA(q_pos) q  ([KPA] §2.3, Def. 2.3)
// Written with the two factors of a head: call F the factor whose feature
// dimension is contracted on the matrix cores (8, 16, 32 or 64 wide) and G
// the other one.
// Head i = (iG, iF), feature j = (jG, jF) in the block order of the Kronecker
// product ([KPA] Def. 2.1).  Then, per query n, rank r and cached slot s,
//   W_r[(n,iG,jG), s] = sum_jF q'[n,iG,iF,jG,jF] F_r[s,iF,jF]   (MFMA 32x32x16:
//        M = (n,iG,jG), N = 32 slots, K = jF -- the queries are the
//        stationary operand, as a grouped-query decode shares K across heads)
//   z[n,iG,iF,s] = sum_r sum_jG G_r[s,iG,jG] W_r[(n,iG,jG),s]   (VALU, in lane)
// which is [KPA] Prop. 2.2 / Eq. (6) with a dense query: contract with one
// factor, then the other; K is never rebuilt.  The value side, per iF,
//   O[(n,iG,jG), jF] += sum_{r,s} (p[n,iG,iF,s] G^V_r[s,iG,jG]) F^V_r[s,iF,jF]
// is a GEMM over slots (MFMA 16x16x32: M = (iG,jG), N = jF, K = 32 slots),
// with the softmax weight folded into the G factor on the VALU.  The online
// softmax (running max and sum per (query, head), rescaling O when the max
// grows) is the blocked online log-sum-exp of FlashTPA decoding ([TPA]).
//
// Work split: a workgroup owns one KV chunk of one sequence for a group of
// queries; its waves are (iF, query subgroup).  The G factors of a tile are
// shared by every wave of the workgroup: they go HBM -> LDS by direct DMA,
// one tile ahead, double-buffered.  Each wave's F slice goes HBM ->
// registers, one tile ahead.  No cross-wave reduction: the (query, head)
// rows of a wave are its own.  With several query groups per chunk, the
// workgroups of one chunk are placed on the same XCD so the tile is fetched
// from HBM once and shared through that XCD's L2.
//
// Precision: bf16 factors exactly; the rotated, scaled query is split into
// bf16 hi + lo parts (two MFMAs) so it carries ~16 bits; the value operand
// p * G^V is formed in fp32 and rounded once to bf16 (relative 2^-8 per
// term, unbiased); the normaliser sums the fp32 weights; all accumulation is
// fp32.  Because each KV chunk rounds against its own running max, results
// for different chunk counts agree to that bf16 rounding, not bit for bit.
#include <atomic>
#include <type_traits>

#include "kpa_append.hpp"
#include "kpa_common.hpp"
#include "kpa_mfma.hpp"

namespace kpa {
namespace {

constexpr int kXcds = 8;  // workgroups are dealt to the 8 XCDs round-robin

constexpr int pow2_at_least(int x) { return x <= 1 ? 1 : 2 * pow2_at_least((x + 1) / 2); }

template <int PG, int QG, int PF, int QF, int RK, int RV, bool F_IS_B, int NQW, int NQG, int MW>
struct Cfg {
    static constexpr int PG_ = PG, QG_ = QG, PF_ = PF, QF_ = QF, RK_ = RK, RV_ = RV;
    static constexpr bool F_IS_B_ = F_IS_B;
    // Kernels with one query per workgroup serve single-query decode, where a
    // tile's bytes are read once per step: their cache loads carry the
    // nontemporal hint (kpa_32k's kernel: 140 -> 126 us).  The multi-query
    // kernels' query groups share each tile through L2: no hint there (it
    // cost multiq_16 2%).
    static constexpr bool NT_ = NQW * NQG == 1;
    static constexpr int NQW_ = NQW;                 // queries per wave
    static constexpr int NQG_ = NQG;                 // query subgroups per workgroup
    static constexpr int QPW = NQW * NQG;            // queries per workgroup
    static constexpr int WAVES = PF * NQG;
    static constexpr int MIN_WAVES = MW;             // waves per SIMD the registers must allow
    static constexpr int M = PG * QG;                // rows (iG, jG) per query
    static constexpr int MB32 = (M + 31) / 32;       // score MFMA row blocks (rows past M are zero)
    static constexpr int MB16 = (M + 15) / 16;       // value MFMA row blocks
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
    // softmax: NQW*PG (query, head) rows per wave, padded to a power of two,
    // spread over 64 lanes
    static constexpr int ROWS = NQW * PG;
    static constexpr int ROWS_P = pow2_at_least(ROWS);
    static constexpr int GROUPS = 64 / ROWS_P;       // lanes per row
    static constexpr int TPG = 32 / GROUPS;          // slots per lane
    // row stride of the per-wave score scratch, padded so that the softmax's
    // reads (TPG consecutive floats per lane, rows = lane % ROWS_P) fall in
    // distinct LDS banks
    static constexpr int ZS = 32 + (ROWS_P >= 8 ? 4 : ROWS_P == 4 ? 8 : 16);
    static constexpr int QROT = F_IS_B ? QF : QG;    // rotary pairs live in B's feature dim
    // cache sets
    static constexpr int SET_GK = F_IS_B ? 0 : 1;
    static constexpr int SET_FK = F_IS_B ? 1 : 0;
    static constexpr int SET_GV = F_IS_B ? 2 : 3;
    static constexpr int SET_FV = F_IS_B ? 3 : 2;
    static_assert(QF == 8 || QF == 16 || QF == 32 || QF == 64, "the MFMA-side feature dimension must be 8, 16, 32 or 64");
    static_assert(QG == 1 || QG == 2 || QG == 4 || QG == 8 || QG == 16 || QG == 32,
                  "G-side feature dimension 1, 2, 4, 8, 16 or 32");
    static_assert(M % 4 == 0, "rows (iG, jG) come in groups of four");
    static_assert(ROWS_P <= 64 && ROWS_P >= 2, "query-head rows of a wave must fit 64 lanes");
    static_assert(QROT <= 64, "rotary table holds 32 pairs");
    static_assert(RK <= 4 && RV <= 4, "ranks up to 4");
    static_assert(WAVES * 64 <= 1024, "at most 16 waves per workgroup");
    __device__ static int head(int iG, int iF) { return F_IS_B ? iG * PF + iF : iF * PG + iG; }
    __device__ static int feat(int jG, int jF) { return F_IS_B ? jG * QF + jF : jF * QG + jG; }
};

// Per-wave LDS scratch: scores, overwritten in place by the softmax weights.
template <class S>
struct alignas(16) WaveScratch {
    float zp[S::ROWS_P][S::ZS];
    float alpha[S::ROWS_P];
    float m_fin[S::ROWS_P];
    float l_fin[S::ROWS_P];
};

// The G blocks of one tile, HBM -> LDS by DMA: 1 KB blocks of the key set,
// then of the value set, dealt to the waves round-robin.  A set's last block
// may be partial: only lanes inside the set copy.  Value set: 16-byte chunk q
// of element row e lands at chunk q ^ ((e >> 1) & 3) of its 64-byte row, so
// the value phase's reads of 16 rows x 4 chunks hit distinct LDS banks; a
// DMA lane writes a fixed LDS position, so it fetches the chunk that belongs
// there.
template <class S>
__device__ __forceinline__ void dma_g_blocks(const uint8_t* gk, const uint8_t* gv, uint8_t* gdst, int wave, int lane) {
    constexpr int KB = S::GK_BLOCKS, NBLK = S::G_BLOCKS;
#pragma unroll
    for (int k = wave; k < NBLK; k += S::WAVES) {
        const bool key = k < KB;
        const int kb = key ? k : k - KB;
        const int left = (key ? S::GK_BYTES : S::GV_BYTES) - kb * 1024;
        const int vchunk = (lane & ~3) | ((lane & 3) ^ ((lane >> 3) & 3));
        const uint8_t* src = (key ? gk : gv) + kb * 1024 + (key ? lane : vchunk) * 16;
        constexpr bool kWholeBlocks = S::GK_BYTES % 1024 == 0 && S::GV_BYTES % 1024 == 0;
        if (kWholeBlocks || lane * 16 < left) dma_to_lds16<S::NT_>(src, lds_addr(gdst + k * 1024));
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
// lanes of columns 8 .. 15 hold zeros.
template <class S>
struct FRegs {
    bf16x8 fk[S::RK_][S::KC];
    bf16x8 fv[S::RV_][S::KC];
};

// The F slice of wave iF: key-set lane (slot s, half) takes 8 features of
// each 16-feature group (both halves the same 8 when F is 8 wide);
// value-set lane (row l16, slot group g16) takes 8 slots of one feature row.
template <class S>
__device__ __forceinline__ void load_f_regs(const uint8_t* tile, int64_t offFK, int64_t offFV, int iF, int half, int s,
                                            int l16, int g16, FRegs<S>& f) {
    constexpr int PF = S::PF_, QF = S::QF_;
#pragma unroll
    for (int r = 0; r < S::RK_; ++r)
#pragma unroll
        for (int kc = 0; kc < S::KC; ++kc)
            f.fk[r][kc] = ld_f<S>(tile + offFK + (int64_t)((r * PF + iF) * (QF / 8) + (S::K8 ? 0 : 2 * kc + half)) * 512 +
                                  s * 16);
#pragma unroll
    for (int r = 0; r < S::RV_; ++r)
#pragma unroll
        for (int nb = 0; nb < S::KC; ++nb) {
            if (S::K8 && l16 >= 8)
                f.fv[r][nb] = bf16x8{};
            else
                f.fv[r][nb] = ld_f<S>(tile + offFV + ((int64_t)((r * PF + iF) * QF + 16 * nb + l16) * 32 + 8 * g16) * 2);
        }
}

// Query elements (iG, iF, jG, jF0 .. jF0 + 7) of row `row`, unrotated.  Dense:
// two 16-byte loads.  Factored ((1/R_Q) sum_r A^Q_r (x) B^Q_r): per rank one
// element of the G-side factor times 8 consecutive elements of the F-side
// factor -- its feature dimension is the 16-wide one, so the 8 are contiguous.
template <class S>
__device__ __forceinline__ void query_group8(const DecodeParams& P, int64_t row, int iG, int iF, int jG, int jF0,
                                             float* out) {
    if (P.a_q == nullptr) {
        const float* src = P.q + (row * S::H + S::head(iG, iF)) * S::DH;
        if constexpr (S::F_IS_B_) {  // feat(jG, jF) = jG * QF + jF: contiguous in jF
            const f32x4 lo = *reinterpret_cast<const f32x4*>(src + S::feat(jG, jF0));
            const f32x4 hi = *reinterpret_cast<const f32x4*>(src + S::feat(jG, jF0) + 4);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                out[k] = lo[k];
                out[4 + k] = hi[k];
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) out[k] = src[S::feat(jG, jF0 + k)];
        }
        return;
    }
    // F = B: A^Q_r[iG][jG] * B^Q_r[iF][jF];  F = A: A^Q_r[iF][jF] * B^Q_r[iG][jG]
    constexpr int PA = S::F_IS_B_ ? S::PG_ : S::PF_, QA = S::F_IS_B_ ? S::QG_ : S::QF_;
    constexpr int PB = S::F_IS_B_ ? S::PF_ : S::PG_, QB = S::F_IS_B_ ? S::QF_ : S::QG_;
    const float* fs = S::F_IS_B_ ? P.b_q : P.a_q;  // the F side's factor (8 contiguous)
    const float* gs = S::F_IS_B_ ? P.a_q : P.b_q;  // the G side's factor (one element)
    constexpr int F_SET = S::F_IS_B_ ? PB * QB : PA * QA, G_SET = S::F_IS_B_ ? PA * QA : PB * QB;
    const float* f = fs + row * P.r_q * F_SET + iF * S::QF_ + jF0;
    const float* g = gs + row * P.r_q * G_SET + iG * S::QG_ + jG;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int r = 0; r < P.r_q; ++r) {
        const float gv = g[(int64_t)r * G_SET];
        const f32x4 lo = *reinterpret_cast<const f32x4*>(f + (int64_t)r * F_SET);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(f + (int64_t)r * F_SET + 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            acc[k] = fmaf(gv, lo[k], acc[k]);
            acc[4 + k] = fmaf(gv, hi[k], acc[4 + k]);
        }
    }
    const float inv = 1.f / (float)P.r_q;
#pragma unroll
    for (int k = 0; k < 8; ++k) out[k] = acc[k] * inv;
}

template <class S>
__global__ void __launch_bounds__(S::WAVES * 64, S::MIN_WAVES) decode_mfma_kernel(DecodeParams P) {
    constexpr int PG = S::PG_, QG = S::QG_, PF = S::PF_, QF = S::QF_, RK = S::RK_, RV = S::RV_;
    constexpr int M = S::M, MB32 = S::MB32, MB16 = S::MB16, NQW = S::NQW_, KC = S::KC;
    // whole row blocks: the bounds checks on rows vanish at compile time
    constexpr bool kFull32 = M % 32 == 0, kFull16 = M % 16 == 0;
    __shared__ WaveScratch<S> scratch[S::WAVES];
    __shared__ float cs_tab[S::QPW][32][2];
    // two separate LDS objects (not one 2-D array) so the compiler can tell the
    // buffer being filled by DMA from the one being read
    __shared__ __attribute__((aligned(1024))) uint8_t gbuf_a[S::G_BLOCKS * 1024];
    __shared__ __attribute__((aligned(1024))) uint8_t gbuf_b[S::G_BLOCKS * 1024];

    const int lane = threadIdx.x & 63;
    const int wave = S::WAVES == 1 ? 0 : (int)(threadIdx.x >> 6);
    const int iF = wave % PF;
    const int qsub = wave / PF;
    const int half = lane >> 5;
    const int s = lane & 31;       // slot within the tile for the score side
    const int l16 = lane & 15;
    const int g16 = lane >> 4;     // 8-slot group for the value side
    const int b = blockIdx.y;
    // workgroup -> (chunk, query group): the query groups of a chunk share an XCD
    const int qwg_count = (P.n_q + S::QPW - 1) / S::QPW;
    const int bx = blockIdx.x;
    const int split = (bx / (kXcds * qwg_count)) * kXcds + bx % kXcds;
    const int qwg = (bx / kXcds) % qwg_count;
    if (split >= P.n_split) return;  // padding of the grid to a multiple of the XCD count
    WaveScratch<S>& ws = scratch[wave];
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
    // elements (8 contiguous per lane and K step when F = B) and the query
    // positions are requested just before.  Loads complete in order, so the
    // prologue's wait for them need not cover the F loads; it still covers
    // the G blocks, whose inline-asm DMA the compiler's wait counts cannot
    // see.
    FRegs<S> fa, fb;
    constexpr bool kEarly = NQW == 1;
    constexpr bool kQPre = kEarly && S::F_IS_B_;
    f32x4 q_pre[MB32][KC][2];
    int qpos_pre = 0;  // this thread's first rotary angle's query position
    if constexpr (kEarly) {
        const int e = threadIdx.x;
        if (e < S::QPW * (S::QROT / 2))
            qpos_pre = P.q_pos[(int64_t)b * P.n_q + min(qwg * S::QPW + e / (S::QROT / 2), P.n_q - 1)];
    }
    if constexpr (kQPre) {
        if (P.a_q == nullptr) {
            const int64_t qrow = (int64_t)b * P.n_q + min(n0, P.n_q - 1);
#pragma unroll
            for (int mb = 0; mb < MB32; ++mb) {
                const int R = mb * 32 + s;
                const bool row_ok = kFull32 || R < M;
                const int iG = row_ok ? R / QG : 0, jG = row_ok ? R % QG : 0;
                const float* src = P.q + (qrow * S::H + S::head(iG, iF)) * S::DH + S::feat(jG, S::K8 ? 0 : 8 * half);
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    q_pre[mb][kc][0] = *reinterpret_cast<const f32x4*>(src + 16 * kc);
                    q_pre[mb][kc][1] = *reinterpret_cast<const f32x4*>(src + 16 * kc + 4);
                }
            }
        }
    }
    int early_first = 0, early_last = 0;
    if constexpr (kEarly) {
        int vis_e = 0;
        for (int n = qwg * S::QPW; n < min(P.n_q, (qwg + 1) * S::QPW); ++n) vis_e = max(vis_e, visible_slots(P, b, n));
        early_first = split * P.chunk_tiles * kTileSlots;
        early_last = min(early_first + P.chunk_tiles * kTileSlots, vis_e);
        if (early_first < early_last) {
            const uint8_t* tile = P.cache + (int64_t)b * L.n_tiles * L.tile_bytes +
                                  (int64_t)(early_first / kTileSlots) * L.tile_bytes;
            dma_g_blocks<S>(tile + L.off[S::SET_GK], tile + L.off[S::SET_GV], gbuf_a, wave, lane);
            load_f_regs<S>(tile, L.off[S::SET_FK], L.off[S::SET_FV], iF, half, s, l16, g16, fa);
        }
    }

    // ---- rotated, scaled queries as MFMA A operands (hi + lo bf16) ----------
    for (int e = threadIdx.x; e < S::QPW * (S::QROT / 2); e += S::WAVES * 64) {
        const int nq = e / (S::QROT / 2), m = e % (S::QROT / 2);
        const int n = min(qwg * S::QPW + nq, P.n_q - 1);
        const double theta = exp2(-(2.0 * m / S::QROT) * log2((double)P.d.rope_base));
        double sn, c;
        const int qp = kEarly && e == (int)threadIdx.x ? qpos_pre : P.q_pos[(int64_t)b * P.n_q + n];
        sincos((double)qp * theta, &sn, &c);
        cs_tab[nq][m][0] = (float)c;
        cs_tab[nq][m][1] = (float)sn;
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
            const int iG = row_ok ? R / QG : 0, jG = row_ok ? R % QG : 0;
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
                        xs[k] = q_pre[mb][kc][0][k];
                        xs[4 + k] = q_pre[mb][kc][1][k];
                    }
                } else {
                    query_group8<S>(P, qrow, iG, iF, jG, jF0, xs);
                }
                if constexpr (!S::F_IS_B_) query_group8<S>(P, qrow, iG, iF, jG ^ 1, jF0, ys);
                float v[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int jF = jF0 + k;
                    float x, y;  // this element and its rotary partner
                    int m, first;
                    if constexpr (S::F_IS_B_) {
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
                    const float c = cs_tab[nq][m][0], sn = cs_tab[nq][m][1];
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
    // padding rows of the softmax scratch never receive scores: keep them at -inf
    for (int e = lane; e < (S::ROWS_P - S::ROWS) * 32; e += 64) ws.zp[S::ROWS + e / 32][e % 32] = -INFINITY;
    // softmax state for row sm_row = (query u, head iG) of this wave; l is this
    // lane's partial sum over its slots
    const int sm_row = lane % S::ROWS_P, sm_g = lane / S::ROWS_P;
    float m_run = -INFINITY, l_run = 0.f;

    // visible slots: per query (causal), and the workgroup's furthest
    int vis[NQW];
#pragma unroll
    for (int u = 0; u < NQW; ++u) vis[u] = n0 + u < P.n_q ? visible_slots(P, b, n0 + u) : 0;
    int vis_wg = 0;
    for (int n = qwg * S::QPW; n < min(P.n_q, (qwg + 1) * S::QPW); ++n) vis_wg = max(vis_wg, visible_slots(P, b, n));
    const int first = split * P.chunk_tiles * kTileSlots;
    int last = first + P.chunk_tiles * kTileSlots;
    if (last > vis_wg) last = vis_wg;
    const uint8_t* seq = P.cache + (int64_t)b * L.n_tiles * L.tile_bytes;
    const int64_t offFK = L.off[S::SET_FK], offGK = L.off[S::SET_GK];
    const int64_t offFV = L.off[S::SET_FV], offGV = L.off[S::SET_GV];

    // Pipeline, one tile ahead for every byte:
    //  * G factors (shared by the workgroup's waves): HBM -> LDS by direct DMA
    //    (global_load_lds_dwordx4), double-buffered, each wave copying 1 KB
    //    blocks.  The DMA is issued from inline asm so the compiler does not
    //    make every LDS read wait for it; the explicit vmcnt(0) below is the
    //    only wait it needs;
    //  * the wave's own F slice: HBM -> registers, double-buffered.
    // At the top of each tile one wait for everything issued a tile earlier
    // and one barrier (all G blocks landed; the other buffer is free).
    constexpr int KB = S::GK_BLOCKS;
    using FRegs = kpa::FRegs<S>;
    auto load_f = [&](const uint8_t* tile, FRegs& f) {
        load_f_regs<S>(tile, offFK, offFV, iF, half, s, l16, g16, f);
    };
    auto issue = [&](const uint8_t* tile, uint8_t* gdst, FRegs& f) {
        dma_g_blocks<S>(tile + offGK, tile + offGV, gdst, wave, lane);
        load_f(tile, f);
    };

    auto process = [&](int s0, const uint8_t* gcur, FRegs& f) {
        const int valid = min(kTileSlots, last - s0);
        // ---- scores: W = q' F (MFMA), z = sum G W (VALU) --------------------
        // This lane holds rows R = mb*32 + 8a + 4half + b (b = 0..3) of W for slot s.
#pragma unroll
        for (int mb = 0; mb < MB32; ++mb) {
            // [query][a][b]: sums over the rank, per row b (G feature dimension 1:
            // every row is a head), per pair of rows (dimension 2) or already
            // summed over the in-lane jG
            constexpr int ZB = QG == 1 ? 4 : QG == 2 ? 2 : 1;
            float zp[NQW][4][ZB];
#pragma unroll
            for (int u = 0; u < NQW; ++u)
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int bb = 0; bb < ZB; ++bb) zp[u][a][bb] = 0.f;
#pragma unroll
            for (int r = 0; r < RK; ++r) {
                // this lane's G values for its rows, shared by every query
                float g[4][4];
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int R0 = mb * 32 + 8 * a + 4 * half;
                    if (kFull32 || R0 < M) {
                        const int e0 = r * M + R0;  // four consecutive elements in one 16-byte chunk
                        const uint2 gk = *reinterpret_cast<const uint2*>(gcur + (e0 >> 3) * 512 + s * 16 + (e0 & 7) * 2);
                        unpack_bf16x4(gk, g[a][0], g[a][1], g[a][2], g[a][3]);
                    } else {
                        g[a][0] = g[a][1] = g[a][2] = g[a][3] = 0.f;
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
                            for (int bb = 0; bb < 4; ++bb) zp[u][a][bb] += w[a * 4 + bb] * g[a][bb];
                        } else if constexpr (ZB == 2) {
#pragma unroll
                            for (int bb = 0; bb < 4; ++bb)
                                zp[u][a][bb >> 1] = fmaf(w[a * 4 + bb], g[a][bb], zp[u][a][bb >> 1]);
                        } else {
                            // a chain of fused multiply-adds into the running sum
#pragma unroll
                            for (int bb = 0; bb < 4; ++bb) zp[u][a][0] = fmaf(w[a * 4 + bb], g[a][bb], zp[u][a][0]);
                        }
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < NQW; ++u) {
                const bool ok = s0 + s < vis[u] && s < valid;  // causal mask per query
                float* zrow = &ws.zp[u * PG][0];
                if constexpr (ZB == 4) {
                    // every row is a head
#pragma unroll
                    for (int a = 0; a < 4; ++a)
#pragma unroll
                        for (int bb = 0; bb < ZB; ++bb) {
                            const int R = mb * 32 + 8 * a + 4 * half + bb;
                            if (kFull32 || R < M) zrow[R * S::ZS + s] = ok ? zp[u][a][bb] : -INFINITY;
                        }
                } else if constexpr (ZB == 2) {
                    // rows 8a + 4half + 2c + {0, 1} form head mb*16 + 4a + 2half + c
#pragma unroll
                    for (int a = 0; a < 4; ++a)
#pragma unroll
                        for (int c = 0; c < 2; ++c) {
                            const int R = mb * 32 + 8 * a + 4 * half + 2 * c;
                            if (kFull32 || R < M) zrow[(R >> 1) * S::ZS + s] = ok ? zp[u][a][c] : -INFINITY;
                        }
                } else {
                    float z4[4];
#pragma unroll
                    for (int a = 0; a < 4; ++a) z4[a] = zp[u][a][0];
                    if constexpr (QG == 4) {
                        // rows 8a + 4half + b: iG = mb*8 + 2a + half, jG = b -- complete in lane
#pragma unroll
                        for (int a = 0; a < 4; ++a)
                            if (kFull32 || mb * 32 + 8 * a + 4 * half < M) zrow[(mb * 8 + 2 * a + half) * S::ZS + s] = ok ? z4[a] : -INFINITY;
                    } else if constexpr (QG == 8) {
                        // iG = mb*4 + a, jG = 4half + b: add the other half
#pragma unroll
                        for (int a = 0; a < 4; ++a) z4[a] = sum_halves(z4[a]);
                        // selects, not a lane-dependent array index (which would go to scratch)
                        const float za = half ? z4[2] : z4[0];
                        const float zb = half ? z4[3] : z4[1];
                        if (kFull32 || mb * 32 + 16 * half < M) zrow[(mb * 4 + 2 * half + 0) * S::ZS + s] = ok ? za : -INFINITY;
                        if (kFull32 || mb * 32 + 16 * half + 8 < M) zrow[(mb * 4 + 2 * half + 1) * S::ZS + s] = ok ? zb : -INFINITY;
                    } else if constexpr (QG == 16) {
                        // iG = mb*2 + a/2, jG = 8(a%2) + 4half + b
                        float z0 = z4[0] + z4[1], z1 = z4[2] + z4[3];
                        z0 = sum_halves(z0);
                        z1 = sum_halves(z1);
                        if (kFull32 || mb * 32 + 16 * half < M) zrow[(mb * 2 + half) * S::ZS + s] = ok ? (half ? z1 : z0) : -INFINITY;
                    } else {
                        // QG == 32: the whole row block is head mb
                        const float z = sum_halves((z4[0] + z4[1]) + (z4[2] + z4[3]));
                        if (half == 0 && (kFull32 || mb * 32 < M)) zrow[mb * S::ZS + s] = ok ? z : -INFINITY;
                    }
                }
            }
        }
        wave_lds_sync();

        // ---- online softmax for the wave's (query, head) rows -----------------
        {
            float zl[S::TPG];
            float mt = -INFINITY;
#pragma unroll
            for (int t = 0; t < S::TPG; ++t) {
                zl[t] = ws.zp[sm_row][sm_g * S::TPG + t];
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
                ws.zp[sm_row][sm_g * S::TPG + t] = p;
                lsum += p;
            }
            l_run = l_run * alpha + lsum;
            m_run = m_new;
            if (sm_g == 0) ws.alpha[sm_row] = alpha;
        }
        wave_lds_sync();

        // ---- values: O = alpha O + (p G^V) F^V (MFMA over slots) -------------
        const uint8_t* gvbase = gcur + KB * 1024;
        auto values = [&](auto partial_tag) {
            constexpr bool kPartial = decltype(partial_tag)::value;
            if constexpr (kPartial) {
                // slots past the end: zero both operands (the cache may hold NaNs there)
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (8 * g16 + k >= valid)
#pragma unroll
                        for (int r = 0; r < RV; ++r)
#pragma unroll
                            for (int nb = 0; nb < KC; ++nb) f.fv[r][nb][k] = (__bf16)0.f;
            }
#pragma unroll
            for (int mb = 0; mb < MB16; ++mb) {
                const int R_row = mb * 16 + l16;               // row of this lane's A operand
                const bool row_ok = kFull16 || R_row < M;
                const int iG_row = row_ok ? R_row / QG : 0;
                float p[NQW][8];
#pragma unroll
                for (int u = 0; u < NQW; ++u) {
                    // rows of this lane's accumulators: mb*16 + 4*g16 + c
                    if constexpr (QG % 4 == 0) {
                        // the four rows share one head
                        const float a = ws.alpha[u * PG + (mb * 16 + 4 * g16) / QG];
#pragma unroll
                        for (int nb = 0; nb < KC; ++nb)
#pragma unroll
                            for (int c = 0; c < 4; ++c) o_acc[u][mb][nb][c] *= a;
                    } else {
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const int R_out = mb * 16 + 4 * g16 + c;
                            const float a = ws.alpha[u * PG + (kFull16 || R_out < M ? R_out / QG : 0)];
#pragma unroll
                            for (int nb = 0; nb < KC; ++nb) o_acc[u][mb][nb][c] *= a;
                        }
                    }
                    ld_lds32(&ws.zp[u * PG + iG_row][8 * g16], p[u]);
                    if (!row_ok)
#pragma unroll
                        for (int k = 0; k < 8; ++k) p[u][k] = 0.f;
                }
#pragma unroll
                for (int r = 0; r < RV; ++r) {
                    float gvf[8];
                    if (row_ok) {
                        const int e = r * M + R_row;  // element row of the value set
                        unpack_bf16x8(*reinterpret_cast<const bf16x8*>(gvbase + e * 64 + ((g16 ^ ((e >> 1) & 3)) * 16)), gvf);
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
    // the workgroup of the chunk whose slots hold it (past every chunk: the
    // last) before it reads it.  The slot0 value arrives behind the first
    // tile's G blocks (loads complete in order), so workgroups owning no token
    // wait here for what the tile loop's first wait would wait for anyway.
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
            const int owner = j < 0 ? 0 : min(j / span, P.n_split - 1);
            if (owner != split) continue;
            append_token<false>(P.d, L, P.cache_w, P.capacity, P.app, P.dev_status, b, n, threadIdx.x,
                                S::WAVES * 64);
            owned = true;
            if (j >= first && j < first + kTileSlots) in_first = true;
        }
        if (owned) {
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's stores are done
            __syncthreads();                     // ... and every other wave's
            if (in_first && first < last) {
                dma_g_blocks<S>(t0 + offGK, t0 + offGV, gbuf_a, wave, lane);
                load_f(t0, fa);
            }
        }
    }
    for (int s0 = first; s0 < last; s0 += 2 * kTileSlots) {
        // tile s0: data in gbuf_a and fa
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the DMA and loads issued one tile ago
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const uint8_t* tile = seq + (int64_t)(s0 / kTileSlots) * L.tile_bytes;
        if (s0 + kTileSlots < last) issue(tile + L.tile_bytes, gbuf_b, fb);
        process(s0, gbuf_a, fa);
        if (s0 + kTileSlots >= last) break;
        // tile s0 + 32: data in gbuf_b and fb
        __builtin_amdgcn_s_waitcnt(0x0f70);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (s0 + 2 * kTileSlots < last) issue(tile + 2 * L.tile_bytes, gbuf_a, fa);
        process(s0 + kTileSlots, gbuf_b, fb);
    }

    // ---- finish: full sums per row, then write --------------------------------
#pragma unroll
    for (int x = S::ROWS_P; x < 64; x <<= 1) l_run += __shfl_xor(l_run, x);
    if (sm_g == 0) {
        ws.m_fin[sm_row] = m_run;
        ws.l_fin[sm_row] = l_run;
    }
    wave_lds_sync();
    const int H = S::H, DH = S::DH;
#pragma unroll
    for (int u = 0; u < NQW; ++u) {
        if (n0 + u >= P.n_q) continue;
        const int64_t row = (int64_t)b * P.n_q + n0 + u;
#pragma unroll
        for (int mb = 0; mb < MB16; ++mb) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int R = mb * 16 + 4 * g16 + c;
                if (R >= M) continue;
                const int iG = R / QG, jG = R % QG;
                const int i = S::head(iG, iF);
                const float l = ws.l_fin[u * PG + iG];
#pragma unroll
                for (int nb = 0; nb < KC; ++nb) {
                    if (S::K8 && l16 >= 8) continue;  // the zero columns of an 8-wide F
                    const int j = S::feat(jG, 16 * nb + l16);
                    const float v = o_acc[u][mb][nb][c] * P.v_scale;
                    if (P.n_split == 1)
                        P.out[(row * H + i) * DH + j] = l > 0.f ? v / l : 0.f;
                    else
                        P.part_o[((row * P.n_split + split) * H + i) * DH + j] = v;
                }
            }
        }
        if (lane < PG) {
            const int i = S::head(lane, iF);
            const float m = ws.m_fin[u * PG + lane], l = ws.l_fin[u * PG + lane];
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

template <class C>
struct Entry {
    static hipError_t launch(const DecodeParams& P, hipStream_t s, const KernelEvents& ev) {
        const int qwg = (P.n_q + C::QPW - 1) / C::QPW;
        const int split_pad = (P.n_split + kXcds - 1) / kXcds * kXcds;
        dim3 grid(split_pad * qwg, P.batch);
        hipExtLaunchKernelGGL(decode_mfma_kernel<C>, grid, dim3(C::WAVES * 64), 0, s, ev.start, ev.stop, 0, P);
        return hipGetLastError();
    }
    // Workgroups of this kernel one CU holds at once (registers and LDS).
    static int blocks_per_cu() {
        static std::atomic<int> cached{0};
        int v = cached.load(std::memory_order_relaxed);
        if (v > 0) return v;
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_mfma_kernel<C>, C::WAVES * 64, 0) != hipSuccess ||
            n <= 0)
            n = 1;
        cached.store(n, std::memory_order_relaxed);
        return n;
    }
    static constexpr int queries_per_group = C::QPW;
};

struct MfmaKernel {
    int p1, p2, q1, q2, r_k, r_v;
    bool multi;  // kernel for n_q > 1
    hipError_t (*launch)(const DecodeParams&, hipStream_t, const KernelEvents&);
    int (*blocks_per_cu)();
    int queries_per_group;
};

#define KPA_MFMA_ENTRY(p1, p2, q1, q2, rk, rv, multi, ...)                                               \
    {p1, p2, q1, q2, rk, rv, multi, Entry<Cfg<__VA_ARGS__>>::launch, Entry<Cfg<__VA_ARGS__>>::blocks_per_cu, \
     Entry<Cfg<__VA_ARGS__>>::queries_per_group}

// Shapes with a matrix-core instantiation.  Cfg arguments: PG, QG, PF, QF
// (F = the factor with feature dimension 16, 32 or 64: B for the first three
// and the last, A for the two multi-query shapes), R_K, R_V, F is B, queries
// per wave, query subgroups, waves/SIMD.
const MfmaKernel kKernels[] = {
    KPA_MFMA_ENTRY(4, 4, 8, 16, 2, 2, false, 4, 8, 4, 16, 2, 2, true, 1, 1, 3),
    KPA_MFMA_ENTRY(4, 4, 8, 16, 1, 1, false, 4, 8, 4, 16, 1, 1, true, 1, 1, 2),
    KPA_MFMA_ENTRY(8, 4, 8, 16, 2, 4, false, 8, 8, 4, 16, 2, 4, true, 1, 1, 2),
    KPA_MFMA_ENTRY(4, 8, 16, 8, 4, 4, false, 8, 8, 4, 16, 4, 4, false, 1, 1, 1),
    KPA_MFMA_ENTRY(4, 8, 16, 8, 4, 4, true, 8, 8, 4, 16, 4, 4, false, 2, 2, 2),
    // TPA split (A: h x 1, B: 1 x d_h): G = A with feature dimension 1, F = B
    KPA_MFMA_ENTRY(12, 1, 1, 64, 2, 2, false, 12, 1, 1, 64, 2, 2, true, 1, 1, 1),
    // FlashTPA's benchmark shapes: d_h = 64, R_K = R_V = 1, h = 16 / 32 / 48
    KPA_MFMA_ENTRY(16, 1, 1, 64, 1, 1, false, 16, 1, 1, 64, 1, 1, true, 1, 1, 2),
    KPA_MFMA_ENTRY(32, 1, 1, 64, 1, 1, false, 32, 1, 1, 64, 1, 1, true, 1, 1, 2),
    KPA_MFMA_ENTRY(48, 1, 1, 64, 1, 1, false, 48, 1, 1, 64, 1, 1, true, 1, 1, 1),
    // The KPA page's head splits (d1 = d2 = 8, R_K = R_V = 2).  F is the
    // factor with fewer heads (fewer waves, more rows per wave), except for
    // 4 x 5, where four waves per workgroup (F = A) spread evenly over a
    // CU's four SIMDs (five waves: 46% -> 62% of 8 TB/s measured)
    KPA_MFMA_ENTRY(8, 2, 8, 8, 2, 2, false, 8, 8, 2, 8, 2, 2, true, 1, 1, 2),
    KPA_MFMA_ENTRY(4, 4, 8, 8, 2, 2, false, 4, 8, 4, 8, 2, 2, true, 1, 1, 3),
    KPA_MFMA_ENTRY(2, 8, 8, 8, 2, 2, false, 8, 8, 2, 8, 2, 2, false, 1, 1, 2),
    KPA_MFMA_ENTRY(10, 2, 8, 8, 2, 2, false, 10, 8, 2, 8, 2, 2, true, 1, 1, 2),
    KPA_MFMA_ENTRY(4, 5, 8, 8, 2, 2, false, 5, 8, 4, 8, 2, 2, false, 1, 1, 2),
    KPA_MFMA_ENTRY(2, 10, 8, 8, 2, 2, false, 10, 8, 2, 8, 2, 2, false, 1, 1, 2),
    KPA_MFMA_ENTRY(5, 5, 8, 8, 2, 2, false, 5, 8, 5, 8, 2, 2, true, 1, 1, 3),
    KPA_MFMA_ENTRY(6, 2, 8, 8, 2, 2, false, 6, 8, 2, 8, 2, 2, true, 1, 1, 2),
    KPA_MFMA_ENTRY(4, 3, 8, 8, 2, 2, false, 4, 8, 3, 8, 2, 2, true, 1, 1, 3),
    KPA_MFMA_ENTRY(3, 4, 8, 8, 2, 2, false, 4, 8, 3, 8, 2, 2, false, 1, 1, 3),
    KPA_MFMA_ENTRY(2, 6, 8, 8, 2, 2, false, 6, 8, 2, 8, 2, 2, false, 1, 1, 2),
};
#undef KPA_MFMA_ENTRY

const MfmaKernel* find_kernel(const kpa_dims& d, int n_q) {
    if (d.dtype != KPA_BF16) return nullptr;
    const bool multi = n_q > 1;
    for (const MfmaKernel& k : kKernels)
        if (k.multi == multi && k.p1 == d.p1 && k.p2 == d.p2 && k.q1 == d.q1 && k.q2 == d.q2 && k.r_k == d.r_k &&
            k.r_v == d.r_v)
            return &k;
    return nullptr;
}

}  // namespace

bool decode_mfma_supported(const kpa_dims& d, int n_q) { return find_kernel(d, n_q) != nullptr; }

int decode_mfma_blocks_per_cu(const kpa_dims& d, int n_q) {
    const MfmaKernel* k = find_kernel(d, n_q);
    return k ? k->blocks_per_cu() : 1;
}

// Workgroups one KV chunk needs (one per group of queries).
int decode_mfma_query_groups(const kpa_dims& d, int n_q) {
    const MfmaKernel* k = find_kernel(d, n_q);
    return k ? (n_q + k->queries_per_group - 1) / k->queries_per_group : 1;
}

hipError_t launch_decode_mfma(const DecodeParams& P, hipStream_t s, const KernelEvents& ev) {
    const MfmaKernel* k = find_kernel(P.d, P.n_q);
    return k ? k->launch(P, s, ev) : hipErrorInvalidValue;
}

}  // namespace kpa
