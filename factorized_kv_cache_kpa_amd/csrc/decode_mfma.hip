// Single-query split-KV decode on the bf16 matrix cores (gfx950 MFMA).
//
// Math ([KPA] = "Kronecker Product Attention: Memory-Efficient KV Compression
// via Structured Factorization"; [TPA] = "Tensor Product Attention Is All You
// Need", summary page):
//   K_s = (1/R_K) sum_r A^K_r (x) B~^K_r, V_s likewise      ([KPA] Eqs. (3)-(4))
//   z_{i,s} = q'_i . k_{s,i} / sqrt(d_h), q' = R_KPA(q_pos) q  ([KPA] §2.3, Def. 2.3)
// Written with the two factors of a head: call F the factor whose feature
// dimension is 16 (it is contracted on the matrix cores) and G the other one.
// Head i = (iG, iF), feature j = (jG, jF) in the block order of the Kronecker
// product ([KPA] Def. 2.1).  Then, per rank r and cached slot s,
//   W_r[(iG,jG), s] = sum_jF q'[iG,iF,jG,jF] F_r[s,iF,jF]      (MFMA 32x32x16:
//        M = (iG,jG), N = 32 slots, K = jF -- the query is the stationary
//        operand, exactly as a grouped-query decode shares K across heads)
//   z[iG,iF,s] = sum_r sum_jG G_r[s,iG,jG] W_r[(iG,jG),s]       (VALU, in lane)
// which is [KPA] Prop. 2.2 / Eq. (6) with a dense query: contract with one
// factor, then the other; K is never rebuilt.  The value side, per iF,
//   O[(iG,jG), jF] += sum_{r,s} (p[iG,iF,s] G^V_r[s,iG,jG]) F^V_r[s,iF,jF]
// is a GEMM over slots (MFMA 16x16x32: M = (iG,jG), N = jF, K = 32 slots),
// with the softmax weight folded into the G factor on the VALU.  The online
// softmax (running max and sum per head, rescaling O when the max grows) is
// the blocked online log-sum-exp of FlashTPA decoding ([TPA]).
//
// Work split: one wave per (sequence, KV chunk, iF).  The PF waves of a
// workgroup share the G factors through L1; each wave reads only its own F
// slice, so every cache byte crosses HBM once.  No cross-wave reduction: the
// heads (., iF) of a wave are its own.
//
// Precision: bf16 factors exactly; the rotated, scaled query is split into
// bf16 hi + lo parts (two MFMAs) so it carries ~16 bits; the value operand
// p * G^V is formed in fp32 and rounded once to bf16 (relative 2^-9 per
// term, unbiased); the normaliser sums the fp32 weights; all accumulation is
// fp32.  Because each KV chunk rounds against its own running max, results
// for different chunk counts agree to that bf16 rounding, not bit for bit.
#include <atomic>
#include <type_traits>

#include "kpa_common.hpp"
#include "kpa_mfma.hpp"

namespace kpa {
namespace {

template <int PG, int QG, int PF, int QF, int RK, int RV, bool F_IS_B>
struct Shape {
    static constexpr int PG_ = PG, QG_ = QG, PF_ = PF, QF_ = QF;
    static constexpr int M = PG * QG;  // rows (iG, jG)
    static constexpr int MB32 = M / 32;
    static constexpr int MB16 = M / 16;
    static constexpr int H = PG * PF;
    static constexpr int DH = QG * QF;
    // G factors of one tile in 1 KB blocks: key set R_K*M elements in 16-byte
    // chunks (M/8 chunks of 512 B per rank), value set R_V*M elements x 32 slots
    static constexpr int GK_BLOCKS = RK * M * 64 / 1024;
    static constexpr int G_BLOCKS = (RK + RV) * M * 64 / 1024;
    static constexpr int GROUPS = 64 / PG;      // softmax: lanes per head
    static constexpr int TPG = 32 / GROUPS;     // softmax: slots per lane
    // cache sets
    static constexpr int SET_GK = F_IS_B ? 0 : 1;
    static constexpr int SET_FK = F_IS_B ? 1 : 0;
    static constexpr int SET_GV = F_IS_B ? 2 : 3;
    static constexpr int SET_FV = F_IS_B ? 3 : 2;
    static_assert(QF == 16, "the MFMA-side feature dimension must be 16");
    static_assert(M % 32 == 0, "rows (iG, jG) must fill 32-row MFMA blocks");
    static_assert(QG == 4 || QG == 8 || QG == 16, "G-side feature dimension 4, 8 or 16");
    static_assert(64 % PG == 0 && PG >= 2, "PG must divide 64");
    static_assert(RK <= 4 && RV <= 4, "ranks up to 4");
    __device__ static int head(int iG, int iF) { return F_IS_B ? iG * PF + iF : iF * PG + iG; }
    __device__ static int feat(int jG, int jF) { return F_IS_B ? jG * QF + jF : jF * QG + jG; }
};

// Per-wave LDS scratch.
template <class S>
struct alignas(16) WaveScratch {
    float z[S::PG_][32];
    float p[S::PG_][32];
    float alpha[S::PG_];
    float m_fin[S::PG_];
    float l_fin[S::PG_];
};

template <class S>
__global__ void __launch_bounds__(S::PF_ * 64, S::MIN_WAVES) decode_mfma_kernel(DecodeParams P) {
    constexpr int PG = S::PG_, QG = S::QG_, PF = S::PF_, QF = S::QF_, RK = S::RK_, RV = S::RV_;
    constexpr int M = S::M, MB32 = S::MB32, MB16 = S::MB16;
    __shared__ WaveScratch<S> scratch[PF];
    __shared__ float cs_tab[16][2];
    // two separate LDS objects (not one 2-D array) so the compiler can tell the
    // buffer being filled by DMA from the one being read
    __shared__ __attribute__((aligned(1024))) uint8_t gbuf_a[S::G_BLOCKS * 1024];
    __shared__ __attribute__((aligned(1024))) uint8_t gbuf_b[S::G_BLOCKS * 1024];

    const int lane = threadIdx.x & 63;
    const int iF = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int s = lane & 31;       // slot within the tile for the score side
    const int l16 = lane & 15;
    const int g16 = lane >> 4;     // 8-slot group for the value side
    const int split = blockIdx.x, b = blockIdx.y;
    WaveScratch<S>& ws = scratch[iF];
    const Layout& L = P.L;

    // ---- rotated, scaled query as MFMA A operands (hi + lo bf16) ------------
    const int qp = P.q_pos[b];
    constexpr int QROT = S::F_IS_B_ ? QF : QG;  // rotary pairs live in B's feature dim
    if (threadIdx.x < QROT / 2) {
        const double theta = exp2(-(2.0 * threadIdx.x / QROT) * log2((double)P.d.rope_base));
        double sn, c;
        sincos((double)qp * theta, &sn, &c);
        cs_tab[threadIdx.x][0] = (float)c;
        cs_tab[threadIdx.x][1] = (float)sn;
    }
    __syncthreads();
    bf16x8 q_hi[MB32], q_lo[MB32];
    {
        const float* qg = P.q + (int64_t)b * S::H * S::DH;
#pragma unroll
        for (int mb = 0; mb < MB32; ++mb) {
            const int R = mb * 32 + s;
            const int iG = R / QG, jG = R % QG;
            const float* qi = qg + (int64_t)S::head(iG, iF) * S::DH;
            float v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int jF = 8 * half + k;
                float x, y;  // this element and its rotary partner
                int m, first;
                if constexpr (S::F_IS_B_) {
                    x = qi[S::feat(jG, jF)];
                    y = qi[S::feat(jG, jF ^ 1)];
                    m = jF >> 1;
                    first = !(jF & 1);
                } else {
                    x = qi[S::feat(jG, jF)];
                    y = qi[S::feat(jG ^ 1, jF)];
                    m = jG >> 1;
                    first = !(jG & 1);
                }
                const float c = cs_tab[m][0], sn = cs_tab[m][1];
                // (x0, x1) -> (x0 c - x1 s, x0 s + x1 c)
                v[k] = (first ? (x * c - y * sn) : (y * sn + x * c)) * P.q_scale;
            }
            split_bf16x8(v, q_hi[mb], q_lo[mb]);
        }
    }

    f32x4 o_acc[MB16];
#pragma unroll
    for (int k = 0; k < MB16; ++k) o_acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    // softmax state for head (iG = lane % PG, iF); l is this lane's partial sum
    const int sm_iG = lane % PG, sm_g = lane / PG;
    float m_run = -INFINITY, l_run = 0.f;

    clear_merge_counters(P, b, split);
    const int vis = visible_slots(P, b, 0);
    const int first = split * P.chunk_tiles * kTileSlots;
    int last = first + P.chunk_tiles * kTileSlots;
    if (last > vis) last = vis;
    const uint8_t* seq = P.cache + (int64_t)b * L.n_tiles * L.tile_bytes;
    const int64_t offFK = L.off[S::SET_FK], offGK = L.off[S::SET_GK];
    const int64_t offFV = L.off[S::SET_FV], offGV = L.off[S::SET_GV];

    // Pipeline, one tile ahead for every byte:
    //  * G factors (shared by the PF waves): HBM -> LDS by direct DMA
    //    (global_load_lds_dwordx4), double-buffered, each wave copying 1 KB
    //    blocks.  The DMA is issued from inline asm so the compiler does not
    //    make every LDS read wait for it; the explicit vmcnt(0) below is the
    //    only wait it needs;
    //  * the wave's own F slice: HBM -> registers, double-buffered.
    // At the top of each tile one wait for everything issued a tile earlier
    // and one barrier (all G blocks landed; the other buffer is free).
    constexpr int KB = S::GK_BLOCKS, NBLK = S::G_BLOCKS;
    struct FRegs {
        bf16x8 fk[RK];
        bf16x8 fv[RV];
    };
    auto issue = [&](const uint8_t* tile, uint8_t* gdst, FRegs& f) {
#pragma unroll
        for (int k = iF; k < NBLK; k += PF) {
            const uint8_t* src = k < KB ? tile + offGK + k * 1024 : tile + offGV + (k - KB) * 1024;
            dma_to_lds16(src + lane * 16, lds_addr(gdst + k * 1024));
        }
#pragma unroll
        for (int r = 0; r < RK; ++r)
            f.fk[r] = ld16<bf16x8>(tile + offFK + (int64_t)((r * PF + iF) * (QF / 8) + half) * 512 + s * 16);
#pragma unroll
        for (int r = 0; r < RV; ++r)
            f.fv[r] = ld16<bf16x8>(tile + offFV + ((int64_t)((r * PF + iF) * QF + l16) * 32 + 8 * g16) * 2);
    };

    auto process = [&](int s0, const uint8_t* gcur, FRegs& f) {
        const int valid = min(kTileSlots, last - s0);
        // ---- scores: W = q' F (MFMA), z = sum G W (VALU) --------------------
#pragma unroll
        for (int mb = 0; mb < MB32; ++mb) {
            float zp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < RK; ++r) {
                f32x16 w = f32x16{};
                w = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q_hi[mb], f.fk[r], w, 0, 0, 0);
                w = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q_lo[mb], f.fk[r], w, 0, 0, 0);
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const uint2 gk = *reinterpret_cast<const uint2*>(gcur + (r * (M / 8) + mb * 4 + a) * 512 + s * 16 + half * 8);
                    float g0, g1, g2, g3;
                    unpack_bf16x4(gk, g0, g1, g2, g3);
                    zp[a] += w[a * 4 + 0] * g0 + w[a * 4 + 1] * g1 + w[a * 4 + 2] * g2 + w[a * 4 + 3] * g3;
                }
            }
            const bool ok = s < valid;
            if constexpr (QG == 4) {
                // rows 8a + 4half + b: iG = mb*8 + 2a + half, jG = b -- complete in lane
#pragma unroll
                for (int a = 0; a < 4; ++a) ws.z[mb * 8 + 2 * a + half][s] = ok ? zp[a] : -INFINITY;
            } else if constexpr (QG == 8) {
                // iG = mb*4 + a, jG = 4half + b: add the other half
#pragma unroll
                for (int a = 0; a < 4; ++a) zp[a] = sum_halves(zp[a]);
                // selects, not a lane-dependent array index (which would go to scratch)
                const float za = half ? zp[2] : zp[0];
                const float zb = half ? zp[3] : zp[1];
                ws.z[mb * 4 + 2 * half + 0][s] = ok ? za : -INFINITY;
                ws.z[mb * 4 + 2 * half + 1][s] = ok ? zb : -INFINITY;
            } else {
                // QG == 16: iG = mb*2 + a/2, jG = 8(a%2) + 4half + b
                float z0 = zp[0] + zp[1], z1 = zp[2] + zp[3];
                z0 = sum_halves(z0);
                z1 = sum_halves(z1);
                ws.z[mb * 2 + half][s] = ok ? (half ? z1 : z0) : -INFINITY;
            }
        }
        wave_lds_sync();

        // ---- online softmax for the wave's PG heads --------------------------
        {
            float zl[S::TPG];
            float mt = -INFINITY;
#pragma unroll
            for (int u = 0; u < S::TPG; ++u) {
                zl[u] = ws.z[sm_iG][sm_g * S::TPG + u];
                mt = fmaxf(mt, zl[u]);
            }
#pragma unroll
            for (int x = PG; x < 64; x <<= 1) mt = fmaxf(mt, __shfl_xor(mt, x));
            const float m_new = fmaxf(m_run, mt);
            // with no slot seen yet (m = -inf) every weight is 0 and alpha 1
            const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_ref);
            float lsum = 0.f;
#pragma unroll
            for (int u = 0; u < S::TPG; ++u) {
                const float p = fast_exp2(zl[u] - m_ref);  // masked slots: 2^-inf = 0
                ws.p[sm_iG][sm_g * S::TPG + u] = p;
                lsum += p;
            }
            l_run = l_run * alpha + lsum;
            m_run = m_new;
            if (sm_g == 0) ws.alpha[sm_iG] = alpha;
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
                        for (int r = 0; r < RV; ++r) f.fv[r][k] = (__bf16)0.f;
            }
#pragma unroll
            for (int mb = 0; mb < MB16; ++mb) {
                const int iG_out = (mb * 16 + 4 * g16) / QG;  // rows of this lane's accumulator
                o_acc[mb] *= ws.alpha[iG_out];
                const int iG_row = (mb * 16 + l16) / QG;      // row of this lane's A operand
                float p[8];
                ld_lds32(&ws.p[iG_row][8 * g16], p);
#pragma unroll
                for (int r = 0; r < RV; ++r) {
                    float gvf[8];
                    unpack_bf16x8(*reinterpret_cast<const bf16x8*>(gvbase + ((r * M + mb * 16 + l16) * 32 + 8 * g16) * 2), gvf);
                    float prod[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        prod[k] = p[k] * gvf[k];
                        if constexpr (kPartial) prod[k] = (8 * g16 + k >= valid) ? 0.f : prod[k];
                    }
                    o_acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pack_bf16x8(prod), f.fv[r], o_acc[mb], 0, 0, 0);
                }
            }
        };
        if (valid < kTileSlots) values(std::true_type{});
        else values(std::false_type{});
    };

    FRegs fa, fb;
    const uint8_t* t0 = seq + (int64_t)(first / kTileSlots) * L.tile_bytes;
    if (first < last) issue(t0, gbuf_a, fa);
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

    // ---- finish: full sums per head, then write -----------------------------
#pragma unroll
    for (int x = PG; x < 64; x <<= 1) l_run += __shfl_xor(l_run, x);
    if (sm_g == 0) {
        ws.m_fin[sm_iG] = m_run;
        ws.l_fin[sm_iG] = l_run;
    }
    wave_lds_sync();
    const int64_t row = b;  // single query
    const int H = S::H, DH = S::DH;
#pragma unroll
    for (int mb = 0; mb < MB16; ++mb) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int R = mb * 16 + 4 * g16 + c;
            const int iG = R / QG, jG = R % QG;
            const int i = S::head(iG, iF), j = S::feat(jG, l16);
            const float v = o_acc[mb][c] * P.v_scale;
            if (P.n_split == 1) {
                const float l = ws.l_fin[iG];
                P.out[(row * H + i) * DH + j] = l > 0.f ? v / l : 0.f;
            } else {
                P.part_o[((row * P.n_split + split) * H + i) * DH + j] = v;
            }
        }
    }
    if (lane < PG) {
        const int i = S::head(lane, iF);
        const float m = ws.m_fin[lane], l = ws.l_fin[lane];
        if (P.n_split == 1) {
            if (P.lse) P.lse[row * H + i] = l > 0.f ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
        } else {
            float* ml = P.part_ml + ((row * P.n_split + split) * H + i) * 2;
            ml[0] = m;
            ml[1] = l;
        }
    }
}

template <int PG, int QG, int PF, int QF, int RK, int RV, bool F_IS_B, int MW = 2>
struct Cfg : Shape<PG, QG, PF, QF, RK, RV, F_IS_B> {
    static constexpr int RK_ = RK, RV_ = RV;
    static constexpr bool F_IS_B_ = F_IS_B;
    static constexpr int MIN_WAVES = MW;  // waves per SIMD the register budget must allow
};

template <class C>
struct Entry {
    static hipError_t launch(const DecodeParams& P, hipStream_t s) {
        dim3 grid(P.n_split, P.batch);
        hipLaunchKernelGGL(decode_mfma_kernel<C>, grid, dim3(C::PF_ * 64), 0, s, P);
        return hipGetLastError();
    }
    // Workgroups of this kernel one CU holds at once (registers and LDS).
    static int blocks_per_cu() {
        static std::atomic<int> cached{0};
        int v = cached.load(std::memory_order_relaxed);
        if (v > 0) return v;
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_mfma_kernel<C>, C::PF_ * 64, 0) != hipSuccess ||
            n <= 0)
            n = 1;
        cached.store(n, std::memory_order_relaxed);
        return n;
    }
};

struct MfmaKernel {
    int p1, p2, q1, q2, r_k, r_v;
    hipError_t (*launch)(const DecodeParams&, hipStream_t);
    int (*blocks_per_cu)();
};

// Shapes with a matrix-core instantiation.  F is the factor whose feature
// dimension is 16 (B for the first three, A for the last).
const MfmaKernel kKernels[] = {
    {4, 4, 8, 16, 2, 2, Entry<Cfg<4, 8, 4, 16, 2, 2, true, 3>>::launch, Entry<Cfg<4, 8, 4, 16, 2, 2, true, 3>>::blocks_per_cu},
    {4, 4, 8, 16, 1, 1, Entry<Cfg<4, 8, 4, 16, 1, 1, true>>::launch, Entry<Cfg<4, 8, 4, 16, 1, 1, true>>::blocks_per_cu},
    {8, 4, 8, 16, 2, 4, Entry<Cfg<8, 8, 4, 16, 2, 4, true>>::launch, Entry<Cfg<8, 8, 4, 16, 2, 4, true>>::blocks_per_cu},
    {4, 8, 16, 8, 4, 4, Entry<Cfg<8, 8, 4, 16, 4, 4, false, 1>>::launch,
     Entry<Cfg<8, 8, 4, 16, 4, 4, false, 1>>::blocks_per_cu},
};

const MfmaKernel* find_kernel(const kpa_dims& d, int n_q) {
    if (d.dtype != KPA_BF16 || n_q != 1) return nullptr;
    for (const MfmaKernel& k : kKernels)
        if (k.p1 == d.p1 && k.p2 == d.p2 && k.q1 == d.q1 && k.q2 == d.q2 && k.r_k == d.r_k && k.r_v == d.r_v)
            return &k;
    return nullptr;
}

}  // namespace

bool decode_mfma_supported(const kpa_dims& d, int n_q) { return find_kernel(d, n_q) != nullptr; }

int decode_mfma_blocks_per_cu(const kpa_dims& d) {
    const MfmaKernel* k = find_kernel(d, 1);
    return k ? k->blocks_per_cu() : 1;
}

hipError_t launch_decode_mfma(const DecodeParams& P, hipStream_t s) {
    const MfmaKernel* k = find_kernel(P.d, P.n_q);
    return k ? k->launch(P, s) : hipErrorInvalidValue;
}

}  // namespace kpa
