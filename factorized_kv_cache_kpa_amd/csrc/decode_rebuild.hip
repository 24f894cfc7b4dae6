// Multi-query split-KV decode with the keys and values rebuilt per tile on
// the matrix cores, then plain attention on the matrix cores.
//
// Math ([KPA] = "Kronecker Product Attention: Memory-Efficient KV Compression
// via Structured Factorization"):
//   K_s = (1/R_K) sum_r A^K_r (x) B~^K_r,  V_s = (1/R_V) sum_r A^V_r (x) B^V_r
//                                                         ([KPA] Eqs. (3)-(4))
//   z_{n,i,s} = q'_{n,i} . K_s[i, :] / sqrt(d_h),  q' = R_KPA(q_pos) q
//                                                         ([KPA] §2.3, Def. 2.3)
// Element (i, j) of K_s, head i = (i1, i2), feature j = (j1, j2) in the
// Kronecker block order ([KPA] Def. 2.1), is sum_r A_r[i1, j1] B~_r[i2, j2]:
// for one cached token and one head a sum of R outer products, i.e. a tiny
// matrix product with the rank as its inner dimension.  With a chunk of
// n_q = 16 queries every rebuilt row serves all 16 of them, so rebuilding
// costs R h d_h products per token -- R h d_h / 16 per (query, token), the
// same count as the factor-space score's second contraction -- but these
// products run on the matrix cores (v_mfma_f32_4x4x4_16b_bf16: 16 blocks of
// 4 x 4 outputs with inner dimension 4 = the ranks, one block per token),
// which leaves the vector ALUs only conversions and the softmax.
//
// Per workgroup: one KV chunk of one sequence, one head group (one A head i1,
// every B head i2) and up to 16 queries; two waves per B head, each taking
// 16 of every tile's 32 slots (so a CU runs 16 waves, 4 per SIMD).  Per
// 32-slot tile:
//   1. The tile's factors go HBM -> registers (one tile ahead) -> LDS with
//      their ranks interleaved: element (slot, row, feature) -> 4 ranks in
//      8 bytes, so each operand of a rebuild MFMA is one 8-byte LDS read.
//      Double-buffered: one barrier per tile.
//   2. Keys: 8 rebuild MFMAs per wave give K[16 slots][128 features] of its
//      head in float32, rounded to bf16.  A rebuild lane holds its slot's
//      features in registers as the score MFMA needs them, but at a lane
//      index rotated by two bits; one ds_bpermute per register moves them.
//   3. Scores: MFMA 16x16x32 with M = 16 slots, N = 16 queries, K = 32
//      features; the query (rotated, scaled) rounded to bf16.  The result
//      holds a query per lane (lane % 16) and its slots in registers and
//      lane bits 4-5 -- exactly the B operand layout of the 16x16x16 value
//      MFMA, so the softmax weights need no data movement.
//   4. Online softmax per (query, head, wave): the running max is shared by
//      a query's four lanes (two lane swaps); it moves only when a score
//      exceeds it by more than 2^8, so the output is rarely rescaled.
//   5. Values: 8 rebuild MFMAs per wave whose outputs already sit in the
//      operand layout of the value MFMA (slots on the inner dimension: rebuild
//      u of 4 covers slot 4 (lane >> 4) + u), then O^T[feature][query] +=
//      V^T P^T, MFMA 16x16x16, eight per tile (one per j2).
//   The running output O^T keeps a query per lane (lane % 16), so the rescale
//   by the softmax correction is a plain multiply.  At the end of the chunk
//   the second wave of each head hands its (m, l, O) to the first through
//   LDS, which combines them as the split-KV merge does.
// The online softmax and the chunk partials (m, l, o) are those of the other
// decode kernels (the blocked online log-sum-exp of FlashTPA decoding,
// "Tensor Product Attention Is All You Need", summary page), merged by the
// same merge kernel.
//
// Shapes: bf16 caches with A's feature dimension q1 = 16 (j1: a lane's 16
// columns) and B's q2 = 8 (j2: 8 consecutive features, the rotary pairs),
// ranks up to 4 (missing ranks are zero rows of the inner dimension), B head
// count p2 = 2, 4, 6 or 8 (two waves each), any A head count p1 (one
// workgroup each), up to 16 queries per workgroup (more queries: more
// workgroups per chunk).  Swapped (SW): q1 = 8, q2 = 16 with p1 = 8 (the
// kernel's 16-wave layout; long_512k's split).  B (x) A is A (x) B with
// heads and features permuted, so the
// kernel runs with the cache's B factors in the A role and its A factors
// in the B role: head (i1, i2) is the kernel's (i2, i1) and feature
// (j1, j2) its (j2, j1).  Only the query's rotary pairs (now along the
// kernel's 16-wide dimension) and the addresses of the query, the output
// and the factor sets change.
//
// Precision: bf16 factors exactly; the rebuilt K and V rows, the rotated
// query and the softmax weights are each rounded once to bf16 (relative 2^-8
// per element at most, unbiased); all sums in float32.
#include <atomic>

#include "kpa_common.hpp"
#include "kpa_mfma.hpp"

namespace kpa {
namespace rebuild {

typedef __attribute__((ext_vector_type(4))) short s16x4;  // 4 bf16: a 4x4x4 MFMA operand

constexpr int kXcds = 8;
constexpr int kNQ = 16;                   // queries per workgroup
constexpr int kQ1 = 16, kQ2 = 8;          // feature dims of A (j1) and B (j2)
constexpr int kDH = kQ1 * kQ2;
constexpr float kSlack = 8.f;          // log2 units the weights may exceed 1 by before a rescale

// LDS layout (bytes) for P2 B heads.
template <int P2>
struct Lds {
    // Rank-interleaved tile: 8 bytes (4 ranks) per (slot, row, feature);
    // offsets inside one of the two tile buffers.
    // Key sets: a row per slot holding its features (the key rebuild reads
    // the rows of 16 slots per instruction), padded by 32 bytes.
    static constexpr int A_ROW = kQ1 * 8 + 32;         // A^K of the group's A head
    static constexpr int B_ROW = P2 * kQ2 * 8 + 32;    // B~^K of every B head
    // value sets: a row per element holding its 32 slots (the value rebuild
    // reads two consecutive slots at once); 272 B rows put the 16 rows one
    // read instruction touches on distinct banks
    static constexpr int V_ROW = kTileSlots * 8 + 16;
    static constexpr int AK = 0;
    static constexpr int BK = AK + kTileSlots * A_ROW;
    static constexpr int AV = BK + kTileSlots * B_ROW;   // [j1][slot]
    static constexpr int BV = AV + kQ1 * V_ROW;          // [i2 q2 + j2][slot]
    static constexpr int TILE = BV + P2 * kQ2 * V_ROW;
    // two tile buffers and the rotary cos/sin [16 queries][up to 8 pairs][2]
    static constexpr int TOTAL = 2 * TILE + kNQ * 8 * 2 * 4;
    static_assert(TOTAL <= 160 * 1024, "LDS of one CU");
};

// bf16 of two floats in one dword (low half = first), round to nearest even.
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Dword of two bf16: element h of x (low half), element h of y (high half),
// h = 0 (low halves) or 1 (high halves).
__device__ __forceinline__ uint32_t pair_lo(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x07060302u); }

// The value of lane l ^ 16 / l ^ 32.
__device__ __forceinline__ float other16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return (threadIdx.x & 16) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}
__device__ __forceinline__ float other32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

template <int P2>
struct Cfg {
    static constexpr int WAVES = 2 * P2;  // two per B head: slots 0-15 and 16-31 of each tile
    static constexpr int THREADS = WAVES * 64;
    // staging units of one tile (64 B of LDS each, from 4 x 16 B of cache):
    // B~^K (slot, i2), B^V (i2, j2, 8-slot group), A^K (slot, 8-feature
    // half), A^V (j1, 8-slot group)
    static constexpr int U_BK = kTileSlots * P2, U_BV = P2 * kQ2 * 4, U_AK = kTileSlots * 2, U_AV = kQ1 * 4;
    static constexpr int UNITS = U_BK + U_BV + U_AK + U_AV;
    static constexpr int UPT = (UNITS + THREADS - 1) / THREADS;  // units per thread
    // kinds of unit start at multiples of 64 (one kind per wave): P2 even
    static_assert(P2 >= 2 && P2 <= 8 && P2 % 2 == 0, "two waves per B head: P2 = 2, 4, 6 or 8");
    static_assert(UPT == 1, "one staging unit per thread");
};

// This thread's staging units of a tile: for each, the four 16-byte source
// chunks (one per rank, consecutive ranks a fixed stride apart; zero for
// ranks past R) and where their 64 interleaved bytes go in LDS.  A unit's
// kind is the same across a wave (kinds start at multiples of 64 units).
template <int P2, bool SW>
struct Stage {
    using C = Cfg<P2>;
    // the cache's factor sets in the kernel's roles (A^K, B~^K, A^V, B^V)
    static constexpr int kSetAK = SW ? 1 : 0, kSetBK = SW ? 0 : 1, kSetAV = SW ? 3 : 2, kSetBV = SW ? 2 : 3;
    enum { kBK = 0, kBV = 1, kAK = 2, kAV = 3, kNone = 4 };
    u32x4 v[C::UPT][4];
    uint32_t src[C::UPT];  // byte offset of rank 0 in the tile
    uint32_t dst[C::UPT];  // LDS byte offset
    int slot[C::UPT];      // the unit's slot (keys) or first of its 8 slots (values)
    int kind[C::UPT];      // wave-uniform

    __device__ __forceinline__ void init(const Layout& L, int i1, int p1) {
        using LY = Lds<P2>;
#pragma unroll
        for (int k = 0; k < C::UPT; ++k) {
            const int u = (int)threadIdx.x + k * C::THREADS;
            int kd;
            if (u < C::U_BK) {  // B~^K chunk (r P2 + i2) of slot s
                const int s = u % kTileSlots, i2 = u / kTileSlots;
                kd = kBK;
                slot[k] = s;
                src[k] = (uint32_t)(L.off[kSetBK] + i2 * (kTileSlots * 16) + s * 16);
                dst[k] = LY::BK + s * LY::B_ROW + i2 * 64;
            } else if (u < C::U_BK + C::U_BV) {  // B^V element (r P2 + i2) q2 + j2, 8 slots
                const int x = u - C::U_BK;
                const int sg = x & 3, e = x >> 2;
                kd = kBV;
                slot[k] = 8 * sg;
                src[k] = (uint32_t)(L.off[kSetBV] + e * 64 + sg * 16);
                dst[k] = LY::BV + e * LY::V_ROW + 64 * sg;
            } else if (u < C::U_BK + C::U_BV + C::U_AK) {  // A^K chunk (r p1 + i1) 2 + hf of slot s
                const int x = u - C::U_BK - C::U_BV;
                const int s = x % kTileSlots, hf = x / kTileSlots;
                kd = kAK;
                slot[k] = s;
                src[k] = (uint32_t)(L.off[kSetAK] + (i1 * 2 + hf) * (kTileSlots * 16) + s * 16);
                dst[k] = LY::AK + s * LY::A_ROW + hf * 64;
            } else if (u < C::UNITS) {  // A^V element (r p1 + i1) q1 + j1, 8 slots
                const int x = u - C::U_BK - C::U_BV - C::U_AK;
                const int sg = x & 3, j1 = x >> 2;
                kd = kAV;
                slot[k] = 8 * sg;
                src[k] = (uint32_t)(L.off[kSetAV] + (i1 * kQ1 + j1) * 64 + sg * 16);
                dst[k] = LY::AV + j1 * LY::V_ROW + 64 * sg;
            } else {
                kd = kNone;
                slot[k] = 0;
                src[k] = 0;
                dst[k] = 0;
            }
            kind[k] = __builtin_amdgcn_readfirstlane(kd);
        }
    }

    // Issue the loads of one tile for this thread's units.  Rank r of a unit
    // is r * stride bytes after rank 0: P2 chunks (B~^K), P2 q2 elements
    // (B^V), 2 p1 chunks (A^K), p1 q1 elements (A^V).  Ranks past the key or
    // value rank count re-read rank 0 (branch-free, so the loads issue back
    // to back); store() writes zeros for them.
    __device__ __forceinline__ void load(const uint8_t* tile, int p1, int rk, int rv) {
#pragma unroll
        for (int k = 0; k < C::UPT; ++k) {
            const int kd = kind[k];
            if (kd == kNone) continue;
            const bool key = kd == kBK || kd == kAK;
            const int nr = key ? rk : rv;
            const uint32_t stride = kd == kBK ? P2 * (kTileSlots * 16)
                                    : kd == kBV ? P2 * kQ2 * 64
                                    : kd == kAK ? 2 * p1 * (kTileSlots * 16)
                                                : p1 * kQ1 * 64;
            const uint8_t* p = tile + src[k];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[k][r] = ld16<u32x4>(p + (r < nr ? r : 0) * stride);
        }
    }

    // Write the loaded units into LDS with the ranks interleaved.
    // Slots at or past `valid` (slot index inside the tile; tail tiles only)
    // are written as zeros: they lie past every query's context and may
    // hold arbitrary bytes, and a zero softmax weight times a NaN value
    // would still poison the value sums.
    __device__ __forceinline__ void store(uint8_t* lds, int rk, int rv, bool tail, int valid) {
#pragma unroll
        for (int k = 0; k < C::UPT; ++k) {
            const int kd = kind[k];
            if (kd == kNone) continue;
            const bool key = kd == kBK || kd == kAK;
            const int nr = key ? rk : rv;
#pragma unroll
            for (int r = 1; r < 4; ++r)
                if (r >= nr) v[k][r] = u32x4{0u, 0u, 0u, 0u};
            if (tail) {
                u32x4 keep;
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    keep[d] = key ? (slot[k] < valid ? 0xffffffffu : 0u)
                                  : ((slot[k] + 2 * d < valid ? 0x0000ffffu : 0u) |
                                     (slot[k] + 2 * d + 1 < valid ? 0xffff0000u : 0u));
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int d = 0; d < 4; ++d) v[k][r][d] &= keep[d];
            }
            // o[d]: items 2d and 2d + 1 (j = element or slot 0..7 of the
            // chunks), each as ranks (0, 1) then (2, 3)
            u32x4 o[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                o[d][0] = pair_lo(v[k][0][d], v[k][1][d]);
                o[d][1] = pair_lo(v[k][2][d], v[k][3][d]);
                o[d][2] = pair_hi(v[k][0][d], v[k][1][d]);
                o[d][3] = pair_hi(v[k][2][d], v[k][3][d]);
            }
            uint8_t* out = lds + dst[k];
            // items = 8 consecutive features of a slot (key sets) or 8
            // consecutive slots of an element (value sets): 64 contiguous bytes
#pragma unroll
            for (int d = 0; d < 4; ++d) *reinterpret_cast<u32x4*>(out + 16 * d) = o[d];
        }
    }
};

__device__ __forceinline__ s16x4 lds8(const uint8_t* p) {
    return __builtin_bit_cast(s16x4, *reinterpret_cast<const uint2*>(p));
}

template <int P2, bool SW>
__global__ void __launch_bounds__(2 * P2 * 64, 1) decode_rebuild_kernel(DecodeParams P) {
    using LY = Lds<P2>;
    constexpr int NP = SW ? kQ1 / 2 : kQ2 / 2;  // rotary pairs along the kernel's A (SW) or B features
    // separate LDS objects, so that the compiler can tell the rebuilt keys
    // (written per tile) from the tile factors (read around those writes)
    __shared__ __attribute__((aligned(16))) uint8_t tiles[2 * LY::TILE];
    __shared__ float cs[kNQ * NP * 2];
    const int lane = threadIdx.x & 63;
    const int wave = (int)(threadIdx.x >> 6);
    const int i2 = wave % P2;   // this wave's B head
    const int hh = wave / P2;   // and its half of every tile: slots 16 hh .. 16 hh + 15
    const int p1 = SW ? P.d.p2 : P.d.p1;  // the kernel's A heads: one workgroup each
    const int H = p1 * P2;
    // workgroup -> (chunk, A head): the head groups (and query groups) of a
    // chunk share an XCD, so the B factors they all read come from HBM once;
    // chunk k of sequence b goes to XCD (b n_split + k) mod 8, so the grid's
    // padding (n_split not a multiple of 8) spreads over the XCDs
    const int bx = blockIdx.x;
    const int b = blockIdx.y;
    const int xcd_off = (int)(((int64_t)b * P.n_split) % kXcds);
    const int split = (bx / (kXcds * p1)) * kXcds + (bx % kXcds - xcd_off + kXcds) % kXcds;
    const int i1 = (bx / kXcds) % p1;
    const int qg = blockIdx.z;  // group of 16 queries
    if (split >= P.n_split) return;
    const Layout& L = P.L;
    const int head = SW ? i2 * p1 + i1 : i1 * P2 + i2;  // in the cache's head order

    // queries of this workgroup: n = 16 qg + (lane & 15)
    const int ql = lane & 15;
    const int n = qg * kNQ + ql;
    const bool q_ok = n < P.n_q;
    const int vis = q_ok ? visible_slots(P, b, n) : 0;
    int vis_max = 0;
    for (int k = 0; k < kNQ && qg * kNQ + k < P.n_q; ++k) vis_max = max(vis_max, visible_slots(P, b, qg * kNQ + k));
    const int first = split * P.chunk_tiles * kTileSlots;
    const int last = min(first + P.chunk_tiles * kTileSlots, vis_max);
    const uint8_t* seq = P.cache + (int64_t)b * L.n_tiles * L.tile_bytes;

    Stage<P2, SW> stage;
    stage.init(L, i1, p1);
    if (first < last) stage.load(seq + (int64_t)(first / kTileSlots) * L.tile_bytes, p1, P.d.r_k, P.d.r_v);

    // ---- rotated, scaled query as the score MFMA's B operand (bf16) --------
    if (threadIdx.x < kNQ * NP) {
        const int nq = threadIdx.x / NP, m = threadIdx.x % NP;
        const int nn = min(qg * kNQ + nq, P.n_q - 1);
        const double theta = exp2(-(2.0 * m / (2 * NP)) * log2((double)P.d.rope_base));
        double sn, c;
        sincos((double)P.q_pos[(int64_t)b * P.n_q + nn] * theta, &sn, &c);
        cs[(nq * NP + m) * 2] = (float)c;
        cs[(nq * NP + m) * 2 + 1] = (float)sn;
    }
    if (i1 == 0)
        for (int k = 0; k < kNQ; ++k)
            if (qg * kNQ + k < P.n_q) clear_merge_counters(P, (int64_t)b * P.n_q + qg * kNQ + k, split);
    __syncthreads();
    bf16x8 q_hi[4];
    {
        const int64_t row = (int64_t)b * P.n_q + min(n, P.n_q - 1);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int j1 = 4 * ks + (lane >> 4);
            float x[8];
            float v[8];
            if constexpr (!SW) {
                // features j1 q2 + 0 .. 7: contiguous, the rotary pairs inside
                if (P.a_q == nullptr) {
                    const float* src = P.q + (row * H + head) * kDH + j1 * kQ2;
                    const f32x4 a = *reinterpret_cast<const f32x4*>(src);
                    const f32x4 c = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        x[k] = a[k];
                        x[4 + k] = c[k];
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < 8; ++k) x[k] = query_elem(P, row, head, j1 * kQ2 + k);
                }
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float c = cs[(ql * NP + m) * 2], sn = cs[(ql * NP + m) * 2 + 1];
                    const float x0 = x[2 * m], x1 = x[2 * m + 1];
                    v[2 * m] = q_ok ? (x0 * c - x1 * sn) * P.q_scale : 0.f;
                    v[2 * m + 1] = q_ok ? (x1 * c + x0 * sn) * P.q_scale : 0.f;
                }
            } else {
                // features k q2 + j1 (k = 0 .. 7) of the cache's order, q2 = 16;
                // the rotary partner of each is k q2 + (j1 ^ 1)
                float y[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int f = k * kQ1 + j1, g = k * kQ1 + (j1 ^ 1);
                    if (P.a_q == nullptr) {
                        x[k] = P.q[(row * H + head) * kDH + f];
                        y[k] = P.q[(row * H + head) * kDH + g];
                    } else {
                        x[k] = query_elem(P, row, head, f);
                        y[k] = query_elem(P, row, head, g);
                    }
                }
                const float c = cs[(ql * NP + (j1 >> 1)) * 2], sn = cs[(ql * NP + (j1 >> 1)) * 2 + 1];
                const bool first_of_pair = (j1 & 1) == 0;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float r = first_of_pair ? (x[k] * c - y[k] * sn) : (x[k] * c + y[k] * sn);
                    v[k] = q_ok ? r * P.q_scale : 0.f;
                }
            }
            q_hi[ks] = pack_bf16x8(v);
        }
    }

    f32x4 o_acc[kQ2];  // O^T block j2: [feature j1 = 4 (lane >> 4) + c][query lane & 15]
#pragma unroll
    for (int j = 0; j < kQ2; ++j) o_acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;  // l_run: this lane's share of the query's sum

    const int l4 = lane & 3;          // row/column inside a 4x4 block
    const int bk = lane >> 2;         // 4x4 block (keys: slot within 16)
    const int g4 = (lane >> 2) & 3;   // values: j1 group
    const int t8 = lane >> 4;         // values: 8-slot group; scores: 4-slot group
    const int sb = 16 * hh;           // this wave's first slot of each tile
    // per-lane LDS offsets of the tile reads (inside a tile buffer) and of
    // the rebuilt keys; the loop adds constants only
    const int a_bk = LY::BK + (sb + bk) * LY::B_ROW + i2 * 64 + l4 * 8;
    const int a_ak = LY::AK + (sb + bk) * LY::A_ROW + l4 * 8;
    const int a_av = LY::AV + (4 * g4 + l4) * LY::V_ROW + (sb + 4 * t8) * 8;
    const int a_bv = LY::BV + (i2 * kQ2 + l4) * LY::V_ROW + (sb + 4 * t8) * 8;
    // source lane (byte address) of the key operand: lane (t + 16 kg) reads
    // rebuild lane (4 t + kg)
    const int k_src = ((ql << 2) | t8) << 2;

    // tiles: the first one staged before the loop, then one barrier per tile;
    // after it each wave writes the next tile (loaded one tile earlier) into
    // the other buffer and issues the loads of the tile after that
    if (first < last) {
        stage.store(tiles, P.d.r_k, P.d.r_v, first + kTileSlots > vis_max, vis_max - first);
        if (first + kTileSlots < last) stage.load(seq + (int64_t)(first / kTileSlots + 1) * L.tile_bytes, p1, P.d.r_k, P.d.r_v);
    }
    // masking is needed only where some query of the group stops seeing slots
    // (queries past n_q are discarded: their columns need no mask)
    int vis_min = q_ok ? vis : INT32_MAX;
    vis_min = min(vis_min, __shfl_xor(vis_min, 1));
    vis_min = min(vis_min, __shfl_xor(vis_min, 2));
    vis_min = min(vis_min, __shfl_xor(vis_min, 4));
    vis_min = min(vis_min, __shfl_xor(vis_min, 8));
    vis_min = __builtin_amdgcn_readfirstlane(vis_min);
    int buf = 0;
    for (int s0 = first; s0 < last; s0 += kTileSlots, buf ^= LY::TILE) {
        __syncthreads();  // tile s0 is in LDS (buffer buf); every wave is done with the other buffer
        if (s0 + kTileSlots < last) {
            stage.store(tiles + (buf ^ LY::TILE), P.d.r_k, P.d.r_v, s0 + 2 * kTileSlots > vis_max,
                        vis_max - (s0 + kTileSlots));
            if (s0 + 2 * kTileSlots < last) stage.load(seq + (int64_t)(s0 / kTileSlots + 2) * L.tile_bytes, p1, P.d.r_k, P.d.r_v);
        }
        const uint8_t* tl = tiles + buf;

        // ---- keys: K[slot][j1][j2] of head (i1, i2) for slots sb .. sb + 15,
        // bf16.  Rebuild lane (4 bk + l4) holds K[sb + bk][j1 = 4 jg + l4][0..7]
        // for jg = 0..3; the score MFMA wants lane (t + 16 kg) to hold
        // K[sb + t][j1 = 4 jg + kg][0..7]: the same registers, lanes rotated
        // by two bits (one ds_bpermute per dword, no LDS memory traffic).
        u32x4 kop[4];
        {
            const s16x4 x0 = lds8(tl + a_bk);       // B~^K, slot sb + bk, j2 = l4
            const s16x4 x1 = lds8(tl + a_bk + 32);  // j2 = 4 + l4
            s16x4 y[4];
#pragma unroll
            for (int jg = 0; jg < 4; ++jg) y[jg] = lds8(tl + a_ak + 32 * jg);  // A^K, j1 = 4 jg + l4
#pragma unroll
            for (int jg = 0; jg < 4; ++jg) {
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                const f32x4 d0 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(x0, y[jg], z, 0, 0, 0);
                const f32x4 d1 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(x1, y[jg], z, 0, 0, 0);
                kop[jg] = u32x4{pack2(d0[0], d0[1]), pack2(d0[2], d0[3]), pack2(d1[0], d1[1]), pack2(d1[2], d1[3])};
            }
#pragma unroll
            for (int jg = 0; jg < 4; ++jg)
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    kop[jg][d] = (uint32_t)__builtin_amdgcn_ds_bpermute(k_src, (int)kop[jg][d]);
        }

        // ---- scores: Z[slot][query] = K q'^T for the wave's 16 slots ---------
        float z[4];
        {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kop[ks]), q_hi[ks], acc, 0,
                                                              0, 0);
            }
            // lane: query ql, slots sb + 4 t8 + c
#pragma unroll
            for (int c = 0; c < 4; ++c) z[c] = acc[c];
        }
        if (s0 + sb + 16 > vis_min) {  // some query of the group stops inside these slots
#pragma unroll
            for (int c = 0; c < 4; ++c) z[c] = (s0 + sb + 4 * t8 + c < vis) ? z[c] : -INFINITY;
        }

        // ---- online softmax ---------------------------------------------------
        // The reference max m_run moves only when some query's scores exceed
        // it by more than kSlack (log2 units); otherwise the weights stay
        // below 2^kSlack and the rescale of the running sums is skipped.  The
        // result is the same for any reference point.
        float mx = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
        mx = fmaxf(mx, other16(mx));
        mx = fmaxf(mx, other32(mx));
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kSlack) != 0) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
            l_run *= alpha;
#pragma unroll
            for (int j = 0; j < kQ2; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c) o_acc[j][c] *= alpha;
            m_run = m_new;
        }
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        float p[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            p[c] = fast_exp2(z[c] - m_use);
            l_run += p[c];
        }
        // ---- values: V^T rebuilt straight into the value MFMA's A layout --------
        // (slots past the context were zeroed when staged).  Rebuild
        // u covers slot sb + 4 (lane >> 4) + u: the inner dimension of the
        // 16x16x16 value MFMA.
        uint32_t vop[kQ2][2];  // block j2: elements e = slot sb + 4 t8 + e of feature j1 = lane & 15
#pragma unroll
        for (int u2 = 0; u2 < 2; ++u2) {  // slots sb + 4 t8 + 2 u2 + (0, 1): one 16-byte read each
            const u32x4 vy = *reinterpret_cast<const u32x4*>(tl + a_av + 16 * u2);                   // A^V, j1 = 4 g4 + l4
            const u32x4 vx0 = *reinterpret_cast<const u32x4*>(tl + a_bv + 16 * u2);                  // B^V, j2 = l4
            const u32x4 vx1 = *reinterpret_cast<const u32x4*>(tl + a_bv + 4 * LY::V_ROW + 16 * u2);  // j2 = 4 + l4
            f32x4 dv[2][2];
            const f32x4 zz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int uu = 0; uu < 2; ++uu) {
                const s16x4 y = __builtin_bit_cast(s16x4, uint2{vy[2 * uu], vy[2 * uu + 1]});
                dv[uu][0] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(
                    __builtin_bit_cast(s16x4, uint2{vx0[2 * uu], vx0[2 * uu + 1]}), y, zz, 0, 0, 0);
                dv[uu][1] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(
                    __builtin_bit_cast(s16x4, uint2{vx1[2 * uu], vx1[2 * uu + 1]}), y, zz, 0, 0, 0);
            }
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int c = 0; c < 4; ++c) vop[4 * hf + c][u2] = pack2(dv[0][hf][c], dv[1][hf][c]);
        }
        // the weights in the score layout are the value MFMA's B operand:
        // lane (query ql), slot sb + 4 t8 + e in element e
        const s16x4 pop = __builtin_bit_cast(s16x4, uint2{pack2(p[0], p[1]), pack2(p[2], p[3])});
#pragma unroll
        for (int j = 0; j < kQ2; ++j)
            o_acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                __builtin_bit_cast(s16x4, uint2{vop[j][0], vop[j][1]}), pop, o_acc[j], 0, 0, 0);
    }

    // ---- the two halves of each head: the second wave hands its (m, l, O)
    // to the first through LDS (the tile buffers are free now), which
    // combines them as the split-KV merge does ----------------------------------
    __syncthreads();
    float* xch = reinterpret_cast<float*>(tiles) + (size_t)i2 * 34 * 64 + lane;
    static_assert(P2 * 34 * 64 * 4 <= 2 * LY::TILE, "exchange fits the tile buffers");
    if (hh == 1) {
        xch[0] = m_run;
        xch[64] = l_run;
#pragma unroll
        for (int j = 0; j < kQ2; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) xch[(2 + 4 * j + c) * 64] = o_acc[j][c];
    }
    __syncthreads();
    if (hh == 1) return;
    {
        const float m1 = xch[0], l1 = xch[64];
        const float mm = fmaxf(m_run, m1);
        const float mref = mm == -INFINITY ? 0.f : mm;
        const float a0 = fast_exp2(m_run - mref), a1 = fast_exp2(m1 - mref);
        l_run = l_run * a0 + l1 * a1;
#pragma unroll
        for (int j = 0; j < kQ2; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) o_acc[j][c] = o_acc[j][c] * a0 + xch[(2 + 4 * j + c) * 64] * a1;
        m_run = mm;
    }

    // ---- finish: the query's sum over its four lanes, then write -------------
    l_run += other16(l_run);
    l_run += other32(l_run);
    if (!q_ok) return;
    const int64_t row = (int64_t)b * P.n_q + n;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int j1 = 4 * t8 + c;
        float v[kQ2];
#pragma unroll
        for (int j = 0; j < kQ2; ++j) v[j] = o_acc[j][c] * P.v_scale;
        float* dst;
        if (P.n_split == 1) {
            const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
            for (int j = 0; j < kQ2; ++j) v[j] = l_run > 0.f ? v[j] * inv : 0.f;
            dst = P.out + (row * H + head) * kDH;
        } else {
            dst = P.part_o + ((row * P.n_split + split) * H + head) * kDH;
        }
        if constexpr (!SW) {
            *reinterpret_cast<f32x4*>(dst + j1 * kQ2) = f32x4{v[0], v[1], v[2], v[3]};
            *reinterpret_cast<f32x4*>(dst + j1 * kQ2 + 4) = f32x4{v[4], v[5], v[6], v[7]};
        } else {
#pragma unroll
            for (int j = 0; j < kQ2; ++j) dst[j * kQ1 + j1] = v[j];  // feature (j, j1) of the cache's order
        }
    }
    if (t8 == 0) {
        if (P.n_split == 1) {
            if (P.lse) P.lse[row * H + head] = l_run > 0.f ? (m_run + log2f(l_run)) * 0.69314718055994531f : -INFINITY;
        } else {
            float* ml = P.part_ml + ((row * P.n_split + split) * H + head) * 2;
            ml[0] = m_run;
            ml[1] = l_run;
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
struct Kernel {
    int p2;   // the kernel's B heads
    bool sw;  // the factors' roles swapped
    hipError_t (*launch)(const DecodeParams&, hipStream_t, const KernelEvents&);
    int (*blocks_per_cu)();
};

template <int P2, bool SW>
struct Entry {
    static hipError_t launch(const DecodeParams& P, hipStream_t s, const KernelEvents& ev) {
        const int split_pad = (P.n_split + kXcds - 1) / kXcds * kXcds;
        const int qgroups = (P.n_q + kNQ - 1) / kNQ;
        dim3 grid(split_pad * (SW ? P.d.p2 : P.d.p1), P.batch, qgroups);
        hipExtLaunchKernelGGL((decode_rebuild_kernel<P2, SW>), grid, dim3(2 * P2 * 64), 0, s, ev.start,
                              ev.stop, 0, P);
        return hipGetLastError();
    }
    static int blocks_per_cu() {
        static std::atomic<int> cached{0};
        int v = cached.load(std::memory_order_relaxed);
        if (v > 0) return v;
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_rebuild_kernel<P2, SW>, 2 * P2 * 64, 0) != hipSuccess ||
            nb <= 0)
            nb = 1;
        cached.store(nb, std::memory_order_relaxed);
        return nb;
    }
};

#define KPA_REBUILD_ENTRY(p2, sw) {p2, sw, Entry<p2, sw>::launch, Entry<p2, sw>::blocks_per_cu}

// The kernel for a shape: q1 = 16, q2 = 8 as they are (B heads p2), or q1 =
// 8, q2 = 16 with the factors' roles swapped (the kernel's B heads are p1).
// Swapped, only p1 = 8 is instantiated: with fewer heads in the kernel's B
// role a workgroup has fewer than 16 waves, and the factor-space kernel was
// as fast or faster on kpa_32k's split (p1 = 4; 8 x 16400 tokens, 16
// queries: 99.7 against 103.8 us, 8 queries 92.1 against 60.9, 32
// sequences x 4096 tokens 370.7 against 188.3).
const Kernel* find(const kpa_dims& d) {
    static const Kernel tab[] = {
        KPA_REBUILD_ENTRY(2, false), KPA_REBUILD_ENTRY(4, false), KPA_REBUILD_ENTRY(6, false),
        KPA_REBUILD_ENTRY(8, false), KPA_REBUILD_ENTRY(8, true),
    };
    if (d.r_k > 4 || d.r_v > 4) return nullptr;
    bool sw;
    if (d.q1 == kQ1 && d.q2 == kQ2) sw = false;
    else if (d.q1 == kQ2 && d.q2 == kQ1) sw = true;
    else return nullptr;
    const int p2 = sw ? d.p1 : d.p2;
    for (const Kernel& k : tab)
        if (k.sw == sw && k.p2 == p2) return &k;
    return nullptr;
}

}  // namespace rebuild

// The rebuild kernel serves bf16 caches with ranks up to 4 and either q1 =
// 16, q2 = 8, p2 = 2, 4, 6 or 8 and at least kRebuildMinQ queries per
// sequence, or q1 = 8, q2 = 16, p1 = 8 and at least kRebuildMinQSwapped.
bool decode_rebuild_supported(const kpa_dims& d, int n_q) {
    if (d.dtype != KPA_BF16) return false;
    const rebuild::Kernel* k = rebuild::find(d);
    return k != nullptr && n_q >= (k->sw ? kRebuildMinQSwapped : kRebuildMinQ);
}

int decode_rebuild_blocks_per_cu(const kpa_dims& d) {
    const rebuild::Kernel* k = rebuild::find(d);
    return k ? k->blocks_per_cu() : 1;
}

int decode_rebuild_query_groups(int n_q) { return (n_q + rebuild::kNQ - 1) / rebuild::kNQ; }

// Workgroups per chunk and query group: one per head of the factor in the
// kernel's A role.
int decode_rebuild_head_groups(const kpa_dims& d) {
    const rebuild::Kernel* k = rebuild::find(d);
    return k && k->sw ? d.p2 : d.p1;
}

hipError_t launch_decode_rebuild(const DecodeParams& P, hipStream_t s, const KernelEvents& ev) {
    const rebuild::Kernel* k = rebuild::find(P.d);
    if (!k) return hipErrorInvalidValue;
    return k->launch(P, s, ev);
}

}  // namespace kpa
