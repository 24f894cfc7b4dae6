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
// every B head i2: one wave per i2) and up to 16 queries.  Per 32-slot tile:
//   1. The tile's factors go HBM -> registers (one tile ahead) -> LDS with
//      their ranks interleaved: element (slot, row, feature) -> 4 ranks in
//      8 bytes, so each operand of a rebuild MFMA is one 8-byte LDS read.
//   2. Keys: 16 rebuild MFMAs per wave give K[32 slots][128 features] of its
//      head in float32; rounded to bf16 and written to the wave's own LDS
//      rows (16-byte chunks, XOR-swizzled so that the writes and the reads
//      below spread over the banks).
//   3. Scores: MFMA 16x16x32 with M = 16 slots, N = 16 queries, K = 32
//      features; the query (rotated, scaled) is carried as bf16 hi + lo, two
//      MFMAs per K step.  The result holds a query per lane (lane % 16) and
//      slots in registers and lane bits 4-5.
//   4. Online softmax per (query, head): the running max is shared by a
//      query's four lanes (two lane swaps); the weights p = 2^(z - m), in
//      bf16, are moved into the value MFMA's operand layout by two
//      permlane swaps (slots into registers and lane bits 4-5).
//   5. Values: 16 rebuild MFMAs per wave whose outputs already sit in the
//      operand layout of the value MFMA (slots on the inner dimension: rebuild
//      u of 8 covers slot 8 (lane >> 4) + u), then O^T[feature][query] +=
//      V^T P^T, MFMA 16x16x32, eight per tile (one per j2).
//   The running output O^T keeps a query per lane (lane % 16), so the rescale
//   by the softmax correction is a plain multiply.
// The online softmax and the chunk partials (m, l, o) are those of the other
// decode kernels (the blocked online log-sum-exp of FlashTPA decoding,
// "Tensor Product Attention Is All You Need", summary page), merged by the
// same merge kernel.
//
// Shapes: bf16 caches with A's feature dimension q1 = 16 (j1: a lane's 16
// columns) and B's q2 = 8 (j2: 8 consecutive features, the rotary pairs),
// ranks up to 4 (missing ranks are zero rows of the inner dimension), B head
// count p2 = 2, 4, 6 or 8 (one wave each), any A head count p1 (one
// workgroup each), up to 16 queries per workgroup (more queries: more
// workgroups per chunk).
//
// Precision: bf16 factors exactly; the rebuilt K and V rows and the softmax
// weights are rounded once to bf16 (relative 2^-8 per element at most,
// unbiased); the query carries ~16 bits (hi + lo); all sums in float32.
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
    // rank-interleaved tile: 8 bytes (4 ranks) per (slot, row, feature);
    // rows of a slot padded so that slot stride = 8 banks mod 32; offsets
    // inside one of the two tile buffers
    static constexpr int A_ROW = kQ1 * 8 + 32;         // A^K or A^V of the group's A head
    static constexpr int B_ROW = P2 * kQ2 * 8 + 32;    // B~^K or B^V of every B head
    static constexpr int AK = 0;
    static constexpr int AV = AK + kTileSlots * A_ROW;
    static constexpr int BK = AV + kTileSlots * A_ROW;
    static constexpr int BV = BK + kTileSlots * B_ROW;
    static constexpr int TILE = BV + kTileSlots * B_ROW;
    // per wave: rebuilt keys [32 slots][16 chunks of 8 features][16 B]
    static constexpr int KS_WAVE = kTileSlots * 256;
    // two tile buffers, the rebuilt keys and the rotary cos/sin [16 queries][4 pairs][2]
    static constexpr int TOTAL = 2 * TILE + P2 * KS_WAVE + kNQ * 4 * 2 * 4;
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

// Chunk swizzle of the rebuilt-key rows: chunk c of slot t sits at
// c ^ swz(t).  swz is a bijection on 0..7 (conflict-free reads of 8 slots
// at one chunk) with swz(2k) ^ swz(2k+1) = 4 (conflict-free writes of the
// 4 chunks of 2 slots).
__device__ __forceinline__ int swz(int t) { return ((t & 1) << 2) | ((t >> 1) & 3); }

template <int P2>
struct Cfg {
    static constexpr int WAVES = P2;
    static constexpr int THREADS = WAVES * 64;
    // staging units of one tile (64 B of LDS each, from 4 x 16 B of cache):
    // B~^K (slot, i2), B^V (i2, j2, 8-slot group), A^K (slot, 8-feature
    // half), A^V (j1, 8-slot group)
    static constexpr int U_BK = kTileSlots * P2, U_BV = P2 * kQ2 * 4, U_AK = kTileSlots * 2, U_AV = kQ1 * 4;
    static constexpr int UNITS = U_BK + U_BV + U_AK + U_AV;
    static constexpr int UPT = (UNITS + THREADS - 1) / THREADS;  // units per thread
    // kinds of unit start at multiples of 64 (one kind per wave): P2 even
    static_assert(P2 >= 2 && P2 <= 8 && P2 % 2 == 0, "one wave per B head: 2, 4, 6 or 8");
    static_assert(UPT <= 2, "at most two staging units per thread");
};

// This thread's staging units of a tile: for each, the four 16-byte source
// chunks (one per rank, consecutive ranks a fixed stride apart; zero for
// ranks past R) and where their 64 interleaved bytes go in LDS.  A unit's
// kind is the same across a wave (kinds start at multiples of 64 units).
template <int P2>
struct Stage {
    using C = Cfg<P2>;
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
                src[k] = (uint32_t)(L.off[1] + i2 * (kTileSlots * 16) + s * 16);
                dst[k] = LY::BK + s * LY::B_ROW + i2 * 64;
            } else if (u < C::U_BK + C::U_BV) {  // B^V element (r P2 + i2) q2 + j2, 8 slots
                const int x = u - C::U_BK;
                const int sg = x & 3, e = x >> 2;
                kd = kBV;
                slot[k] = 8 * sg;
                src[k] = (uint32_t)(L.off[3] + e * 64 + sg * 16);
                dst[k] = LY::BV + (8 * sg) * LY::B_ROW + e * 8;
            } else if (u < C::U_BK + C::U_BV + C::U_AK) {  // A^K chunk (r p1 + i1) 2 + hf of slot s
                const int x = u - C::U_BK - C::U_BV;
                const int s = x % kTileSlots, hf = x / kTileSlots;
                kd = kAK;
                slot[k] = s;
                src[k] = (uint32_t)(L.off[0] + (i1 * 2 + hf) * (kTileSlots * 16) + s * 16);
                dst[k] = LY::AK + s * LY::A_ROW + hf * 64;
            } else if (u < C::UNITS) {  // A^V element (r p1 + i1) q1 + j1, 8 slots
                const int x = u - C::U_BK - C::U_BV - C::U_AK;
                const int sg = x & 3, j1 = x >> 2;
                kd = kAV;
                slot[k] = 8 * sg;
                src[k] = (uint32_t)(L.off[2] + (i1 * kQ1 + j1) * 64 + sg * 16);
                dst[k] = LY::AV + (8 * sg) * LY::A_ROW + j1 * 8;
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
        using LY = Lds<P2>;
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
            if (kd == kBK || kd == kAK) {  // items = 8 consecutive features: 64 contiguous bytes
#pragma unroll
                for (int d = 0; d < 4; ++d) *reinterpret_cast<u32x4*>(out + 16 * d) = o[d];
            } else {  // items = 8 consecutive slots: one 8-byte entry per slot row
                const int row = kd == kBV ? LY::B_ROW : LY::A_ROW;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    *reinterpret_cast<uint2*>(out + (2 * d) * row) = uint2{o[d][0], o[d][1]};
                    *reinterpret_cast<uint2*>(out + (2 * d + 1) * row) = uint2{o[d][2], o[d][3]};
                }
            }
        }
    }
};

__device__ __forceinline__ s16x4 lds8(const uint8_t* p) {
    return __builtin_bit_cast(s16x4, *reinterpret_cast<const uint2*>(p));
}

template <int P2>
__global__ void __launch_bounds__(P2 * 64, 1) decode_rebuild_kernel(DecodeParams P) {
    using LY = Lds<P2>;
    // separate LDS objects, so that the compiler can tell the rebuilt keys
    // (written per tile) from the tile factors (read around those writes)
    __shared__ __attribute__((aligned(16))) uint8_t tiles[2 * LY::TILE];
    __shared__ __attribute__((aligned(16))) uint8_t kscr[P2 * LY::KS_WAVE];
    __shared__ float cs[kNQ * 4 * 2];
    const int lane = threadIdx.x & 63;
    const int i2 = (int)(threadIdx.x >> 6);  // this wave's B head
    const int p1 = P.d.p1;
    const int H = p1 * P2;
    // workgroup -> (chunk, A head): the head groups of a chunk share an XCD,
    // so the B factors they all read come from HBM once
    const int bx = blockIdx.x;
    const int split = (bx / (kXcds * p1)) * kXcds + bx % kXcds;
    const int i1 = (bx / kXcds) % p1;
    const int b = blockIdx.y;
    const int qg = blockIdx.z;  // group of 16 queries
    if (split >= P.n_split) return;
    const Layout& L = P.L;
    const int head = i1 * P2 + i2;

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

    Stage<P2> stage;
    stage.init(L, i1, p1);
    if (first < last) stage.load(seq + (int64_t)(first / kTileSlots) * L.tile_bytes, p1, P.d.r_k, P.d.r_v);

    // ---- rotated, scaled query as the score MFMA's B operand (hi + lo) -----
    if (threadIdx.x < kNQ * 4) {
        const int nq = threadIdx.x >> 2, m = threadIdx.x & 3;
        const int nn = min(qg * kNQ + nq, P.n_q - 1);
        const double theta = exp2(-(2.0 * m / kQ2) * log2((double)P.d.rope_base));
        double sn, c;
        sincos((double)P.q_pos[(int64_t)b * P.n_q + nn] * theta, &sn, &c);
        cs[(nq * 4 + m) * 2] = (float)c;
        cs[(nq * 4 + m) * 2 + 1] = (float)sn;
    }
    if (i1 == 0)
        for (int k = 0; k < kNQ; ++k)
            if (qg * kNQ + k < P.n_q) clear_merge_counters(P, (int64_t)b * P.n_q + qg * kNQ + k, split);
    __syncthreads();
    bf16x8 q_hi[4], q_lo[4];
    {
        const int64_t row = (int64_t)b * P.n_q + min(n, P.n_q - 1);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int j1 = 4 * ks + (lane >> 4);
            float x[8];
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
            float v[8];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float c = cs[(ql * 4 + m) * 2], sn = cs[(ql * 4 + m) * 2 + 1];
                const float x0 = x[2 * m], x1 = x[2 * m + 1];
                v[2 * m] = q_ok ? (x0 * c - x1 * sn) * P.q_scale : 0.f;
                v[2 * m + 1] = q_ok ? (x1 * c + x0 * sn) * P.q_scale : 0.f;
            }
            split_bf16x8(v, q_hi[ks], q_lo[ks]);
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
    uint8_t* ks_w = kscr + i2 * LY::KS_WAVE;

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

        // ---- keys: K[slot][j1][j2] of head (i1, i2), bf16, into ks_w ----------
#pragma unroll
        for (int th = 0; th < 2; ++th) {
            const int s = 16 * th + bk;
            const s16x4 x0 = lds8(tl + LY::BK + s * LY::B_ROW + i2 * 64 + l4 * 8);        // B~^K, j2 = l4
            const s16x4 x1 = lds8(tl + LY::BK + s * LY::B_ROW + i2 * 64 + (4 + l4) * 8);  // j2 = 4 + l4
#pragma unroll
            for (int jg = 0; jg < 4; ++jg) {
                const s16x4 y = lds8(tl + LY::AK + s * LY::A_ROW + (4 * jg + l4) * 8);  // A^K, j1 = 4 jg + l4
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                const f32x4 d0 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(x0, y, z, 0, 0, 0);
                const f32x4 d1 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(x1, y, z, 0, 0, 0);
                // lane (4 bk + l4): K[s][j1 = 4 jg + l4][j2 = 0..7]
                const u32x4 w = {pack2(d0[0], d0[1]), pack2(d0[2], d0[3]), pack2(d1[0], d1[1]), pack2(d1[2], d1[3])};
                *reinterpret_cast<u32x4*>(ks_w + s * 256 + (((4 * jg + l4) ^ swz(s & 7)) << 4)) = w;
            }
        }

        // ---- values: V^T rebuilt straight into the value MFMA's A layout --------
        // (independent of the scores: issued before them, so that the two
        // overlap; slots past the context were zeroed when staged)
        uint32_t vop[kQ2][4];  // block j2: element e = slot 8 t8 + e of feature j1 = lane & 15
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {  // slots 8 t8 + 4 h2 + uu
            s16x4 vy[4], vx0[4], vx1[4];
#pragma unroll
            for (int uu = 0; uu < 4; ++uu) {
                const int s = 8 * t8 + 4 * h2 + uu;
                vy[uu] = lds8(tl + LY::AV + s * LY::A_ROW + (4 * g4 + l4) * 8);        // A^V, j1 = 4 g4 + l4
                vx0[uu] = lds8(tl + LY::BV + s * LY::B_ROW + i2 * 64 + l4 * 8);        // B^V, j2 = l4
                vx1[uu] = lds8(tl + LY::BV + s * LY::B_ROW + i2 * 64 + (4 + l4) * 8);  // j2 = 4 + l4
            }
            f32x4 dv[4][2];
            const f32x4 zz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int uu = 0; uu < 4; ++uu) {
                dv[uu][0] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(vx0[uu], vy[uu], zz, 0, 0, 0);
                dv[uu][1] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(vx1[uu], vy[uu], zz, 0, 0, 0);
            }
#pragma unroll
            for (int u2 = 0; u2 < 2; ++u2)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        vop[4 * hf + c][2 * h2 + u2] = pack2(dv[2 * u2][hf][c], dv[2 * u2 + 1][hf][c]);
        }
        wave_lds_sync();  // this wave's keys are in ks_w

        // ---- scores: Z[slot][query] = K q'^T ----------------------------------
        float z[2][4];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int t = 16 * tb + ql;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 kop = ld_lds16(reinterpret_cast<const uint16_t*>(
                    ks_w + t * 256 + (((4 * ks + t8) ^ swz(t & 7)) << 4)));
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, q_hi[ks], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, q_lo[ks], acc, 0, 0, 0);
            }
            // lane: query ql, slots 16 tb + 4 t8 + c
#pragma unroll
            for (int c = 0; c < 4; ++c) z[tb][c] = acc[c];
        }
        if (s0 + kTileSlots > vis_min) {  // some query of the group stops inside this tile
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int c = 0; c < 4; ++c) z[tb][c] = (s0 + 16 * tb + 4 * t8 + c < vis) ? z[tb][c] : -INFINITY;
        }

        // ---- online softmax ---------------------------------------------------
        // The reference max m_run moves only when some query's scores exceed
        // it by more than kSlack (log2 units); otherwise the weights stay
        // below 2^kSlack and the rescale of the running sums is skipped.  The
        // result is the same for any reference point.
        float mx = fmaxf(fmaxf(fmaxf(z[0][0], z[0][1]), fmaxf(z[0][2], z[0][3])),
                         fmaxf(fmaxf(z[1][0], z[1][1]), fmaxf(z[1][2], z[1][3])));
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
        float p[2][4];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                p[tb][c] = fast_exp2(z[tb][c] - m_use);
                l_run += p[tb][c];
            }

        // weights into the value MFMA's B layout: lane (query ql, 8-slot
        // group lane >> 4), slot 8 (lane >> 4) + e in element e
        bf16x8 pop;
        {
            uint32_t pk[2][2];
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int d = 0; d < 2; ++d) pk[tb][d] = pack2(p[tb][2 * d], p[tb][2 * d + 1]);
            uint32_t x[2][2], y[2][2];
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const auto r = __builtin_amdgcn_permlane32_swap(pk[0][d], pk[1][d], false, false);
                x[0][d] = r[0];
                x[1][d] = r[1];
            }
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const auto r = __builtin_amdgcn_permlane16_swap(x[0][d], x[1][d], false, false);
                y[0][d] = r[0];
                y[1][d] = r[1];
            }
            pop = __builtin_bit_cast(bf16x8, u32x4{y[0][0], y[0][1], y[1][0], y[1][1]});
        }
#pragma unroll
        for (int j = 0; j < kQ2; ++j)
            o_acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, u32x4{vop[j][0], vop[j][1], vop[j][2], vop[j][3]}), pop, o_acc[j], 0, 0,
                0);
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
            dst = P.out + (row * H + head) * kDH + j1 * kQ2;
        } else {
            dst = P.part_o + ((row * P.n_split + split) * H + head) * kDH + j1 * kQ2;
        }
        *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{v[4], v[5], v[6], v[7]};
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
    int p2;
    hipError_t (*launch)(const DecodeParams&, hipStream_t, const KernelEvents&);
    int (*blocks_per_cu)();
};

template <int P2>
struct Entry {
    static hipError_t launch(const DecodeParams& P, hipStream_t s, const KernelEvents& ev) {
        const int split_pad = (P.n_split + kXcds - 1) / kXcds * kXcds;
        const int qgroups = (P.n_q + kNQ - 1) / kNQ;
        dim3 grid(split_pad * P.d.p1, P.batch, qgroups);
        hipExtLaunchKernelGGL(decode_rebuild_kernel<P2>, grid, dim3(P2 * 64), 0, s, ev.start,
                              ev.stop, 0, P);
        return hipGetLastError();
    }
    static int blocks_per_cu() {
        static std::atomic<int> cached{0};
        int v = cached.load(std::memory_order_relaxed);
        if (v > 0) return v;
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_rebuild_kernel<P2>, P2 * 64, 0) != hipSuccess ||
            nb <= 0)
            nb = 1;
        cached.store(nb, std::memory_order_relaxed);
        return nb;
    }
};

#define KPA_REBUILD_ENTRY(p2) {p2, Entry<p2>::launch, Entry<p2>::blocks_per_cu}

const Kernel* find(const kpa_dims& d) {
    static const Kernel tab[] = {
        KPA_REBUILD_ENTRY(2), KPA_REBUILD_ENTRY(4), KPA_REBUILD_ENTRY(6), KPA_REBUILD_ENTRY(8),
    };
    if (d.r_k > 4 || d.r_v > 4) return nullptr;
    for (const Kernel& k : tab)
        if (k.p2 == d.p2) return &k;
    return nullptr;
}

}  // namespace rebuild

// The rebuild kernel serves bf16 caches with q1 = 16, q2 = 8, p2 = 2, 4, 6
// or 8, ranks up to 4 and at least kRebuildMinQ queries per sequence.
bool decode_rebuild_supported(const kpa_dims& d, int n_q) {
    if (d.dtype != KPA_BF16 || n_q < kRebuildMinQ) return false;
    if (d.q1 != rebuild::kQ1 || d.q2 != rebuild::kQ2) return false;
    return rebuild::find(d) != nullptr;
}

int decode_rebuild_blocks_per_cu(const kpa_dims& d) {
    const rebuild::Kernel* k = rebuild::find(d);
    return k ? k->blocks_per_cu() : 1;
}

int decode_rebuild_query_groups(int n_q) { return (n_q + rebuild::kNQ - 1) / rebuild::kNQ; }

hipError_t launch_decode_rebuild(const DecodeParams& P, hipStream_t s, const KernelEvents& ev) {
    const rebuild::Kernel* k = rebuild::find(P.d);
    if (!k || P.d.q1 != rebuild::kQ1 || P.d.q2 != rebuild::kQ2) return hipErrorInvalidValue;
    return k->launch(P, s, ev);
}

}  // namespace kpa
