// General-shape split-KV decode on the vector ALUs (any split/rank within the
// kpa.h limits, float32 or bfloat16 factors, one or many queries).  Used for
// float32 caches and for bf16 shapes outside the matrix-core kernels' families.
//
// Per (chunk of the cache, query, sequence) one workgroup:
//   1. rotates the query (dense, or expanded from its Kronecker factors) with
//      R_KPA(q_pos) and folds in log2(e)/(R_K sqrt(d_h))
//      ([KPA] Def. 2.3, §2.3);
//   2. per 32-slot tile, scores every (head, slot) in factor space: the query
//      is contracted with B~^K over j2, then with A^K over j1 and summed over
//      the rank ([KPA] Prop. 2.2 / Eq. (6) with a dense query);
//   3. keeps an online softmax per head (running max and sum, rescaling the
//      accumulators when the max grows -- the blocked online log-sum-exp of
//      FlashTPA decoding, "Tensor Product Attention Is All You Need" summary
//      page);
//   4. accumulates sum_s p_s v_{s,i} with v rebuilt element by element from
//      A^V, B^V ([KPA] Eq. (4)); K and V are never stored;
//   5. writes either the final output or a partial (m, l, o) for the merge.
// [KPA] = "Kronecker Product Attention: Memory-Efficient KV Compression via
// Structured Factorization".
#include <map>
#include <mutex>
#include <utility>

#include "kpa_common.hpp"

namespace kpa {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxPerThread = KPA_MAX_HD / kThreads;  // output elements per thread

template <bool kF32>
__device__ __forceinline__ float load_factor(const uint8_t* p) {
    if constexpr (kF32) return *reinterpret_cast<const float*>(p);
    else return bf16_to_f32(*reinterpret_cast<const uint16_t*>(p));
}

// Byte offset of element e of set c for slot t inside a tile (the cache
// layout's rule, with the element size fixed at compile time so that the
// chunk arithmetic is shifts and masks).
template <bool kF32>
__device__ __forceinline__ int eoff(const Layout& L, int c, int e, int t) {
    constexpr int ES = kF32 ? 4 : 2, PC = kChunkBytes / ES;
    if (c < 2) return (int)L.off[c] + (e / PC) * (kTileSlots * kChunkBytes) + t * kChunkBytes + (e % PC) * ES;
    return (int)L.off[c] + (e * kTileSlots + t) * ES;
}

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4v;

// 8 consecutive elements (16 bytes of bf16 or 32 of float32, 16-byte aligned)
template <bool kF32>
__device__ __forceinline__ void load8(const uint8_t* p, float* v) {
    if constexpr (kF32) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x4v w = *reinterpret_cast<const u32x4v*>(p + 16 * h);
#pragma unroll
            for (int k = 0; k < 4; ++k) v[4 * h + k] = __uint_as_float(w[k]);
        }
    } else {
        const u32x4v w = *reinterpret_cast<const u32x4v*>(p);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = __uint_as_float(w[k] << 16);
            v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
    }
}

// kStage: each tile is first copied into LDS with 16-byte loads (when it fits
// beside the query and score buffers), so that the many element reads of the
// score and value loops are LDS reads instead of scattered global loads.
// Output element of accumulator k of thread tid.  kG4 (q2 a multiple of 4):
// each thread owns runs of 4 consecutive outputs, which share the head and
// j1, so the value loop forms p * A^V once for four B^V rows.
template <bool kG4>
__device__ __forceinline__ int out_index(int tid, int k) {
    if constexpr (kG4) return 4 * (tid + (k / 4) * kThreads) + k % 4;
    return tid + k * kThreads;
}

template <bool kF32, bool kStage, bool kG4>
__global__ void __launch_bounds__(kThreads) decode_valu_kernel(DecodeParams P, int stage_off) {
    extern __shared__ float smem[];
    const kpa_dims& d = P.d;
    const Layout& L = P.L;
    const int h = d.p1 * d.p2, dh = d.q1 * d.q2;
    const int split = blockIdx.x, n = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;

    float* qr = smem;                      // [h][dh] rotated, scaled query
    float* zs = qr + (h * dh + 3) / 4 * 4;  // [h][32] scores, then probabilities (16-byte aligned rows)
    float* m_run = zs + h * kTileSlots;    // [h] running max (log2 units)
    float* l_run = m_run + h;              // [h] running sum
    float* alpha = l_run + h;              // [h] rescale factor of this tile
    float* cs = alpha + h;                 // [q2/2][2] cos, sin

    clear_merge_counters(P, (int64_t)b * P.n_q + n, split);
    const int vis = visible_slots(P, b, n);
    const int first = split * P.chunk_tiles * kTileSlots;
    int last = first + P.chunk_tiles * kTileSlots;
    if (last > vis) last = vis;

    // 1. rotate the query ---------------------------------------------------
    const int qp = P.q_pos[(int64_t)b * P.n_q + n];
    const int half = d.q2 / 2;
    if (tid < half) {
        const double theta = exp2(-(2.0 * tid / d.q2) * log2((double)d.rope_base));
        double sn, c;
        sincos((double)qp * theta, &sn, &c);
        cs[2 * tid] = (float)c;
        cs[2 * tid + 1] = (float)sn;
    }
    for (int i = tid; i < h; i += kThreads) {
        m_run[i] = -INFINITY;
        l_run[i] = 0.f;
    }
    __syncthreads();
    const int64_t qrow = (int64_t)b * P.n_q + n;
    for (int pr = tid; pr < h * dh / 2; pr += kThreads) {
        const int e = 2 * pr;
        const int m = (e % d.q2) / 2;
        const float x0 = query_elem(P, qrow, e / dh, e % dh), x1 = query_elem(P, qrow, e / dh, e % dh + 1);
        const float c = cs[2 * m], sn = cs[2 * m + 1];
        qr[e] = (x0 * c - x1 * sn) * P.q_scale;
        qr[e + 1] = (x0 * sn + x1 * c) * P.q_scale;
    }

    float acc[kMaxPerThread];
#pragma unroll
    for (int k = 0; k < kMaxPerThread; ++k) acc[k] = 0.f;
    __syncthreads();

    const uint8_t* seq_base = P.cache + (int64_t)b * L.n_tiles * L.tile_bytes;
    const int es = L.elem_bytes;
    for (int s0 = first; s0 < last; s0 += kTileSlots) {
        const uint8_t* gtile = seq_base + (int64_t)(s0 / kTileSlots) * L.tile_bytes;
        const int valid = (last - s0) < kTileSlots ? (last - s0) : kTileSlots;
        const uint8_t* tile;
        if constexpr (kStage) {
            // (the previous tile's readers passed the barrier that ends the loop)
            uint8_t* st = reinterpret_cast<uint8_t*>(smem) + stage_off;
            const u32x4v* src = reinterpret_cast<const u32x4v*>(gtile);
            u32x4v* dst = reinterpret_cast<u32x4v*>(st);
            for (int v = tid; v < (int)(L.tile_bytes / kChunkBytes); v += kThreads) dst[v] = src[v];
            __syncthreads();
            tile = st;
        } else {
            tile = gtile;
        }

        // 2.-3. factor-space scores for every (head, slot), then the online
        // softmax per head: the 32 slots of a head sit in 32 consecutive lanes
        // (h * 32 is a multiple of 32, so a lane group is all in or all out),
        // which reduce their max and sum with shuffles.
        constexpr int PC = kChunkBytes / (kF32 ? 4 : 2);  // elements per 16-byte chunk
        const bool bk_chunks = d.q2 % PC == 0;            // B~^K rows are whole chunks
        for (int pi = tid; pi < h * kTileSlots; pi += kThreads) {
            const int i = pi / kTileSlots, t = pi % kTileSlots;
            float z = -INFINITY;
            if (t < valid) {
                const int i1 = i / d.p2, i2 = i % d.p2;
                const float* qi = qr + i * dh;
                z = 0.f;
                for (int r = 0; r < d.r_k; ++r) {
                    const int bk_row = (r * d.p2 + i2) * d.q2;
                    const int ak_row = (r * d.p1 + i1) * d.q1;
                    for (int j1 = 0; j1 < d.q1; ++j1) {
                        float w = 0.f;  // sum_j2 q'[i, j1, j2] B~^K_r[i2, j2]
                        const float* qj = qi + j1 * d.q2;
                        if (bk_chunks) {
                            for (int c = 0; c < d.q2; c += PC) {
                                float bq[PC];
                                const uint8_t* src = tile + eoff<kF32>(L, 1, bk_row + c, t);
                                if constexpr (kF32) {
                                    const u32x4v v4 = *reinterpret_cast<const u32x4v*>(src);
#pragma unroll
                                    for (int k = 0; k < 4; ++k) bq[k] = __uint_as_float(v4[k]);
                                } else {
                                    load8<false>(src, bq);
                                }
                                // q2 and d_h are multiples of 4 here: qj + c is 16-byte aligned
#pragma unroll
                                for (int k = 0; k < PC; k += 4) {
                                    const float4 q4 = *reinterpret_cast<const float4*>(qj + c + k);
                                    w += q4.x * bq[k] + q4.y * bq[k + 1] + q4.z * bq[k + 2] + q4.w * bq[k + 3];
                                }
                            }
                        } else {
                            for (int j2 = 0; j2 < d.q2; ++j2)
                                w += qj[j2] * load_factor<kF32>(tile + eoff<kF32>(L, 1, bk_row + j2, t));
                        }
                        z += load_factor<kF32>(tile + eoff<kF32>(L, 0, ak_row + j1, t)) * w;
                    }
                }
            }
            float mx = z;
            for (int o = kTileSlots / 2; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
            const float m_old = m_run[i];
            const float m_new = fmaxf(m_old, mx);
            const float a = (m_new == -INFINITY) ? 1.f : exp2f(m_old - m_new);
            const float p = (z == -INFINITY) ? 0.f : exp2f(z - m_new);
            float sum = p;
            for (int o = kTileSlots / 2; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
            zs[i * kTileSlots + t] = p;
            if (t == 0) {  // (every lane of the group has read m_run[i] above)
                alpha[i] = a;
                m_run[i] = m_new;
                l_run[i] = l_run[i] * a + sum;
            }
        }
        __syncthreads();

        // 4. value accumulation in factor space ---------------------------------
        if constexpr (kG4) {
#pragma unroll
            for (int g = 0; g < kMaxPerThread / 4; ++g) {
                const int o0 = out_index<true>(tid, 4 * g);
                if (o0 < h * dh) {
                    const int i = o0 / dh, j = o0 % dh;
                    const int i1 = i / d.p2, i2 = i % d.p2;
                    const int j1 = j / d.q2, j20 = j % d.q2;  // outputs j20 .. j20 + 3
                    const float* pi = zs + i * kTileSlots;
                    float sum[4] = {0.f, 0.f, 0.f, 0.f};
                    for (int r = 0; r < d.r_v; ++r) {
                        const uint8_t* av = tile + eoff<kF32>(L, 2, (r * d.p1 + i1) * d.q1 + j1, 0);
                        const uint8_t* bv = tile + eoff<kF32>(L, 3, (r * d.p2 + i2) * d.q2 + j20, 0);
                        for (int t0 = 0; t0 < valid; t0 += 8) {
                            float a8[8];
                            load8<kF32>(av + t0 * es, a8);
                            const float4 p0 = *reinterpret_cast<const float4*>(pi + t0);
                            const float4 p1 = *reinterpret_cast<const float4*>(pi + t0 + 4);
                            const float p8[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
                            float pa[8];
#pragma unroll
                            for (int k = 0; k < 8; ++k) pa[k] = p8[k] * a8[k];
#pragma unroll
                            for (int u = 0; u < 4; ++u) {
                                float b8[8];  // B^V element j20 + u: the next 32-slot row
                                load8<kF32>(bv + (u * kTileSlots + t0) * es, b8);
#pragma unroll
                                for (int k = 0; k < 8; ++k)  // slots past the context may hold anything
                                    if (t0 + k < valid) sum[u] += pa[k] * b8[k];
                            }
                        }
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u) acc[4 * g + u] = acc[4 * g + u] * alpha[i] + sum[u];
                }
            }
        } else {
#pragma unroll
        for (int k = 0; k < kMaxPerThread; ++k) {
            const int o = tid + k * kThreads;
            if (o < h * dh) {
                const int i = o / dh, j = o % dh;
                const int i1 = i / d.p2, i2 = i % d.p2;
                const int j1 = j / d.q2, j2 = j % d.q2;
                const float* pi = zs + i * kTileSlots;
                float sum = 0.f;
                for (int r = 0; r < d.r_v; ++r) {
                    // a value-set element's 32 slots are contiguous (64-byte aligned rows)
                    const uint8_t* av = tile + eoff<kF32>(L, 2, (r * d.p1 + i1) * d.q1 + j1, 0);
                    const uint8_t* bv = tile + eoff<kF32>(L, 3, (r * d.p2 + i2) * d.q2 + j2, 0);
                    for (int t0 = 0; t0 < valid; t0 += 8) {
                        float a8[8], b8[8];
                        load8<kF32>(av + t0 * es, a8);
                        load8<kF32>(bv + t0 * es, b8);
                        // a head's 32 weights are a 128-byte aligned row
                        const float4 p0 = *reinterpret_cast<const float4*>(pi + t0);
                        const float4 p1 = *reinterpret_cast<const float4*>(pi + t0 + 4);
                        const float p8[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
                        for (int k = 0; k < 8; ++k)  // slots past the context may hold anything
                            if (t0 + k < valid) sum += p8[k] * a8[k] * b8[k];
                    }
                }
                acc[k] = acc[k] * alpha[i] + sum;
            }
        }
        }
        __syncthreads();
    }

    // 5. write out -------------------------------------------------------------
    const int64_t row = ((int64_t)b * P.n_q + n);
    if (P.n_split == 1) {
#pragma unroll
        for (int k = 0; k < kMaxPerThread; ++k) {
            const int o = out_index<kG4>(tid, k);
            if (o < h * dh) {
                const int i = o / dh;
                const float l = l_run[i];
                P.out[row * h * dh + o] = l > 0.f ? acc[k] * P.v_scale / l : 0.f;
            }
        }
        if (P.lse)
            for (int i = tid; i < h; i += kThreads)
                P.lse[row * h + i] = l_run[i] > 0.f ? (m_run[i] + log2f(l_run[i])) * 0.69314718055994531f : -INFINITY;
    } else {
        const int64_t prow = row * P.n_split + split;
#pragma unroll
        for (int k = 0; k < kMaxPerThread; ++k) {
            const int o = out_index<kG4>(tid, k);
            if (o < h * dh) P.part_o[prow * h * dh + o] = acc[k] * P.v_scale;
        }
        for (int i = tid; i < h; i += kThreads) {
            P.part_ml[(prow * h + i) * 2] = m_run[i];
            P.part_ml[(prow * h + i) * 2 + 1] = l_run[i];
        }
    }
}

}  // namespace

size_t decode_valu_smem(const kpa_dims& d) {
    const int h = d.p1 * d.p2, dh = d.q1 * d.q2;
    return sizeof(float) * (((size_t)h * dh + 3) / 4 * 4 + (size_t)h * kTileSlots + 3 * (size_t)h + d.q2);
}

namespace {

// The variant and LDS size a shape launches with: the tile is staged when it
// fits in 64 KB beside the query and score buffers; outputs go in runs of
// four when q2 is a multiple of 4.
struct ValuChoice {
    bool f32, stage, g4;
    size_t smem;
    int stage_off;
};

ValuChoice valu_choice(const kpa_dims& d) {
    const Layout L = make_layout(d, 1, kTileSlots);  // the tile size depends on the dims only
    ValuChoice c{};
    c.f32 = d.dtype == KPA_F32;
    const size_t base = (decode_valu_smem(d) + kChunkBytes - 1) / kChunkBytes * kChunkBytes;
    const size_t staged = base + (size_t)L.tile_bytes;
    c.stage = staged <= 65536 && L.tile_bytes % kChunkBytes == 0;
    c.g4 = d.q2 % 4 == 0;
    c.smem = c.stage ? staged : decode_valu_smem(d);
    c.stage_off = (int)base;
    return c;
}

template <bool kF32, bool kStage, bool kG4>
const void* valu_kernel() {
    return reinterpret_cast<const void*>(&decode_valu_kernel<kF32, kStage, kG4>);
}

const void* valu_kernel_of(const ValuChoice& c) {
    if (c.f32) {
        if (c.stage) return c.g4 ? valu_kernel<true, true, true>() : valu_kernel<true, true, false>();
        return c.g4 ? valu_kernel<true, false, true>() : valu_kernel<true, false, false>();
    }
    if (c.stage) return c.g4 ? valu_kernel<false, true, true>() : valu_kernel<false, true, false>();
    return c.g4 ? valu_kernel<false, false, true>() : valu_kernel<false, false, false>();
}

template <bool kF32, bool kStage, bool kG4>
void launch_valu_variant(const DecodeParams& P, dim3 grid, const ValuChoice& c, hipStream_t s,
                         const KernelEvents& ev) {
    hipExtLaunchKernelGGL((decode_valu_kernel<kF32, kStage, kG4>), grid, dim3(kThreads), c.smem, s, ev.start, ev.stop,
                          0, P, c.stage_off);
}

template <bool kF32>
void launch_valu_dtype(const DecodeParams& P, dim3 grid, const ValuChoice& c, hipStream_t s, const KernelEvents& ev) {
    if (c.stage) {
        if (c.g4) launch_valu_variant<kF32, true, true>(P, grid, c, s, ev);
        else launch_valu_variant<kF32, true, false>(P, grid, c, s, ev);
    } else {
        if (c.g4) launch_valu_variant<kF32, false, true>(P, grid, c, s, ev);
        else launch_valu_variant<kF32, false, false>(P, grid, c, s, ev);
    }
}

}  // namespace

// Workgroups of the vector-ALU kernel one CU holds at once for this shape
// (registers of the chosen variant, its LDS), as the runtime reports it;
// looked up once per (variant, LDS size).
int decode_valu_blocks_per_cu(const kpa_dims& d) {
    static std::mutex mu;
    static std::map<std::pair<const void*, size_t>, int> cache;
    const ValuChoice c = valu_choice(d);
    const void* k = valu_kernel_of(c);
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find({k, c.smem});
    if (it != cache.end()) return it->second;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, kThreads, c.smem) != hipSuccess || n <= 0) n = 1;
    cache[{k, c.smem}] = n;
    return n;
}

hipError_t launch_decode_valu(const DecodeParams& P, hipStream_t s, const KernelEvents& ev) {
    dim3 grid(P.n_split, P.n_q, P.batch);
    const ValuChoice c = valu_choice(P.d);
    if (c.f32)
        launch_valu_dtype<true>(P, grid, c, s, ev);
    else
        launch_valu_dtype<false>(P, grid, c, s, ev);
    return hipGetLastError();
}

}  // namespace kpa
