// Log-sum-exp merge of split-KV partial results.
//
// Each chunk k of a (sequence, query) wrote, per head, its running max m_k
// (log2 units), its sum l_k = sum_s 2^(z_s - m_k) and o_k = sum_s
// 2^(z_s - m_k) v_s.  With M = max_k m_k and w_k = 2^(m_k - M):
//   out = sum_k w_k o_k / sum_k w_k l_k,   lse = ln 2 * (M + log2 sum_k w_k l_k).
// This is the exact combination of blocked online softmax (FlashTPA decoding
// blocks over the cache with an online log-sum-exp: "Tensor Product Attention
// Is All You Need", summary page).  Chunks that saw no slot carry m = -inf,
// l = 0 and drop out; if every chunk is empty the output is 0 and lse -inf.
//
// One block merges all chunks of one (row, head) when they fit one pass of a
// block (up to kMaxSingleLevel chunks, 1024 threads for more than
// kMergeGroup).  Otherwise the blocks of a (row, head) each merge kMergeGroup
// chunks and write a second-level partial (M_g, L_g, O_g) -- the same
// triple, so the same rule combines them -- and the last block to arrive
// (an arrival counter, cleared by the decode kernel) merges those.  The
// planner keeps the chunk count <= kMergeGroup^2.
//
// The merge is latency-bound (a few MB at most), so each block makes a single
// memory round trip: every thread issues all of its o loads (vectors of VEC
// floats, one output column block per thread, chunks spread over the block)
// together with the (m, l) loads, and only then waits; the weights need a
// block-wide max, computed while the o loads are in flight.
#include "kpa_common.hpp"
#include "kpa_dispatch.hpp"

namespace kpa {
namespace {

constexpr float kLn2 = 0.69314718055994531f;

template <int VEC>
struct Vec;
template <>
struct Vec<2> {
    using T = float2;
};
template <>
struct Vec<4> {
    using T = float4;
};

template <int VEC>
__device__ __forceinline__ void axpy(float w, const typename Vec<VEC>::T& x, float* acc) {
    acc[0] += w * x.x;
    acc[1] += w * x.y;
    if constexpr (VEC == 4) {
        acc[2] += w * x.z;
        acc[3] += w * x.w;
    }
}

struct MergeOut {
    float M, L;
    float acc[4];  // this thread's VEC output elements (valid for threadIdx.x < d_h / VEC)
};

struct MergeLds {
    float red[16];             // per-wave maxima / sums
    float w[kMaxSingleLevel];  // chunk weights
};

// Merges n <= T chunks of one (row, head) with a block of T
// threads.  ml: chunk k's (m, l) at ml + k * ml_stride; o: chunk k's d_h
// outputs at o + k * o_stride.  Thread t owns column block c = t % CB
// (CB = d_h / VEC) of chunks k = t / CB + u * (T / CB), u < U, issued all at
// once; chunks beyond U passes (only for shapes the launcher did not size U
// for) are added one by one.  The per-thread sums are then added across the
// threads sharing a column block through LDS (part: T * VEC floats).
template <int VEC, int U, int T>
__device__ MergeOut merge_group(const float* ml, int64_t ml_stride, const float* o, int64_t o_stride, int n, int dh,
                                MergeLds& sh, float* part) {
    using V = typename Vec<VEC>::T;
    constexpr int NW = T / 64;
    const int t = threadIdx.x;
    const int CB = dh / VEC;          // column blocks (<= 128)
    const int KL = T / CB;            // chunks per pass
    const int c = t % CB, k0 = t / CB;
    const bool active = k0 < KL;      // T may not be a multiple of CB
    // (m, l) of chunk t, then every o vector of this thread: one round trip
    float m = -INFINITY, l = 0.f;
    if (t < n) {
        m = ml[(int64_t)t * ml_stride];
        l = ml[(int64_t)t * ml_stride + 1];
    }
    V v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int k = k0 + u * KL;
        if (active && k < n) v[u] = *reinterpret_cast<const V*>(o + (int64_t)k * o_stride + c * VEC);
    }
    // block max of the chunk maxima
    float M = m;
    for (int x = 32; x > 0; x >>= 1) M = fmaxf(M, __shfl_xor(M, x));
    if ((t & 63) == 0) sh.red[t >> 6] = M;
    __syncthreads();
    M = sh.red[0];
#pragma unroll
    for (int x = 1; x < NW; ++x) M = fmaxf(M, sh.red[x]);
    const float wk = (m == -INFINITY) ? 0.f : exp2f(m - M);
    float L = wk * l;
    for (int x = 32; x > 0; x >>= 1) L += __shfl_xor(L, x);
    __syncthreads();
    if ((t & 63) == 0) sh.red[t >> 6] = L;
    if (t < n) sh.w[t] = wk;
    __syncthreads();
    L = 0.f;
#pragma unroll
    for (int x = 0; x < NW; ++x) L += sh.red[x];
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int k = k0 + u * KL;
        if (active && k < n) axpy<VEC>(sh.w[k], v[u], acc);
    }
    for (int k = k0 + U * KL; active && k < n; k += KL)
        axpy<VEC>(sh.w[k], *reinterpret_cast<const V*>(o + (int64_t)k * o_stride + c * VEC), acc);
    // add the KL partial sums of each column block
    MergeOut r{M, L, {0.f, 0.f, 0.f, 0.f}};
    if ((CB & (CB - 1)) == 0 && CB <= 64) {
        // CB a power of two: the lanes of a column block sit CB apart in every
        // wave, so the wave adds them with shuffles, then the NW wave sums
        // meet in LDS
        if (!active)
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
        for (int x = CB; x < 64; x <<= 1)
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] += __shfl_xor(acc[e], x);
        if ((t & 63) < CB)
#pragma unroll
            for (int e = 0; e < VEC; ++e) part[((t >> 6) * CB + c) * VEC + e] = acc[e];
        __syncthreads();
        if (t < CB)
            for (int w = 0; w < NW; ++w)
#pragma unroll
                for (int e = 0; e < VEC; ++e) r.acc[e] += part[(w * CB + t) * VEC + e];
    } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) part[t * VEC + e] = acc[e];
        __syncthreads();
        if (t < CB) {
            for (int j = 0; j < KL; ++j)
#pragma unroll
                for (int e = 0; e < VEC; ++e) r.acc[e] += part[(j * CB + t) * VEC + e];
        }
    }
    __syncthreads();  // the LDS is reused by the caller
    return r;
}

template <int VEC>
__device__ __forceinline__ void store_out(float* dst, const MergeOut& r, float scale) {
    using V = typename Vec<VEC>::T;
    V x;
    x.x = r.acc[0] * scale;
    x.y = r.acc[1] * scale;
    if constexpr (VEC == 4) {
        x.z = r.acc[2] * scale;
        x.w = r.acc[3] * scale;
    }
    *reinterpret_cast<V*>(dst) = x;
}

// One block per (row, head, group of chunks) -- or, for a single level, per
// (row, head, slice of the d_h columns): blockIdx.y is the group with a second
// level (n_group > 1), else the column slice (col_split slices; every slice's
// block reads all (m, l) pairs for the weights and merges its own columns, so
// a long chunk list is spread over more blocks).  group_size = n_split for a
// single level, kMergeGroup with a second level.
template <int VEC, int U, int T>
__global__ void __launch_bounds__(T) merge_kernel(DecodeParams P, int group_size, int col_split) {
    __shared__ MergeLds sh;
    __shared__ float part[T * VEC];
    __shared__ int is_last;
    const int h = P.d.p1 * P.d.p2, dh = P.d.q1 * P.d.q2;
    const int64_t row = blockIdx.x / h;  // (b, n)
    const int i = blockIdx.x % h;
    const int S = P.n_split, G = P.n_group;
    const int g = G > 1 ? blockIdx.y : 0;
    const int dh_part = dh / col_split;                   // columns of this block
    const int col0 = G > 1 ? 0 : blockIdx.y * dh_part;    // first column of this block
    const int k0 = g * group_size;
    const int n = min(S - k0, group_size);
    const int t = threadIdx.x;
    const bool has_out = t < dh_part / VEC;

    MergeOut r = merge_group<VEC, U, T>(P.part_ml + ((row * S + k0) * h + i) * 2, (int64_t)h * 2,
                                        P.part_o + ((row * S + k0) * h + i) * (int64_t)dh + col0, (int64_t)h * dh, n,
                                        dh_part, sh, part);
    if (T > 256 || G == 1) {  // the 1024-thread blocks are single-level only
        const float inv = r.L > 0.f ? 1.f / r.L : 0.f;
        if (has_out) store_out<VEC>(P.out + (row * h + i) * dh + col0 + t * VEC, r, inv);
        if (P.lse && t == 0 && col0 == 0) P.lse[row * h + i] = r.L > 0.f ? (r.M + log2f(r.L)) * kLn2 : -INFINITY;
        return;
    }

    // second level: publish this group's triple, the last block merges all groups
    const int64_t prow = (row * G + g) * h + i;
    if (has_out) store_out<VEC>(P.part2_o + prow * dh + t * VEC, r, 1.f);
    if (t == 0) {
        P.part2_ml[prow * 2] = r.M;
        P.part2_ml[prow * 2 + 1] = r.L;
    }
    __threadfence();
    __syncthreads();
    if (t == 0) is_last = atomicAdd(&P.merge_count[row * h + i], 1u) == (uint32_t)(G - 1);
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    // G <= kMergeGroup (the planner caps the chunk count) and T >= kMergeGroup
    r = merge_group<VEC, U, T>(P.part2_ml + (row * G * h + i) * 2, (int64_t)h * 2,
                               P.part2_o + (row * G * h + i) * (int64_t)dh, (int64_t)h * dh, G, dh, sh, part);
    const float inv = r.L > 0.f ? 1.f / r.L : 0.f;
    if (has_out) store_out<VEC>(P.out + (row * h + i) * dh + t * VEC, r, inv);
    if (t == 0) {
        if (P.lse) P.lse[row * h + i] = r.L > 0.f ? (r.M + log2f(r.L)) * kLn2 : -INFINITY;
        P.merge_count[row * h + i] = 0u;
    }
}

template <int VEC, int U, int T>
void launch_one(const DecodeParams& P, int group_size, int col_split, hipStream_t s) {
    const int h = P.d.p1 * P.d.p2;
    const int gy = P.n_group > 1 ? P.n_group : col_split;
    hipLaunchKernelGGL((merge_kernel<VEC, U, T>), dim3(P.batch * P.n_q * h, gy), dim3(T), 0, s, P, group_size,
                       col_split);
}

// Loads per thread: the smallest power of two covering the group's chunks.
template <int VEC, int T>
void launch_u(const DecodeParams& P, int group_size, int col_split, hipStream_t s) {
    const int dh = P.d.q1 * P.d.q2;
    const int KL = T / (dh / col_split / VEC);
    const int need = (group_size + KL - 1) / KL;
    if (need <= 1) launch_one<VEC, 1, T>(P, group_size, col_split, s);
    else if (need <= 2) launch_one<VEC, 2, T>(P, group_size, col_split, s);
    else if (need <= 4) launch_one<VEC, 4, T>(P, group_size, col_split, s);
    else if (need <= 8) launch_one<VEC, 8, T>(P, group_size, col_split, s);
    else launch_one<VEC, 16, T>(P, group_size, col_split, s);
}

// Block size: the smallest of 64 / 128 / 256 threads that covers the group
// with at most 8 loads per thread (fewer threads per output, fewer
// block-wide barriers); 1024 threads for a wide single level, whose columns
// are split over blocks until there are ~256 of them (the block count is
// otherwise rows x heads, 32 for a single long sequence).
template <int VEC>
void launch_vec(const DecodeParams& P, hipStream_t s) {
    const int gs = P.n_group > 1 ? kMergeGroup : P.n_split;  // chunks per block
    if (gs > kMergeGroup) {
        const int64_t blocks = (int64_t)P.batch * P.n_q * P.d.p1 * P.d.p2;
        const int cb = P.d.q1 * P.d.q2 / VEC;  // column blocks of d_h
        int cs = 1;
        while (cb % (2 * cs) == 0 && blocks * cs < 256) cs *= 2;
        return launch_u<VEC, 1024>(P, gs, cs, s);
    }
    const int CB = P.d.q1 * P.d.q2 / VEC;
    auto need = [&](int T) { return T / CB > 0 ? (gs + T / CB - 1) / (T / CB) : 1 << 30; };
    if (need(64) <= 8) return launch_u<VEC, 64>(P, gs, 1, s);
    if (need(128) <= 8) return launch_u<VEC, 128>(P, gs, 1, s);
    return launch_u<VEC, 256>(P, gs, 1, s);
}

}  // namespace

hipError_t launch_merge(const DecodeParams& P, hipStream_t s) {
    // d_h is even (q2 is); float4 vectors when it is a multiple of 4.  The
    // workspace partials start 16-byte aligned and every row of them is d_h
    // floats long, so the vectors are aligned.
    if (P.d.q1 * P.d.q2 % 4 == 0)
        launch_vec<4>(P, s);
    else
        launch_vec<2>(P, s);
    return hipGetLastError();
}

}  // namespace kpa
