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
// One block merges up to kMergeGroup chunks of one (row, head).  With more
// chunks (a long single sequence split over the whole chip) the blocks of a
// (row, head) each write a second-level partial (M_g, L_g, O_g) -- the same
// triple, so the same rule combines them -- and the last block to arrive
// (an arrival counter, cleared by the decode kernel) merges those.
#include "kpa_common.hpp"
#include "kpa_dispatch.hpp"

namespace kpa {
namespace {

constexpr float kLn2 = 0.69314718055994531f;

// Combine n (max, sum) pairs into weights w[k] = 2^(m_k - M) (0 for empty
// chunks); returns M and L = sum_k w_k l_k through LDS.  Block-wide.
__device__ void merge_weights(const float* ml, int stride, int n, float* w, float* red, float& M_out,
                              float& L_out) {
    float m = -INFINITY;
    for (int k = threadIdx.x; k < n; k += blockDim.x) m = fmaxf(m, ml[(int64_t)k * stride]);
    for (int x = 32; x > 0; x >>= 1) m = fmaxf(m, __shfl_xor(m, x));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    float M = -INFINITY;
    for (int k = 0; k < (int)(blockDim.x >> 6); ++k) M = fmaxf(M, red[k]);
    __syncthreads();
    float l = 0.f;
    for (int k = threadIdx.x; k < n; k += blockDim.x) {
        const float mk = ml[(int64_t)k * stride];
        const float wk = (mk == -INFINITY) ? 0.f : exp2f(mk - M);
        w[k] = wk;
        l += wk * ml[(int64_t)k * stride + 1];
    }
    for (int x = 32; x > 0; x >>= 1) l += __shfl_xor(l, x);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = l;
    __syncthreads();
    float L = 0.f;
    for (int k = 0; k < (int)(blockDim.x >> 6); ++k) L += red[k];
    M_out = M;
    L_out = L;
    __syncthreads();
}

// sum_k w[k] * o[k * stride + j] with several loads in flight.
__device__ __forceinline__ float weighted_sum(const float* w, const float* o, int64_t stride, int n) {
    float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
    int k = 0;
    for (; k + 4 <= n; k += 4) {
        acc0 += w[k] * o[k * stride];
        acc1 += w[k + 1] * o[(k + 1) * stride];
        acc2 += w[k + 2] * o[(k + 2) * stride];
        acc3 += w[k + 3] * o[(k + 3) * stride];
    }
    for (; k < n; ++k) acc0 += w[k] * o[k * stride];
    return (acc0 + acc1) + (acc2 + acc3);
}

__global__ void __launch_bounds__(256) merge_kernel(DecodeParams P) {
    __shared__ float w[kMergeGroup];
    __shared__ float red[4];
    __shared__ int is_last;
    extern __shared__ float w2[];  // [n_group] second-level weights
    const int h = P.d.p1 * P.d.p2, dh = P.d.q1 * P.d.q2;
    const int64_t row = blockIdx.x / h;  // (b, n)
    const int i = blockIdx.x % h;
    const int g = blockIdx.y;
    const int S = P.n_split, G = P.n_group;
    const int k0 = g * kMergeGroup;
    const int n = min(S - k0, kMergeGroup);

    const float* ml = P.part_ml + ((row * S + k0) * h + i) * 2;
    const float* po = P.part_o + ((row * S + k0) * h + i) * (int64_t)dh;
    float M, L;
    merge_weights(ml, h * 2, n, w, red, M, L);
    float acc[2];
    int nj = 0;
    for (int j = threadIdx.x; j < dh; j += blockDim.x) acc[nj++] = weighted_sum(w, po + j, (int64_t)h * dh, n);

    if (G == 1) {
        const float inv = L > 0.f ? 1.f / L : 0.f;
        nj = 0;
        for (int j = threadIdx.x; j < dh; j += blockDim.x) P.out[(row * h + i) * dh + j] = acc[nj++] * inv;
        if (P.lse && threadIdx.x == 0) P.lse[row * h + i] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
        return;
    }

    // second level: publish this group's triple, the last block merges all groups
    const int64_t prow = (row * G + g) * h + i;
    nj = 0;
    for (int j = threadIdx.x; j < dh; j += blockDim.x) P.part2_o[prow * dh + j] = acc[nj++];
    if (threadIdx.x == 0) {
        P.part2_ml[prow * 2] = M;
        P.part2_ml[prow * 2 + 1] = L;
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) is_last = atomicAdd(&P.merge_count[row * h + i], 1u) == (uint32_t)(G - 1);
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    const float* ml2 = P.part2_ml + (row * G * h + i) * 2;
    const float* po2 = P.part2_o + (row * G * h + i) * (int64_t)dh;
    merge_weights(ml2, h * 2, G, w2, red, M, L);
    const float inv = L > 0.f ? 1.f / L : 0.f;
    for (int j = threadIdx.x; j < dh; j += blockDim.x)
        P.out[(row * h + i) * dh + j] = weighted_sum(w2, po2 + j, (int64_t)h * dh, G) * inv;
    if (threadIdx.x == 0) {
        if (P.lse) P.lse[row * h + i] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
        P.merge_count[row * h + i] = 0u;
    }
}

}  // namespace

hipError_t launch_merge(const DecodeParams& P, hipStream_t s) {
    const int h = P.d.p1 * P.d.p2, dh = P.d.q1 * P.d.q2;
    const int threads = dh <= 64 ? 64 : (dh <= 128 ? 128 : 256);
    const size_t smem = P.n_group > 1 ? P.n_group * sizeof(float) : 0;
    hipLaunchKernelGGL(merge_kernel, dim3(P.batch * P.n_q * h, P.n_group), dim3(threads), smem, s, P);
    return hipGetLastError();
}

}  // namespace kpa
