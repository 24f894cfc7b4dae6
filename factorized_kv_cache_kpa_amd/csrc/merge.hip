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
// (an arrival counter, cleared by the decode kernel) merges those.  The
// planner keeps the chunk count <= kMergeGroup^2.
#include "kpa_common.hpp"
#include "kpa_dispatch.hpp"

namespace kpa {
namespace {

constexpr float kLn2 = 0.69314718055994531f;

// One (row, head) over n <= kMergeGroup chunks, for the thread's output
// element j (j < dh).  Every load -- the chunk maxima, sums and outputs -- is
// issued up front; the weights need only a block-wide max, so the whole merge
// costs one memory round trip.  Returns (M, L) and the unnormalised sum.
struct MergeOut {
    float M, L, acc;
};

__device__ MergeOut merge_group(const float* ml, int ml_stride, const float* o, int64_t o_stride, int n,
                                int j, bool has_j, float* red) {
    float m = -INFINITY, l = 0.f;
    if ((int)threadIdx.x < n) {  // one chunk's (max, sum) per thread
        m = ml[(int64_t)threadIdx.x * ml_stride];
        l = ml[(int64_t)threadIdx.x * ml_stride + 1];
    }
    // block max of the chunk maxima
    float M = m;
    for (int x = 32; x > 0; x >>= 1) M = fmaxf(M, __shfl_xor(M, x));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = M;
    __syncthreads();
    M = -INFINITY;
    for (int k = 0; k < (int)(blockDim.x >> 6); ++k) M = fmaxf(M, red[k]);
    // this thread's chunk weight, the weighted sum of sums, and every weight in LDS
    const float wk = (m == -INFINITY) ? 0.f : exp2f(m - M);
    float L = wk * l;
    for (int x = 32; x > 0; x >>= 1) L += __shfl_xor(L, x);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = L;
    red[4 + threadIdx.x] = wk;  // red[4 .. 4 + blockDim)
    __syncthreads();
    L = 0.f;
    for (int k = 0; k < (int)(blockDim.x >> 6); ++k) L += red[k];
    float acc = 0.f;
    if (has_j) {
        const float* oj = o + j;
        int k = 0;
        for (; k + 8 <= n; k += 8) {  // eight loads in flight
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = oj[(k + u) * o_stride];
#pragma unroll
            for (int u = 0; u < 8; ++u) acc += red[4 + k + u] * v[u];
        }
        for (; k < n; ++k) acc += red[4 + k] * oj[k * o_stride];
    }
    __syncthreads();
    return {M, L, acc};
}

__global__ void __launch_bounds__(256) merge_kernel(DecodeParams P) {
    __shared__ float red[4 + 256];
    __shared__ int is_last;
    const int h = P.d.p1 * P.d.p2, dh = P.d.q1 * P.d.q2;
    const int64_t row = blockIdx.x / h;  // (b, n)
    const int i = blockIdx.x % h;
    const int g = blockIdx.y;
    const int S = P.n_split, G = P.n_group;
    const int k0 = g * kMergeGroup;
    const int n = min(S - k0, kMergeGroup);
    const int j = threadIdx.x;  // blockDim.x >= dh and >= kMergeGroup
    const bool has_j = j < dh;

    MergeOut r = merge_group(P.part_ml + ((row * S + k0) * h + i) * 2, h * 2,
                             P.part_o + ((row * S + k0) * h + i) * (int64_t)dh, (int64_t)h * dh, n, j, has_j, red);
    if (G == 1) {
        const float inv = r.L > 0.f ? 1.f / r.L : 0.f;
        if (has_j) P.out[(row * h + i) * dh + j] = r.acc * inv;
        if (P.lse && threadIdx.x == 0) P.lse[row * h + i] = r.L > 0.f ? (r.M + log2f(r.L)) * kLn2 : -INFINITY;
        return;
    }

    // second level: publish this group's triple, the last block merges all groups
    const int64_t prow = (row * G + g) * h + i;
    if (has_j) P.part2_o[prow * dh + j] = r.acc;
    if (threadIdx.x == 0) {
        P.part2_ml[prow * 2] = r.M;
        P.part2_ml[prow * 2 + 1] = r.L;
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) is_last = atomicAdd(&P.merge_count[row * h + i], 1u) == (uint32_t)(G - 1);
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    // G <= kMergeGroup (the planner caps the chunk count)
    r = merge_group(P.part2_ml + (row * G * h + i) * 2, h * 2, P.part2_o + (row * G * h + i) * (int64_t)dh,
                    (int64_t)h * dh, G, j, has_j, red);
    const float inv = r.L > 0.f ? 1.f / r.L : 0.f;
    if (has_j) P.out[(row * h + i) * dh + j] = r.acc * inv;
    if (threadIdx.x == 0) {
        if (P.lse) P.lse[row * h + i] = r.L > 0.f ? (r.M + log2f(r.L)) * kLn2 : -INFINITY;
        P.merge_count[row * h + i] = 0u;
    }
}

}  // namespace

hipError_t launch_merge(const DecodeParams& P, hipStream_t s) {
    const int h = P.d.p1 * P.d.p2, dh = P.d.q1 * P.d.q2;
    const int threads = dh <= 64 ? 64 : (dh <= 128 ? 128 : 256);  // >= kMergeGroup as well
    hipLaunchKernelGGL(merge_kernel, dim3(P.batch * P.n_q * h, P.n_group), dim3(threads), 0, s, P);
    return hipGetLastError();
}

}  // namespace kpa
