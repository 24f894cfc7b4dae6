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
#include "kpa_common.hpp"

namespace kpa {
namespace {

// One block per (sequence, query, head); threads over the head dimension.
__global__ void __launch_bounds__(256) merge_kernel(DecodeParams P) {
    const int h = P.d.p1 * P.d.p2, dh = P.d.q1 * P.d.q2;
    const int64_t row = blockIdx.x;  // (b, n)
    const int i = blockIdx.y;        // head
    const int S = P.n_split;
    const float* ml = P.part_ml + row * S * h * 2;
    const float* po = P.part_o + row * S * h * dh;

    float M = -INFINITY;
    for (int k = 0; k < S; ++k) M = fmaxf(M, ml[(k * h + i) * 2]);
    float l = 0.f;
    if (M != -INFINITY)
        for (int k = 0; k < S; ++k) {
            const float mk = ml[(k * h + i) * 2];
            if (mk != -INFINITY) l += exp2f(mk - M) * ml[(k * h + i) * 2 + 1];
        }
    const float inv_l = l > 0.f ? 1.f / l : 0.f;
    if (P.lse && threadIdx.x == 0)
        P.lse[row * h + i] = l > 0.f ? (M + log2f(l)) * 0.69314718055994531f : -INFINITY;
    for (int j = threadIdx.x; j < dh; j += blockDim.x) {
        float acc = 0.f;
        if (M != -INFINITY)
            for (int k = 0; k < S; ++k) {
                const float mk = ml[(k * h + i) * 2];
                if (mk != -INFINITY) acc += exp2f(mk - M) * po[((int64_t)k * h + i) * dh + j];
            }
        P.out[(row * h + i) * dh + j] = acc * inv_l;
    }
}

}  // namespace

hipError_t launch_merge(const DecodeParams& P, hipStream_t s) {
    const int h = P.d.p1 * P.d.p2, dh = P.d.q1 * P.d.q2;
    const int threads = dh <= 64 ? 64 : (dh <= 128 ? 128 : 256);
    hipLaunchKernelGGL(merge_kernel, dim3(P.batch * P.n_q, h), dim3(threads), 0, s, P);
    return hipGetLastError();
}

}  // namespace kpa
