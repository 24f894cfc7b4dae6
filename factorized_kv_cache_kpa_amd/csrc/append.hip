// kpa_cache_append kernel: writes new tokens' factors into the tiled cache and
// applies the Kronecker-separable RoPE to B^K once, at write time.
//
// [KPA] "Kronecker Product Attention: Memory-Efficient KV Compression via
//       Structured Factorization": Def. 2.3 (R_KPA = I_{d1} (x) R^(2)),
//       Thm. 2.4 and consequence (i) after it (only B^K is pre-rotated;
//       A^K, A^V, B^V are stored as they are), §2.5 (what the cache holds).
// The rotation pairs consecutive features (2m, 2m+1) of each B row with
// angle pos * theta_m, theta_m = base^(-2m/q2) ("Tensor Product Attention Is
// All You Need", summary page, "RoPE Compatibility and Acceleration").
#include "kpa_common.hpp"

namespace kpa {
namespace {

template <typename T>
__device__ __forceinline__ void store_elem(uint8_t* p, T v) { *reinterpret_cast<T*>(p) = v; }

// One block per (new token n, sequence b).  Threads stride over the token's
// elements; B^K is handled one rotation pair per thread.
template <bool kF32>
__global__ void __launch_bounds__(256) append_kernel(AppendParams P) {
    const int n = blockIdx.x;
    const int b = blockIdx.y;
    const int slot = P.slot0[b] + n;
    const int pos = P.positions[(int64_t)b * P.n_new + n];
    if (slot < 0 || slot >= P.capacity || pos < 0) {
        if (threadIdx.x == 0 && P.dev_status) {
            uint32_t bits = 0;
            if (slot < 0 || slot >= P.capacity) bits |= KPA_DEV_SLOT_OUT_OF_RANGE;
            if (pos < 0) bits |= KPA_DEV_NEGATIVE_POSITION;
            atomicOr(P.dev_status, bits);
        }
        return;
    }
    const Layout& L = P.L;
    const int tile = slot / kTileSlots;
    const int t = slot % kTileSlots;
    uint8_t* tile_base = P.cache + ((int64_t)b * L.n_tiles + tile) * L.tile_bytes;
    const int64_t tok = (int64_t)b * P.n_new + n;
    using E = typename std::conditional<kF32, float, uint16_t>::type;

    // Verbatim copies: A^K (set 0), A^V (set 2), B^V (set 3).
    const void* srcs[4] = {P.a_k, nullptr, P.a_v, P.b_v};
    for (int c = 0; c < 4; ++c) {
        if (c == 1) continue;
        const E* src = reinterpret_cast<const E*>(srcs[c]) + tok * L.elems[c];
        for (int e = threadIdx.x; e < L.elems[c]; e += blockDim.x)
            store_elem<E>(tile_base + elem_offset(L, c, e, t), src[e]);
    }

    // B~^K = R^(2)(pos) B^K row by row, in float64, rounded once.
    const int q2 = P.d.q2;
    const int half = q2 / 2;
    const int pairs = L.elems[1] / 2;
    const E* bk = reinterpret_cast<const E*>(P.b_k) + tok * L.elems[1];
    const double log2_base = log2((double)P.d.rope_base);
    for (int pr = threadIdx.x; pr < pairs; pr += blockDim.x) {
        const int row = pr / half;       // (r, i2)
        const int m = pr % half;         // pair index inside the row
        const int e0 = row * q2 + 2 * m;
        double x0, x1;
        if constexpr (kF32) {
            x0 = bk[e0];
            x1 = bk[e0 + 1];
        } else {
            x0 = bf16_to_f32(bk[e0]);
            x1 = bf16_to_f32(bk[e0 + 1]);
        }
        const double theta = exp2(-(2.0 * m / q2) * log2_base);
        double sn, cs;
        sincos((double)pos * theta, &sn, &cs);
        const double y0 = x0 * cs - x1 * sn;
        const double y1 = x0 * sn + x1 * cs;
        if constexpr (kF32) {
            store_elem<float>(tile_base + elem_offset(L, 1, e0, t), (float)y0);
            store_elem<float>(tile_base + elem_offset(L, 1, e0 + 1, t), (float)y1);
        } else {
            store_elem<uint16_t>(tile_base + elem_offset(L, 1, e0, t), f64_to_bf16_rne(y0));
            store_elem<uint16_t>(tile_base + elem_offset(L, 1, e0 + 1, t), f64_to_bf16_rne(y1));
        }
    }
    if (threadIdx.x == 0) {
        int32_t* positions = reinterpret_cast<int32_t*>(P.cache + L.positions_off);
        positions[(int64_t)b * L.n_tiles * kTileSlots + slot] = pos;
    }
}

}  // namespace

hipError_t launch_append(const AppendParams& P, hipStream_t s) {
    dim3 grid(P.n_new, P.batch);
    if (P.d.dtype == KPA_F32)
        hipLaunchKernelGGL(append_kernel<true>, grid, dim3(256), 0, s, P);
    else
        hipLaunchKernelGGL(append_kernel<false>, grid, dim3(256), 0, s, P);
    return hipGetLastError();
}

}  // namespace kpa
