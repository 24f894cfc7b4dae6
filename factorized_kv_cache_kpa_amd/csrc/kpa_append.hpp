// Writing one new token into the tiled factor cache, with the
// Kronecker-separable RoPE applied to B^K once, at write time.  Used by the
// append kernel and by the decode kernels' fused append.
//
// [KPA] "Kronecker Product Attention: Memory-Efficient KV Compression via
//       Structured Factorization": Def. 2.3 (R_KPA = I_{d1} (x) R^(2)),
//       Thm. 2.4 and consequence (i) after it (only B^K is pre-rotated;
//       A^K, A^V, B^V are stored as they are), §2.5 (what the cache holds).
// The rotation pairs consecutive features (2m, 2m+1) of each B row with
// angle pos * theta_m, theta_m = base^(-2m/q2) ("Tensor Product Attention Is
// All You Need", summary page, "RoPE Compatibility and Acceleration").
#pragma once

#include <type_traits>

#include "kpa_common.hpp"

namespace kpa {

template <typename T>
__device__ __forceinline__ void store_elem(uint8_t* p, T v) { *reinterpret_cast<T*>(p) = v; }

// The RoPE angle of pair m at position pos, in float64: sin and cos of
// pos * theta_m, theta_m = base^(-2m/q2).
__device__ __forceinline__ void rope_angle(int pos, int m, int q2, double log2_base, double& sn, double& cs) {
    const double theta = exp2(-(2.0 * m / q2) * log2_base);
    sincos((double)pos * theta, &sn, &cs);
}

// (x0, x1) turned by that angle.  Products and sums stay separate roundings
// (no fused multiply-add), so every kernel that rotates gets the same bits.
__device__ __forceinline__ void rope_rotate(double x0, double x1, double sn, double cs, double& y0, double& y1) {
#pragma clang fp contract(off)
    y0 = x0 * cs - x1 * sn;
    y1 = x0 * sn + x1 * cs;
}

// One RoPE pair of a B^K row, in float64: (x0, x1) at features (2m, 2m+1)
// turned by pos * theta_m.
__device__ __forceinline__ void rope_pair(double x0, double x1, int pos, int m, int q2, double log2_base,
                                          double& y0, double& y1) {
    double sn, cs;
    rope_angle(pos, m, q2, log2_base, sn, cs);
    rope_rotate(x0, x1, sn, cs, y0, y1);
}

// Slot of token n of sequence b (may be out of range; the writer checks).
__device__ __forceinline__ int append_slot(const AppendInputs& in, int b, int n) { return slot_add(in.slot0[b], n); }

// Token n of sequence b, written by threads tid = 0 .. nthr - 1 of the
// calling workgroup (elements strided over them; B^K one rotation pair per
// thread).  An out-of-range slot or a negative position skips the token and
// sets the dev_status bits.
template <bool kF32>
__device__ __forceinline__ void append_token(const kpa_dims& d, const Layout& L, uint8_t* cache, int capacity,
                             const AppendInputs& in, uint32_t* dev_status, int b, int n, int tid, int nthr) {
    const int slot = append_slot(in, b, n);
    const int pos = in.positions[(int64_t)b * in.n_new + n];
    if (slot < 0 || slot >= capacity || pos < 0) {
        if (tid == 0 && dev_status) {
            uint32_t bits = 0;
            if (slot < 0 || slot >= capacity) bits |= KPA_DEV_SLOT_OUT_OF_RANGE;
            if (pos < 0) bits |= KPA_DEV_NEGATIVE_POSITION;
            atomicOr(dev_status, bits);
        }
        return;
    }
    const int tile = slot / kTileSlots;
    const int t = slot % kTileSlots;
    uint8_t* tile_base = cache + ((int64_t)b * L.n_tiles + tile) * L.tile_bytes;
    const int64_t tok = (int64_t)b * in.n_new + n;
    using E = typename std::conditional<kF32, float, uint16_t>::type;

    // Verbatim copies: A^K (set 0), A^V (set 2), B^V (set 3).
    auto copy_set = [&](int c, const void* from) {
        const E* src = reinterpret_cast<const E*>(from) + tok * L.elems[c];
        for (int e = tid; e < L.elems[c]; e += nthr) store_elem<E>(tile_base + elem_offset(L, c, e, t), src[e]);
    };
    copy_set(0, in.a_k);
    copy_set(2, in.a_v);
    copy_set(3, in.b_v);

    // B~^K = R^(2)(pos) B^K row by row, in float64, rounded once.
    const int q2 = d.q2;
    const int half = q2 / 2;
    const int pairs = L.elems[1] / 2;
    const E* bk = reinterpret_cast<const E*>(in.b_k) + tok * L.elems[1];
    const double log2_base = log2((double)d.rope_base);
    for (int pr = tid; pr < pairs; pr += nthr) {
        const int row = pr / half;  // (r, i2)
        const int m = pr % half;    // pair index inside the row
        const int e0 = row * q2 + 2 * m;
        double x0, x1;
        if constexpr (kF32) {
            x0 = bk[e0];
            x1 = bk[e0 + 1];
        } else {
            x0 = bf16_to_f32(bk[e0]);
            x1 = bf16_to_f32(bk[e0 + 1]);
        }
        double y0, y1;
        rope_pair(x0, x1, pos, m, q2, log2_base, y0, y1);
        if constexpr (kF32) {
            store_elem<float>(tile_base + elem_offset(L, 1, e0, t), (float)y0);
            store_elem<float>(tile_base + elem_offset(L, 1, e0 + 1, t), (float)y1);
        } else {
            store_elem<uint16_t>(tile_base + elem_offset(L, 1, e0, t), f64_to_bf16_rne(y0));
            store_elem<uint16_t>(tile_base + elem_offset(L, 1, e0 + 1, t), f64_to_bf16_rne(y1));
        }
    }
    if (tid == 0) {
        int32_t* positions = reinterpret_cast<int32_t*>(cache + L.positions_off);
        positions[(int64_t)b * L.n_tiles * kTileSlots + slot] = pos;
    }
}

}  // namespace kpa
